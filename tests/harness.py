"""Shared test plumbing: upload seeded workloads to a DeviceLayer and build
oracle sequences over the same bytes.  Test infrastructure only."""
from __future__ import annotations

import numpy as np

import oracle as O
from workloads import gen as G
from workloads.configs import LayerShape

BF16_TOL = (2e-2, 1e-3)   # (rtol, atol) for bf16 / fp32 outputs
FP8_TOL = (5e-2, 1e-3)    # when the K=V cache is fp8
Q_NORM_FLAG = 64          # ckv_layer_desc.flags bit of the query norm


def device_layer(cfg: LayerShape, weights, cache: G.CacheInit = None, max_chunk: int = 0, batch=None, flags=None):
    from compressed_kv_sparse_amd import DeviceLayer
    dl = DeviceLayer(ratio=cfg.ratio, hidden=cfg.hidden, head_dim=cfg.head_dim, n_heads=cfg.n_heads,
                     batch=cfg.batch if batch is None else batch, idx_heads=cfg.idx_heads, idx_dim=cfg.idx_dim,
                     top_k=cfg.top_k, comp_cap=cfg.comp_cap, kv_fmt=cfg.kv_fmt, idx_fmt=cfg.idx_fmt,
                     act_fmt=cfg.act_fmt, w_fmt=cfg.w_fmt, rope_base=cfg.rope_base, norm_eps=cfg.norm_eps,
                     n_rot=cfg.n_rot, swa=cfg.swa, max_chunk=max_chunk, rope_base_comp=cfg.rope_base_comp or 0.0,
                     flags=cfg.flags if flags is None else flags)
    if weights is not None:
        dl.set_weights(wkv=weights.wkv, wgate=weights.wgate, ape=weights.ape, gamma=weights.gamma,
                       idx_wkv=weights.idx_wkv, idx_wgate=weights.idx_wgate, idx_ape=weights.idx_ape,
                       idx_gamma=weights.idx_gamma)
    if cache is not None:
        dl.load_cache(raw=cache.raw, comp=cache.comp, idx=cache.idx, st_kv=cache.st_kv, st_sc=cache.st_sc,
                      ist_kv=cache.ist_kv, ist_sc=cache.ist_sc, n_tokens=cache.first_live)
    return dl


def dev(a, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def oracle_layer(cfg, weights):
    L = O.layer_from(cfg, weights)
    L.q_norm = bool(cfg.flags & Q_NORM_FLAG)
    return L


def oracle_seq_from_init(L, cache: G.CacheInit, b: int) -> O.OracleSequence:
    """Oracle sequence b starting from the drawn cache (tokens before
    first_live come from the drawn bytes)."""
    return O.OracleSequence(
        L, raw_rec=cache.raw[b], comp_rec=None if cache.comp is None else cache.comp[b],
        idx_vals=None if cache.idx is None else cache.idx[b],
        st_kv=None if cache.st_kv is None else cache.st_kv[b], st_sc=None if cache.st_sc is None else cache.st_sc[b],
        ist_kv=None if cache.ist_kv is None else cache.ist_kv[b],
        ist_sc=None if cache.ist_sc is None else cache.ist_sc[b], first_live=int(cache.first_live[b]))


def oracle_seq_from_bytes(L, raw, comp, idx, live_from: int) -> O.OracleSequence:
    """Oracle sequence that reads every row from the given stored bytes
    (nothing is computed: no token is live before ``live_from``)."""
    return O.OracleSequence(L, raw_rec=raw, comp_rec=comp, idx_vals=idx, first_live=live_from)


def close(gpu, ref, tol, what=""):
    """|g - o| <= atol + rtol |o| element-wise; returns (ok, max_abs, max_rel)."""
    rtol, atol = tol
    g = np.asarray(gpu, np.float64)
    o = np.asarray(ref, np.float64)
    err = np.abs(g - o)
    ok = bool(np.all(err <= atol + rtol * np.abs(o)))
    rel = float(np.max(err / np.maximum(np.abs(o), 1e-30))) if err.size else 0.0
    return ok, float(err.max() if err.size else 0.0), rel


def assert_close(gpu, ref, tol, what=""):
    ok, ma, mr = close(gpu, ref, tol)
    if not ok:
        g = np.asarray(gpu, np.float64)
        o = np.asarray(ref, np.float64)
        bad = np.abs(g - o) > tol[1] + tol[0] * np.abs(o)
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside tol {tol}; max abs {ma:.3g}; "
                             f"first {idx.tolist()} gpu {g[bad][:5]} ref {o[bad][:5]}")


def e4m3_ordinal(c):
    c = np.asarray(c).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def compare_rows(gpu_rec, ref_z, fmt, d, n_rot, what):
    """Stored row(s) from the GPU vs the oracle's pre-cast values.  f32 / bf16:
    tolerance on values.  e4m3: codes within one step of the oracle's own
    encoding, tail within tolerance, scale within 1e-5."""
    gpu_rec = np.asarray(gpu_rec, np.uint8)
    ref_z = np.atleast_2d(np.asarray(ref_z, np.float64))
    gpu_rec = gpu_rec.reshape(ref_z.shape[0], -1)
    if fmt in ("f32", "bf16"):
        assert_close(O.decode_rows(gpu_rec, fmt, d, n_rot), ref_z, BF16_TOL, what)
        return
    dn = d - n_rot
    for n in range(ref_z.shape[0]):
        rec, _ = O.encode_row(ref_z[n], "e4m3", d, n_rot)
        dist = np.abs(e4m3_ordinal(gpu_rec[n, :dn]) - e4m3_ordinal(rec[:dn]))
        assert dist.max() <= 1, f"{what} row {n}: fp8 code distance {dist.max()}"
        gs = gpu_rec[n, dn + 2 * n_rot:dn + 2 * n_rot + 4].copy().view(np.float32)[0]
        rs = rec[dn + 2 * n_rot:dn + 2 * n_rot + 4].copy().view(np.float32)[0]
        assert abs(gs - rs) <= 1e-5 * abs(rs), f"{what} row {n}: scale {gs} vs {rs}"
        gt = O.bf16_decode(gpu_rec[n, dn:dn + 2 * n_rot].copy().view(np.uint16))
        assert_close(gt, ref_z[n, dn:], BF16_TOL, f"{what} row {n} tail")


FP4_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])   # E2M1 rounding boundaries
FP4_T_MARGIN = 2e-5    # distance (in units of the block scale) taken as a possible rounding flip
FP4_E_MARGIN = 1e-5    # relative distance of a block max from a power of two


def fp4_ordinal(codes):
    c = np.asarray(codes).astype(np.int64)
    return np.where(c & 8, -(c & 7), c & 7)


def fp4_unpack(rec, n):
    rec = np.asarray(rec, np.uint8)
    codes = np.empty(rec.shape[:-1] + (n,), np.uint8)
    codes[..., 0::2] = rec[..., :n // 2] & 15
    codes[..., 1::2] = rec[..., :n // 2] >> 4
    return codes, rec[..., n // 2:n // 2 + n // 32].astype(np.int64) - 127


def fp4_fragile(h):
    """Per value of Hadamard-domain vectors h [..., n]: True where a float32
    computation of h could round to another MXFP4 code than fp64 does (the
    scaled value lies within FP4_T_MARGIN of a rounding boundary, or its
    block's max lies within FP4_E_MARGIN of a power of two)."""
    h = np.asarray(h, np.float64)
    blk = h.reshape(h.shape[:-1] + (h.shape[-1] // 32, 32))
    amax = np.abs(blk).max(-1)
    with np.errstate(divide="ignore"):
        lg = np.log2(np.where(amax > 0, amax, 1.0))
    near_pow2 = (amax > 0) & (np.abs(lg - np.round(lg)) < FP4_E_MARGIN)
    e = np.where(amax > 0, np.floor(lg) - 2, -127)
    t = np.abs(blk) / np.ldexp(1.0, e.astype(np.int64))[..., None]
    near_mid = np.min(np.abs(t[..., None] - FP4_MIDPOINTS), axis=-1) < FP4_T_MARGIN
    return (near_mid | near_pow2[..., None]).reshape(h.shape)


def compare_fp4_rows(gpu_rec, pre, what):
    """GPU fp4 indexer records vs the oracle's pre-rounding (Hadamard-domain)
    values: block scales and codes equal to the oracle's own encoding, except
    where fp4_fragile marks the value, where the neighbouring code (and for a
    block max at a power of two, the neighbouring scale) is accepted."""
    pre = np.atleast_2d(np.asarray(pre, np.float64))
    n = pre.shape[-1]
    gpu_rec = np.asarray(gpu_rec, np.uint8).reshape(pre.shape[0], -1)
    ref_rec = O.fp4_encode_rows(pre)
    cg, eg = fp4_unpack(gpu_rec, n)
    cr, er = fp4_unpack(ref_rec, n)
    frag = fp4_fragile(pre)
    blk_frag = frag.reshape(pre.shape[0], n // 32, 32).any(-1)
    bad_e = (eg != er) & ~((np.abs(eg - er) == 1) & blk_frag)
    assert not bad_e.any(), f"{what}: block scale differs at {np.argwhere(bad_e)[:5].tolist()}"
    same_e = np.repeat(eg == er, 32, axis=-1)
    dist = np.abs(fp4_ordinal(cg) - fp4_ordinal(cr))
    bad = same_e & (dist > 0) & ~((dist == 1) & frag)
    assert not bad.any(), (f"{what}: {int(bad.sum())} fp4 codes differ (first {np.argwhere(bad)[:5].tolist()})")


def fp4_query_fragile(L, p, qI):
    """True when the indexer query's MXFP4 codes at position p could differ
    between a float32 and an fp64 computation (see fp4_fragile)."""
    qh = L.rope(O.decode_values(qI, L.act_fmt), p, L.base_comp, min(L.n_rot, L.idx_dim))
    return bool(fp4_fragile(O.hadamard(qh)).any())


def topk_margin(scores: np.ndarray, k: int) -> float:
    """Gap between the k-th and (k+1)-th largest score, relative to max|s|
    (inf when every row is selected)."""
    if len(scores) <= k:
        return np.inf
    s = np.sort(scores)[::-1]
    return float((s[k - 1] - s[k]) / max(np.max(np.abs(s)), 1e-30))


def sets_equal(gpu_topk: np.ndarray, ref_topk: np.ndarray) -> bool:
    return np.array_equal(np.sort(gpu_topk), np.sort(ref_topk))


def tie_free_queries(cfg, seqs, pos, qI, w, attempts=40, margin=1e-4):
    """Redraw q^I / w of any query whose oracle score gap at the k boundary is
    below ``margin``, or (fp4 indexer) whose MXFP4 codes are fragile (same
    generator, sub-seed per query and attempt)."""
    qI, w = qI.copy(), w.copy()
    for b, seq in enumerate(seqs):
        for a in range(attempts):
            if not (cfg.idx_fmt == "fp4" and fp4_query_fragile(seq.L, int(pos[b]), qI[b])):
                sc = seq.index_scores(int(pos[b]), qI[b], w[b])
                if topk_margin(sc, cfg.top_k) > margin:
                    break
            nq, nw = G.draw_query_index(cfg, 1, sub=b, attempt=a + 1)
            qI[b], w[b] = nq[0], nw[0]
        else:
            raise AssertionError(f"no tie-free indexer query for sequence {b}")
    return qI, w


def compare_out_fp8(rec_gpu, o_ref, rtol, what, atol=1e-3):
    """fp8 attention-output records (CKV_FLAG_OUT_FP8) [H, d + 4 d/128] vs the
    oracle's output o_ref [H, d] (pre-cast): every group's scale within rtol of
    the oracle's max|o| / 448 and its largest code at 448 (or an all-zero
    group with scale 1); decoded values within the attention tolerance plus
    half an E4M3 step (2^-4 relative, 2^-10 of the scale below the normal
    range)."""
    o_ref = np.atleast_2d(np.asarray(o_ref, np.float64))
    H, d = o_ref.shape
    ng = d // 128
    rec = np.asarray(rec_gpu, np.uint8).reshape(H, d + 4 * ng)
    ref_rec, _ = O.encode_out_fp8(o_ref)
    sg = rec[:, d:].copy().view(np.float32).reshape(H, ng).astype(np.float64)
    sr = ref_rec[:, d:].copy().view(np.float32).reshape(H, ng).astype(np.float64)
    assert np.all(np.abs(sg - sr) <= rtol * sr + atol / 448.0), f"{what}: group scales {sg.ravel()[:4]} vs {sr.ravel()[:4]}"
    mag = (rec[:, :d] & 0x7F).reshape(H, ng, 128).max(axis=-1)
    assert np.all((mag == 0x7E) | ((mag == 0) & (sg == 1.0))), f"{what}: a group's largest code is not 448"
    deq = O.decode_out_fp8(rec, d)
    bound = (atol + (rtol + 2.0 ** -4 * (1 + rtol)) * np.abs(o_ref)
             + np.repeat(2.0 ** -10 * sg, 128, axis=1)) * 1.01
    bad = np.abs(deq - o_ref) > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} fp8 outputs outside; first {np.argwhere(bad)[:3].tolist()} "
                           f"gpu {deq[bad][:3]} ref {o_ref[bad][:3]}")
