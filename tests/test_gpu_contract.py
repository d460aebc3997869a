"""GPU tests of the library's contract beyond plain parity: the sequence
check on the token counts, one RoPE base per row class on the MFMA path, and
the fp16 range guard of the attention tiles.  Every call goes through the C
ABI; expected values come from the CPU oracle.
"""
import numpy as np
import pytest

import oracle as O
from harness import (BF16_TOL, assert_close, dev, device_layer, oracle_layer, oracle_seq_from_bytes,
                     oracle_seq_from_init, sets_equal, topk_margin)
from test_gpu_parity import cpu, log, out_values, run_decode_stage_checks, run_decode_step_checks
from workloads import get_config, make_decode_inputs, make_layer_weights, make_prefill_inputs
from workloads import gen as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_kv_sparse_amd  # noqa: F401


# ---------------------------------------------------------------------------
# sequence contract (cache->n_tokens)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("api", ["calls", "step"])
def test_out_of_step_positions_are_refused_per_sequence(api):
    """Sequences hold n_b tokens.  One step appends at n_0 (next), n_1 + 1 (a
    token skipped), n_2 (next) and n_3 - 2 (behind): sequences 1 and 3 get the
    sequence status bit and keep every cache byte and their count; 0 and 2 are
    stored and advance.  The same step again is a re-run of the last position
    for 0 and 2 (accepted, same bytes) and still refused for 1 and 3."""
    from compressed_kv_sparse_amd import _lib as L
    cfg = get_config("c2").with_(batch=4, comp_cap=256, top_k=16, seed=61, name=f"seq_{api}")
    n = np.array([100, 200, 300, 400])
    inp = make_decode_inputs(cfg, n_ctx=n)
    wts = make_layer_weights(cfg)
    dl = device_layer(cfg, wts, inp.cache)
    assert list(cpu(dl.n_tokens)) == list(inp.pos)
    pos = inp.pos.copy()
    pos[1] += 1
    pos[3] -= 2
    before = {k: cpu(getattr(dl, k)).copy() for k in ("raw", "comp", "idx", "st_kv", "st_sc")}
    x, u, q, qI, w = dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w)
    for rep in range(2):
        if api == "calls":
            dl.compress_decode(x, u, dev(pos))
        else:
            dl.decode_step(x, u, q, qI, w, dev(pos))
        torch.cuda.synchronize()
        st = cpu(dl.status)
        log(f"[seq {api}] rep {rep} status {st} n_tokens {cpu(dl.n_tokens)}")
        assert st[0] == 0 and st[2] == 0
        assert st[1] & L.CKV_STATUS_SEQUENCE and st[3] & L.CKV_STATUS_SEQUENCE
        assert list(cpu(dl.n_tokens)) == [pos[0] + 1, inp.pos[1], pos[2] + 1, inp.pos[3]]
        after = {k: cpu(getattr(dl, k)) for k in before}
        for k in before:
            for b in (1, 3):
                np.testing.assert_array_equal(after[k][b], before[k][b], err_msg=f"{k} of sequence {b}")
        for b in (0, 2):
            assert not np.array_equal(after["raw"][b], before["raw"][b])
        if rep == 0:
            first = {k: v.copy() for k, v in after.items()}
        else:
            for k in first:
                np.testing.assert_array_equal(after[k], first[k], err_msg=f"re-run changed {k}")


def test_prefill_out_of_sequence_leaves_the_cache():
    """A chunk whose pos0 is not the sequence's count: no cache byte changes,
    the count stays, the status bit is set; the chunk at the right pos0 then
    runs and advances the count by T."""
    from compressed_kv_sparse_amd import _lib as L
    cfg = get_config("c2").with_(batch=1, comp_cap=1024, top_k=64, idx_heads=8, seed=62, name="seq_prefill")
    inp = make_prefill_inputs(cfg, pos0=1000, T=100)
    wts = make_layer_weights(cfg)
    dl = device_layer(cfg, wts, inp.cache, max_chunk=100)
    before = {k: cpu(getattr(dl, k)).copy() for k in ("raw", "comp", "idx", "st_kv", "st_sc")}
    args = (dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w))
    dl.prefill(0, 1004, *args)
    torch.cuda.synchronize()
    assert cpu(dl.status)[0] & L.CKV_STATUS_SEQUENCE
    assert cpu(dl.n_tokens)[0] == 1000
    for k in before:
        np.testing.assert_array_equal(cpu(getattr(dl, k)), before[k], err_msg=k)
    dl.status.zero_()
    dl.prefill(0, 1000, *args)
    torch.cuda.synchronize()
    assert cpu(dl.status)[0] == 0 and cpu(dl.n_tokens)[0] == 1100
    # the host mirror refuses before any work
    dl.set_host_tokens(np.array([1100], np.int32))
    with pytest.raises(L.CkvError) as e:
        dl.prefill(0, 1000, *args)
    assert e.value.code == L.CKV_E_SEQUENCE


# ---------------------------------------------------------------------------
# one RoPE base per row class on the MFMA path
# ---------------------------------------------------------------------------

def _two_base_cfg(name, **kw):
    return get_config("c2").with_(rope_base=10000.0, rope_base_comp=160000.0, name=name, **kw)


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_two_bases_decode_on_the_tile_path(fmt):
    """Raw rows at base 10000, compressed and indexer rows at 160000: the
    compressor, the indexer and the tiled attention (query rotated per class,
    the output's two shares rotated back each in its frame) against the
    oracle, with short contexts (no compressed rows, a split holding both
    classes) and long ones, through the stage calls and the fused step."""
    cfg = _two_base_cfg(f"two_bases_{fmt}", batch=6, comp_cap=1024, top_k=64, kv_fmt=fmt, seed=63)
    n = np.array([1, 4, 100, 131, 1027, 4096], np.int64)
    inp = make_decode_inputs(cfg, n_ctx=n)
    wts = make_layer_weights(cfg)
    tol = (5e-2, 1e-3) if fmt == "e4m3" else BF16_TOL
    run_decode_stage_checks(cfg, inp, wts, tol)
    run_decode_step_checks(cfg, inp, wts, tol)


def test_two_bases_prefill_chunk():
    """A 600-token chunk at an unaligned position with the two bases: every
    emitted row, and sampled queries' top-k sets and outputs."""
    cfg = _two_base_cfg("two_bases_prefill", batch=1, comp_cap=1024, top_k=64, idx_heads=8, seed=64)
    _prefill_sampled(cfg, pos0=501, T=600)


def _prefill_sampled(cfg, pos0, T, sample=None, margin=1e-4):
    """Prefill one chunk from a drawn cache; stored rows, state and raw ring
    compared with the oracle's history run, sampled queries' top-k (on the
    GPU's index bytes) and outputs (with the GPU's lists)."""
    wts = make_layer_weights(cfg)
    inp = make_prefill_inputs(cfg, pos0=pos0, T=T)
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, inp.cache, 0)
    seq.feed(pos0, inp.x, inp.u)
    sample = sorted(set(sample or {0, 1, 2, 3, 63, 64, T // 2, T - 2, T - 1}) & set(range(T)))
    qI, w = (inp.qI.copy(), inp.w.copy()) if cfg.ratio == 4 else (None, None)
    if cfg.ratio == 4:
        for n_ in sample:
            for a in range(40):
                if topk_margin(seq.index_scores(pos0 + n_, qI[n_], w[n_]), cfg.top_k) > margin:
                    break
                nq, nw = G.draw_query_index(cfg, 1, sub=7000 + n_, attempt=a + 1)
                qI[n_], w[n_] = nq[0], nw[0]
    dl = device_layer(cfg, wts, inp.cache, max_chunk=T)
    out, tk = dl.prefill(0, pos0, dev(inp.x), dev(inp.u), dev(inp.q), None if qI is None else dev(qI),
                         None if w is None else dev(w))
    torch.cuda.synchronize()
    assert cpu(dl.status)[0] == 0 and cpu(dl.n_tokens)[0] == pos0 + T
    _check_chunk_state(cfg, dl, seq, pos0, T)
    og = out_values(out, cfg.act_fmt)
    tkg = cpu(tk) if tk is not None else None
    comp_g = cpu(dl.comp)[0] if dl.comp is not None else None
    idx_g = cpu(dl.idx)[0] if dl.idx is not None else None
    bseq = oracle_seq_from_bytes(L, None, comp_g, idx_g, 0)
    cb = chunk_bytes(dl)
    tol = (5e-2, 1e-3) if cfg.kv_fmt == "e4m3" else BF16_TOL
    for n_ in sample:
        p = pos0 + n_
        if cfg.ratio == 4:
            sc = bseq.index_scores(p, qI[n_], w[n_])
            assert sets_equal(tkg[n_], O.topk_select(sc, cfg.top_k)), f"top-k of query {n_}"
        # attention on the GPU's bytes (fp8 rows: one code step is 2^-3 relative,
        # so only identical bytes compare within the fp8 bar); bf16 / f32 rows
        # also on the oracle's own rows
        sel = None if tkg is None else tkg[n_]
        ref = gpu_bytes_seq(L, cfg, cb, p, pos0).attend(p, inp.q[n_], sel)
        assert_close(og[n_], ref, tol, f"{cfg.name} output of query {n_} (p={p}), GPU bytes")
        if cfg.kv_fmt != "e4m3":
            ref = seq.attend(p, inp.q[n_], sel)
            assert_close(og[n_], ref, tol, f"{cfg.name} output of query {n_} (p={p}), oracle rows")
    return dl, seq


def chunk_bytes(dl):
    """Host copies of what a chunk's attention read: (stage, comp, idx)."""
    return (cpu(dl.stage), cpu(dl.comp)[0] if dl.comp is not None else None,
            cpu(dl.idx)[0] if dl.idx is not None else None)


def gpu_bytes_seq(L, cfg, cb, p, pos0):
    """Oracle sequence over exactly the bytes the GPU attends at query p of a
    chunk starting at pos0: its window rows from the staging rows (ring slot
    t % swa), its compressed and indexer rows from the caches (cb from
    chunk_bytes)."""
    stage, comp, idx = cb
    ring = np.zeros((cfg.swa, stage.shape[1]), np.uint8)
    for t in range(max(0, p - cfg.swa + 1), p + 1):
        ring[t % cfg.swa] = stage[t - pos0 + cfg.swa - 1]
    return oracle_seq_from_bytes(L, ring, comp, idx, p + 1)


def _check_chunk_state(cfg, dl, seq, pos0, T):
    """Rows the chunk emitted, the compressor window state and the raw ring
    after the chunk, against the oracle's history."""
    from harness import compare_rows
    d, r = cfg.head_dim, cfg.ratio
    end = pos0 + T
    raw_g = cpu(dl.raw)[0]
    for t in range(max(0, end - cfg.swa), end):
        if seq.is_live(t):
            compare_rows(raw_g[t % cfg.swa], seq.raw_row(t)[0], cfg.kv_fmt, d, cfg.n_rot, f"raw ring t={t}")
        else:   # a row from before the first chunk stays as it was stored
            np.testing.assert_array_equal(raw_g[t % cfg.swa], seq.raw_rec[t % cfg.swa], err_msg=f"raw ring t={t}")
    if not r:
        return
    comp_g = cpu(dl.comp)[0]
    for i in range(pos0 // r, end // r):
        compare_rows(comp_g[i], seq.comp_row(i)[0], cfg.kv_fmt, d, cfg.n_rot, f"comp row {i}")
        if r == 4:
            assert_close(O.decode_values(cpu(dl.idx)[0][i], cfg.idx_fmt), seq.idx_row(i)[0], BF16_TOL,
                         f"idx row {i}")
    W = cfg.window
    st_kv, st_sc = cpu(dl.st_kv)[0], cpu(dl.st_sc)[0]
    for t in range(max(0, end - W), end):
        assert_close(st_kv[t % W], seq.kap[t], (1e-4, 1e-5), f"state kappa t={t}")
        assert_close(st_sc[t % W], seq.sig[t], (1e-4, 1e-5), f"state sigma t={t}")
    if r == 4:
        ist_kv = cpu(dl.ist_kv)[0]
        for t in range(max(0, end - 8), end):
            assert_close(ist_kv[t % 8], seq.ikap[t], (1e-4, 1e-5), f"indexer state t={t}")


# ---------------------------------------------------------------------------
# fp16 range guard of the attention tiles
# ---------------------------------------------------------------------------

def _scale_bf16_rows(rec, rows, factor):
    """Multiply stored bf16 rows (uint8 records) by ``factor`` (input
    preparation: float32 product, high half kept)."""
    v = rec[rows].copy().view(np.uint16).astype(np.uint32) << 16
    f = (v.view(np.float32) * np.float32(factor)).astype(np.float32)
    rec[rows] = G.bf16_bits_of_draw(f).view(np.uint8).reshape(rec[rows].shape)


def test_attention_range_guard_decode():
    """bf16 rows and queries far outside fp16 (1e5) and far below its normal
    range (1e-6): the tiled attention with its guard against the oracle, with
    each sequence's split partials merged."""
    cfg = get_config("c2").with_(batch=4, comp_cap=512, top_k=64, seed=71, name="range_decode")
    n = np.array([2000, 1500, 700, 2048], np.int64)
    inp = make_decode_inputs(cfg, n_ctx=n)
    c = inp.cache
    rng = np.random.default_rng(5)
    for b in range(cfg.batch):
        big = rng.choice(cfg.swa, 3, replace=False)
        _scale_bf16_rows(c.raw[b], big, 1e5)
        _scale_bf16_rows(c.comp[b], rng.choice(int(c.n_drawn_comp[b]), 40, replace=False), 1e5)
        _scale_bf16_rows(c.comp[b], rng.choice(int(c.n_drawn_comp[b]), 40, replace=False), 1e-6)
    q = inp.q.copy()
    qf = (q.astype(np.uint32) << 16).view(np.float32).copy()
    qf[0, 3] *= 1e5                 # one head of sequence 0 far above fp16
    qf[1] *= 1e-6                   # every head of sequence 1 tiny
    qf[2, :, -64:] *= 1e5           # the RoPE tail of sequence 2's heads
    q = G.bf16_bits_of_draw(qf)
    wts = make_layer_weights(cfg)
    dl = device_layer(cfg, wts, c)
    L = oracle_layer(cfg, wts)
    tk = np.full((cfg.batch, cfg.top_k), -1, np.int32)
    for b in range(cfg.batch):
        V = (int(inp.pos[b]) + 1) // 4
        tk[b] = np.sort(rng.choice(V, cfg.top_k, replace=False))
    out = dl.new_out(cfg.batch)
    dl.attn_decode(dev(q), dev(inp.pos), dev(tk), out)
    torch.cuda.synchronize()
    og = out_values(out, cfg.act_fmt)
    assert np.all(np.isfinite(og))
    raw_g, comp_g = cpu(dl.raw), cpu(dl.comp)
    for b in range(cfg.batch):
        p = int(inp.pos[b])
        seq = oracle_seq_from_bytes(L, raw_g[b], comp_g[b], None, p + 1)
        ref = seq.attend(p, q[b], tk[b])
        assert_close(og[b], ref, BF16_TOL, f"guarded output b={b}")


def test_attention_range_guard_prefill():
    """The same guard on a single-split prefill (c128a, every visible row
    attended): drawn rows at 1e5 and 1e-6, and chunk tokens whose raw rows
    reach 1e5."""
    cfg = get_config("c3").with_(batch=1, comp_cap=64, seed=72, ctx_range=None, name="range_prefill")
    pos0, T = 4000, 96
    inp = make_prefill_inputs(cfg, pos0=pos0, T=T)
    c = inp.cache
    rng = np.random.default_rng(6)
    nd = int(c.n_drawn_comp[0])
    _scale_bf16_rows(c.comp[0], rng.choice(nd, 4, replace=False), 1e5)
    _scale_bf16_rows(c.comp[0], rng.choice(nd, 4, replace=False), 1e-6)
    uf = (inp.u.astype(np.uint32) << 16).view(np.float32).copy()
    uf[[5, 40]] *= 1e5
    u = G.bf16_bits_of_draw(uf)
    wts = make_layer_weights(cfg)
    dl = device_layer(cfg, wts, c, max_chunk=T)
    out, _ = dl.prefill(0, pos0, dev(inp.x), dev(u), dev(inp.q))
    torch.cuda.synchronize()
    og = out_values(out, cfg.act_fmt)
    assert np.all(np.isfinite(og))
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, c, 0)
    seq.feed(pos0, inp.x, u)
    for n_ in (0, 4, 5, 6, 39, 40, 41, 95):
        ref = seq.attend(pos0 + n_, inp.q[n_], None)
        assert_close(og[n_], ref, BF16_TOL, f"guarded prefill output {n_}")


# ---------------------------------------------------------------------------
# debug stage skips (desc.flags)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("which", ["norm", "rope", "both"])
def test_debug_stage_skips_decode_and_prefill(which):
    """C1 (f32) with the boundary's SKIP_NORM / SKIP_ROPE against the oracle
    with the same skips: 300 compress_append steps from token 0 (every stored
    row compared), index + attend at the last token; then the same tokens
    prefilled in chunks of 150 + 150 on a fresh layer, with top-k sets and
    outputs of sampled queries compared."""
    from harness import compare_rows, tie_free_queries
    from compressed_kv_sparse_amd import _lib as L
    fl = {"norm": L.CKV_FLAG_SKIP_NORM, "rope": L.CKV_FLAG_SKIP_ROPE,
          "both": L.CKV_FLAG_SKIP_NORM | L.CKV_FLAG_SKIP_ROPE}[which]
    cfg = get_config("c1")
    wts = make_layer_weights(cfg)
    T = 300
    x, u, q, qI, w = G.make_token_stream(cfg, T)
    Lo = oracle_layer(cfg, wts)
    Lo.skip_norm = bool(fl & L.CKV_FLAG_SKIP_NORM)
    Lo.skip_rope = bool(fl & L.CKV_FLAG_SKIP_ROPE)
    seq = O.OracleSequence(Lo)
    seq.feed(0, x, u)
    dl = device_layer(cfg, wts, flags=fl)
    xd, ud = dev(x), dev(u)
    for p in range(T):
        dl.compress_decode(xd[p:p + 1], ud[p:p + 1], dev(np.array([p], np.int32)), B=1)
    torch.cuda.synchronize()
    comp_g, idx_g, raw_g = cpu(dl.comp)[0], cpu(dl.idx)[0], cpu(dl.raw)[0]
    for i in range(T // 4):
        compare_rows(comp_g[i], seq.comp_row(i)[0], "f32", cfg.head_dim, cfg.n_rot, f"[{which}] comp row {i}")
        assert_close(idx_g[i], seq.idx_row(i)[0], BF16_TOL, f"[{which}] idx row {i}")
    for t in range(T - 128, T):
        compare_rows(raw_g[t % 128], seq.raw_row(t)[0], "f32", cfg.head_dim, cfg.n_rot, f"[{which}] raw {t}")
    p = T - 1
    qI1, w1 = tie_free_queries(cfg, [seq], [p], qI[p:p + 1], w[p:p + 1])
    pos_d = dev(np.array([p], np.int32))
    topk_d = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda")
    dl.indexer_decode(dev(qI1), dev(w1), pos_d, topk_d, B=1)
    out = dl.new_out(1)
    dl.attn_decode(dev(q[p:p + 1]), pos_d, topk_d, out, B=1)
    torch.cuda.synchronize()
    ref = seq.query(p, q[p], qI1[0], w1[0])
    assert sets_equal(cpu(topk_d)[0], ref["topk"])
    assert_close(cpu(out)[0], ref["out_f64"], BF16_TOL, f"[{which}] decode output")
    log(f"[skips {which}] decode rows, top-k and output match")

    qI2, w2 = qI.copy(), w.copy()
    want = [0, 1, 3, 99, 149, 150, 151, 203, 255, 299]
    for n in want:
        for a in range(40):
            if topk_margin(seq.index_scores(n, qI2[n], w2[n]), cfg.top_k) > 1e-4:
                break
            nq, nw = G.draw_query_index(cfg, 1, sub=7000 + n, attempt=a + 1)
            qI2[n], w2[n] = nq[0], nw[0]
    dp = device_layer(cfg, wts, max_chunk=150, flags=fl)
    for p0 in (0, 150):
        sl = slice(p0, p0 + 150)
        o, tk = dp.prefill(0, p0, dev(x[sl]), dev(u[sl]), dev(q[sl]), dev(qI2[sl]), dev(w2[sl]))
        torch.cuda.synchronize()
        og, tkg = cpu(o), cpu(tk)
        for n in want:
            if not p0 <= n < p0 + 150:
                continue
            r = seq.query(n, q[n], qI2[n], w2[n])
            assert sets_equal(tkg[n - p0], r["topk"]), f"[{which}] prefill top-k of query {n}"
            assert_close(og[n - p0], r["out_f64"], BF16_TOL, f"[{which}] prefill output {n}")
    log(f"[skips {which}] prefill matches")


def test_keep_f32_changes_nothing_on_f32_layers():
    """KEEP_F32 declares that every cast is the identity; on an f32 layer
    (C1) it is accepted and the stored bytes and outputs are those of the
    same calls without it."""
    from compressed_kv_sparse_amd import _lib as L
    cfg = get_config("c1")
    wts = make_layer_weights(cfg)
    T = 160
    x, u, q, qI, w = G.make_token_stream(cfg, T)
    res = []
    for fl in (0, L.CKV_FLAG_KEEP_F32):
        dl = device_layer(cfg, wts, flags=fl)
        xd, ud = dev(x), dev(u)
        for p in range(T):
            dl.compress_decode(xd[p:p + 1], ud[p:p + 1], dev(np.array([p], np.int32)), B=1)
        p = T - 1
        pos_d = dev(np.array([p], np.int32))
        topk_d = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda")
        dl.indexer_decode(dev(qI[p:p + 1]), dev(w[p:p + 1]), pos_d, topk_d, B=1)
        out = dl.new_out(1)
        dl.attn_decode(dev(q[p:p + 1]), pos_d, topk_d, out, B=1)
        torch.cuda.synchronize()
        res.append((cpu(dl.comp), cpu(dl.idx), cpu(dl.raw), cpu(topk_d), cpu(out)))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
