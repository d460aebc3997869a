"""Decode attention on E4M3 rows (the tiled fp16-MFMA kernel, its split
merge and its range guard) against the oracle on the bytes the GPU holds.

Batches of 3, 5 and 11 sequences, ratios 4, 128 and 0, short contexts (raw
slots before position 0, fewer visible rows than top_k, a ratio-128 layer
with no compressed row yet), top-k lists with -1 entries and a list that ends
early (an entry >= V cuts it), fp8 output records with the query norm on a
layer with two RoPE bases, and the range guard on E4M3 rows (RoPE tails and
query heads beyond fp16's range) with its fp32 recompute.  Every call goes
through the C ABI.
"""
import numpy as np
import pytest

import oracle as O
from harness import BF16_TOL, assert_close, compare_out_fp8, dev, device_layer, oracle_layer, oracle_seq_from_bytes
from workloads import get_config, make_decode_inputs, make_layer_weights
from workloads import gen as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

OUT_FP8 = 32
C5 = {4: "c5_c4a_decode_b16_ctx131072_fp8", 128: "c5_c128a_decode_b16_ctx131072_fp8",
      0: "c5_swa_decode_b16_ctx131072_fp8"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_kv_sparse_amd  # noqa: F401  (fails loudly if libckv.so is missing)


def log(msg):
    print(msg, flush=True)


def cpu(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _topk_lists(cfg, pos, rng, cut_b=None):
    """Sorted top-k lists: all visible rows then -1 padding when V <= k,
    otherwise k distinct rows; sequence cut_b gets an entry >= V in the
    middle of its list (the list ends there)."""
    k = cfg.top_k
    tk = np.full((cfg.batch, k), -1, np.int32)
    for b in range(cfg.batch):
        V = min((int(pos[b]) + 1) // 4, cfg.comp_cap)
        if V <= k:
            tk[b, :V] = np.arange(V)
        else:
            tk[b] = np.sort(rng.choice(V, k, replace=False))
        if b == cut_b and V > 2:
            tk[b, k // 2] = V + 5
    return tk


def _oracle_topk(tk_b, V):
    """The list as the consumer reads it: it ends at its first entry >= V."""
    t = tk_b.copy()
    bad = np.nonzero(t >= V)[0]
    if bad.size:
        t[bad[0]:] = -1
    return t


def _run(cfg, inp, q, tk, flags):
    dl = device_layer(cfg, make_layer_weights(cfg), inp.cache, flags=flags)
    out = dl.new_out(cfg.batch)
    dl.attn_decode(dev(q), dev(inp.pos), None if tk is None else dev(tk), out)
    torch.cuda.synchronize()
    return dl, out


def _check(cfg, inp, q, tk, dl, out, flags, what):
    L = oracle_layer(cfg, make_layer_weights(cfg))
    raw_g = cpu(dl.raw)
    comp_g = cpu(dl.comp) if dl.comp is not None else None   # window-only layers have none
    o = cpu(out)
    for b in range(cfg.batch):
        p = int(inp.pos[b])
        V = min((p + 1) // 4, cfg.comp_cap) if cfg.ratio == 4 else 0
        t = _oracle_topk(tk[b], V) if tk is not None else None
        ref = oracle_seq_from_bytes(L, raw_g[b], None if comp_g is None else comp_g[b], None, p + 1).attend(p, q[b], t)
        if flags & OUT_FP8:
            compare_out_fp8(o[b], ref, BF16_TOL[0], f"{what} b={b}")
        else:
            assert_close(O.decode_values(o[b], cfg.act_fmt), ref, BF16_TOL, f"{what} b={b}")


@pytest.mark.parametrize("ratio,B", [(4, 3), (4, 11), (128, 11), (0, 5)])
def test_dec_attention_ragged_batches(ratio, B):
    cap = {4: 4096, 128: 256, 0: 0}[ratio]
    cfg = get_config(C5[ratio]).with_(batch=B, comp_cap=cap, seed=170 + B + ratio, name=f"attn_dec_r{ratio}_b{B}")
    rng = np.random.default_rng(cfg.seed)
    # short contexts first: raw slots before position 0, V <= top_k, a c128a
    # layer with no compressed row yet; then long ones
    short = [1, 60, 129, 700, 2051]
    n = np.array([short[b] if b < len(short) else int(rng.integers(2100, 16384)) for b in range(B)], np.int64)
    if ratio == 128:
        n[-1] = 128 * cap   # every compressed row visible
    inp = make_decode_inputs(cfg, n_ctx=n)
    tk = _topk_lists(cfg, inp.pos, rng, cut_b=B - 1) if ratio == 4 else None
    log(f"[attn_dec] ratio={ratio} B={B} n={n.tolist()}")
    dl, out = _run(cfg, inp, inp.q, tk, 0)
    _check(cfg, inp, inp.q, tk, dl, out, 0, f"attn_dec r{ratio} B{B}")


@pytest.mark.parametrize("flags", [0, OUT_FP8])
def test_dec_attention_range_guard_e4m3(flags):
    """E4M3 rows whose bf16 RoPE tails reach 1e5 and query heads at 1e5
    (beyond fp16) or 1e-6: the blocks holding them take the fp32 recompute,
    the others the fp16 tiles; every output against the oracle."""
    cfg = get_config(C5[4]).with_(batch=5, comp_cap=2048, top_k=128, seed=181 + flags, name="attn_dec_guard")
    rng = np.random.default_rng(cfg.seed)
    n = np.array([3000, 1500, 700, 8192, 4000], np.int64)
    inp = make_decode_inputs(cfg, n_ctx=n)
    c = inp.cache
    rb = c.raw.shape[-1]
    dn = cfg.head_dim - 64
    for b in (0, 2):   # RoPE tails of a few raw rows and compressed rows at 1e5
        for rows, arr in ((rng.choice(cfg.swa, 3, replace=False), c.raw[b]),
                          (rng.choice(int(c.n_drawn_comp[b]), 20, replace=False), c.comp[b])):
            tail = arr[rows, dn:dn + 128].copy().view(np.uint16).astype(np.uint32) << 16
            f = (tail.view(np.float32) * np.float32(1e5)).astype(np.float32)
            arr[rows, dn:dn + 128] = G.bf16_bits_of_draw(f).view(np.uint8).reshape(len(rows), 128)
    assert rb >= dn + 132
    q = inp.q.copy()
    qf = (q.astype(np.uint32) << 16).view(np.float32).copy()
    qf[1, 17] *= 1e5     # one head of sequence 1 far above fp16
    qf[3] *= 1e-6        # every head of sequence 3 tiny
    q = G.bf16_bits_of_draw(qf)
    tk = _topk_lists(cfg, inp.pos, rng)
    log(f"[attn_dec guard] flags={flags}")
    dl, out = _run(cfg, inp, q, tk, flags)
    if not flags:
        assert np.all(np.isfinite(O.decode_values(cpu(out), cfg.act_fmt)))
    _check(cfg, inp, q, tk, dl, out, flags, "attn_dec guard")


def test_dec_attention_out_fp8_qnorm_two_bases():
    """fp8 output records with the query norm, on a layer whose raw and
    compressed rows have their own RoPE bases (the waves switch frames
    after their raw tile; a wave with no compressed tile joins the others'
    frame before the combine)."""
    from workloads.configs import ROPE_BASE_COMPRESSED, ROPE_BASE_RAW
    flags = OUT_FP8 | 64
    cfg = get_config(C5[4]).with_(batch=4, comp_cap=1024, top_k=32, seed=191, name="attn_dec_two_bases",
                                  rope_base=ROPE_BASE_RAW, rope_base_comp=ROPE_BASE_COMPRESSED, flags=flags)
    n = np.array([300, 4096, 2000, 129], np.int64)   # top_k 32: tile 4 only (wave 0) holds compressed rows
    inp = make_decode_inputs(cfg, n_ctx=n)
    tk = _topk_lists(cfg, inp.pos, np.random.default_rng(cfg.seed))
    dl, out = _run(cfg, inp, inp.q, tk, flags)
    _check(cfg, inp, inp.q, tk, dl, out, flags, "attn_dec two bases")
