"""The query norm inside the attention (CKV_FLAG_Q_NORM: each head's query
divided by its RMS over head_dim, before its RoPE) against the oracle's
attention with the same reading: the tiled kernel through the split merge at
the 16 x 131072-token c4a shape (fp8 K=V), bf16 decode, the vector kernel
(f32, head_dim 128), a prefill chunk (one split per query) and the range
guard's fp32 recompute.  Queries carry per-head factors 2^-8 .. 2^8 (exact in
bf16) so that the norm changes every head by a different amount; each case
also checks that the output moves against the oracle without the norm."""
import numpy as np
import pytest

import oracle as O
from harness import BF16_TOL, FP8_TOL, assert_close, dev, device_layer, oracle_layer, oracle_seq_from_bytes, \
    oracle_seq_from_init
from test_gpu_contract import _scale_bf16_rows
from workloads import get_config, make_decode_inputs, make_layer_weights, make_prefill_inputs
from workloads import gen as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def cpu(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def log(msg):
    print(msg, flush=True)


def head_scaled(q, act_fmt, rng):
    """q [..., H, d] with head h multiplied by 2^k_h, k_h in -8..8."""
    H = q.shape[-2]
    f = np.exp2(rng.integers(-8, 9, H)).astype(np.float32)[:, None]
    if act_fmt == "bf16":
        v = (q.astype(np.uint32) << 16).view(np.float32) * f
        return G.bf16_bits_of_draw(v)
    return (q * f).astype(q.dtype)


def flag():
    from compressed_kv_sparse_amd import _lib as Lb
    return Lb.CKV_FLAG_Q_NORM


def random_topk(cfg, pos, rng):
    return np.stack([np.sort(rng.choice(max((int(p) + 1) // 4, cfg.top_k), cfg.top_k, replace=False))
                     for p in pos]).astype(np.int32)


def check(og, q, pos, tk, seqs, L, tol, what, must_move=True):
    moved = 0.0
    for b in range(len(seqs)):
        p = int(pos[b])
        L.q_norm = True
        ref = seqs[b].attend(p, q[b], None if tk is None else tk[b])
        assert_close(og[b], ref, tol, f"{what} b={b}")
        L.q_norm = False
        moved = max(moved, float(np.abs(seqs[b].attend(p, q[b], None if tk is None else tk[b]) - ref).max()))
    assert moved > 1e-2 or not must_move, f"{what}: the norm does not change the output ({moved})"


@pytest.mark.parametrize("name", ["c5", "c2_small", "c1"])
def test_qnorm_decode(name):
    """Attention alone on the drawn cache with random top-k lists."""
    rng = np.random.default_rng(321)
    if name == "c2_small":
        cfg = get_config("c2").with_(batch=3, comp_cap=1024, top_k=128, seed=81, name="qnorm_c2_small")
        inp = make_decode_inputs(cfg, n_ctx=np.array([4000, 2500, 129], np.int64))
    else:
        cfg = get_config(name)
        inp = make_decode_inputs(cfg)
    wts = make_layer_weights(cfg)
    log(f"[qnorm decode] {cfg.name}")
    q = head_scaled(inp.q, cfg.act_fmt, rng)
    dl = device_layer(cfg, wts, inp.cache, flags=flag())
    tk = random_topk(cfg, inp.pos, rng) if cfg.ratio == 4 else None
    out = dl.new_out(cfg.batch)
    dl.attn_decode(dev(q), dev(inp.pos), None if tk is None else dev(tk), out)
    torch.cuda.synchronize()
    L = oracle_layer(cfg, wts)
    raw_g, comp_g = cpu(dl.raw), cpu(dl.comp)
    seqs = [oracle_seq_from_bytes(L, raw_g[b], comp_g[b], None, int(inp.pos[b]) + 1) for b in range(cfg.batch)]
    og = O.decode_values(cpu(out), cfg.act_fmt)
    tol = FP8_TOL if cfg.kv_fmt == "e4m3" else BF16_TOL
    check(og, q, inp.pos, tk, seqs, L, tol, "q-norm output")


def test_qnorm_prefill_chunk():
    """A c4a prefill chunk (compressor, indexer, attention) with the norm:
    sampled queries against the oracle on the GPU's top-k lists."""
    cfg = get_config("c4")
    T = 256
    inp = make_prefill_inputs(cfg, pos0=cfg.pos0, T=T)
    wts = make_layer_weights(cfg)
    q = head_scaled(inp.q, cfg.act_fmt, np.random.default_rng(5))
    log(f"[qnorm prefill] T={T}")
    dl = device_layer(cfg, wts, inp.cache, max_chunk=T, flags=flag())
    out, tk = dl.prefill(0, inp.pos0, dev(inp.x), dev(inp.u), dev(q), dev(inp.qI), dev(inp.w))
    torch.cuda.synchronize()
    og, tkg = O.decode_values(cpu(out), cfg.act_fmt), cpu(tk)
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, inp.cache, 0)
    seq.feed(inp.pos0, inp.x, inp.u)
    picks = [0, 7, 100, 200, T - 1]
    check(og[picks], q[picks], [inp.pos0 + n for n in picks], tkg[picks], [seq] * len(picks), L, BF16_TOL,
          "q-norm prefill output")


def test_qnorm_range_guard():
    """Stored rows at 1e5 send the splits to the fp32 recompute, which applies
    the norm on its own (32 threads per head)."""
    rng = np.random.default_rng(17)
    cfg = get_config("c2").with_(batch=2, comp_cap=512, top_k=64, seed=91, name="qnorm_guard")
    inp = make_decode_inputs(cfg, n_ctx=np.array([2000, 1500], np.int64))
    c = inp.cache
    for b in range(cfg.batch):
        _scale_bf16_rows(c.raw[b], rng.choice(cfg.swa, 3, replace=False), 1e5)
    q = head_scaled(inp.q, cfg.act_fmt, rng)
    wts = make_layer_weights(cfg)
    log("[qnorm guard]")
    dl = device_layer(cfg, wts, c, flags=flag())
    tk = random_topk(cfg, inp.pos, rng)
    out = dl.new_out(cfg.batch)
    dl.attn_decode(dev(q), dev(inp.pos), dev(tk), out)
    torch.cuda.synchronize()
    L = oracle_layer(cfg, wts)
    raw_g, comp_g = cpu(dl.raw), cpu(dl.comp)
    seqs = [oracle_seq_from_bytes(L, raw_g[b], comp_g[b], None, int(inp.pos[b]) + 1) for b in range(cfg.batch)]
    # (rows at 1e5 dominate both softmaxes, so the output need not move)
    check(O.decode_values(cpu(out), cfg.act_fmt), q, inp.pos, tk, seqs, L, BF16_TOL, "guarded q-norm output",
          must_move=False)
