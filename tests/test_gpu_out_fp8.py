"""The attention output written as fp8 records (CKV_FLAG_OUT_FP8: the inverse
RoPE fused with an E4M3 quantisation in groups of 128 channels) against the
oracle's output and its fp8 encoding: decode at the 16 x 131072-token c4a
shape through the split merge, a prefill chunk (one split, the tile kernel's
own epilogue), and both range-guard recompute paths."""
import numpy as np
import pytest

import oracle as O
from harness import (BF16_TOL, FP8_TOL, compare_out_fp8, dev, device_layer, oracle_layer, oracle_seq_from_bytes,
                     oracle_seq_from_init, tie_free_queries)
from test_gpu_contract import _scale_bf16_rows
from workloads import get_config, make_decode_inputs, make_layer_weights, make_prefill_inputs
from workloads import gen as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def cpu(t):
    return t.detach().cpu().numpy()


def log(msg):
    print(msg, flush=True)


def test_out_fp8_decode_full_size():
    """C5 c4a decode (fp8 K=V): compressor, indexer, then the attention with
    fp8 output records, against the oracle on the cache the GPU wrote."""
    from compressed_kv_sparse_amd import _lib as Lb
    cfg = get_config("c5")
    inp = make_decode_inputs(cfg)
    wts = make_layer_weights(cfg)
    log(f"[out_fp8 decode] {cfg.name}")
    dl = device_layer(cfg, wts, inp.cache, flags=Lb.CKV_FLAG_OUT_FP8)
    pos_d = dev(inp.pos)
    dl.compress_decode(dev(inp.x), dev(inp.u), pos_d)
    torch.cuda.synchronize()
    L = oracle_layer(cfg, wts)
    raw_g, comp_g, idx_g = cpu(dl.raw), cpu(dl.comp), cpu(dl.idx).view(np.uint16)
    bseqs = [oracle_seq_from_bytes(L, raw_g[b], comp_g[b], idx_g[b], int(inp.pos[b]) + 1) for b in range(cfg.batch)]
    qI, w = tie_free_queries(cfg, bseqs, inp.pos, inp.qI, inp.w)
    topk = torch.empty((cfg.batch, cfg.top_k), dtype=torch.int32, device="cuda")
    dl.indexer_decode(dev(qI), dev(w), pos_d, topk)
    out = dl.new_out(cfg.batch)
    assert out.dtype == torch.uint8 and out.shape[-1] == 528
    dl.attn_decode(dev(inp.q), pos_d, topk, out)
    torch.cuda.synchronize()
    og, tk = cpu(out), cpu(topk)
    for b in range(cfg.batch):
        ref = bseqs[b].attend(int(inp.pos[b]), inp.q[b], tk[b])
        compare_out_fp8(og[b], ref, FP8_TOL[0], f"fp8 output b={b}")


def test_out_fp8_prefill_chunk():
    """A c4a prefill chunk (bf16 caches, one split per query): sampled queries'
    fp8 records against the oracle's outputs on the GPU's top-k lists."""
    from compressed_kv_sparse_amd import _lib as Lb
    cfg = get_config("c4")
    T = 512
    inp = make_prefill_inputs(cfg, pos0=cfg.pos0, T=T)
    wts = make_layer_weights(cfg)
    log(f"[out_fp8 prefill] T={T}")
    dl = device_layer(cfg, wts, inp.cache, max_chunk=T, flags=Lb.CKV_FLAG_OUT_FP8)
    out, tk = dl.prefill(0, inp.pos0, dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w))
    torch.cuda.synchronize()
    og, tkg = cpu(out), cpu(tk)
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, inp.cache, 0)
    seq.feed(inp.pos0, inp.x, inp.u)
    for n in (0, 3, 100, 257, T - 1):
        ref = seq.attend(inp.pos0 + n, inp.q[n], tkg[n])
        compare_out_fp8(og[n], ref, BF16_TOL[0], f"fp8 prefill output {n}")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_out_fp8_range_guard(mode):
    """Rows and queries at 1e5 and 1e-6 (the range guard's fp32 recompute)
    with fp8 output records: through the merge (decode) and the recompute's
    own epilogue (a one-split prefill)."""
    from compressed_kv_sparse_amd import _lib as Lb
    f8 = Lb.CKV_FLAG_OUT_FP8
    rng = np.random.default_rng(9)
    if mode == "decode":
        cfg = get_config("c2").with_(batch=2, comp_cap=512, top_k=64, seed=73, name="range_fp8_decode")
        inp = make_decode_inputs(cfg, n_ctx=np.array([2000, 1500], np.int64))
        c = inp.cache
        for b in range(cfg.batch):
            _scale_bf16_rows(c.raw[b], rng.choice(cfg.swa, 3, replace=False), 1e5)
            _scale_bf16_rows(c.comp[b], rng.choice(int(c.n_drawn_comp[b]), 30, replace=False), 1e-6)
        q = inp.q.copy()
        qf = (q.astype(np.uint32) << 16).view(np.float32).copy()
        qf[0, 3] *= 1e5
        q = G.bf16_bits_of_draw(qf)
        wts = make_layer_weights(cfg)
        dl = device_layer(cfg, wts, c, flags=f8)
        tk = np.stack([np.sort(rng.choice((int(inp.pos[b]) + 1) // 4, cfg.top_k, replace=False))
                       for b in range(cfg.batch)]).astype(np.int32)
        out = dl.new_out(cfg.batch)
        dl.attn_decode(dev(q), dev(inp.pos), dev(tk), out)
        torch.cuda.synchronize()
        og = cpu(out)
        L = oracle_layer(cfg, wts)
        raw_g, comp_g = cpu(dl.raw), cpu(dl.comp)
        for b in range(cfg.batch):
            p = int(inp.pos[b])
            ref = oracle_seq_from_bytes(L, raw_g[b], comp_g[b], None, p + 1).attend(p, q[b], tk[b])
            compare_out_fp8(og[b], ref, BF16_TOL[0], f"guarded fp8 output b={b}")
    else:
        cfg = get_config("c3").with_(batch=1, comp_cap=64, seed=74, ctx_range=None, name="range_fp8_prefill")
        pos0, T = 4000, 64
        inp = make_prefill_inputs(cfg, pos0=pos0, T=T)
        c = inp.cache
        nd = int(c.n_drawn_comp[0])
        _scale_bf16_rows(c.comp[0], rng.choice(nd, 4, replace=False), 1e5)
        _scale_bf16_rows(c.comp[0], rng.choice(nd, 4, replace=False), 1e-6)
        wts = make_layer_weights(cfg)
        dl = device_layer(cfg, wts, c, max_chunk=T, flags=f8)
        out, _ = dl.prefill(0, pos0, dev(inp.x), dev(inp.u), dev(inp.q))
        torch.cuda.synchronize()
        og = cpu(out)
        L = oracle_layer(cfg, wts)
        seq = oracle_seq_from_init(L, c, 0)
        seq.feed(pos0, inp.x, inp.u)
        for n in (0, 5, 40, T - 1):
            compare_out_fp8(og[n], seq.attend(pos0 + n, inp.q[n], None), BF16_TOL[0], f"guarded fp8 prefill {n}")
