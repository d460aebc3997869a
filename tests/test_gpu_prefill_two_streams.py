"""ckv_prefill_chunk (the chunk's three prefill calls in one, the indexer
branch on a second stream beside the attention lane's compression and the raw
staging) against the three separate calls on the same inputs: outputs, top-k
lists and every cache byte the chunk writes must be identical, for the
4096-token c4a chunk (bf16 and fp4 indexer caches), short chunks (the
projection's other kernels), a c128a chunk and a window-only chunk (no
indexer: one stream), plus sampled queries of the two-stream run against the
oracle."""
import numpy as np
import pytest

import oracle as O
from harness import BF16_TOL, assert_close, dev, device_layer, oracle_layer, oracle_seq_from_init, sets_equal
from workloads import get_config, make_layer_weights, make_prefill_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def cpu(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def log(msg):
    print(msg, flush=True)


def cache_bytes(dl):
    return {n: cpu(getattr(dl, n)).copy() for n in ("raw", "comp", "idx", "st_kv", "st_sc", "ist_kv", "ist_sc",
                                                     "n_tokens")
            if getattr(dl, n, None) is not None}


def run_both(cfg, pos0, T, side=True):
    inp = make_prefill_inputs(cfg, pos0=pos0, T=T)
    wts = make_layer_weights(cfg)
    args = [dev(inp.x), dev(inp.u), dev(inp.q)]
    extra = [dev(inp.qI), dev(inp.w)] if cfg.ratio == 4 else [None, None]
    ref_dl = device_layer(cfg, wts, inp.cache, max_chunk=T)
    o_ref, tk_ref = ref_dl.prefill(0, pos0, *args, *extra)
    torch.cuda.synchronize()
    ref = (cpu(o_ref), None if tk_ref is None else cpu(tk_ref), cache_bytes(ref_dl))
    del ref_dl, o_ref, tk_ref
    dl = device_layer(cfg, wts, inp.cache, max_chunk=T)
    s = torch.cuda.Stream() if side else None
    out, tk = dl.prefill_chunk(0, pos0, *args, *extra, side_stream=s)
    torch.cuda.synchronize()
    got = (cpu(out), None if tk is None else cpu(tk), cache_bytes(dl))
    np.testing.assert_array_equal(got[0], ref[0], err_msg="outputs differ")
    if cfg.ratio == 4:
        np.testing.assert_array_equal(got[1], ref[1], err_msg="top-k lists differ")
    for n in ref[2]:
        np.testing.assert_array_equal(got[2][n], ref[2][n], err_msg=f"cache {n} differs")
    return inp, wts, got


@pytest.mark.parametrize("name,T", [("c4", None), ("c4_fp4idx", None), ("c4", 100), ("c4", 37)])
def test_prefill_chunk_two_streams_equal_three_calls(name, T):
    cfg = get_config(name)
    T = cfg.chunk if T is None else T
    log(f"[prefill two streams] {cfg.name} T={T}")
    inp, wts, (og, tkg, _) = run_both(cfg, cfg.pos0, T)
    if name != "c4" or T != cfg.chunk:
        return
    # sampled queries of the two-stream run against the oracle
    L = oracle_layer(cfg, wts)
    seq = oracle_seq_from_init(L, inp.cache, 0)
    seq.feed(inp.pos0, inp.x, inp.u)
    for n in (0, 511, 512, 2047, 4095):
        p = inp.pos0 + n
        assert sets_equal(tkg[n], O.topk_select(seq.index_scores(p, inp.qI[n], inp.w[n]), cfg.top_k)), n
        assert_close(O.decode_values(og[n], cfg.act_fmt), seq.attend(p, inp.q[n], tkg[n]), BF16_TOL,
                     f"two-stream output {n}")


@pytest.mark.parametrize("name,pos0,T", [("c3", 4000, 300), ("c5_swa", 1000, 200)])
def test_prefill_chunk_without_indexer(name, pos0, T):
    """Layers without an indexer ignore the side stream: one stream, same bytes."""
    cfg = get_config(name)
    if name == "c3":
        cfg = cfg.with_(comp_cap=64, ctx_range=None)
    log(f"[prefill two streams] {cfg.name} pos0={pos0} T={T}")
    run_both(cfg.with_(batch=1), pos0, T)


def test_prefill_chunk_one_stream():
    """No side stream: the three calls in order, one launch sequence."""
    cfg = get_config("c4")
    log("[prefill two streams] one stream")
    run_both(cfg, cfg.pos0, 1000, side=False)
