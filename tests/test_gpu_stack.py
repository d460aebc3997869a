"""The layer-stack decode driver against the oracle.

A 43-layer Flash stack (two window-only layers, then c4a on even and c128a on
odd layers; "ds4.c を読み解く (#3)", section 1) at a short context, one decode
step of every layer through ``DeviceStack`` (all layers launched back to back
on one stream), then every layer checked on the bytes its caches hold:
the rows the step wrote against the oracle's compressor run from the drawn
state, the top-k set bit-exact, the output within the fp8 bar.
"""
import numpy as np
import pytest

import oracle as O
from harness import (FP8_TOL, assert_close, compare_rows, dev, oracle_layer, oracle_seq_from_bytes,
                     oracle_seq_from_init, sets_equal, tie_free_queries, topk_margin)
from workloads import make_decode_inputs, make_layer_weights
from workloads.configs import flash_ratio, stack_layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_kv_sparse_amd  # noqa: F401


def cpu(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@pytest.mark.parametrize("paged", [False, True])
def test_flash_stack_decode_every_layer(paged):
    """paged: every layer's compressed rows in pages of pools the 43 layers
    share (three page sizes), through per-layer block tables."""
    from compressed_kv_sparse_amd.stack import DeviceStack, StackShape

    B, n = 2, 4096 + 4          # p = 4099: c4a boundary (row 1024 emitted), c128a mid-window
    shape = StackShape(batch=B, n_ctx=8192, paged=paged)
    stk = DeviceStack(shape)
    assert len(stk) == 43
    assert stk.ratios == [O.flash_ratio(il) for il in range(43)]
    inputs, cases = [], []
    for il, dl in enumerate(stk.layers):
        r = flash_ratio(il)
        cfg = stack_layer(il).with_(batch=B, n_ctx=n, comp_cap=(8192 // r) if r else 0)
        assert dl.ratio == cfg.ratio
        wts = make_layer_weights(cfg)
        inp = make_decode_inputs(cfg)
        if wts is not None:
            dl.set_weights(wkv=wts.wkv, wgate=wts.wgate, ape=wts.ape, gamma=wts.gamma, idx_wkv=wts.idx_wkv,
                           idx_wgate=wts.idx_wgate, idx_ape=wts.idx_ape, idx_gamma=wts.idx_gamma)
        c = inp.cache
        dl.load_cache(raw=c.raw, comp=c.comp, idx=c.idx, st_kv=c.st_kv, st_sc=c.st_sc, ist_kv=c.ist_kv,
                      ist_sc=c.ist_sc, n_tokens=c.first_live)
        L = oracle_layer(cfg, wts)
        seqs = [oracle_seq_from_init(L, c, b) for b in range(B)]
        for b in range(B):
            seqs[b].feed(int(inp.pos[b]), inp.x[b][None], inp.u[b][None])
        qI, w = inp.qI, inp.w
        if r == 4:   # wide gap on the oracle's own rows; re-checked on the GPU's bytes below
            qI, w = tie_free_queries(cfg, seqs, inp.pos, qI, w, margin=3e-4)
        inputs.append(dict(x=dev(inp.x), u=dev(inp.u), q=dev(inp.q), pos=dev(inp.pos),
                           qI=None if qI is None else dev(qI), w=None if w is None else dev(w)))
        cases.append((cfg, L, inp, seqs, qI, w))
    outs, topks = stk.buffers()
    stk.decode(inputs, outs, topks)
    torch.cuda.synchronize()
    print(f"[stack] 43 layers stepped at p={n - 1} (paged: {paged})", flush=True)
    if paged:
        assert len(stk.pools.page_sizes()) == 3

    for il, (dl, (cfg, L, inp, seqs, qI, w)) in enumerate(zip(stk.layers, cases)):
        assert int(np.abs(cpu(dl.status)).sum()) == 0, f"layer {il}: status set"
        d, r = cfg.head_dim, cfg.ratio
        raw_g = cpu(dl.raw)
        comp_g = cpu(dl.comp_rows()) if dl.comp is not None else None
        idx_g = cpu(dl.idx_rows()) if dl.idx is not None else None
        for b in range(B):
            p = int(inp.pos[b])
            compare_rows(raw_g[b, p % cfg.swa], seqs[b].raw_row(p)[0], cfg.kv_fmt, d, cfg.n_rot,
                         f"layer {il} raw row b={b}")
            if r and (p + 1) % r == 0:
                i = (p + 1) // r - 1
                compare_rows(comp_g[b, i], seqs[b].comp_row(i)[0], cfg.kv_fmt, d, cfg.n_rot,
                             f"layer {il} comp row {i} b={b}")
        tk = cpu(topks[il]) if topks[il] is not None else None
        og = O.decode_values(cpu(outs[il]), cfg.act_fmt)
        for b in range(B):
            p = int(inp.pos[b])
            bs = oracle_seq_from_bytes(L, raw_g[b], None if comp_g is None else comp_g[b],
                                       None if idx_g is None else idx_g[b], p + 1)
            sel = None
            if r == 4:
                sc = bs.index_scores(p, qI[b], w[b])
                assert topk_margin(sc, cfg.top_k) > 1e-4, f"layer {il} b={b}: near-tie on the GPU's rows"
                assert sets_equal(tk[b], O.topk_select(sc, cfg.top_k)), f"layer {il}: top-k set differs b={b}"
                sel = tk[b]
            ref = bs.attend(p, inp.q[b], sel)
            assert_close(og[b], ref, FP8_TOL, f"layer {il} (ratio {r}) output b={b}")
