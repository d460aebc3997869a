"""The paged compressed caches (256-position blocks through a block table,
pages scattered in a shared pool) against the contiguous layout on the same
inputs: outputs, top-k lists and every compressed and indexer row must be
identical, through the single-call decode step at the 16 x 131072-token c4a
shape (fp8 K=V; bf16 and fp4 indexer rows), the three separate decode calls,
a c128a layer, the f32 vector kernels, a 4096-token prefill chunk (its
indexer GEMM reads two lane tables of pages) and an fp4 prefill chunk; and a
block-table entry outside the pool, which drops that row's store and flags
only its own sequence."""
import numpy as np
import pytest

from harness import dev, device_layer
from workloads import get_config, make_decode_inputs, make_layer_weights, make_prefill_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def cpu(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def paged_layer(cfg, wts, cache, seed, max_chunk=0, batch=None, spare=37):
    """A layer whose compressed rows live in scattered pages of a pool with
    ``spare`` more pages than the layer needs."""
    from compressed_kv_sparse_amd import DeviceLayer, PagePools
    from compressed_kv_sparse_amd import _lib as L
    B = cfg.batch if batch is None else batch
    rpb = 256 // cfg.ratio
    nb = cfg.comp_cap // rpb
    rb = L.row_bytes(L.FMT[cfg.kv_fmt], cfg.head_dim, cfg.n_rot)
    irb = L.idx_row_bytes(L.FMT[cfg.idx_fmt], cfg.idx_dim) if cfg.ratio == 4 else 0
    n = B * nb + spare
    pools = PagePools(kv_row_bytes=rb, idx_row_bytes=irb, pages_c4a=n if cfg.ratio == 4 else 0,
                      pages_c128a=n if cfg.ratio == 128 else 0)
    dl = DeviceLayer(ratio=cfg.ratio, hidden=cfg.hidden, head_dim=cfg.head_dim, n_heads=cfg.n_heads, batch=B,
                     idx_heads=cfg.idx_heads, idx_dim=cfg.idx_dim, top_k=cfg.top_k, comp_cap=cfg.comp_cap,
                     kv_fmt=cfg.kv_fmt, idx_fmt=cfg.idx_fmt, act_fmt=cfg.act_fmt, w_fmt=cfg.w_fmt,
                     rope_base=cfg.rope_base, norm_eps=cfg.norm_eps, n_rot=cfg.n_rot, swa=cfg.swa,
                     max_chunk=max_chunk, rope_base_comp=cfg.rope_base_comp or 0.0, flags=cfg.flags, pages=pools)
    perm = np.random.default_rng(seed).permutation(n)
    for b in range(B):
        dl.map_rows(b, cfg.comp_cap, order=perm[b * nb:(b + 1) * nb])
    dl.set_weights(wkv=wts.wkv, wgate=wts.wgate, ape=wts.ape, gamma=wts.gamma, idx_wkv=wts.idx_wkv,
                   idx_wgate=wts.idx_wgate, idx_ape=wts.idx_ape, idx_gamma=wts.idx_gamma)
    dl.load_cache(raw=cache.raw, comp=cache.comp, idx=cache.idx, st_kv=cache.st_kv, st_sc=cache.st_sc,
                  ist_kv=cache.ist_kv, ist_sc=cache.ist_sc, n_tokens=cache.first_live)
    return dl


def same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    bad = np.argwhere(a != b)
    assert bad.size == 0, f"{what}: {len(bad)} elements differ, first {bad[:3].tolist()}"


def compare_layers(cont, paged, what):
    same(cpu(cont.comp_rows()), cpu(paged.comp_rows()), f"{what}: compressed rows")
    if cont.ratio == 4:
        same(cpu(cont.idx_rows()), cpu(paged.idx_rows()), f"{what}: indexer rows")
    same(cpu(cont.raw), cpu(paged.raw), f"{what}: raw rows")
    same(cpu(cont.status), cpu(paged.status), f"{what}: status")


def decode_both(cfg, inp, wts, call, seed):
    cont = device_layer(cfg, wts, inp.cache)
    pg = paged_layer(cfg, wts, inp.cache, seed)
    args = [dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI) if cfg.ratio == 4 else None,
            dev(inp.w) if cfg.ratio == 4 else None, dev(inp.pos)]
    oc, tc = getattr(cont, call)(*args)
    op, tp = getattr(pg, call)(*args)
    torch.cuda.synchronize()
    same(cpu(oc), cpu(op), f"{cfg.name} {call}: outputs")
    if cfg.ratio == 4:
        same(cpu(tc), cpu(tp), f"{cfg.name} {call}: top-k lists")
    compare_layers(cont, pg, f"{cfg.name} {call}")
    return cont, pg


@pytest.mark.parametrize("name,call", [("c5", "decode_step"), ("c5_fp4idx", "decode_step"),
                                       ("c2_small", "decode"), ("c2_small", "decode_step"), ("c3_small", "decode"),
                                       ("c1", "decode")])
def test_paged_decode_equals_contiguous(name, call):
    if name == "c2_small":
        cfg = get_config("c2").with_(batch=3, comp_cap=1024, top_k=128, seed=83, name="paged_c2_small")
        inp = make_decode_inputs(cfg, n_ctx=np.array([4000, 2500, 129], np.int64))
    elif name == "c3_small":
        cfg = get_config("c3").with_(batch=2, comp_cap=1024, seed=84, ctx_range=None, name="paged_c3_small")
        inp = make_decode_inputs(cfg, n_ctx=np.array([100000, 66560], np.int64))
    else:
        cfg = get_config(name)
        inp = make_decode_inputs(cfg)
    wts = make_layer_weights(cfg)
    log(f"[paged decode] {cfg.name} {call}")
    decode_both(cfg, inp, wts, call, seed=len(name) * 7 + len(call))


@pytest.mark.parametrize("name", ["c4", "c4_fp4idx"])
def test_paged_prefill_chunk_equals_contiguous(name):
    cfg = get_config(name)
    inp = make_prefill_inputs(cfg)
    wts = make_layer_weights(cfg)
    T = inp.T
    log(f"[paged prefill] {cfg.name} T={T}")
    cont = device_layer(cfg, wts, inp.cache, max_chunk=T)
    pg = paged_layer(cfg, wts, inp.cache, seed=5, max_chunk=T)
    args = [dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w)]
    oc, tc = cont.prefill(0, inp.pos0, *args)
    op, tp = pg.prefill(0, inp.pos0, *args)
    torch.cuda.synchronize()
    same(cpu(oc), cpu(op), f"{cfg.name} prefill: outputs")
    same(cpu(tc), cpu(tp), f"{cfg.name} prefill: top-k lists")
    compare_layers(cont, pg, f"{cfg.name} prefill")


def test_paged_entry_outside_the_pool():
    """Sequence 0's block holding the row its token closes points past the
    pool: that row is not stored and CKV_STATUS_PAGE is set for sequence 0
    only; the other sequences' outputs, lists and rows match the contiguous
    run."""
    from compressed_kv_sparse_amd import _lib as L
    cfg = get_config("c2").with_(batch=3, comp_cap=1024, top_k=128, seed=85, name="paged_bad_entry")
    inp = make_decode_inputs(cfg, n_ctx=np.array([4000, 2500, 1600], np.int64))
    wts = make_layer_weights(cfg)
    log("[paged decode] entry outside the pool")
    cont = device_layer(cfg, wts, inp.cache)
    pg = paged_layer(cfg, wts, inp.cache, seed=9)
    i = (int(inp.pos[0]) + 1) // 4 - 1          # the row sequence 0's token closes
    assert (int(inp.pos[0]) + 1) % 4 == 0
    n_pages = pg.cache.n_pages
    pg.table.dev[0, i // 64] = n_pages + 3
    args = [dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w), dev(inp.pos)]
    oc, tc = cont.decode_step(*args)
    op, tp = pg.decode_step(*args)
    torch.cuda.synchronize()
    st = cpu(pg.status)
    assert st[0] & L.CKV_STATUS_PAGE and not st[1:].any(), st
    same(cpu(oc)[1:], cpu(op)[1:], "other sequences' outputs")
    same(cpu(tc)[1:], cpu(tp)[1:], "other sequences' lists")
    rows_c, rows_p = cpu(cont.comp_rows()), cpu(pg.comp_rows())
    same(rows_c[1:], rows_p[1:], "other sequences' rows")
