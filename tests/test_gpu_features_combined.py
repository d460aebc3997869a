"""The optional parts together on one c4a layer: two-lane compressors, the
query norm, fp8 attention output records and the fp4 indexer cache, on a
paged cache against the same layer on a contiguous one (bit-exact), and the
contiguous run against the oracle with every one of those readings on; then
a prefill chunk with the indexer on a second stream, paged against
contiguous."""
import numpy as np
import pytest

from harness import FP8_TOL, compare_out_fp8, dev, device_layer, oracle_layer, oracle_seq_from_bytes, \
    tie_free_queries
from test_gpu_paged import cpu, paged_layer, same
from workloads import get_config, make_decode_inputs, make_layer_weights, make_prefill_inputs
from workloads.configs import TWO_LANE_FLAG

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ALL = TWO_LANE_FLAG | 64 | 32   # two lanes, query norm, fp8 output records


def log(msg):
    print(msg, flush=True)


def test_decode_with_every_option():
    cfg = get_config("c5_fp4idx").with_(batch=4, flags=ALL, seed=91, name="c5_all_options_b4")
    inp = make_decode_inputs(cfg)
    wts = make_layer_weights(cfg)
    log(f"[combined decode] {cfg.name}")
    cont = device_layer(cfg, wts, inp.cache)
    pg = paged_layer(cfg, wts, inp.cache, seed=3)
    pos_d = dev(inp.pos)
    # tie-free indexer queries on the rows the compressor writes
    cont.compress_decode(dev(inp.x), dev(inp.u), pos_d)
    torch.cuda.synchronize()
    L = oracle_layer(cfg, wts)
    assert L.two_lane and L.q_norm
    raw_g, comp_g, idx_g = cpu(cont.raw), cpu(cont.comp), cpu(cont.idx)
    seqs = [oracle_seq_from_bytes(L, raw_g[b], comp_g[b], idx_g[b], int(inp.pos[b]) + 1) for b in range(cfg.batch)]
    qI, w = tie_free_queries(cfg, seqs, inp.pos, inp.qI, inp.w)
    cont2 = device_layer(cfg, wts, inp.cache)
    args = [dev(inp.x), dev(inp.u), dev(inp.q), dev(qI), dev(w), pos_d]
    oc, tc = cont2.decode_step(*args)
    op, tp = pg.decode_step(*args)
    torch.cuda.synchronize()
    same(cpu(oc), cpu(op), "outputs")
    same(cpu(tc), cpu(tp), "top-k lists")
    same(cpu(cont2.comp_rows()), cpu(pg.comp_rows()), "compressed rows")
    same(cpu(cont2.idx_rows()), cpu(pg.idx_rows()), "indexer rows")
    same(cpu(cont2.st_kv), cpu(pg.st_kv), "state")
    og, tk = cpu(oc), cpu(tc)
    for b in range(cfg.batch):
        ref = seqs[b].attend(int(inp.pos[b]), inp.q[b], tk[b])
        compare_out_fp8(og[b], ref, FP8_TOL[0], f"fp8 output b={b}")


def test_prefill_with_every_option_two_streams():
    cfg = get_config("c4").with_(flags=ALL, name="c4_all_options")
    T = 1024
    inp = make_prefill_inputs(cfg, pos0=cfg.pos0, T=T)
    wts = make_layer_weights(cfg)
    log(f"[combined prefill] {cfg.name} T={T}")
    cont = device_layer(cfg, wts, inp.cache, max_chunk=T)
    pg = paged_layer(cfg, wts, inp.cache, seed=4, max_chunk=T)
    args = [dev(inp.x), dev(inp.u), dev(inp.q), dev(inp.qI), dev(inp.w)]
    oc, tc = cont.prefill(0, inp.pos0, *args)
    op, tp = pg.prefill_chunk(0, inp.pos0, *args, side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    same(cpu(oc), cpu(op), "outputs")
    same(cpu(tc), cpu(tp), "top-k lists")
    same(cpu(cont.comp_rows()), cpu(pg.comp_rows()), "compressed rows")
    same(cpu(cont.idx_rows()), cpu(pg.idx_rows()), "indexer rows")
    same(cpu(cont.st_kv), cpu(pg.st_kv), "state")
