"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/ckv.h declares, and rejects bad arguments before any
work is enqueued.  Every call here fails validation on the host, so no
kernel is ever launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ckv = pytest.importorskip("compressed_kv_sparse_amd", reason="libckv.so not built")
from compressed_kv_sparse_amd import _lib as L  # noqa: E402


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ckv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ckv_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 21, names
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTS) == names


def desc(**kw):
    base = dict(ratio=4, hidden=4096, head_dim=512, n_rot=64, n_heads=64, swa=128, idx_heads=64, idx_dim=128,
                top_k=512, comp_cap=32768, batch=16, kv_fmt=L.CKV_E4M3, idx_fmt=L.CKV_BF16, act_fmt=L.CKV_BF16,
                w_fmt=L.CKV_BF16, flags=0, rope_base=160000.0, norm_eps=1e-6, softmax_scale=0.0)
    base.update(kw)
    return L.LayerDesc(**base)


def test_validate_accepts_the_workload_shapes():
    assert L.validate(desc()) == 0
    assert L.validate(desc(ratio=128, comp_cap=8192, kv_fmt=L.CKV_BF16)) == 0
    assert L.validate(desc(ratio=0, comp_cap=0)) == 0
    assert L.validate(desc(hidden=1024, head_dim=128, n_heads=16, idx_heads=4, idx_dim=64, top_k=32,
                           comp_cap=256, batch=1, kv_fmt=0, idx_fmt=0, act_fmt=0, w_fmt=0)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(ratio=3), L.CKV_E_UNSUPPORTED), (dict(n_rot=32), L.CKV_E_UNSUPPORTED),
    (dict(swa=64), L.CKV_E_UNSUPPORTED), (dict(head_dim=1024), L.CKV_E_UNSUPPORTED),
    (dict(head_dim=500), L.CKV_E_UNSUPPORTED), (dict(n_heads=24), L.CKV_E_UNSUPPORTED),
    (dict(idx_dim=96), L.CKV_E_UNSUPPORTED), (dict(idx_heads=65), L.CKV_E_UNSUPPORTED),
    (dict(top_k=0), L.CKV_E_UNSUPPORTED), (dict(kv_fmt=7), L.CKV_E_UNSUPPORTED),
    (dict(act_fmt=L.CKV_E4M3), L.CKV_E_UNSUPPORTED), (dict(comp_cap=0), L.CKV_E_INVAL),
    (dict(batch=0), L.CKV_E_INVAL), (dict(rope_base=0.0), L.CKV_E_INVAL),
    (dict(flags=0x200), L.CKV_E_UNSUPPORTED), (dict(flags=0x100), L.CKV_E_UNSUPPORTED), (dict(hidden=100), L.CKV_E_UNSUPPORTED),
    (dict(top_k=2049), L.CKV_E_UNSUPPORTED), (dict(rope_base_comp=-1.0), L.CKV_E_INVAL),
])
def test_validate_rejects(kw, code):
    assert L.validate(desc(**kw)) == code


def test_debug_stage_flags():
    """The header's debug stage skips are accepted (SKIP_NORM, SKIP_ROPE on any
    formats; KEEP_F32 only with f32 caches, activations and weights); other
    bits are not."""
    both = L.CKV_FLAG_SKIP_NORM | L.CKV_FLAG_SKIP_ROPE
    assert L.validate(desc(flags=both)) == 0
    assert L.validate(desc(flags=both | L.CKV_FLAG_NO_INV_ROPE | L.CKV_FLAG_IDX_NO_RELU)) == 0
    assert L.validate(desc(flags=L.CKV_FLAG_KEEP_F32)) == L.CKV_E_UNSUPPORTED
    f32 = dict(kv_fmt=L.CKV_F32, idx_fmt=L.CKV_F32, act_fmt=L.CKV_F32, w_fmt=L.CKV_F32)
    assert L.validate(desc(flags=L.CKV_FLAG_KEEP_F32, **f32)) == 0
    assert L.validate(desc(flags=L.CKV_FLAG_KEEP_F32, **dict(f32, idx_fmt=L.CKV_BF16))) == L.CKV_E_UNSUPPORTED
    assert L.validate(desc(flags=L.CKV_FLAG_KEEP_F32, ratio=0, comp_cap=0, **dict(f32, idx_fmt=L.CKV_BF16))) == 0
    assert L.validate(desc(flags=256)) == L.CKV_E_UNSUPPORTED


def test_validate_bounds_match_the_header():
    """top_k 1..2048 (the header's stated range), a separate compressed-class
    base, and c128a caches of any row count: the attention kernels compute
    the addresses of all-visible compressed rows, so no per-split table
    bounds them (a c128a cache of 8192 rows is the 1M-token workload's)."""
    assert L.validate(desc(top_k=2048)) == 0
    assert L.validate(desc(top_k=1)) == 0
    assert L.validate(desc(rope_base=10000.0, rope_base_comp=160000.0)) == 0
    for cap in (8192, 65536):
        d = desc(ratio=128, comp_cap=cap, kv_fmt=L.CKV_BF16)
        assert L.validate(d) == 0
        assert L.workspace_bytes(d, L.CKV_MODE_PREFILL, 4096) > 0


def test_fp4_indexer_rows():
    """CKV_FP4 indexer rows: 68-byte records at idx_dim 128, accepted on ratio-4
    layers with idx_dim 128 and bf16 activations only; KEEP_F32 excludes it."""
    assert L.idx_row_bytes(L.CKV_FP4, 128) == 68
    assert L.idx_row_bytes(L.CKV_FP4, 64) == 34
    assert L.idx_row_bytes(L.CKV_FP4, 100) == 0
    assert L.idx_row_bytes(L.CKV_BF16, 128) == 256
    assert L.idx_row_bytes(L.CKV_F32, 64) == 256
    assert L.idx_row_bytes(L.CKV_E4M3, 128) == 0
    assert L.row_bytes(L.CKV_FP4, 512) == 0            # not a K=V row format
    assert L.validate(desc(idx_fmt=L.CKV_FP4)) == 0
    assert L.validate(desc(idx_fmt=L.CKV_FP4, kv_fmt=L.CKV_BF16, idx_heads=8)) == 0
    assert L.validate(desc(idx_fmt=L.CKV_FP4, idx_dim=64)) == L.CKV_E_UNSUPPORTED
    assert L.validate(desc(idx_fmt=L.CKV_FP4, act_fmt=L.CKV_F32)) == L.CKV_E_UNSUPPORTED
    assert L.validate(desc(kv_fmt=L.CKV_FP4)) == L.CKV_E_UNSUPPORTED
    assert L.validate(desc(idx_fmt=4)) == L.CKV_E_UNSUPPORTED
    f32 = dict(kv_fmt=L.CKV_F32, act_fmt=L.CKV_F32, w_fmt=L.CKV_F32)
    assert L.validate(desc(flags=L.CKV_FLAG_KEEP_F32, idx_fmt=L.CKV_FP4, **f32)) == L.CKV_E_UNSUPPORTED
    # the decode workspace also holds each query's fp4 form (64 heads x 68 bytes)
    d4, d16 = desc(idx_fmt=L.CKV_FP4), desc()
    assert L.workspace_bytes(d4, L.CKV_MODE_DECODE, 16) == L.workspace_bytes(d16, L.CKV_MODE_DECODE, 16) + 16 * 64 * 68
    assert L.workspace_bytes(d4, L.CKV_MODE_PREFILL, 4096) == L.workspace_bytes(d16, L.CKV_MODE_PREFILL, 4096)


def test_row_bytes_and_workspace():
    assert L.row_bytes(L.CKV_E4M3, 512) == 640
    assert L.row_bytes(L.CKV_BF16, 512) == 1024
    assert L.row_bytes(L.CKV_F32, 128) == 512
    assert L.row_bytes(9, 128) == 0
    d = desc()
    ws = L.workspace_bytes(d, L.CKV_MODE_DECODE, 16)
    assert ws >= 16 * 32768 * 4 + 16 * 4096 * 4   # keys + histogram
    assert L.workspace_bytes(d, 7, 16) == 0
    assert L.workspace_bytes(desc(ratio=9), L.CKV_MODE_DECODE, 16) == 0
    assert L.strerror(L.CKV_E_CAPACITY).startswith("capacity")


FAKE = 1 << 40          # aligned, never dereferenced: every call below fails first
MIS = FAKE + 4          # misaligned


def cache(**kw):
    c = dict(raw=FAKE, comp=FAKE, idx=FAKE, st_kv=FAKE, st_sc=FAKE, ist_kv=FAKE, ist_sc=FAKE, raw_stage=FAKE,
             stage_rows=4096 + 127, status=None)
    c.update(kw)
    return L.LayerCache(**c)


def weights(**kw):
    w = {n: FAKE for n in ("wkv", "wgate", "ape", "gamma", "idx_wkv", "idx_wgate", "idx_ape", "idx_gamma")}
    w.update(kw)
    return L.LayerWeights(**w)


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="fake device addresses are only passed where no GPU exists")
def test_host_errors_before_any_enqueue():
    d = desc()
    ws = L.workspace_bytes(d, L.CKV_MODE_DECODE, 16)
    c, w = cache(), weights()
    # batch beyond the cache
    assert L.compress_append_decode(d, w, c, FAKE, FAKE, FAKE, 17, FAKE, ws) == L.CKV_E_CAPACITY
    assert L.compress_append_decode(d, w, c, FAKE, FAKE, FAKE, 0, FAKE, ws) == L.CKV_E_INVAL
    # workspace too small / missing / misaligned
    assert L.compress_append_decode(d, w, c, FAKE, FAKE, FAKE, 16, FAKE, ws - 1) == L.CKV_E_WORKSPACE
    assert L.indexer_topk_decode(d, c, FAKE, FAKE, FAKE, 16, FAKE, None, ws) == L.CKV_E_WORKSPACE
    assert L.indexer_topk_decode(d, c, FAKE, FAKE, FAKE, 16, FAKE, MIS, ws) == L.CKV_E_WORKSPACE
    # NULL / misaligned pointers
    assert L.compress_append_decode(d, w, c, None, FAKE, FAKE, 16, FAKE, ws) == L.CKV_E_INVAL
    assert L.compress_append_decode(d, weights(ape=MIS), c, FAKE, FAKE, FAKE, 16, FAKE, ws) == L.CKV_E_INVAL
    assert L.compress_append_decode(d, w, cache(comp=None), FAKE, FAKE, FAKE, 16, FAKE, ws) == L.CKV_E_INVAL
    assert L.sparse_swa_attn_decode(d, c, FAKE, FAKE, None, 16, FAKE, FAKE, ws) == L.CKV_E_INVAL  # r=4 needs topk
    assert L.sparse_swa_attn_decode(d, c, MIS, FAKE, FAKE, 16, FAKE, FAKE, ws) == L.CKV_E_INVAL
    # indexer on a ratio-128 layer
    d128 = desc(ratio=128, comp_cap=1024)
    assert L.indexer_topk_decode(d128, c, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 1 << 30) == L.CKV_E_UNSUPPORTED
    assert L.sparse_swa_attn_decode(d128, c, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 1 << 30) == L.CKV_E_INVAL
    # prefill limits
    wp = L.workspace_bytes(d, L.CKV_MODE_PREFILL, 4096)
    assert L.compress_append_prefill(d, w, c, FAKE, FAKE, 0, 0, 4097, FAKE, 1 << 40) == L.CKV_E_CAPACITY
    assert L.compress_append_prefill(d, w, c, FAKE, FAKE, 16, 0, 16, FAKE, wp) == L.CKV_E_CAPACITY
    assert L.compress_append_prefill(d, w, c, FAKE, FAKE, 0, -1, 16, FAKE, wp) == L.CKV_E_INVAL
    assert L.compress_append_prefill(d, w, c, FAKE, FAKE, 0, 4 * 32768 - 8, 16, FAKE, wp) == L.CKV_E_CAPACITY
    assert L.compress_append_prefill(d, w, cache(stage_rows=100), FAKE, FAKE, 0, 0, 16, FAKE, wp) == L.CKV_E_CAPACITY
    assert L.compress_append_prefill(d, w, cache(raw_stage=None), FAKE, FAKE, 0, 0, 16, FAKE, wp) == L.CKV_E_INVAL
    assert L.indexer_topk_prefill(d, c, FAKE, FAKE, 0, 0, 5000, FAKE, FAKE, wp) == L.CKV_E_CAPACITY
    assert L.sparse_swa_attn_prefill(d, c, FAKE, 0, 0, 16, FAKE, FAKE, FAKE, 16) == L.CKV_E_WORKSPACE
    # the single-call prefill chunk: the three calls' checks
    pc = lambda **k: L.prefill_chunk(k.get("d", d), k.get("w", w), k.get("c", c), k.get("x", FAKE), FAKE,
                                     k.get("q", FAKE), k.get("qI", FAKE), k.get("iw", FAKE), 0, k.get("pos0", 0),
                                     k.get("T", 16), k.get("topk", FAKE), k.get("out", FAKE), FAKE, k.get("wsb", wp),
                                     None, k.get("side", FAKE))
    assert pc(T=4097) == L.CKV_E_CAPACITY
    assert pc(pos0=-1) == L.CKV_E_INVAL
    assert pc(wsb=16) == L.CKV_E_WORKSPACE
    assert pc(topk=None) == L.CKV_E_INVAL and pc(topk=MIS) == L.CKV_E_INVAL
    assert pc(qI=None) == L.CKV_E_INVAL and pc(iw=None) == L.CKV_E_INVAL
    assert pc(x=None) == L.CKV_E_INVAL and pc(out=None) == L.CKV_E_INVAL
    assert pc(c=cache(stage_rows=100)) == L.CKV_E_CAPACITY
    assert pc(w=weights(idx_gamma=None)) == L.CKV_E_INVAL
    # the single-call decode step: same checks, all before anything is enqueued
    st = lambda **k: L.decode_step(k.get("d", d), k.get("w", w), k.get("c", c), k.get("x", FAKE), FAKE,
                                   k.get("q", FAKE), k.get("qI", FAKE), k.get("iw", FAKE), FAKE, k.get("B", 16),
                                   k.get("topk", FAKE), k.get("out", FAKE), k.get("ws", FAKE), k.get("wsb", ws))
    assert st(B=17) == L.CKV_E_CAPACITY
    assert st(B=0) == L.CKV_E_INVAL
    assert st(wsb=ws - 1) == L.CKV_E_WORKSPACE
    assert st(ws=MIS) == L.CKV_E_WORKSPACE
    assert st(topk=None) == L.CKV_E_INVAL          # ratio 4 needs the top-k output
    assert st(qI=None) == L.CKV_E_INVAL
    assert st(iw=MIS) == L.CKV_E_INVAL
    assert st(out=None) == L.CKV_E_INVAL
    assert st(q=MIS) == L.CKV_E_INVAL
    assert st(x=None) == L.CKV_E_INVAL
    assert st(w=weights(idx_gamma=None)) == L.CKV_E_INVAL
    assert st(c=cache(idx=None)) == L.CKV_E_INVAL
    assert st(d=desc(ratio=5)) == L.CKV_E_UNSUPPORTED
    d0 = desc(ratio=0, comp_cap=0)
    assert st(d=d0, wsb=L.workspace_bytes(d0, L.CKV_MODE_DECODE, 16), out=MIS) == L.CKV_E_INVAL
    # invalid description
    assert L.compress_append_decode(desc(ratio=5), w, c, FAKE, FAKE, FAKE, 1, FAKE, ws) == L.CKV_E_UNSUPPORTED
    assert L.lib.ckv_validate(None) == L.CKV_E_INVAL
    # misaligned token counts / status words
    assert L.compress_append_decode(d, w, cache(n_tokens=FAKE + 2), FAKE, FAKE, FAKE, 16, FAKE, ws) == L.CKV_E_INVAL
    assert L.compress_append_decode(d, w, cache(status=FAKE + 1), FAKE, FAKE, FAKE, 16, FAKE, ws) == L.CKV_E_INVAL


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="fake device addresses are only passed where no GPU exists")
def test_static_workspace_step_refuses_what_does_not_fit():
    """The workspace-free decode step checks everything on the host first: a
    batch whose workspace exceeds the library's array, and the ordinary
    argument errors, return before any GPU call."""
    d = desc(batch=128, comp_cap=32768)
    assert L.workspace_bytes(d, L.CKV_MODE_DECODE, 128) > L.CKV_STATIC_WORKSPACE_BYTES
    st = lambda d, B, **k: L.decode_step_static(d, weights(), cache(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B,
                                                k.get("topk", FAKE), FAKE)
    assert st(d, 128) == L.CKV_E_WORKSPACE
    assert st(desc(), 17) == L.CKV_E_CAPACITY
    assert st(desc(), 0) == L.CKV_E_INVAL
    assert st(desc(), 16, topk=None) == L.CKV_E_INVAL
    assert st(desc(ratio=5), 16) == L.CKV_E_UNSUPPORTED
    assert L.workspace_bytes(desc(), L.CKV_MODE_DECODE, 16) <= L.CKV_STATIC_WORKSPACE_BYTES


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="fake device addresses are only passed where no GPU exists")
def test_prefill_out_of_sequence_is_refused_on_the_host():
    """With the host mirror of the token counts, a chunk that does not start
    at its sequence's next position returns CKV_E_SEQUENCE before any work is
    enqueued (the pages' engine refuses KV state whose token prefix does not
    match).  A matching pos0 passes that check and fails later, on the
    missing workspace, still before any enqueue."""
    import numpy as np
    d = desc()
    counts = np.array([61440] + [0] * 15, np.int32)
    c = cache(n_tokens=FAKE, n_tokens_host=counts.ctypes.data)
    w = weights()
    wp = L.workspace_bytes(d, L.CKV_MODE_PREFILL, 4096)
    for pos0 in (61439, 61441, 0, 65536):
        assert L.compress_append_prefill(d, w, c, FAKE, FAKE, 0, pos0, 4096, FAKE, wp) == L.CKV_E_SEQUENCE
    assert L.compress_append_prefill(d, w, c, FAKE, FAKE, 0, 61440, 4096, None, wp) == L.CKV_E_WORKSPACE
    assert L.compress_append_prefill(d, w, c, FAKE, FAKE, 3, 8, 16, FAKE, wp) == L.CKV_E_SEQUENCE
    assert L.strerror(L.CKV_E_SEQUENCE).startswith("position")


def test_stack_schedule_matches_the_oracle():
    """The stack driver's per-layer ratio rule against the oracle's schedules."""
    import oracle as O
    from compressed_kv_sparse_amd.stack import layer_ratio
    for il in range(61):
        assert layer_ratio(il, "flash") == O.flash_ratio(il)
        assert layer_ratio(il, "pro") == O.pro_ratio(il)
    with pytest.raises(ValueError):
        layer_ratio(0, "other")


def test_score_timing_arms_and_disarms_without_a_device():
    # arming only records two handles for the calling thread; no GPU call
    assert L.time_next_score(None, None) == 0
    assert L.lib.ckv_time_next_score(None, None) == 0


def test_hc_validate():
    """The Hyper-Connection mixer's description: 4 streams, hidden a multiple of
    8 up to 65536, 1..100 Sinkhorn iterations, finite eps >= 0, f32 / bf16."""
    good = dict(hidden=4096, n_hc=4, sinkhorn_iters=20, eps=1e-6, act_fmt=L.CKV_BF16)
    assert L.hc_validate(L.HcDesc(**good)) == 0
    assert L.hc_validate(L.HcDesc(**dict(good, act_fmt=L.CKV_F32, hidden=8, sinkhorn_iters=1, eps=0.0))) == 0
    for kw in (dict(n_hc=2), dict(hidden=100), dict(hidden=65544), dict(hidden=0), dict(sinkhorn_iters=0),
               dict(sinkhorn_iters=101), dict(eps=-1.0), dict(eps=float("inf")), dict(eps=float("nan")),
               dict(act_fmt=L.CKV_E4M3)):
        assert L.hc_validate(L.HcDesc(**dict(good, **kw))) == L.CKV_E_UNSUPPORTED, kw
    d = L.HcDesc(**good)
    # NULL or misaligned pointers and T < 1 fail before any enqueue (no device needed)
    assert L.hc_pre(d, 0, FAKE, 4, FAKE, FAKE, None) == L.CKV_E_INVAL
    assert L.hc_pre(d, FAKE, FAKE, 4, MIS, FAKE, None) == L.CKV_E_INVAL
    assert L.hc_pre(d, FAKE, FAKE, 0, FAKE + (1 << 30), FAKE, None) == L.CKV_E_INVAL
    assert L.hc_post(d, FAKE, FAKE, FAKE, 4, 0, None) == L.CKV_E_INVAL
    # outputs overlapping their inputs
    assert L.hc_pre(d, FAKE, FAKE, 4, FAKE + 16, FAKE + (1 << 30), None) == L.CKV_E_INVAL
    assert L.hc_post(d, FAKE + (1 << 30), FAKE, FAKE + (1 << 31), 4, FAKE + 4096, None) == L.CKV_E_INVAL


def test_out_fp8_flag():
    """CKV_FLAG_OUT_FP8 (attention output as E4M3 records with group scales) is
    accepted on the tiled attention's shapes only."""
    f = L.CKV_FLAG_OUT_FP8
    assert L.validate(desc(flags=f)) == 0
    assert L.validate(desc(flags=f, kv_fmt=L.CKV_BF16, ratio=128, comp_cap=8192)) == 0
    assert L.validate(desc(flags=f, ratio=0, comp_cap=0)) == 0
    for kw in (dict(act_fmt=L.CKV_F32), dict(kv_fmt=L.CKV_F32), dict(head_dim=256), dict(n_heads=32)):
        assert L.validate(desc(flags=f, **kw)) == L.CKV_E_UNSUPPORTED, kw


def test_q_norm_flag():
    """CKV_FLAG_Q_NORM (each head's query RMS-normalised in the attention) is
    accepted on every layer shape and combines with the other flags; its value
    is the one the test harness gives the oracle."""
    from harness import Q_NORM_FLAG
    f = L.CKV_FLAG_Q_NORM
    assert f == Q_NORM_FLAG == 64
    for kw in (dict(), dict(act_fmt=L.CKV_F32, kv_fmt=L.CKV_F32, w_fmt=L.CKV_F32, idx_fmt=L.CKV_F32),
               dict(head_dim=256), dict(n_heads=32), dict(ratio=0, comp_cap=0)):
        assert L.validate(desc(flags=f, **kw)) == 0, kw
    assert L.validate(desc(flags=f | L.CKV_FLAG_OUT_FP8 | L.CKV_FLAG_NO_INV_ROPE)) == 0


def test_two_lane_flag():
    """CKV_FLAG_TWO_LANE: ratio-4 layers only; the projection doubles (the
    prefill workspace's projection region grows with it)."""
    f = L.CKV_FLAG_TWO_LANE
    assert f == 128
    assert L.validate(desc(flags=f)) == 0
    assert L.validate(desc(flags=f, idx_fmt=L.CKV_FP4)) == 0
    assert L.validate(desc(flags=f, ratio=128, comp_cap=8192)) == L.CKV_E_UNSUPPORTED
    assert L.validate(desc(flags=f, ratio=0, comp_cap=0)) == L.CKV_E_UNSUPPORTED
    one, two = desc(), desc(flags=f)
    grow = L.workspace_bytes(two, L.CKV_MODE_PREFILL, 4096) - L.workspace_bytes(one, L.CKV_MODE_PREFILL, 4096)
    assert grow >= 4096 * (2 * 512 + 2 * 128) * 4 - 256
