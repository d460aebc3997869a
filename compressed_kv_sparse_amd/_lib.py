"""ctypes binding of libckv.so (the C ABI declared in include/ckv.h).

Argument marshalling only: every entry point takes plain integers / device
addresses and forwards them to the library.  Importing this module loads the
library and fails loudly when it has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libckv.so")

CKV_OK = 0
CKV_E_INVAL = -1
CKV_E_UNSUPPORTED = -2
CKV_E_CAPACITY = -3
CKV_E_WORKSPACE = -4
CKV_E_HIP = -5
CKV_E_SEQUENCE = -6

CKV_F32, CKV_BF16, CKV_E4M3, CKV_FP4 = 0, 1, 2, 3
FMT = {"f32": CKV_F32, "bf16": CKV_BF16, "e4m3": CKV_E4M3, "fp4": CKV_FP4}
CKV_FLAG_NO_INV_ROPE = 1
CKV_FLAG_IDX_NO_RELU = 2
CKV_FLAG_SKIP_NORM = 4
CKV_FLAG_SKIP_ROPE = 8
CKV_FLAG_KEEP_F32 = 16
CKV_FLAG_OUT_FP8 = 32
CKV_FLAG_Q_NORM = 64
CKV_FLAG_TWO_LANE = 128
CKV_MODE_DECODE, CKV_MODE_PREFILL = 0, 1
CKV_MAX_CHUNK = 4096
CKV_STATIC_WORKSPACE_BYTES = 48 << 20
CKV_STATUS_BAD_POS = 1
CKV_STATUS_CAPACITY = 2
CKV_STATUS_SEQUENCE = 4
CKV_STATUS_PAGE = 8


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("ratio", ctypes.c_int32), ("hidden", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_rot", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("swa", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("comp_cap", ctypes.c_int32), ("batch", ctypes.c_int32), ("kv_fmt", ctypes.c_int32),
        ("idx_fmt", ctypes.c_int32), ("act_fmt", ctypes.c_int32), ("w_fmt", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("rope_base", ctypes.c_double), ("norm_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float), ("rope_base_comp", ctypes.c_double),
    ]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("wkv", "wgate", "ape", "gamma", "idx_wkv", "idx_wgate", "idx_ape", "idx_gamma")]


class LayerCache(ctypes.Structure):
    _fields_ = [
        ("raw", ctypes.c_void_p), ("comp", ctypes.c_void_p), ("idx", ctypes.c_void_p),
        ("st_kv", ctypes.c_void_p), ("st_sc", ctypes.c_void_p), ("ist_kv", ctypes.c_void_p),
        ("ist_sc", ctypes.c_void_p), ("raw_stage", ctypes.c_void_p), ("stage_rows", ctypes.c_int32),
        ("status", ctypes.c_void_p), ("n_tokens", ctypes.c_void_p), ("n_tokens_host", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("n_pages", ctypes.c_int32),
    ]


class HcDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_hc", ctypes.c_int32), ("sinkhorn_iters", ctypes.c_int32),
                ("eps", ctypes.c_float), ("act_fmt", ctypes.c_int32)]


class CkvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        extra = f" [{lib.ckv_last_hip_error().decode()}]" if code == CKV_E_HIP else ""
        super().__init__(f"{where}: {strerror(code)} ({code}){extra}")


def _load() -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime whose libraries ask for it by a file
    # name that does not match an already-mapped /opt/rocm runtime, so loading
    # libckv first would leave two HIP runtimes in the process (the second sees
    # no device).  With torch loaded first, libckv's libamdhip64.so.7 and
    # libhsa-runtime64.so.1 dependencies resolve to the copies torch mapped.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libckv.so is not built at {LIB_PATH}; run "
                          "`python compressed_kv_sparse_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    D, Wt, C = P(LayerDesc), P(LayerWeights), P(LayerCache)
    lib.ckv_row_bytes.argtypes = [I32, I32, I32]
    lib.ckv_row_bytes.restype = SZ
    lib.ckv_idx_row_bytes.argtypes = [I32, I32]
    lib.ckv_idx_row_bytes.restype = SZ
    lib.ckv_validate.argtypes = [D]
    lib.ckv_validate.restype = ctypes.c_int
    lib.ckv_strerror.argtypes = [ctypes.c_int]
    lib.ckv_strerror.restype = ctypes.c_char_p
    lib.ckv_last_hip_error.argtypes = []
    lib.ckv_last_hip_error.restype = ctypes.c_char_p
    lib.ckv_time_next_score.argtypes = [VP, VP]
    lib.ckv_time_next_score.restype = I32
    lib.ckv_workspace_bytes.argtypes = [D, I32, I32]
    lib.ckv_workspace_bytes.restype = SZ
    lib.ckv_workspace_sync_bytes.argtypes = [D, I32, I32]
    lib.ckv_workspace_sync_bytes.restype = SZ
    sig = {
        "ckv_compress_append_decode": [D, Wt, C, VP, VP, VP, I32, VP, SZ, VP],
        "ckv_compress_append_prefill": [D, Wt, C, VP, VP, I32, I32, I32, VP, SZ, VP],
        "ckv_indexer_topk_decode": [D, C, VP, VP, VP, I32, VP, VP, SZ, VP],
        "ckv_indexer_topk_prefill": [D, C, VP, VP, I32, I32, I32, VP, VP, SZ, VP],
        "ckv_indexer_score_decode": [D, C, VP, VP, VP, I32, VP, VP],
        "ckv_sparse_swa_attn_decode": [D, C, VP, VP, VP, I32, VP, VP, SZ, VP],
        "ckv_sparse_swa_attn_prefill": [D, C, VP, I32, I32, I32, VP, VP, VP, SZ, VP],
        "ckv_decode_step": [D, Wt, C, VP, VP, VP, VP, VP, VP, I32, VP, VP, VP, SZ, VP],
        "ckv_decode_step_static": [D, Wt, C, VP, VP, VP, VP, VP, VP, I32, VP, VP, VP],
        "ckv_prefill_chunk": [D, Wt, C, VP, VP, VP, VP, VP, I32, I32, I32, VP, VP, VP, SZ, VP, VP],
        "ckv_hc_validate": [P(HcDesc)],
        "ckv_hc_pre": [P(HcDesc), VP, VP, I32, VP, VP, VP],
        "ckv_hc_post": [P(HcDesc), VP, VP, VP, I32, VP, VP],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    return lib


lib = _load()

EXPORTS = ("ckv_row_bytes", "ckv_idx_row_bytes", "ckv_validate", "ckv_strerror", "ckv_last_hip_error", "ckv_workspace_bytes",
           "ckv_workspace_sync_bytes",
           "ckv_compress_append_decode", "ckv_compress_append_prefill", "ckv_indexer_topk_decode",
           "ckv_indexer_topk_prefill", "ckv_indexer_score_decode", "ckv_sparse_swa_attn_decode",
           "ckv_sparse_swa_attn_prefill", "ckv_decode_step", "ckv_time_next_score", "ckv_decode_step_static",
           "ckv_hc_validate", "ckv_hc_pre", "ckv_hc_post", "ckv_prefill_chunk")


def strerror(code: int) -> str:
    return lib.ckv_strerror(int(code)).decode()


def row_bytes(fmt: int, head_dim: int, n_rot: int = 64) -> int:
    return int(lib.ckv_row_bytes(fmt, head_dim, n_rot))


def idx_row_bytes(fmt: int, idx_dim: int) -> int:
    return int(lib.ckv_idx_row_bytes(fmt, idx_dim))


def validate(desc: LayerDesc) -> int:
    return int(lib.ckv_validate(ctypes.byref(desc)))


def workspace_bytes(desc: LayerDesc, mode: int, n: int) -> int:
    return int(lib.ckv_workspace_bytes(ctypes.byref(desc), mode, n))


def workspace_sync_bytes(desc: LayerDesc, mode: int, n: int) -> int:
    return int(lib.ckv_workspace_sync_bytes(ctypes.byref(desc), mode, n))


def _p(x) -> int:
    """Device address of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _ref(s):
    return None if s is None else ctypes.byref(s)


def compress_append_decode(desc, weights, cache, x, u, pos, B, ws, ws_bytes, stream=None) -> int:
    return lib.ckv_compress_append_decode(_ref(desc), _ref(weights), _ref(cache), _p(x), _p(u), _p(pos),
                                          int(B), _p(ws), int(ws_bytes), stream)


def compress_append_prefill(desc, weights, cache, x, u, seq, pos0, T, ws, ws_bytes, stream=None) -> int:
    return lib.ckv_compress_append_prefill(_ref(desc), _ref(weights), _ref(cache), _p(x), _p(u), int(seq),
                                           int(pos0), int(T), _p(ws), int(ws_bytes), stream)


def indexer_topk_decode(desc, cache, qI, w, pos, B, topk, ws, ws_bytes, stream=None) -> int:
    return lib.ckv_indexer_topk_decode(_ref(desc), _ref(cache), _p(qI), _p(w), _p(pos), int(B), _p(topk),
                                       _p(ws), int(ws_bytes), stream)


def time_next_score(start_event, stop_event) -> int:
    """Arm this thread's next indexer score launch to stamp two timing events
    (torch.cuda.Event objects, already recorded once so that they exist, or
    raw hipEvent_t handles; None disarms)."""
    def h(e):
        if e is None:
            return None
        return int(getattr(e, "cuda_event", e))
    return lib.ckv_time_next_score(h(start_event), h(stop_event))


def indexer_score_decode(desc, cache, qI, w, pos, B, keys, stream=None) -> int:
    return lib.ckv_indexer_score_decode(_ref(desc), _ref(cache), _p(qI), _p(w), _p(pos), int(B), _p(keys),
                                        stream)


def indexer_topk_prefill(desc, cache, qI, w, seq, pos0, T, topk, ws, ws_bytes, stream=None) -> int:
    return lib.ckv_indexer_topk_prefill(_ref(desc), _ref(cache), _p(qI), _p(w), int(seq), int(pos0), int(T),
                                        _p(topk), _p(ws), int(ws_bytes), stream)


def sparse_swa_attn_decode(desc, cache, q, pos, topk, B, out, ws, ws_bytes, stream=None) -> int:
    return lib.ckv_sparse_swa_attn_decode(_ref(desc), _ref(cache), _p(q), _p(pos), _p(topk), int(B), _p(out),
                                          _p(ws), int(ws_bytes), stream)


def sparse_swa_attn_prefill(desc, cache, q, seq, pos0, T, topk, out, ws, ws_bytes, stream=None) -> int:
    return lib.ckv_sparse_swa_attn_prefill(_ref(desc), _ref(cache), _p(q), int(seq), int(pos0), int(T),
                                           _p(topk), _p(out), _p(ws), int(ws_bytes), stream)


def decode_step(desc, weights, cache, x, u, q, qI, w, pos, B, topk, out, ws, ws_bytes, stream=None) -> int:
    return lib.ckv_decode_step(_ref(desc), _ref(weights), _ref(cache), _p(x), _p(u), _p(q), _p(qI), _p(w),
                               _p(pos), int(B), _p(topk), _p(out), _p(ws), int(ws_bytes), stream)


def decode_step_static(desc, weights, cache, x, u, q, qI, w, pos, B, topk, out, stream=None) -> int:
    return lib.ckv_decode_step_static(_ref(desc), _ref(weights), _ref(cache), _p(x), _p(u), _p(q), _p(qI), _p(w),
                                      _p(pos), int(B), _p(topk), _p(out), stream)


def prefill_chunk(desc, weights, cache, x, u, q, qI, w, seq, pos0, T, topk, out, ws, ws_bytes, stream=None,
                  side_stream=None) -> int:
    return lib.ckv_prefill_chunk(_ref(desc), _ref(weights), _ref(cache), _p(x), _p(u), _p(q), _p(qI), _p(w),
                                 int(seq), int(pos0), int(T), _p(topk), _p(out), _p(ws), int(ws_bytes), stream,
                                 side_stream)


def hc_validate(desc: HcDesc) -> int:
    return int(lib.ckv_hc_validate(ctypes.byref(desc)))


def hc_pre(desc: HcDesc, mix: int, h: int, T: int, x: int, coef: int, stream) -> int:
    return int(lib.ckv_hc_pre(ctypes.byref(desc), mix, h, T, x, coef, stream))


def hc_post(desc: HcDesc, coef: int, h: int, y: int, T: int, h_out: int, stream) -> int:
    return int(lib.ckv_hc_post(ctypes.byref(desc), coef, h, y, T, h_out, stream))
