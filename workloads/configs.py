"""Workload registry: the five layer shapes the method is exercised on.

Shapes follow the DeepSeek-V4 Flash attention layout described in
"ds4.c を読み解く (#3)" (section 1 for the per-layer ratio schedule, section 2
for the 128-row sliding window, section 6 for the 64x128 indexer with top-k
512, section 8 for head_dim 512 with a 64-dim RoPE tail) and in the vLLM
DeepSeek V4 page ("DeepSeek V4 attention architecture": c4a = 8 tokens at
stride 4, c128a = 128 tokens at stride 128, SWA 128, shared K=V).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

# RoPE bases.  The pages name a normal base and a separate base for
# compressed layers ("ds4.c を読み解く (#3)", section 8) without values; the
# values are the workload's: 10000 for uncompressed layers and raw rows,
# 160000 for compressed ones.  The layers of the 1024-token tiny workload keep
# one base per row class (raw rows 10000, compressed and indexer rows 160000,
# as its description states); the other workloads use one base per layer
# (the layer's choice applies to the query, the raw rows, the compressed rows
# and the indexer alike).
ROPE_BASE_RAW = 10000.0
ROPE_BASE_COMPRESSED = 160000.0


def flash_ratio(il: int) -> int:
    """Compression ratio of layer ``il`` in the Flash stack.

    Layers 0-1 are uncompressed; from layer 2 on, even layers are ratio 4 and
    odd layers ratio 128 ("ds4.c を読み解く (#3)", section 1).
    """
    if il < 2:
        return 0
    return 4 if (il & 1) == 0 else 128


def window_of(ratio: int) -> int:
    """Compressor window: 8 tokens for ratio 4, 128 for ratio 128 (vLLM page, c4a/c128a)."""
    return {4: 8, 128: 128}.get(ratio, 0)


# ckv_layer_desc.flags bit of the two-lane c4a compressors
TWO_LANE_FLAG = 128


@dataclass(frozen=True)
class LayerShape:
    name: str
    ratio: int                 # 0, 4 or 128
    hidden: int                # D
    head_dim: int              # d
    n_heads: int               # H (query heads; one shared K=V head)
    idx_heads: int             # H_I (0 when ratio != 4)
    idx_dim: int               # D_I
    top_k: int                 # k
    batch: int                 # sequences (decode) or 1 (prefill)
    n_ctx: int                 # tokens seen including the query (decode)
    comp_cap: int              # compressed rows per sequence the cache holds
    kv_fmt: str = "bf16"       # f32 | bf16 | e4m3
    idx_fmt: str = "bf16"      # f32 | bf16 | fp4 (Hadamard + MXFP4 records)
    act_fmt: str = "bf16"      # f32 | bf16
    w_fmt: str = "bf16"        # f32 | bf16
    n_rot: int = 64
    swa: int = 128
    rope_base: float = ROPE_BASE_COMPRESSED
    # base of the compressed-row class (compressed rows, indexer rows and the
    # query's rotation against them); None: ``rope_base`` serves every class
    rope_base_comp: Optional[float] = None
    norm_eps: float = 1e-6
    seed: int = 1
    # distributions (standard deviations)
    w_std: Optional[float] = None     # None -> 1/sqrt(hidden)
    ape_std: Optional[float] = None   # None -> 1/sqrt(head_dim)
    gamma_std: float = 0.0            # gamma = 1 + gamma_std * N(0,1)
    # prefill
    pos0: int = 0
    chunk: int = 0
    # variable context lengths per sequence (inclusive range); None -> all n_ctx
    ctx_range: Optional[Tuple[int, int]] = None
    layer: int = 0
    flags: int = 0                    # ckv_layer_desc.flags (e.g. 32: attention output as fp8 records)
    paged: bool = False               # compressed rows in scattered 256-position pages (block table)

    @property
    def two_lane(self) -> bool:
        """Ratio 4 with two-lane compressors (projections 2 d / 2 D_I, APE [4, 2 w])."""
        return bool(self.flags & TWO_LANE_FLAG) and self.ratio == 4

    @property
    def lanes(self) -> int:
        return 2 if self.two_lane else 1

    @property
    def window(self) -> int:
        return window_of(self.ratio)

    @property
    def d_nope(self) -> int:
        return self.head_dim - self.n_rot

    @property
    def scale(self) -> float:
        return self.head_dim ** -0.5

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


def _c1() -> LayerShape:
    return LayerShape(
        name="c1_tiny_c4a_decode_ctx1024_f32", ratio=4, hidden=1024, head_dim=128,
        n_heads=16, idx_heads=4, idx_dim=64, top_k=32, batch=1, n_ctx=1024,
        comp_cap=256, kv_fmt="f32", idx_fmt="f32", act_fmt="f32", w_fmt="f32",
        w_std=0.02, ape_std=0.1, seed=1,
        rope_base=ROPE_BASE_RAW, rope_base_comp=ROPE_BASE_COMPRESSED)


def _c2() -> LayerShape:
    return LayerShape(
        name="c2_c4a_decode_b32_ctx65536_bf16", ratio=4, hidden=4096, head_dim=512,
        n_heads=64, idx_heads=8, idx_dim=128, top_k=512, batch=32, n_ctx=65536,
        comp_cap=16384, seed=2)


def _c3() -> LayerShape:
    return LayerShape(
        name="c3_c128a_decode_b8_ctx1m_bf16", ratio=128, hidden=4096, head_dim=512,
        n_heads=64, idx_heads=0, idx_dim=0, top_k=0, batch=8, n_ctx=1 << 20,
        comp_cap=8192, ctx_range=(524288, 1048576), seed=3)


def _c4() -> LayerShape:
    return LayerShape(
        name="c4_c4a_prefill_T4096_at61440_bf16", ratio=4, hidden=4096, head_dim=512,
        n_heads=64, idx_heads=64, idx_dim=128, top_k=512, batch=1, n_ctx=65536,
        comp_cap=16384, pos0=61440, chunk=4096, seed=4)


def _c5(ratio: int = 4, layer: int = 2) -> LayerShape:
    name = {4: "c5_c4a_decode_b16_ctx131072_fp8",
            128: "c5_c128a_decode_b16_ctx131072_fp8",
            0: "c5_swa_decode_b16_ctx131072_fp8"}[ratio]
    return LayerShape(
        name=name, ratio=ratio, hidden=4096, head_dim=512, n_heads=64,
        idx_heads=64 if ratio == 4 else 0, idx_dim=128 if ratio == 4 else 0,
        top_k=512 if ratio == 4 else 0, batch=16, n_ctx=131072,
        comp_cap={4: 32768, 128: 1024, 0: 0}[ratio], kv_fmt="e4m3", idx_fmt="bf16",
        rope_base=ROPE_BASE_COMPRESSED if ratio else ROPE_BASE_RAW,
        gamma_std=0.1, seed=5, layer=layer)


CONFIGS: Dict[str, LayerShape] = {}
for _f in (_c1, _c2, _c3, _c4):
    _c = _f()
    CONFIGS[_c.name] = _c
for _r, _l in ((4, 2), (128, 3), (0, 0)):
    _c = _c5(_r, _l)
    CONFIGS[_c.name] = _c
# the same c4a decode and prefill workloads with the indexer cache in the
# quantisation-aware fp4 form (Hadamard-128 + MXFP4 records of 68 bytes)
for _c in (_c5(4, 2).with_(name="c5_c4a_decode_b16_ctx131072_fp8_fp4idx", idx_fmt="fp4"),
           _c4().with_(name="c4_c4a_prefill_T4096_at61440_bf16_fp4idx", idx_fmt="fp4")):
    CONFIGS[_c.name] = _c
# the C5 c4a decode with the attention output written as fp8 records (the
# inverse RoPE fused with the output's E4M3 quantisation)
_c = _c5(4, 2).with_(name="c5_c4a_decode_b16_ctx131072_fp8_out8", flags=32)
CONFIGS[_c.name] = _c
# ... and with each head's query RMS-normalised inside the attention
_c = _c5(4, 2).with_(name="c5_c4a_decode_b16_ctx131072_fp8_qnorm", flags=64)
CONFIGS[_c.name] = _c
# the C5 c4a decode and the C4 chunk with two-lane compressors
for _c in (_c5(4, 2).with_(name="c5_c4a_decode_b16_ctx131072_fp8_two_lane", flags=TWO_LANE_FLAG),
           _c4().with_(name="c4_c4a_prefill_T4096_at61440_bf16_two_lane", flags=TWO_LANE_FLAG)):
    CONFIGS[_c.name] = _c
# ... and with the compressed and indexer rows in scattered pages of a pool
_c = _c5(4, 2).with_(name="c5_c4a_decode_b16_ctx131072_fp8_paged", paged=True)
CONFIGS[_c.name] = _c

# short aliases
ALIASES = {
    "c1": "c1_tiny_c4a_decode_ctx1024_f32",
    "c2": "c2_c4a_decode_b32_ctx65536_bf16",
    "c3": "c3_c128a_decode_b8_ctx1m_bf16",
    "c4": "c4_c4a_prefill_T4096_at61440_bf16",
    "c5": "c5_c4a_decode_b16_ctx131072_fp8",
    "c5_c128a": "c5_c128a_decode_b16_ctx131072_fp8",
    "c5_swa": "c5_swa_decode_b16_ctx131072_fp8",
    "c5_fp4idx": "c5_c4a_decode_b16_ctx131072_fp8_fp4idx",
    "c4_fp4idx": "c4_c4a_prefill_T4096_at61440_bf16_fp4idx",
    "c5_out8": "c5_c4a_decode_b16_ctx131072_fp8_out8",
    "c5_qnorm": "c5_c4a_decode_b16_ctx131072_fp8_qnorm",
    "c5_paged": "c5_c4a_decode_b16_ctx131072_fp8_paged",
    "c5_two_lane": "c5_c4a_decode_b16_ctx131072_fp8_two_lane",
    "c4_two_lane": "c4_c4a_prefill_T4096_at61440_bf16_two_lane",
}


def get_config(name: str) -> LayerShape:
    return CONFIGS[ALIASES.get(name, name)]


def stack_layer(il: int) -> LayerShape:
    """Layer ``il`` of the 43-layer Flash attention stack at 128k context."""
    r = flash_ratio(il)
    return _c5(r, il).with_(name=f"c5_stack_L{il:02d}_r{r}", seed=5000 + il, layer=il)
