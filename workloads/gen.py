"""Seeded input draws for the compressed-KV layer.

Every tensor gets its own PCG64 stream keyed by (config seed, tensor name,
layer, optional sub-key), so adding a tensor never shifts another one's
values.  Values are returned as the exact stored bit patterns:

* ``f32``  -> float32 arrays
* ``bf16`` -> uint16 arrays holding bfloat16 bit patterns (a float32 draw with
  its low 16 bits dropped: a draw from a bf16-valued distribution, not a
  rounding step of the method)
* ``e4m3`` -> uint8 row records (see :func:`row_bytes`) whose fp8 codes are
  drawn directly as sign / exponent / mantissa fields.
* ``fp4`` (indexer rows) -> uint8 records (see :func:`idx_row_bytes`) whose
  4-bit codes and block-scale bytes are drawn directly.

Nothing here projects, pools, normalises, rotates, scores, selects or
attends.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from .configs import LayerShape

# ---------------------------------------------------------------------------
# stored row layout (an interface fact shared by the library and its checker)
# ---------------------------------------------------------------------------

ROW_ALIGN = 128


def row_bytes(fmt: str, d: int, n_rot: int = 64) -> int:
    """Bytes one stored K=V row occupies in a cache of format ``fmt``.

    ``e4m3`` rows hold the d - n_rot non-RoPE channels as one fp8 E4M3 code
    each, then the n_rot RoPE channels as bfloat16, then one float32 row
    scale; the record is padded to a multiple of 128 bytes so that every row
    starts on a cache-line boundary.
    """
    if fmt == "f32":
        return 4 * d
    if fmt == "bf16":
        return 2 * d
    if fmt == "e4m3":
        raw = (d - n_rot) + 2 * n_rot + 4
        return (raw + ROW_ALIGN - 1) // ROW_ALIGN * ROW_ALIGN
    raise ValueError(fmt)


def idx_row_bytes(fmt: str, dim: int) -> int:
    """Bytes one stored indexer row occupies: f32 4 dim, bf16 2 dim; ``fp4``
    records hold dim/2 bytes of 4-bit codes (two channels a byte, the even
    channel in the low nibble) and then dim/32 one-byte block scales."""
    if fmt == "f32":
        return 4 * dim
    if fmt == "bf16":
        return 2 * dim
    if fmt == "fp4":
        return dim // 2 + dim // 32
    raise ValueError(fmt)


def e4m3_row_offsets(d: int, n_rot: int = 64):
    """(tail offset, scale offset) inside an e4m3 row record."""
    return d - n_rot, (d - n_rot) + 2 * n_rot


# ---------------------------------------------------------------------------
# streams
# ---------------------------------------------------------------------------

def _rng(seed: int, name: str, *sub: int) -> np.random.Generator:
    key = [zlib.crc32(name.encode()) & 0x7FFFFFFF] + [int(s) & 0x7FFFFFFF for s in sub]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _normal32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def bf16_bits_of_draw(a32: np.ndarray) -> np.ndarray:
    """Keep the high 16 bits of float32 draws (a bf16-valued draw)."""
    return (np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def draw_values(rng, shape, fmt: str, std: float = 1.0) -> np.ndarray:
    a = _normal32(rng, shape, std)
    if fmt == "f32":
        return a
    if fmt == "bf16":
        return bf16_bits_of_draw(a)
    raise ValueError(fmt)


def draw_e4m3_codes(rng, shape) -> np.ndarray:
    """fp8 E4M3 codes with roughly normal magnitudes around 2^6.

    Sign and magnitude octave follow a normal draw g (exponent field
    floor(log2|g|) + 13, clipped to 1..15); the 3 mantissa bits are uniform.
    The NaN pattern (exponent 15, mantissa 7) is never produced.
    """
    g = rng.standard_normal(size=shape, dtype=np.float32)
    sign = (g < 0).astype(np.uint8)
    mag = np.maximum(np.abs(g), np.float32(1e-30))
    e = np.clip(np.floor(np.log2(mag)).astype(np.int32) + 13, 1, 15).astype(np.uint8)
    m = rng.integers(0, 8, size=shape, dtype=np.uint8)
    m = np.where((e == 15) & (m == 7), np.uint8(6), m).astype(np.uint8)
    return (sign << 7) | (e << 3) | m


def draw_rows(rng, n_rows_shape, fmt: str, d: int, n_rot: int = 64) -> np.ndarray:
    """Draw stored K=V rows; returns uint8 records [..., row_bytes]."""
    shape = tuple(n_rows_shape)
    rb = row_bytes(fmt, d, n_rot)
    if fmt in ("f32", "bf16"):
        v = draw_values(rng, shape + (d,), fmt)
        return np.ascontiguousarray(v).view(np.uint8).reshape(shape + (rb,))
    out = np.zeros(shape + (rb,), dtype=np.uint8)
    dn = d - n_rot
    toff, soff = e4m3_row_offsets(d, n_rot)
    out[..., :dn] = draw_e4m3_codes(rng, shape + (dn,))
    tail = bf16_bits_of_draw(_normal32(rng, shape + (n_rot,), 1.0))
    out[..., toff:toff + 2 * n_rot] = tail.view(np.uint8).reshape(shape + (2 * n_rot,))
    scale = rng.uniform(0.75 / 64, 1.25 / 64, size=shape).astype(np.float32)
    out[..., soff:soff + 4] = scale.view(np.uint8).reshape(shape + (4,))
    return out


FP4_SCALE_BYTES = (125, 127)   # block scales 2^-2 .. 2^0 (E8M0 bytes e + 127)


def draw_fp4_records(rng, shape, dim: int) -> np.ndarray:
    """fp4 indexer records with every 4-bit code uniform over its 16 values and
    block-scale bytes uniform in FP4_SCALE_BYTES (inclusive)."""
    shape = tuple(shape)
    out = np.empty(shape + (idx_row_bytes("fp4", dim),), np.uint8)
    out[..., :dim // 2] = rng.integers(0, 256, size=shape + (dim // 2,), dtype=np.uint8)
    lo, hi = FP4_SCALE_BYTES
    out[..., dim // 2:] = rng.integers(lo, hi + 1, size=shape + (dim // 32,), dtype=np.uint8)
    return out


def draw_idx_rows(rng, shape, fmt: str, dim: int) -> np.ndarray:
    if fmt == "fp4":
        return draw_fp4_records(rng, shape, dim)
    return draw_values(rng, tuple(shape) + (dim,), fmt)


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

@dataclass
class LayerWeights:
    wkv: np.ndarray          # [d, D]   (w_fmt)
    wgate: np.ndarray        # [d, D]
    ape: np.ndarray          # [W, d]   float32
    gamma: np.ndarray        # [d]      float32
    idx_wkv: Optional[np.ndarray] = None    # [D_I, D]
    idx_wgate: Optional[np.ndarray] = None  # [D_I, D]
    idx_ape: Optional[np.ndarray] = None    # [8, D_I]
    idx_gamma: Optional[np.ndarray] = None  # [D_I]


def make_layer_weights(cfg: LayerShape) -> Optional[LayerWeights]:
    if cfg.ratio == 0:
        return None
    s, L = cfg.seed, cfg.layer
    d, D, W = cfg.head_dim, cfg.hidden, cfg.window
    w_std = cfg.w_std if cfg.w_std is not None else D ** -0.5
    ape_std = cfg.ape_std if cfg.ape_std is not None else d ** -0.5
    nl = cfg.lanes   # two-lane c4a: projections of 2 d rows, APE [4, 2 d]
    lw = LayerWeights(
        wkv=draw_values(_rng(s, "wkv", L), (nl * d, D), cfg.w_fmt, w_std),
        wgate=draw_values(_rng(s, "wgate", L), (nl * d, D), cfg.w_fmt, w_std),
        ape=_normal32(_rng(s, "ape", L), (W // nl, nl * d), ape_std),
        gamma=(1.0 + _normal32(_rng(s, "gamma", L), (d,), cfg.gamma_std)).astype(np.float32)
        if cfg.gamma_std else np.ones(d, np.float32),
    )
    if cfg.ratio == 4:
        DI = cfg.idx_dim
        iape_std = cfg.ape_std if cfg.ape_std is not None else DI ** -0.5
        lw.idx_wkv = draw_values(_rng(s, "idx_wkv", L), (nl * DI, D), cfg.w_fmt, w_std)
        lw.idx_wgate = draw_values(_rng(s, "idx_wgate", L), (nl * DI, D), cfg.w_fmt, w_std)
        lw.idx_ape = _normal32(_rng(s, "idx_ape", L), (8 // nl, nl * DI), iape_std)
        lw.idx_gamma = ((1.0 + _normal32(_rng(s, "idx_gamma", L), (DI,), cfg.gamma_std))
                        .astype(np.float32) if cfg.gamma_std else np.ones(DI, np.float32))
    return lw


# ---------------------------------------------------------------------------
# caches and per-step inputs
# ---------------------------------------------------------------------------

@dataclass
class CacheInit:
    """Initial cache contents (stored bytes), per sequence b."""
    raw: np.ndarray                 # [B, swa, rb] uint8
    comp: Optional[np.ndarray]      # [B, cap, rb] uint8
    idx: Optional[np.ndarray]       # [B, cap, D_I] f32 / uint16
    st_kv: Optional[np.ndarray]     # [B, W, d] float32
    st_sc: Optional[np.ndarray]
    ist_kv: Optional[np.ndarray]    # [B, 8, D_I] float32
    ist_sc: Optional[np.ndarray]
    n_drawn_comp: np.ndarray        # [B] rows 0..n-1 hold drawn values
    first_live: np.ndarray          # [B] first token position that runs through the path


@dataclass
class DecodeInputs:
    cfg: LayerShape
    pos: np.ndarray        # [B] int32, the query token position p = n - 1
    x: np.ndarray          # [B, D]
    u: np.ndarray          # [B, d]
    q: np.ndarray          # [B, H, d]
    qI: Optional[np.ndarray]   # [B, H_I, D_I]
    w: Optional[np.ndarray]    # [B, H_I] float32
    cache: CacheInit


@dataclass
class PrefillInputs:
    cfg: LayerShape
    pos0: int
    T: int
    x: np.ndarray          # [T, D]
    u: np.ndarray          # [T, d]
    q: np.ndarray          # [T, H, d]
    qI: Optional[np.ndarray]
    w: Optional[np.ndarray]
    cache: CacheInit


def _draw_cache(cfg: LayerShape, first_live: np.ndarray, empty: bool) -> CacheInit:
    """Cache state as it stands just before token ``first_live[b]`` is processed.

    Compressed rows already emitted before that token are drawn; so are the
    raw window rows of positions first_live-127 .. first_live-1 and the
    compressor window state of the pending tokens.  With ``empty`` the cache
    starts from zero (a whole history runs through the path).
    """
    B, d, swa = cfg.batch, cfg.head_dim, cfg.swa
    s, L = cfg.seed, cfg.layer
    rb = row_bytes(cfg.kv_fmt, d, cfg.n_rot)
    raw = np.zeros((B, swa, rb), np.uint8)
    comp = idx = st_kv = st_sc = ist_kv = ist_sc = None
    r, W, cap = cfg.ratio, cfg.window, cfg.comp_cap
    n_drawn = np.zeros(B, np.int64)
    nl = cfg.lanes   # a two-lane state slot holds both lanes of its token
    if r:
        comp = np.zeros((B, cap, rb), np.uint8)
        st_kv = np.zeros((B, W, nl * d), np.float32)
        st_sc = np.zeros((B, W, nl * d), np.float32)
    if r == 4:
        DI = cfg.idx_dim
        if cfg.idx_fmt == "fp4":
            idx = np.zeros((B, cap, idx_row_bytes("fp4", DI)), np.uint8)
        else:
            idx = np.zeros((B, cap, DI), np.float32 if cfg.idx_fmt == "f32" else np.uint16)
        ist_kv = np.zeros((B, 8, nl * DI), np.float32)
        ist_sc = np.zeros((B, 8, nl * DI), np.float32)
    if empty:
        return CacheInit(raw, comp, idx, st_kv, st_sc, ist_kv, ist_sc, n_drawn, first_live)
    for b in range(B):
        t0 = int(first_live[b])
        # raw window rows t0-swa+1 .. t0-1 (slot t mod swa)
        lo = max(0, t0 - (swa - 1))
        if t0 > lo:
            rows = draw_rows(_rng(s, "raw", L, b), (t0 - lo,), cfg.kv_fmt, d, cfg.n_rot)
            slots = np.arange(lo, t0) % swa
            raw[b, slots] = rows
        if not r:
            continue
        # compressed rows emitted before t0: floor(t0 / r); plus the row the
        # step may emit, so an overwrite is observable
        nd = min(cap, t0 // r + 1)
        n_drawn[b] = nd
        comp[b, :nd] = draw_rows(_rng(s, "comp", L, b), (nd,), cfg.kv_fmt, d, cfg.n_rot)
        if r == 4:
            idx[b, :nd] = draw_idx_rows(_rng(s, "idx", L, b), (nd,), cfg.idx_fmt, cfg.idx_dim)
        # pending compressor state: tokens [t0 - W, t0) that are >= 0
        ts = np.arange(max(0, t0 - W), t0)
        if len(ts):
            st_kv[b, ts % W] = _normal32(_rng(s, "st_kv", L, b), (len(ts), nl * d), 1.0)
            st_sc[b, ts % W] = _normal32(_rng(s, "st_sc", L, b), (len(ts), nl * d), 1.0)
            if r == 4:
                ts8 = ts[ts >= t0 - 8]
                ist_kv[b, ts8 % 8] = _normal32(_rng(s, "ist_kv", L, b), (len(ts8), nl * cfg.idx_dim), 1.0)
                ist_sc[b, ts8 % 8] = _normal32(_rng(s, "ist_sc", L, b), (len(ts8), nl * cfg.idx_dim), 1.0)
    return CacheInit(raw, comp, idx, st_kv, st_sc, ist_kv, ist_sc, n_drawn, first_live)


def context_lengths(cfg: LayerShape) -> np.ndarray:
    """Per-sequence context length n_b (tokens including the query)."""
    if cfg.ctx_range is None:
        return np.full(cfg.batch, cfg.n_ctx, np.int64)
    lo, hi = cfg.ctx_range
    n = _rng(cfg.seed, "ctx_len", cfg.layer).integers(lo, hi + 1, size=cfg.batch)
    # the cache must hold every row a sequence can see
    return np.minimum(n, cfg.comp_cap * max(cfg.ratio, 1)).astype(np.int64)


def draw_query_index(cfg: LayerShape, rows: int, sub: int = 0, attempt: int = 0):
    """Indexer query q^I [rows, H_I, D_I] and head weights w [rows, H_I] ~ U(0,1)."""
    s, L = cfg.seed, cfg.layer
    qI = draw_values(_rng(s, "qI", L, sub, attempt), (rows, cfg.idx_heads, cfg.idx_dim), cfg.act_fmt)
    w = _rng(s, "w", L, sub, attempt).uniform(0.0, 1.0, size=(rows, cfg.idx_heads)).astype(np.float32)
    return qI, w


def make_decode_inputs(cfg: LayerShape, n_ctx: Optional[np.ndarray] = None,
                       empty_cache: bool = False) -> DecodeInputs:
    """Inputs of one decode step at p = n - 1 for every sequence."""
    B = cfg.batch
    n = context_lengths(cfg) if n_ctx is None else np.asarray(n_ctx, np.int64)
    pos = (n - 1).astype(np.int32)
    s, L = cfg.seed, cfg.layer
    x = draw_values(_rng(s, "x", L), (B, cfg.hidden), cfg.act_fmt)
    u = draw_values(_rng(s, "u", L), (B, cfg.head_dim), cfg.act_fmt)
    q = draw_values(_rng(s, "q", L), (B, cfg.n_heads, cfg.head_dim), cfg.act_fmt)
    qI = w = None
    if cfg.ratio == 4:
        qI, w = draw_query_index(cfg, B)
    cache = _draw_cache(cfg, pos.astype(np.int64), empty_cache)
    return DecodeInputs(cfg, pos, x, u, q, qI, w, cache)


def make_token_stream(cfg: LayerShape, T: int, sub: int = 0):
    """Per-token inputs x, u, q (and q^I, w) for T consecutive tokens of one sequence."""
    s, L = cfg.seed, cfg.layer
    x = draw_values(_rng(s, "px", L, sub), (T, cfg.hidden), cfg.act_fmt)
    u = draw_values(_rng(s, "pu", L, sub), (T, cfg.head_dim), cfg.act_fmt)
    q = draw_values(_rng(s, "pq", L, sub), (T, cfg.n_heads, cfg.head_dim), cfg.act_fmt)
    qI = w = None
    if cfg.ratio == 4:
        qI, w = draw_query_index(cfg, T, sub=1000 + sub)
    return x, u, q, qI, w


def make_prefill_inputs(cfg: LayerShape, pos0: Optional[int] = None, T: Optional[int] = None,
                        empty_cache: Optional[bool] = None) -> PrefillInputs:
    """One sequence's chunk of T tokens starting at absolute position pos0."""
    pos0 = cfg.pos0 if pos0 is None else pos0
    T = cfg.chunk if T is None else T
    c1 = cfg.with_(batch=1)
    empty = (pos0 == 0) if empty_cache is None else empty_cache
    cache = _draw_cache(c1, np.array([pos0], np.int64), empty)
    x, u, q, qI, w = make_token_stream(c1, T)
    return PrefillInputs(c1, pos0, T, x, u, q, qI, w, cache)


def as_float(a: np.ndarray, fmt: str) -> np.ndarray:
    """Reinterpret stored f32 / bf16 bit patterns as float32 (bit extension only)."""
    if fmt == "f32":
        return a.astype(np.float32)
    if fmt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(fmt)
