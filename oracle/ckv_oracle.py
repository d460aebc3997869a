"""Plain, slow fp64 CPU oracle of one DeepSeek-V4-style compressed-KV attention layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.  It shares no code
with the HIP library: its number codecs, rotation, pooling, normalisation,
scoring, selection and attention are written here from the pages alone.

Sources (cited by page title and section):

* P1 = "【#3】ds4.c を読み解く" (Metal graph + compressed KV, DwarfStar ds4)
* P4 = "vLLM DeepSeek V4 サポート: 効率的な長文コンテキスト注意機構"

What it computes, per layer of compression ratio r (0, 4 or 128):

1. compressor (P1 s4, s5; P4 "KV Cache Compression"): for every token t,
   kappa_t = W_kv x_t and sigma_t = W_gate x_t.  Compressed row i pools the
   window of W tokens (W = 8 at stride 4 for c4a, 128 at stride 128 for
   c128a) channel by channel with a softmax over the window of
   sigma + APE[slot]; then RMS normalisation, RoPE on the last n_rot
   channels at position i*r, and the cast into the cache format.  Ratio-4
   layers run a second, narrower compressor of the same form for the indexer
   (P1 s6).
2. raw sliding window (P1 s2, s7; P4 "Short Sliding Window"): the last
   min(128, p+1) tokens' rows u_t, RoPE'd at t.
3. indexer (P1 s6; P4 "DSA"), ratio 4 only: score every visible compressed
   row, keep the top k.
4. attention (P1 s7; P4 "Shared Key and Value"): one softmax over the raw
   window plus the selected (r=4) or all visible (r=128) compressed rows, the
   same row serving as key and value, then inverse RoPE on the output tail.
5. chunked prefill (P1 s3) is defined as the sequence of decode steps.

Readings taken where the pages are silent (each also listed in the design
notes): APE row = the token's slot in the window being pooled; a compressed
row sits at position i*r; RoPE rotates adjacent channel pairs of the tail
with theta_j = base^(-2j/n_rot); one RoPE base per layer by default, or one
base for the raw rows and another for the compressed class (compressed and
indexer rows), the output's two shares rotated back each in its own frame;
RMSNorm eps 1e-6;
logit scale 1/sqrt(d); indexer score = sum_h w_h * relu(qI_h . kI_s) with the
rotated indexer query cast to the indexer-cache format; top-k ties go to the
lower index, output ascending with -1 padding; an fp8 row keeps its RoPE tail
in bf16 and scales its other channels by max|z|/448; an fp4 indexer cache is
the QAT round trip of P1 s9 read as orthonormal Hadamard-128 then OCP MXFP4
(E2M1 in blocks of 32 with a power-of-two block scale), applied alike to the
rotated indexer query; the optional query norm (P4 "GPU compute
saturation") divides each head's query by its RMS, with no learned weight,
before the RoPE.  Optionally (two_lane) a ratio-4 compressor is
two lanes wide: lane A of a token serves the window its block ends, lane B
the window of its own row (P1 s5, the alternative reading of its lane
comment).

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64

# ===========================================================================
# number formats (own codecs; textbook definitions)
# ===========================================================================


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> values: the pattern is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(F64)


def _round_to_quantum(x: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round-to-nearest-even onto a binary grid with ``mant_bits`` significant
    bits and smallest quantum 2**min_exp (covers normal and subnormal ranges)."""
    x = np.asarray(x, dtype=F64)
    out = np.array(x, dtype=F64, copy=True)  # zeros keep their sign; inf / nan pass
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])                   # x = m * 2**e with 0.5 <= |m| < 1
    qexp = np.maximum(e - mant_bits, min_exp)
    scaled = np.ldexp(x[nz], -qexp)          # exact (power-of-two scaling)
    out[nz] = np.ldexp(np.rint(scaled), qexp)  # np.rint rounds half to even
    return out


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bfloat16 value (8 significant bits, RNE, overflow to inf)."""
    y = _round_to_quantum(x, 8, -133)
    return np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, y), y)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """fp64 -> bfloat16 bit patterns (RNE)."""
    v = bf16_round(x).astype(np.float32)     # exact: bf16 values are float32 values
    return (v.view(np.uint32) >> 16).astype(np.uint16)


E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN code -> value.  Exponent bias 7, 3 mantissa bits, no
    infinities; S.1111.111 is NaN; exponent field 0 holds subnormals m * 2^-9."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest E4M3 value (4 significant bits, smallest quantum 2^-9,
    RNE), saturated to +-448."""
    y = _round_to_quantum(x, 4, -9)
    return np.clip(y, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp64 -> E4M3 code of ``e4m3_round(x)``."""
    y = e4m3_round(x)
    sign = (np.signbit(y)).astype(np.int64) << 7
    a = np.abs(y)
    code = np.zeros(a.shape, np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        _, e = np.frexp(a[nrm])              # a = f * 2**e, f in [0.5, 1)
        ef = e - 1 + 7                        # unbiased exponent e-1
        m = np.rint((a[nrm] / np.ldexp(1.0, e - 1) - 1.0) * 8).astype(np.int64)
        code[nrm] = (ef << 3) | m
    return (code | sign).astype(np.uint8)


def f32_round(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, F64).astype(np.float32).astype(F64)


# ---------------------------------------------------------------------------
# indexer QAT: Hadamard-128 and FP4 (P1 s9: the indexer's compressed rows and
# its query pass through a Hadamard transform of width 128 and an FP4
# activation-quantisation round trip; P4 "DeepSeek V4 attention
# architecture": the indexer cache may be fp4).  The pages name neither the
# FP4 element format nor its scaling; the reading taken here is OCP MXFP4:
# E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in blocks of 32
# consecutive channels, each block sharing a power-of-two scale 2^e with
# e = floor(log2 max|x|) - 2 (2 = the largest E2M1 exponent), elements rounded
# to nearest with ties to the even code and saturated at 6.  The Hadamard
# transform is the orthonormal one (Sylvester order, H / sqrt(n), symmetric),
# applied to the 128 channels after the tail RoPE.
# ---------------------------------------------------------------------------

FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # E2M1 magnitude of codes 0..7
FP4_BLOCK = 32


def hadamard(x: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform along the last axis (length a
    power of two): x @ H_n / sqrt(n), H_n the Sylvester matrix."""
    from scipy.linalg import hadamard as sylvester
    x = np.asarray(x, F64)
    n = x.shape[-1]
    return x @ (sylvester(n).astype(F64) / math.sqrt(n))


def fp4_decode(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes (bit 3 = sign) -> values."""
    c = np.asarray(codes, np.int64)
    mag = FP4_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def fp4_encode(v: np.ndarray) -> np.ndarray:
    """Values (already divided by their block scale) -> E2M1 codes: nearest
    grid magnitude, a tie going to the even code, saturated at 6; the sign bit
    is set for negative values (zero keeps code 0)."""
    v = np.asarray(v, F64)
    a = np.minimum(np.abs(v), FP4_GRID[-1])
    dist = np.abs(a[..., None] - FP4_GRID)                     # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = np.isclose(dist, best, rtol=0.0, atol=0.0) | (dist == best)
    # among equally near codes (at most two, adjacent) take the even one
    even = cand & ((np.arange(8) & 1) == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (code | np.where((v < 0) & (code > 0), 8, 0)).astype(np.uint8)


def mxfp4_encode(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Blocks of 32 along the last axis -> (E2M1 codes [..., n], block
    exponents e [..., n/32] as ints).  e = floor(log2 max|x|) - 2, clamped to
    [-127, 127]; an all-zero block takes e = -127."""
    x = np.asarray(x, F64)
    shp = x.shape
    blk = x.reshape(shp[:-1] + (shp[-1] // FP4_BLOCK, FP4_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    codes = fp4_encode(blk / np.ldexp(1.0, e)[..., None])
    return codes.reshape(shp), e


def mxfp4_decode(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    c = np.asarray(codes)
    shp = c.shape
    blk = fp4_decode(c).reshape(shp[:-1] + (shp[-1] // FP4_BLOCK, FP4_BLOCK))
    return (blk * np.ldexp(1.0, np.asarray(e, np.int64))[..., None]).reshape(shp)


def mxfp4_round_trip(x: np.ndarray) -> np.ndarray:
    return mxfp4_decode(*mxfp4_encode(x))


def fp4_row_bytes(n: int) -> int:
    """One stored fp4 indexer row: n/2 bytes of codes (channel 2j in the low
    nibble of byte j, 2j + 1 in the high one), then n/32 E8M0 bytes (e + 127)."""
    return n // 2 + n // FP4_BLOCK


def fp4_encode_rows(x: np.ndarray) -> np.ndarray:
    """Rows [..., n] (already in the Hadamard domain) -> records [..., n/2 + n/32] uint8."""
    codes, e = mxfp4_encode(x)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return np.concatenate([packed, (e + 127).astype(np.uint8)], axis=-1)


def fp4_decode_rows(rec: np.ndarray, n: int) -> np.ndarray:
    rec = np.asarray(rec, np.uint8)
    packed = rec[..., :n // 2]
    codes = np.empty(rec.shape[:-1] + (n,), np.uint8)
    codes[..., 0::2] = packed & 15
    codes[..., 1::2] = packed >> 4
    e = rec[..., n // 2:n // 2 + n // FP4_BLOCK].astype(np.int64) - 127
    return mxfp4_decode(codes, e)


def idx_quantise(z: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """An indexer vector (a row after its RoPE, or the rotated query) as it
    enters the scores: (value before rounding, value after).  fp4 is the QAT
    round trip, Hadamard then MXFP4 (P1 s9); f32 / bf16 a plain cast."""
    if fmt == "fp4":
        h = hadamard(z)
        return h, mxfp4_round_trip(h)
    return np.asarray(z, F64), cast_values(z, fmt)


# ---------------------------------------------------------------------------
# stored-row formats
# ---------------------------------------------------------------------------

def stored_row_bytes(fmt: str, d: int, n_rot: int) -> int:
    """Size of one stored K=V row: f32 4d, bf16 2d; an fp8 row keeps
    d - n_rot E4M3 codes, the n_rot RoPE channels in bf16 and one fp32 scale,
    padded to a multiple of 128 bytes.  ``f64`` (8d, no rounding at all) is
    not a cache format of the method: it lets the exact pins compare two runs
    of the oracle to fp64 precision."""
    if fmt == "f64":
        return 8 * d
    if fmt == "f32":
        return 4 * d
    if fmt == "bf16":
        return 2 * d
    raw = (d - n_rot) + 2 * n_rot + 4
    return (raw + 127) // 128 * 128


def decode_values(a: np.ndarray, fmt: str) -> np.ndarray:
    """Stored values -> fp64.  fp4 takes indexer-row records [..., n/2 + n/32]
    (values in the Hadamard domain)."""
    if fmt == "fp4":
        a = np.asarray(a, np.uint8)
        n = a.shape[-1] * 32 // 17
        return fp4_decode_rows(a, n)
    if fmt == "f64":
        return np.asarray(a, F64).copy()
    if fmt == "f32":
        return np.asarray(a, np.float32).astype(F64)
    if fmt == "bf16":
        return bf16_decode(a)
    raise ValueError(fmt)


def cast_values(z: np.ndarray, fmt: str) -> np.ndarray:
    """Value after storing ``z`` in format ``fmt`` (f32 or bf16, RNE; f64 keeps it)."""
    if fmt == "f64":
        return np.asarray(z, F64).copy()
    if fmt == "f32":
        return f32_round(z)
    if fmt == "bf16":
        return bf16_round(z)
    raise ValueError(fmt)


def decode_rows(rec: np.ndarray, fmt: str, d: int, n_rot: int) -> np.ndarray:
    """Stored row records [..., rb] uint8 -> row values [..., d] fp64."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    shp = rec.shape[:-1]
    if fmt == "f64":
        return rec[..., :8 * d].copy().view(F64).reshape(shp + (d,))
    if fmt == "f32":
        return rec[..., :4 * d].copy().view(np.float32).reshape(shp + (d,)).astype(F64)
    if fmt == "bf16":
        return bf16_decode(rec[..., :2 * d].copy().view(np.uint16).reshape(shp + (d,)))
    dn = d - n_rot
    codes = rec[..., :dn]
    tail = rec[..., dn:dn + 2 * n_rot].copy().view(np.uint16).reshape(shp + (n_rot,))
    scale = rec[..., dn + 2 * n_rot:dn + 2 * n_rot + 4].copy().view(np.float32).reshape(shp)
    out = np.empty(shp + (d,), F64)
    out[..., :dn] = e4m3_decode(codes) * scale.astype(F64)[..., None]
    out[..., dn:] = bf16_decode(tail)
    return out


def encode_row(z: np.ndarray, fmt: str, d: int, n_rot: int) -> Tuple[np.ndarray, np.ndarray]:
    """Store one row ``z`` [d]: returns (record bytes, stored value fp64).

    fp8 rows (P1 s9: the FP8 round trip covers the non-RoPE part only): the
    tail is kept as bf16; the other channels use the row scale
    s = max|z_c| / 448 (1 when the row is all zero), kept as fp32, and the
    codes RNE(z_c / s) saturated to +-448.
    """
    z = np.asarray(z, F64)
    rb = stored_row_bytes(fmt, d, n_rot)
    rec = np.zeros(rb, np.uint8)
    if fmt == "f64":
        rec[:] = z.view(np.uint8)
        return rec, z.copy()
    if fmt == "f32":
        v = z.astype(np.float32)
        rec[:4 * d] = v.view(np.uint8)
        return rec, v.astype(F64)
    if fmt == "bf16":
        bits = bf16_encode(z)
        rec[:2 * d] = bits.view(np.uint8)
        return rec, bf16_decode(bits)
    dn = d - n_rot
    amax = float(np.max(np.abs(z[:dn]))) if dn else 0.0
    s32 = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    codes = e4m3_encode(z[:dn] / F64(s32))
    tail = bf16_encode(z[dn:])
    rec[:dn] = codes
    rec[dn:dn + 2 * n_rot] = tail.view(np.uint8)
    rec[dn + 2 * n_rot:dn + 2 * n_rot + 4] = np.array([s32], np.float32).view(np.uint8)
    val = np.concatenate([e4m3_decode(codes) * F64(s32), bf16_decode(tail)])
    return rec, val


# ===========================================================================
# method steps
# ===========================================================================


# ---------------------------------------------------------------------------
# attention output in fp8 (P4 "GPU compute saturation": the inverse RoPE of the
# attention output is fused with its fp8 quantisation).  The page names the
# fusion, not the format; the reading taken here: E4M3 codes of the output
# (after the inverse RoPE) in groups of 128 consecutive channels of a head,
# each group scaled by s = max|o| / 448 over the group (1 when all zero), s
# kept as fp32; a head's record is its d codes then its d/128 scales.

OUT_FP8_GROUP = 128


def out_fp8_record_bytes(d: int) -> int:
    return d + 4 * (d // OUT_FP8_GROUP)


def encode_out_fp8(o: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Output rows o [..., d] -> (records [..., d + 4 d/128] uint8, decoded
    values [..., d])."""
    o = np.asarray(o, F64)
    d = o.shape[-1]
    g = o.reshape(o.shape[:-1] + (d // OUT_FP8_GROUP, OUT_FP8_GROUP))
    amax = np.abs(g).max(axis=-1)
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    codes = e4m3_encode(g / s.astype(F64)[..., None])
    rec = np.concatenate([codes.reshape(o.shape[:-1] + (d,)),
                          np.ascontiguousarray(s).view(np.uint8).reshape(o.shape[:-1] + (4 * (d // OUT_FP8_GROUP),))],
                         axis=-1)
    return rec, decode_out_fp8(rec, d)


def decode_out_fp8(rec: np.ndarray, d: int) -> np.ndarray:
    rec = np.asarray(rec, np.uint8)
    ng = d // OUT_FP8_GROUP
    s = np.ascontiguousarray(rec[..., d:d + 4 * ng]).view(np.float32).astype(F64)
    v = e4m3_decode(rec[..., :d]).reshape(rec.shape[:-1] + (ng, OUT_FP8_GROUP))
    return (v * s[..., None]).reshape(rec.shape[:-1] + (d,))


def rope_theta(base: float, n_rot: int) -> np.ndarray:
    """theta_j = base^(-2j/n_rot), j = 0 .. n_rot/2 - 1."""
    j = np.arange(n_rot // 2, dtype=F64)
    return np.power(F64(base), -2.0 * j / n_rot)


def rope_tail(x: np.ndarray, pos, base: float, n_rot: int) -> np.ndarray:
    """Rotate only the last n_rot channels of each vector (P1 s8: the head's
    first d - n_rot channels are left alone).  Channel pair
    (d - n_rot + 2j, d - n_rot + 2j + 1) turns by the angle pos * theta_j;
    a negative ``pos`` undoes the rotation at -pos.  ``pos`` may be an array
    broadcasting against x[..., 0]."""
    x = np.array(x, dtype=F64, copy=True)
    d = x.shape[-1]
    dn = d - n_rot
    ang = np.multiply.outer(np.asarray(pos, F64), rope_theta(base, n_rot))  # [..., n_rot/2]
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., dn + 0::2].copy()
    b = x[..., dn + 1::2].copy()
    # broadcast the angle over the head axis when x has one more axis than pos
    while c.ndim < a.ndim:
        c = c[..., None, :]
        s = s[..., None, :]
    x[..., dn + 0::2] = a * c - b * s
    x[..., dn + 1::2] = a * s + b * c
    return x


def rmsnorm(y: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """z = gamma * y / sqrt(mean(y^2) + eps) (P1 s4 step 6)."""
    y = np.asarray(y, F64)
    return np.asarray(gamma, F64) * y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)


def query_rms_norm(q: np.ndarray, eps: float) -> np.ndarray:
    """Each head's query divided by its RMS: q_h / sqrt(mean(q_h^2) + eps).

    P4 "GPU compute saturation" lists a query norm among the steps fused with
    the raw keys' RoPE and insertion, without its form.  Reading: an RMS
    normalisation over each head's head_dim channels with no learned weight,
    eps = the layer's RMSNorm eps, applied before the query's RoPE (a rotation
    of channel pairs keeps every pair's sum of squares, so the order does not
    change the result)."""
    q = np.asarray(q, F64)
    return q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps)


def window_positions(i: int, ratio: int) -> np.ndarray:
    """Token position held by each slot j of compressed row i's window.

    c4a: 8 tokens at stride 4, row i pooling the previous stride block (slots
    0-3) and its own (slots 4-7): t_j = 4i - 4 + j (P1 s5, P4 c4a).
    c128a: 128 tokens at stride 128: t_j = 128 i + j (P4 c128a)."""
    if ratio == 4:
        return 4 * i - 4 + np.arange(8)
    if ratio == 128:
        return 128 * i + np.arange(128)
    raise ValueError(ratio)


def softmax_pool(kappa: np.ndarray, score: np.ndarray) -> np.ndarray:
    """Per-channel softmax-weighted pooling over the window axis (P1 s4):
    for each channel, m = max_j score, w_j = exp(score_j - m),
    y = sum_j w_j kappa_j / sum_j w_j (0 when the sum is 0).  Slots with score
    -inf get weight 0."""
    kappa = np.asarray(kappa, F64)
    score = np.asarray(score, F64)
    m = np.max(score, axis=0)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(score - m)
    w = np.where(np.isfinite(score), w, 0.0)
    den = np.sum(w, axis=0)
    num = np.sum(w * np.where(np.isfinite(score), kappa, 0.0), axis=0)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def pool_window(kappa_win: np.ndarray, sigma_win: np.ndarray, ape: np.ndarray,
                valid: np.ndarray) -> np.ndarray:
    """Pool one window: slot j scores sigma_j + APE[j] (P1 s4 step 3); slots
    before token 0 are empty and carry no weight."""
    e = np.asarray(sigma_win, F64) + np.asarray(ape, F64)
    e = np.where(np.asarray(valid)[:, None], e, -np.inf)
    return softmax_pool(kappa_win, e)


def indexer_scores(qhat: np.ndarray, w: np.ndarray, rows: np.ndarray, relu: bool = True) -> np.ndarray:
    """I(s) = sum_h w_h * relu(qhat_h . k_s) for every row s (P1 s6: the
    narrow indexer representation scores every compressed row)."""
    dots = np.asarray(rows, F64) @ np.asarray(qhat, F64).T       # [V, H_I]
    if relu:
        dots = np.maximum(dots, 0.0)
    return dots @ np.asarray(w, F64)


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """The k largest scores' indices (ties to the lower index), listed in
    ascending index order, -1-padded to length k; every index when there are
    at most k scores (P1 s6, s7: negative entries are skipped by the
    consumer)."""
    V = len(scores)
    out = np.full(k, -1, np.int32)
    if V <= k:
        out[:V] = np.arange(V)
        return out
    sc = np.asarray(scores, F64) + 0.0               # -0 compares equal to +0
    order = np.lexsort((np.arange(V), -sc))          # full sort: score descending, then index
    out[:] = np.sort(order[:k]).astype(np.int32)
    return out


def attention(qhat: np.ndarray, rows: np.ndarray, scale: float) -> np.ndarray:
    """Shared-K=V attention (P4 "Shared Key and Value"): logits
    l_hj = scale * qhat_h . k_j, a = softmax_j(l), o_h = sum_j a_hj k_j.
    Two-pass softmax over the explicit row set."""
    rows = np.asarray(rows, F64)
    l = scale * (np.asarray(qhat, F64) @ rows.T)                  # [H, S]
    l = l - np.max(l, axis=1, keepdims=True)
    a = np.exp(l)
    a = a / np.sum(a, axis=1, keepdims=True)
    return a @ rows


def attention_two_class(q_a: np.ndarray, rows_a: np.ndarray, q_b: np.ndarray, rows_b: np.ndarray,
                        scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One softmax over the union of two row classes whose keys carry their
    positions in different rotation frames (raw rows and compressed rows when
    each class has its own RoPE base): class a's logits use the query q_a,
    class b's use q_b.  Returns the two classes' shares of o = sum_j a_j k_j,
    so that each can be rotated back in its own frame."""
    rows_a = np.asarray(rows_a, F64).reshape(-1, np.shape(q_a)[-1])
    rows_b = np.asarray(rows_b, F64).reshape(-1, np.shape(q_b)[-1])
    l = scale * np.concatenate([np.asarray(q_a, F64) @ rows_a.T, np.asarray(q_b, F64) @ rows_b.T], axis=1)
    l = l - np.max(l, axis=1, keepdims=True)
    a = np.exp(l)
    a = a / np.sum(a, axis=1, keepdims=True)
    na = rows_a.shape[0]
    return a[:, :na] @ rows_a, a[:, na:] @ rows_b


# ===========================================================================
# one layer, history based
# ===========================================================================


@dataclass
class OracleLayer:
    """Layer parameters (fp64 copies of the stored weights)."""
    ratio: int
    head_dim: int
    n_heads: int
    idx_heads: int
    idx_dim: int
    top_k: int
    n_rot: int
    swa: int
    rope_base: float
    norm_eps: float
    kv_fmt: str
    idx_fmt: str
    act_fmt: str
    wkv: Optional[np.ndarray] = None
    wgate: Optional[np.ndarray] = None
    ape: Optional[np.ndarray] = None
    gamma: Optional[np.ndarray] = None
    idx_wkv: Optional[np.ndarray] = None
    idx_wgate: Optional[np.ndarray] = None
    idx_ape: Optional[np.ndarray] = None
    idx_gamma: Optional[np.ndarray] = None
    relu: bool = True
    # RoPE base of the compressed-row class (compressed rows, indexer rows and
    # the query's rotation against them).  None: the layer's one base serves
    # every class (per-layer reading); a value: raw rows and the query against
    # them keep ``rope_base``, the compressed class takes this one
    # (per-row-class reading).
    rope_base_comp: Optional[float] = None
    # Debug stage skips of the library's layer description (used to isolate a
    # stage in tests): no RMSNorm (neither 1/rms nor gamma) on compressed rows;
    # no tail rotation anywhere (every angle zero).
    skip_norm: bool = False
    skip_rope: bool = False
    # query norm of the layer description's flags: each head's attention
    # query RMS-normalised (query_rms_norm) before its RoPE
    q_norm: bool = False
    # two-lane c4a compressor (P1 s5: a ratio-4 compressor is twice as wide
    # as its rows): every token projects to two lanes (wkv, wgate [2 w, D]),
    # lane A serving the window it ends (slots 0-3 of the next row), lane B the
    # window of its own row (slots 4-7); APE [4, 2 w] holds lane A's slot s in
    # row s, channels :w, and lane B's in channels w:.  Both compressors of a
    # ratio-4 layer take it (the indexer's at width D_I).
    two_lane: bool = False

    def rope(self, x, pos, base: float, n_rot: int) -> np.ndarray:
        """rope_tail, or the identity when the layer skips RoPE."""
        return np.asarray(x, F64) if self.skip_rope else rope_tail(x, pos, base, n_rot)

    @property
    def base_raw(self) -> float:
        return self.rope_base

    @property
    def base_comp(self) -> float:
        return self.rope_base if self.rope_base_comp is None else self.rope_base_comp

    @property
    def window(self) -> int:
        return {4: 8, 128: 128}.get(self.ratio, 0)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def layer_from(cfg, weights) -> OracleLayer:
    """Build an OracleLayer from a workload shape and its stored weights."""
    def w(a, fmt):
        return None if a is None else decode_values(a, fmt)
    L = OracleLayer(ratio=cfg.ratio, head_dim=cfg.head_dim, n_heads=cfg.n_heads,
                    idx_heads=cfg.idx_heads, idx_dim=cfg.idx_dim, top_k=cfg.top_k,
                    n_rot=cfg.n_rot, swa=cfg.swa, rope_base=cfg.rope_base,
                    norm_eps=cfg.norm_eps, kv_fmt=cfg.kv_fmt, idx_fmt=cfg.idx_fmt,
                    act_fmt=cfg.act_fmt, rope_base_comp=getattr(cfg, "rope_base_comp", None),
                    two_lane=bool(getattr(cfg, "two_lane", False)) and cfg.ratio == 4)
    if weights is not None:
        L.wkv = w(weights.wkv, cfg.w_fmt)
        L.wgate = w(weights.wgate, cfg.w_fmt)
        L.ape = weights.ape.astype(F64)
        L.gamma = weights.gamma.astype(F64)
        if weights.idx_wkv is not None:
            L.idx_wkv = w(weights.idx_wkv, cfg.w_fmt)
            L.idx_wgate = w(weights.idx_wgate, cfg.w_fmt)
            L.idx_ape = weights.idx_ape.astype(F64)
            L.idx_gamma = weights.idx_gamma.astype(F64)
    return L


class OracleSequence:
    """One sequence's token history and the cache it implies.

    Tokens fed through :meth:`feed` are live: their projections and raw rows
    are computed here.  Everything from before the first live token comes
    from the drawn cache bytes: compressed rows whose window ends before it,
    raw rows, and the pending compressor window values (kappa, sigma) of the
    tokens just before it.
    """

    def __init__(self, L: OracleLayer, raw_rec=None, comp_rec=None, idx_vals=None,
                 st_kv=None, st_sc=None, ist_kv=None, ist_sc=None, first_live: int = 0):
        self.L = L
        self.first_live = int(first_live)
        self.raw_rec = raw_rec          # [swa, rb] uint8 (ring, slot t mod swa)
        self.comp_rec = comp_rec        # [cap, rb] uint8
        self.idx_vals = idx_vals        # [cap, D_I] stored f32 / bf16 bits
        self.kap: Dict[int, np.ndarray] = {}
        self.sig: Dict[int, np.ndarray] = {}
        self.ikap: Dict[int, np.ndarray] = {}
        self.isig: Dict[int, np.ndarray] = {}
        self.u: Dict[int, np.ndarray] = {}
        self._row_cache: Dict[Tuple[str, int], Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
        # memo of raw rows of live tokens and of the indexer matrix (cleared by feed)
        self._raw_cache: Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
        self._idx_mat: Optional[np.ndarray] = None
        W = L.window
        if W and st_kv is not None:
            for t in range(max(0, first_live - W), first_live):
                self.kap[t] = np.asarray(st_kv[t % W], F64)
                self.sig[t] = np.asarray(st_sc[t % W], F64)
        if L.ratio == 4 and ist_kv is not None:
            for t in range(max(0, first_live - 8), first_live):
                self.ikap[t] = np.asarray(ist_kv[t % 8], F64)
                self.isig[t] = np.asarray(ist_sc[t % 8], F64)

    # -- tokens ------------------------------------------------------------
    def feed(self, t0: int, x: np.ndarray, u: np.ndarray) -> None:
        """Make tokens t0 .. t0+len(x)-1 live: kappa = W_kv x, sigma = W_gate x
        for the attention lane and (ratio 4) the indexer lane (P1 s4 steps 1-2)."""
        L = self.L
        X = decode_values(x, L.act_fmt).reshape(len(x), -1)
        U = decode_values(u, L.act_fmt).reshape(len(u), -1)
        if L.ratio:
            K, S = X @ L.wkv.T, X @ L.wgate.T
            has_idx = L.ratio == 4 and L.idx_wkv is not None
            if has_idx:
                KI, SI = X @ L.idx_wkv.T, X @ L.idx_wgate.T
        self._idx_mat = None
        for n in range(len(X)):
            t = t0 + n
            self.u[t] = U[n]
            self._raw_cache.pop(t, None)
            if L.ratio:
                self.kap[t], self.sig[t] = K[n], S[n]
                if has_idx:
                    self.ikap[t], self.isig[t] = KI[n], SI[n]
            for key in [k for k in self._row_cache if k[1] >= (t // max(L.ratio, 1)) - 1]:
                del self._row_cache[key]

    def is_live(self, t: int) -> bool:
        return t in self.u

    # -- compressed rows -----------------------------------------------------
    def pooled(self, i: int, lane: str = "attn") -> np.ndarray:
        """Row i's window pooled channel by channel, before normalisation."""
        L = self.L
        ts = window_positions(i, L.ratio)
        kap, sig = (self.kap, self.sig) if lane == "attn" else (self.ikap, self.isig)
        ape = np.asarray(L.ape if lane == "attn" else L.idx_ape, F64)
        two = L.two_lane and L.ratio == 4
        if two:   # slot j < 4: lane A (first half), slot j >= 4: lane B (second half)
            width = ape.shape[1] // 2
            ape = np.concatenate([ape[:, :width], ape[:, width:]])
        width = ape.shape[1]
        valid = ts >= 0
        kw = np.zeros((len(ts), width))
        sw = np.zeros((len(ts), width))
        for j, t in enumerate(ts):
            if t >= 0:
                k, sg = kap[int(t)], sig[int(t)]
                if two:
                    h = slice(0, width) if j < 4 else slice(width, 2 * width)
                    k, sg = k[h], sg[h]
                kw[j], sw[j] = k, sg
        return pool_window(kw, sw, ape, valid)

    def _pool_row(self, i: int, lane: str) -> np.ndarray:
        """Pool, RMS-normalise, then rotate the tail at the row position i*r
        (P1 s4 steps 5-7) with the compressed class's base."""
        L = self.L
        y = self.pooled(i, lane)
        gamma = L.gamma if lane == "attn" else L.idx_gamma
        z = y if L.skip_norm else rmsnorm(y, gamma, L.norm_eps)
        n_rot = min(L.n_rot, len(z))
        return L.rope(z, i * L.ratio, L.base_comp, n_rot)

    def _row_is_computed(self, i: int) -> bool:
        """Row i is computed from history when its last window token is live."""
        last = i * self.L.ratio + self.L.ratio - 1
        return self.is_live(last)

    def comp_row(self, i: int) -> Tuple[np.ndarray, Optional[np.ndarray], np.ndarray]:
        """(pre-cast value, stored record or None, stored value) of attention row i."""
        key = ("attn", i)
        if key not in self._row_cache:
            L = self.L
            if self._row_is_computed(i):
                z = self._pool_row(i, "attn")
                rec, val = encode_row(z, L.kv_fmt, L.head_dim, L.n_rot)
                self._row_cache[key] = (z, rec, val)
            else:
                val = decode_rows(self.comp_rec[i], L.kv_fmt, L.head_dim, L.n_rot)
                self._row_cache[key] = (val, None, val)
        return self._row_cache[key]

    def idx_row(self, i: int) -> Tuple[np.ndarray, np.ndarray]:
        """(pre-cast value, stored value) of indexer row i (for an fp4 cache
        both in the Hadamard domain: before and after the MXFP4 round trip)."""
        key = ("idx", i)
        if key not in self._row_cache:
            L = self.L
            if self._row_is_computed(i):
                z = self._pool_row(i, "idx")
                pre, val = idx_quantise(z, L.idx_fmt)
                self._row_cache[key] = (pre, val, None)
            else:
                v = decode_values(self.idx_vals[i], L.idx_fmt)
                self._row_cache[key] = (v, v, None)
        return self._row_cache[key][:2]

    # -- raw window ----------------------------------------------------------
    def raw_row(self, t: int) -> Tuple[np.ndarray, Optional[np.ndarray], np.ndarray]:
        """(pre-cast, record, stored value) of the raw row of token t: u_t RoPE'd
        at t with the raw class's base (P4: the SWA rows carry their position)."""
        L = self.L
        if self.is_live(t):
            if t not in self._raw_cache:
                z = L.rope(self.u[t], t, L.base_raw, L.n_rot)
                rec, val = encode_row(z, L.kv_fmt, L.head_dim, L.n_rot)
                self._raw_cache[t] = (z, rec, val)
            return self._raw_cache[t]
        val = decode_rows(self.raw_rec[t % L.swa], L.kv_fmt, L.head_dim, L.n_rot)
        return val, None, val

    # -- one query -------------------------------------------------------------
    def visible_rows(self, p: int) -> int:
        """V_p = floor((p+1)/r): rows whose window has closed by token p."""
        return (p + 1) // self.L.ratio if self.L.ratio else 0

    def raw_window(self, p: int) -> range:
        """Raw positions max(0, p-swa+1) .. p (P1 s7 window rule)."""
        return range(max(0, p + 1 - self.L.swa), p + 1)

    def computed_rows(self, V: int):
        """Indices < V of the rows whose window closes at a live token."""
        r = self.L.ratio
        return sorted({(t + 1) // r - 1 for t in self.u if (t + 1) % r == 0 and (t + 1) // r - 1 < V})

    def idx_matrix(self, V: int) -> np.ndarray:
        """Stored values of indexer rows 0..V-1 (drawn rows decoded in bulk,
        computed rows from the history)."""
        L = self.L
        if V == 0:
            return np.zeros((0, L.idx_dim))
        if self._idx_mat is not None and len(self._idx_mat) >= V:
            return self._idx_mat[:V].copy()
        if self.idx_vals is not None:
            rows = decode_values(self.idx_vals[:V], L.idx_fmt)
        else:
            rows = np.zeros((V, L.idx_dim))
        for i in self.computed_rows(V):
            rows[i] = self.idx_row(i)[1]
        self._idx_mat = rows
        return rows.copy()

    def comp_matrix(self, idx: Sequence[int]) -> np.ndarray:
        """Stored values of attention rows ``idx``."""
        L = self.L
        idx = np.asarray(idx, np.int64)
        if len(idx) == 0:
            return np.zeros((0, L.head_dim))
        comp = set(self.computed_rows(int(idx.max()) + 1))
        if self.comp_rec is not None:
            rows = decode_rows(self.comp_rec[idx], L.kv_fmt, L.head_dim, L.n_rot)
        else:
            rows = np.zeros((len(idx), L.head_dim))
        for n, i in enumerate(idx):
            if int(i) in comp:
                rows[n] = self.comp_row(int(i))[2]
        return rows

    def index_scores(self, p: int, qI: np.ndarray, w: np.ndarray) -> np.ndarray:
        """Indexer scores of every visible row for query p.  The indexer query
        gets the tail RoPE at p (the compressed class's base: it is matched
        against compressed rows) and is cast to the indexer-cache format (for
        fp4: the Hadamard + MXFP4 round trip of its rows, P1 s9)."""
        L = self.L
        V = self.visible_rows(p)
        qh = L.rope(decode_values(qI, L.act_fmt), p, L.base_comp, min(L.n_rot, L.idx_dim))
        qh = idx_quantise(qh, L.idx_fmt)[1]
        return indexer_scores(qh, np.asarray(w, F64), self.idx_matrix(V), relu=L.relu)

    def attend(self, p: int, q: np.ndarray, topk: Optional[np.ndarray]) -> np.ndarray:
        """Output o [H, d] (pre-cast) for query p over raw window + compressed
        set: one softmax over both classes, the query rotated at p against
        each class in that class's frame, and each class's share of the output
        rotated back by -p in its own frame (inverse RoPE, P4; with one base
        per layer the two rotations are the same and this is o rotated by -p)."""
        L = self.L
        raw = np.stack([self.raw_row(t)[2] for t in self.raw_window(p)])
        V = self.visible_rows(p)
        sel = []
        if L.ratio == 4:
            for i in topk:
                if i < 0:
                    continue
                if i >= V:
                    break
                sel.append(int(i))
        elif L.ratio == 128:
            sel = list(range(V))
        comp = self.comp_matrix(sel)
        qv = decode_values(q, L.act_fmt).reshape(L.n_heads, L.head_dim)
        if L.q_norm:
            qv = query_rms_norm(qv, L.norm_eps)
        q_raw = L.rope(qv, p, L.base_raw, L.n_rot)
        q_comp = L.rope(qv, p, L.base_comp, L.n_rot)
        o_raw, o_comp = attention_two_class(q_raw, raw, q_comp, comp, L.scale)
        # inverse RoPE (P4), class by class
        return L.rope(o_raw, -p, L.base_raw, L.n_rot) + L.rope(o_comp, -p, L.base_comp, L.n_rot)

    def step(self, p: int, x, u, q, qI=None, w=None, topk_override=None) -> dict:
        """One decode step at token p: make p live, then index, select, attend."""
        self.feed(p, np.asarray(x)[None], np.asarray(u)[None])
        return self.query(p, q, qI, w, topk_override)

    def query(self, p: int, q, qI=None, w=None, topk_override=None) -> dict:
        L = self.L
        res = {"p": p, "V": self.visible_rows(p)}
        topk = None
        if L.ratio == 4:
            sc = self.index_scores(p, qI, w)
            res["scores"] = sc
            topk = topk_select(sc, L.top_k)
            res["topk"] = topk
            if topk_override is not None:
                topk = np.asarray(topk_override)
        o = self.attend(p, q, topk)
        res["out_f64"] = o
        res["out"] = cast_values(o, L.act_fmt)
        return res


def prefill(seq: OracleSequence, pos0: int, x, u, q, qI=None, w=None, queries=None) -> Dict[int, dict]:
    """Chunked prefill, defined as the run of decode steps pos0 .. pos0+T-1
    (P1 s3: the chunking keeps absolute compressor and indexer boundaries).
    ``queries`` limits which positions' outputs are computed (all by default);
    every token is made live regardless."""
    T = len(x)
    seq.feed(pos0, np.asarray(x), np.asarray(u))
    want = range(pos0, pos0 + T) if queries is None else queries
    out = {}
    for p in want:
        n = p - pos0
        out[p] = seq.query(p, q[n], None if qI is None else qI[n], None if w is None else w[n])
    return out


# ===========================================================================
# closed forms used as pins
# ===========================================================================


def flash_ratio(il: int) -> int:
    """Flash layer schedule (P1 s1): layers 0-1 uncompressed, then even
    layers ratio 4 and odd layers ratio 128."""
    if il < 2:
        return 0
    return 4 if il % 2 == 0 else 128


def pro_ratio(il: int) -> int:
    """Pro layer schedule (P1 s1): layers 0-1 ratio 128, then alternating 4 / 128."""
    if il < 2:
        return 128
    return 4 if il % 2 == 0 else 128


def kv_bytes_per_sequence(n_tokens: int, ratios: Sequence[int], head_dim: int = 512,
                          idx_dim: int = 128, swa: int = 128, attn_bytes_per_row: float = 1024,
                          idx_bytes_per_row: float = 256) -> float:
    """Bytes of KV cache one sequence of ``n_tokens`` needs over a stack with
    the given per-layer ratios: c4a layers keep n/4 attention rows plus n/4
    indexer rows, c128a layers n/128 attention rows, and every layer its
    sliding window of ``swa`` raw rows (P4 "KV Cache Compression" and the
    9.62 GiB figure)."""
    total = 0.0
    for r in ratios:
        total += swa * attn_bytes_per_row
        if r == 4:
            total += n_tokens / 4 * (attn_bytes_per_row + idx_bytes_per_row)
        elif r == 128:
            total += n_tokens / 128 * attn_bytes_per_row
    return total
