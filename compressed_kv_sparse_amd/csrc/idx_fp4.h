// The fp4 indexer format: Hadamard-128 + MXFP4 ("ds4.c を読み解く (#3)",
// section 9: the indexer's quantisation-aware path rotates its vectors with a
// 128-point Hadamard transform and rounds them to 4-bit floats).
//
// The page names the transform and the 4-bit width; the block size, scale rule
// and bit layout are those of the OCP microscaling format MXFP4:
//   * y = x H / sqrt(128), H the Sylvester-order Hadamard matrix (symmetric,
//     H[j][k] = (-1)^popcount(j & k));
//   * per block of 32 consecutive channels one power-of-two scale 2^e with
//     e = floor(log2 max|y|) - 2, clamped to [-127, 127] (-127 for a block of
//     zeros), stored as the E8M0 byte e + 127;
//   * each y / 2^e rounded to the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}:
//     nearest, a tie going to the even code, saturated at 6; bit 3 is the sign
//     and is set only for a nonzero magnitude.
// A stored row is 64 code bytes (channel 2j in the low nibble of byte j) and
// then the 4 scale bytes: 68 bytes.
//
// Lane layout.  A vector is held by the four lanes l, l ^ 16, l ^ 32, l ^ 48 of
// a wave: the lane in 16-lane row g holds channels 32 g .. 32 g + 31, i.e. one
// MXFP4 block.  That is the operand layout of the gfx950 scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 operands (lane (r, g) supplies
// k = 32 g .. 32 g + 31 of row r of A, or of column r of B, as 16 bytes with
// k at nibble k % 8 of dword k / 8, plus that block's E8M0 scale), so a block
// encoded by a lane is the operand that lane feeds to the MFMA, and a stored
// row's 16-byte block g is the B operand of lane (r, g) as it lies in memory.
#pragma once

#include "ckv_device.h"

namespace ckv {

constexpr int kFp4RowBytes = 68;   // 128 channels
typedef int i32x8 __attribute__((ext_vector_type(8)));
// a 16-byte vector at a 4-byte aligned address (stored rows are 68 bytes apart)
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));

// Butterfly on the lane bit that permlane swap S exchanges: the lane with the
// bit clear receives a + b, the other a - b (a from the lane with the bit clear).
// neg: 0x80000000 on the lanes with the bit set, else 0 (a + (-b) is a - b
// exactly).
__device__ __forceinline__ float hbfly32(float v, uint32_t neg) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // s[0]: the value of the lane with bit 5 clear, s[1]: with bit 5 set
  return __uint_as_float(s[0]) + __uint_as_float(s[1] ^ neg);
}
__device__ __forceinline__ float hbfly16(float v, uint32_t neg) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1] ^ neg);
}

// Orthonormal 128-point Walsh-Hadamard transform of the vector held by lanes
// l, l ^ 16, l ^ 32, l ^ 48 (this lane: channels 32 g .. 32 g + 31, g = lane
// bits 4-5).  Channel bits 0-4 are butterflies inside the lane; bits 5 and 6
// are lane bits 4 and 5.  All lanes of the wave must be active.
__device__ __forceinline__ void fwht128(float (&v)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  const int lane = threadIdx.x & 63;
  const uint32_t n16 = (lane & 16) ? 0x80000000u : 0u, n32 = (lane & 32) ? 0x80000000u : 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = hbfly16(v[i], n16);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = hbfly32(v[i], n32) * 0.08838834764831845f;   // 1 / sqrt(128)
}

// E2M1 magnitude of code m (0..7)
__device__ __forceinline__ float e2m1_value(uint32_t m) {
  return m < 4 ? 0.5f * (float)m : m == 4 ? 2.f : m == 5 ? 3.f : m == 6 ? 4.f : 6.f;
}

// Block exponent of a block whose largest magnitude is am: e = floor(log2 am)
// - 2 (frexp's exponent is floor(log2 am) + 1), -127 for am = 0 or below
// 2^-125; at most 125 for any finite float.
__device__ __forceinline__ int mxfp4_exponent(float am) {
  return am > 0.f ? max(__builtin_amdgcn_frexp_expf(am) - 3, -127) : -127;
}

// E2M1 codes of 8 values divided by 2^e (value i at nibble i), by the gfx950
// conversion v_cvt_scalef32_pk_fp4_f32, which divides by its scale operand
// and rounds to the nearest grid point, ties to the even code, saturating at
// 6 -- measured against the rounding rule on MI355X for values around every
// boundary and tie and for scales 2^-100 .. 2^10.  It keeps the sign of a
// negative value that rounds to zero (code 8); the stored form has code 0
// there, so those sign bits are cleared.  The scale 2^-127 is not a normal
// float: that case divides 2 x by 2^-126 instead (both exact).
__device__ __forceinline__ uint32_t fp4_codes8(float v0, float v1, float v2, float v3, float v4, float v5, float v6,
                                               float v7, int e) {
  const float s = __uint_as_float((uint32_t)(127 + max(e, -126)) << 23);
  const float pre = e == -127 ? 2.f : 1.f;
  uint32_t r = 0u;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v0 * pre, v1 * pre, s, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v2 * pre, v3 * pre, s, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v4 * pre, v5 * pre, s, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v6 * pre, v7 * pre, s, 3);
  const uint32_t m = r & 0x77777777u;
  const uint32_t nz = (m | (m >> 1) | (m >> 2)) & 0x11111111u;   // bit 0 of each nibble: magnitude != 0
  return r & (0x77777777u | (nz << 3));
}

// MXFP4 encoding of this lane's block of 32 values: the codes (channel j at
// nibble j % 8 of dword j / 8) are returned, the scale byte e + 127 in
// scale_byte.
__device__ __forceinline__ u32x4 mxfp4_block(const float (&v)[32], uint32_t& scale_byte) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  const int e = mxfp4_exponent(am);
  u32x4 codes;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    codes[q] = fp4_codes8(v[8 * q], v[8 * q + 1], v[8 * q + 2], v[8 * q + 3], v[8 * q + 4], v[8 * q + 5],
                          v[8 * q + 6], v[8 * q + 7], e);
  scale_byte = (uint32_t)(e + 127);
  return codes;
}

// The scaled fp4 MFMA: D = A (16 x 128) * B (128 x 16) + C, each lane's block
// weighted by its E8M0 scale byte (bits 0-7 of sa / sb).
__device__ __forceinline__ f32x4 mfma_fp4(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb, f32x4 c) {
  const i32x8 A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // operand formats 4 and 4: E2M1 for both A and B
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// Decoded values of 8 stored codes (channel i at nibble i) of a block with
// E8M0 scale byte sb.
__device__ __forceinline__ void fp4_decode8(uint32_t codes, uint32_t sb, float (&v)[8]) {
  const int e = (int)(sb & 255u) - 127;
  const float sc = __uint_as_float((uint32_t)(127 + min(max(e, -126), 127)) << 23) * (e == -127 ? 0.5f : 1.f);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = (codes >> (4 * i)) & 15u;
    const float mag = e2m1_value(c & 7u) * sc;
    v[i] = (c & 8u) ? -mag : mag;
  }
}

// One RoPE pair (a, b) rotated by the angle with cosine c and sine s, with
// explicit fmas (the rounding does not depend on the compiler's contraction
// choices).
__device__ __forceinline__ float2 rope_pair(float a, float b, float c, float s) {
  return make_float2(fmaf(a, c, -(b * s)), fmaf(a, s, b * c));
}

// RoPE of this lane's block of an indexer vector (channels 32 g .. 32 g + 31,
// pairs 16 g .. 16 g + 15 of the 128 channels), cos / sin of its pairs at
// cs[0..15], sn[0..15] (16-byte aligned): every pair is rotated, the pairs
// before the tail with cos 1, sin 0, which leaves them exactly as they are.
__device__ __forceinline__ void rope_block32(float (&v)[32], const float* cs, const float* sn) {
  float c[16], s[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 a = *(const float4*)(cs + 4 * q), b = *(const float4*)(sn + 4 * q);
    c[4 * q] = a.x; c[4 * q + 1] = a.y; c[4 * q + 2] = a.z; c[4 * q + 3] = a.w;
    s[4 * q] = b.x; s[4 * q + 1] = b.y; s[4 * q + 2] = b.z; s[4 * q + 3] = b.w;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float2 r = rope_pair(v[2 * j], v[2 * j + 1], c[j], s[j]);
    v[2 * j] = r.x;
    v[2 * j + 1] = r.y;
  }
}

// ---- the same transform on 16 lanes x 8 channels -------------------------
// Lane s = lane % 16 of each 16-lane row holds channels 8 s .. 8 s + 7 of one
// vector (one MXFP4 block = 4 consecutive lanes).  For kernels that cannot
// spare 32 registers per lane.  The butterflies run in the same bit order
// with the same operands as fwht128 (bit-clear value a, bit-set value b:
// a + b and a - b), so both give bit-identical results.

// v of lane s ^ m (m = 1, 2, 4, 8) within the 16-lane row, through DPP
template <int M>
__device__ __forceinline__ float xor16(float v) {
  if constexpr (M == 1) return dpp_f32<0xb1>(0.f, v);                         // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_f32<0x4e>(0.f, v);                    // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return dpp_f32<0x1b>(0.f, dpp_f32<0x141>(0.f, v));   // half-mirror (s ^ 7), then s ^ 3
  else return dpp_f32<0x128>(0.f, v);                                         // row_ror:8
}

// butterfly on lane bit M: the bit-clear lane keeps a + b, the other a - b
template <int M>
__device__ __forceinline__ void bfly16(float (&v)[8], bool hi) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = xor16<M>(v[i]);
    v[i] = hi ? o - v[i] : v[i] + o;
  }
}

__device__ __forceinline__ void fwht128_x8(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!(i & h)) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  const int s = threadIdx.x & 15;
  bfly16<1>(v, s & 1);
  bfly16<2>(v, s & 2);
  bfly16<4>(v, s & 4);
  bfly16<8>(v, s & 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= 0.08838834764831845f;
}

// MXFP4 of the block of 4 lanes (s / 4): this lane's 8 codes (channel 8 s + i
// at nibble i) are returned, the block's scale byte in scale_byte.
__device__ __forceinline__ uint32_t mxfp4_x8(const float (&v)[8], uint32_t& scale_byte) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  am = fmaxf(am, xor16<1>(am));
  am = fmaxf(am, xor16<2>(am));
  const int e = mxfp4_exponent(am);
  scale_byte = (uint32_t)(e + 127);
  return fp4_codes8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], e);
}

// Encode one indexer row held in LDS (z[0..127], after its RoPE) and store
// the 68-byte record at dst; called by a whole wave (every 16-lane row
// computes the row; lanes 0-15 store it, unless store is false).  With rt !=
// NULL the decoded values (Hadamard domain) are written to rt[0..127] by the
// same lanes (rt may be z).
__device__ __forceinline__ void fp4_store_row(const float* z, uint8_t* dst, float* rt, bool store = true) {
  const int lane = threadIdx.x & 63, s = lane & 15;
  const float4 t0 = *(const float4*)(z + 8 * s), t1 = *(const float4*)(z + 8 * s + 4);
  float v[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
  fwht128_x8(v);
  uint32_t sb;
  const uint32_t codes = mxfp4_x8(v, sb);
  if (rt) fp4_decode8(codes, sb, v);
  if (lane < 16) {
    if (store) {
      *(uint32_t*)(dst + 4 * s) = codes;
      if ((s & 3) == 0) dst[64 + (s >> 2)] = (uint8_t)sb;
    }
    if (rt) {
      *(float4*)(rt + 8 * s) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(rt + 8 * s + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

}  // namespace ckv
