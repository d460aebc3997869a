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
__device__ __forceinline__ float hbfly32(float v, bool hi) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // s[0]: the value of the lane with bit 5 clear, s[1]: with bit 5 set
  const float a = __uint_as_float(s[0]), b = __uint_as_float(s[1]);
  return hi ? a - b : a + b;
}
__device__ __forceinline__ float hbfly16(float v, bool hi) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(s[0]), b = __uint_as_float(s[1]);
  return hi ? a - b : a + b;
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
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = hbfly16(v[i], lane & 16);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = hbfly32(v[i], lane & 32) * 0.08838834764831845f;   // 1 / sqrt(128)
}

// E2M1 magnitude code of a >= 0 (a value already divided by its block scale):
// nearest grid point, ties to the even code, 6 and above -> 7.
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}
__device__ __forceinline__ float e2m1_value(uint32_t m) {
  return m < 4 ? 0.5f * (float)m : m == 4 ? 2.f : m == 5 ? 3.f : m == 6 ? 4.f : 6.f;
}

// MXFP4 encoding of this lane's block of 32 values: the codes (channel j at
// nibble j % 8 of dword j / 8) and the scale byte e + 127 are returned; with
// ROUND_TRIP, v is replaced by the decoded values.
template <bool ROUND_TRIP>
__device__ __forceinline__ u32x4 mxfp4_block(float (&v)[32], uint32_t& scale_byte) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  // floor(log2 am) = frexp exponent - 1; e <= 125 for any finite float
  const int e = am > 0.f ? max(__builtin_amdgcn_frexp_expf(am) - 3, -127) : -127;
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, a normal float
  const float sc = __uint_as_float((uint32_t)(127 + max(e, -126)) << 23);
  u32x4 codes = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float x = v[i] * inv;   // exact: a power-of-two scaling
    const uint32_t m = e2m1_mag(fabsf(x));
    const uint32_t c = m | (x < 0.f && m ? 8u : 0u);
    codes[i >> 3] |= c << (4 * (i & 7));
    if constexpr (ROUND_TRIP) {
      // 2^e: for e = -127 (sc holds 2^-126) the extra halving is exact
      const float mag = e2m1_value(m) * sc * (e == -127 ? 0.5f : 1.f);
      v[i] = x < 0.f ? -mag : mag;
    }
  }
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

// One RoPE pair (a, b) rotated by the angle with cosine c and sine s, written
// with explicit fmas so that every kernel rotating an indexer query rounds
// alike (the decode step's scan and its selection block must derive the same
// fp4 query).
__device__ __forceinline__ float2 rope_pair(float a, float b, float c, float s) {
  return make_float2(fmaf(a, c, -(b * s)), fmaf(a, s, b * c));
}

// Tail RoPE of this lane's block of an indexer vector (channels 32 g .. +31;
// the tail is channels DI - n_rot .. DI - 1, pair j = channels dn + 2 j,
// dn + 2 j + 1), with cos / sin of pair j at cs[j], sn[j].
__device__ __forceinline__ void rope_block32(float (&v)[32], int g, int dn, const float* cs, const float* sn) {
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    const int c = 32 * g + i;
    if (c >= dn) {
      const int j = (c - dn) >> 1;
      const float2 r = rope_pair(v[i], v[i + 1], cs[j], sn[j]);
      v[i] = r.x;
      v[i + 1] = r.y;
    }
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
// at nibble i) are returned, the block's scale byte in scale_byte; with
// ROUND_TRIP v receives the decoded values.
template <bool ROUND_TRIP>
__device__ __forceinline__ uint32_t mxfp4_x8(float (&v)[8], uint32_t& scale_byte) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
  am = fmaxf(am, xor16<1>(am));
  am = fmaxf(am, xor16<2>(am));
  const int e = am > 0.f ? max(__builtin_amdgcn_frexp_expf(am) - 3, -127) : -127;
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  const float sc = __uint_as_float((uint32_t)(127 + max(e, -126)) << 23);
  uint32_t codes = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = v[i] * inv;
    const uint32_t m = e2m1_mag(fabsf(x));
    codes |= (m | (x < 0.f && m ? 8u : 0u)) << (4 * i);
    if constexpr (ROUND_TRIP) {
      const float mag = e2m1_value(m) * sc * (e == -127 ? 0.5f : 1.f);
      v[i] = x < 0.f ? -mag : mag;
    }
  }
  scale_byte = (uint32_t)(e + 127);
  return codes;
}

// Encode one indexer row held in LDS (z[0..127], after its RoPE) and store
// the 68-byte record at dst; called by a whole wave (every 16-lane row
// computes the row; lanes 0-15 store it).  With rt != NULL the decoded values
// (Hadamard domain) are written to rt[0..127] by the same lanes (rt may be z).
__device__ __forceinline__ void fp4_store_row(const float* z, uint8_t* dst, float* rt) {
  const int lane = threadIdx.x & 63, s = lane & 15;
  const float4 t0 = *(const float4*)(z + 8 * s), t1 = *(const float4*)(z + 8 * s + 4);
  float v[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
  fwht128_x8(v);
  uint32_t sb;
  const uint32_t codes = mxfp4_x8<true>(v, sb);
  if (lane < 16) {
    *(uint32_t*)(dst + 4 * s) = codes;
    if ((s & 3) == 0) dst[64 + (s >> 2)] = (uint8_t)sb;
    if (rt) {
      *(float4*)(rt + 8 * s) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(rt + 8 * s + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

}  // namespace ckv
