// Device helpers shared by the CDNA4 (gfx950) kernels of libckv.
//
// Number formats: bfloat16 (round to nearest even) and OCP FP8 E4M3FN with a
// float32 row scale (the attention-cache format of "ds4.c を読み解く (#3)",
// section 9: the non-RoPE channels go through FP8, the RoPE tail does not).
// Both codecs are written from the format definitions with integer bit
// arithmetic, so their rounding does not depend on the hardware converters.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ckv_internal.h"

namespace ckv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bfloat16 bits, round to nearest, ties to even (NaN stays NaN):
// the conversion instruction of gfx950 (v_cvt_pk_bf16_f32), two values at a time.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- E4M3FN

// code -> value.  Exponent field 0 holds subnormals m * 2^-9; otherwise the
// value is (1 + m/8) * 2^(e-7).  The NaN pattern is never stored.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// value -> code, round to nearest even on the E4M3 grid, saturated to +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  if (!(a < 448.0f)) return sign | 0x7eu;           // also catches values that round past 448
  if (a < 0.015625f) {                               // below 2^-6: quantum 2^-9
    const float m = __builtin_rintf(a * 512.0f);     // exact scaling, RNE
    return sign | (uint32_t)m;                        // m == 8 encodes 2^-6 itself
  }
  uint32_t u = __float_as_uint(a);
  u += 0x7ffffu + ((u >> 20) & 1u);                  // RNE to 3 mantissa bits
  const uint32_t e = (u >> 23) - 120u;               // E4M3 exponent field
  const uint32_t m = (u >> 20) & 7u;
  if (e > 15u || (e == 15u && m == 7u)) return sign | 0x7eu;
  return sign | (e << 3) | m;
}

// ---------------------------------------------------------------- RoPE

// cos / sin of pos * theta_j.  The angle is formed in fp64 and reduced to
// [-pi, pi] with a two-part 2*pi (error ~1e-11 rad at positions near 2^20);
// the reduced angle then goes through float sincos.  theta_j comes from the
// host (LayerParams::theta, base^(-2j/n_rot) in fp64).  All RoPE tails here
// have n_rot = 64, so pair j of every tail uses theta_j.
__device__ __forceinline__ void rope_cs_theta(double theta, double pos, float* c, float* s) {
  const double a = pos * theta;
  const double k = rint(a * 0.15915494309189535);      // a / (2 pi)
  double r = fma(-k, 6.283185307179586, a);            // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);              // 2 pi, low part
  sincosf((float)r, s, c);
}
// Pair j at position pos in the raw rows' frame (raw rows, the query against
// them) and in the compressed class's frame (compressed rows, indexer rows,
// the query against them); the two coincide when the layer has one base.
__device__ __forceinline__ void rope_cs(const LayerParams& P, int j, double pos, float* c, float* s) {
  rope_cs_theta(P.theta[j], pos, c, s);
}
__device__ __forceinline__ void rope_cs_c(const LayerParams& P, int j, double pos, float* c, float* s) {
  rope_cs_theta(P.theta_c[j], pos, c, s);
}
// theta_c[j] (theta[j]) for a lane-dependent j, chosen among the 32 entries read as
// scalars: indexing the kernel-argument array with a per-lane j compiles to a
// vector load from the argument segment, which a kernel that has issued its
// own vector loads first then waits for behind all of them.
__device__ __forceinline__ double theta_c_sel(const LayerParams& P, int j) {
  double t = 0.0;
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) t = j == jj ? P.theta_c[jj] : t;
  return t;
}
__device__ __forceinline__ double theta_sel(const LayerParams& P, int j) {
  double t = 0.0;
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) t = j == jj ? P.theta[jj] : t;
  return t;
}
// Rotation that takes a vector turned by pos in the raw frame to the same
// vector turned by pos in the compressed frame: angle pos (theta_c - theta).
__device__ __forceinline__ void rope_cs_switch(const LayerParams& P, int j, double pos, float* c, float* s) {
  rope_cs_theta(P.theta_c[j] - P.theta[j], pos, c, s);
}

// ---------------------------------------------------------------- MFMA

// D = A(16x32) * B(32x16) + C on bf16 inputs with fp32 accumulation.
// Lane l holds A[l%16][8(l/16) .. 8(l/16)+7], B[8(l/16) .. +7][l%16] and
// returns D[4(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- barriers

// Workgroup barrier that orders LDS only.  __syncthreads() also drains every
// outstanding global memory operation (its release fence must cover global
// stores, and on this architecture loads and stores share one counter), which
// would stall prefetched loads at every barrier.  Use this one where the
// barrier protects LDS data only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- reductions

// Cross-lane steps on DPP (data-parallel primitives: a lane reads another
// lane's register within the VALU operation, no LDS round trip).  Controls:
// quad_perm [1,0,3,2] = 0xb1, [2,3,0,1] = 0x4e, row_half_mirror = 0x141,
// row_mirror = 0x140, row_shr:n = 0x110 + n, row_bcast:15 = 0x142 (lane 15
// of each row to the next row), row_bcast:31 = 0x143 (lane 31 to rows 2, 3).
// Lanes whose source is masked off or out of range receive `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf,
                                                    false));
}

// Wave-wide sum / max, returned to every lane: butterflies inside each row of
// 16 lanes, then the row totals chained through lanes 15 and 31 up to lane 63,
// which is read back as a scalar.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xb1>(0.f, v);
  v += dpp_f32<0x4e>(0.f, v);
  v += dpp_f32<0x141>(0.f, v);
  v += dpp_f32<0x140>(0.f, v);
  v += dpp_f32<0x142, 0xa>(0.f, v);
  v += dpp_f32<0x143, 0xc>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xb1>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x4e>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x141>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x140>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x142, 0xa>(-INFINITY, v));
  v = fmaxf(v, dpp_f32<0x143, 0xc>(-INFINITY, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Sum over each row of 16 lanes, every lane of the row receiving it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xb1>(0.f, v);
  v += dpp_f32<0x4e>(0.f, v);
  v += dpp_f32<0x141>(0.f, v);
  v += dpp_f32<0x140>(0.f, v);
  return v;
}

// Sum / max over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (the same lane of the
// four 16-lane rows), every lane receiving the result: v_permlane32_swap and
// v_permlane16_swap exchange rows in the VALU, with no LDS round trip.
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Inclusive prefix sum over the wave's lanes (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<0x111>(0u, x);
  x += dpp_u32<0x112>(0u, x);
  x += dpp_u32<0x114>(0u, x);
  x += dpp_u32<0x118>(0u, x);
  x += dpp_u32<0x142, 0xa>(0u, x);
  x += dpp_u32<0x143, 0xc>(0u, x);
  return x;
}

// Block-wide sum; `red` is LDS scratch of at least blockDim.x/64 floats.
// Every thread returns the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

// ---------------------------------------------------------------- format IO

// ---- row slots of the compressed caches -------------------------------------
// Compressed row i of sequence b sits at slot b * cap + i of a contiguous
// cache.  A paged cache ("vLLM DeepSeek V4", KV cache memory management: one
// logical block of 256 token positions for every compressed layer) keeps it
// at slot page * rpb + i % rpb of its page pools, rpb = 256 / ratio rows a
// page, page = blocks[b * max_blocks + i / rpb]; the K=V and the indexer rows
// of a c4a layer share the page index.  An entry outside the pool gives -1.
__device__ __forceinline__ long long row_slot(const LayerParams& P, int b, int i) {
  if (!P.blocks) return (long long)b * P.cap + i;
  const int pg = P.blocks[(size_t)b * P.max_blocks + (i >> P.rpb_shift)];
  const int m = (1 << P.rpb_shift) - 1;
  return (pg >= 0 && pg < P.n_pages) ? ((long long)pg << P.rpb_shift) + (i & m) : -1;
}
// the slot a read takes: a bad entry reads page 0 (the write that stored the
// row reported it)
__device__ __forceinline__ long long row_slot_rd(const LayerParams& P, int b, int i) {
  const long long s = row_slot(P, b, i);
  return s >= 0 ? s : (long long)(i & ((1 << P.rpb_shift) - 1));
}
// the slot a store takes, or -1 after flagging the sequence
__device__ __forceinline__ long long row_slot_wr(const LayerParams& P, uint32_t* status, int b, int i) {
  const long long s = row_slot(P, b, i);
  if (s < 0 && status) atomicOr(&status[b], CKV_STATUS_PAGE);
  return s;
}

template <int FMT>
__device__ __forceinline__ float load_val(const void* p, long i) {
  if constexpr (FMT == CKV_F32) return ((const float*)p)[i];
  else return bf16_to_f32(((const uint16_t*)p)[i]);
}

template <int FMT>
__device__ __forceinline__ void store_val(void* p, long i, float v) {
  if constexpr (FMT == CKV_F32) ((float*)p)[i] = v;
  else ((uint16_t*)p)[i] = (uint16_t)f32_to_bf16(v);
}

// float key that orders like the float (larger float -> larger key); -0 is
// first folded onto +0 so the two compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace ckv
