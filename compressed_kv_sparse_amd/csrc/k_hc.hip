// Hyper-Connection mixer around the attention block ("ds4.c を読み解く (#3)",
// section 10): the hidden state is carried as four residual streams; a
// per-token mixer row is split into pre weights, post gates and a 4 x 4
// coupling matrix normalised by Sinkhorn iterations.
//
// Per token (mixer row m of 24 floats, streams h_0..h_3 of D channels):
//   pre_i  = sigmoid(m[i]),  post_j = sigmoid(m[4 + j]),
//   C      = Sinkhorn(m[8 ..], iters, eps): a softmax along each row, a column
//            normalisation, then (iters - 1) times a row and a column
//            normalisation, each dividing by (sum + eps);
//   x      = sum_i pre_i h_i                          (k_hc_pre: the block input)
//   h'_j   = sum_i C[j][i] h_i + post_j y             (k_hc_post: y = the block output)
// The page gives the split, the matrix size, the iteration count and the
// alternating normalisation with eps; the row layout, the logistic gates and
// the build step are this library's reading of it.
//
// k_hc_pre computes the split once per block with 16 lanes of wave 0 (lane
// 4 j + i holds C[j][i]: row sums over a quad, column sums over lanes 4 apart,
// both by DPP), leaves (pre, post, C) in coef for k_hc_post, and applies the
// pre weights over its channel slice.  Both kernels stream 8 channels per
// thread with 16-byte loads; grid (tokens, channel slices of 2048).
#include <hip/hip_runtime.h>

#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kHcThreads = 256;
constexpr int kHcSlice = kHcThreads * 8;   // channels per block

// v of lane ^ M within a 16-lane row (M = 1, 2, 4, 8), by DPP
template <int M>
__device__ __forceinline__ float hc_xor(float v) {
  if constexpr (M == 1) return dpp_f32<0xb1>(0.f, v);
  else if constexpr (M == 2) return dpp_f32<0x4e>(0.f, v);
  else if constexpr (M == 4) return dpp_f32<0x1b>(0.f, dpp_f32<0x141>(0.f, v));   // (l ^ 7) ^ 3
  else return dpp_f32<0x128>(0.f, v);                                            // row_ror:8
}

// 8 channels of a row in format F as floats (16 or 32 bytes)
template <int F>
__device__ __forceinline__ void load8(const void* p, size_t i, float (&v)[8]) {
  if constexpr (F == CKV_F32) {
    const float4 a = *(const float4*)((const float*)p + i), b = *(const float4*)((const float*)p + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const u32x4 a = *(const u32x4*)((const uint16_t*)p + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_to_f32(a[k] & 0xffffu);
      v[2 * k + 1] = bf16_to_f32(a[k] >> 16);
    }
  }
}

template <int F>
__device__ __forceinline__ void store8(void* p, size_t i, const float (&v)[8]) {
  if constexpr (F == CKV_F32) {
    *(float4*)((float*)p + i) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)((float*)p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    const u32x4 a = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    *(u32x4*)((uint16_t*)p + i) = a;
  }
}

__device__ __forceinline__ float hc_sigmoid(float x) { return 1.f / (1.f + expf(-x)); }

template <int ACTF>
__global__ __launch_bounds__(kHcThreads) void k_hc_pre(HcParams Hp, const float* __restrict__ mix,
                                                       const void* __restrict__ h, void* __restrict__ x,
                                                       float* __restrict__ coef) {
  __shared__ float pre_s[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const size_t D = (size_t)Hp.hidden;
  const int c0 = blockIdx.y * kHcSlice + 8 * tid;
  // this thread's channels of the four streams, issued before the split
  float hv[4][8];
  const bool act = c0 < (int)D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (act) load8<ACTF>(h, ((size_t)t * 4 + i) * D + c0, hv[i]);
  }
  if (tid < 64) {   // wave 0: the split; lanes 0-15 hold C[lane / 4][lane % 4]
    const int l = tid & 15;
    const float* m = mix + (size_t)t * 24;
    float c = m[8 + l];
    // row softmax: maximum and sum over the quad (the row)
    float mx = fmaxf(c, hc_xor<1>(c));
    mx = fmaxf(mx, hc_xor<2>(mx));
    c = expf(c - mx);
    float s = c + hc_xor<1>(c);
    s = s + hc_xor<2>(s);
    c = c / s;
    auto col_norm = [&] {
      float cs = c + hc_xor<4>(c);
      cs = cs + hc_xor<8>(cs);
      c = c / (cs + Hp.eps);
    };
    col_norm();
    for (int it = 1; it < Hp.iters; ++it) {
      float rs = c + hc_xor<1>(c);
      rs = rs + hc_xor<2>(rs);
      c = c / (rs + Hp.eps);
      col_norm();
    }
    const float g = tid < 8 ? hc_sigmoid(m[tid]) : 0.f;
    if (blockIdx.y == 0) {
      if (tid < 16) coef[(size_t)t * 24 + 8 + l] = c;
      if (tid < 8) coef[(size_t)t * 24 + tid] = g;
    }
    if (tid < 4) pre_s[tid] = g;
  }
  __syncthreads();
  if (!act) return;
  float o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float a = pre_s[0] * hv[0][k];
#pragma unroll
    for (int i = 1; i < 4; ++i) a = fmaf(pre_s[i], hv[i][k], a);
    o[k] = a;
  }
  store8<ACTF>(x, (size_t)t * D + c0, o);
}

template <int ACTF>
__global__ __launch_bounds__(kHcThreads) void k_hc_post(HcParams Hp, const float* __restrict__ coef,
                                                        const void* __restrict__ h, const void* __restrict__ y,
                                                        void* __restrict__ hout) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const size_t D = (size_t)Hp.hidden;
  const int c0 = blockIdx.y * kHcSlice + 8 * tid;
  if (c0 >= (int)D) return;
  const float* cf = coef + (size_t)t * 24;   // wave-uniform: scalar loads
  float hv[4][8], yv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) load8<ACTF>(h, ((size_t)t * 4 + i) * D + c0, hv[i]);
  load8<ACTF>(y, (size_t)t * D + c0, yv);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = cf[4 + j] * yv[k];
#pragma unroll
      for (int i = 0; i < 4; ++i) a = fmaf(cf[8 + 4 * j + i], hv[i][k], a);
      o[k] = a;
    }
    store8<ACTF>(hout, ((size_t)t * 4 + j) * D + c0, o);
  }
}

int launch_hc_pre(const HcParams& Hp, const float* mix, const void* h, int T, void* x, float* coef, void* stream) {
  dim3 grid(T, (Hp.hidden + kHcSlice - 1) / kHcSlice);
  hipStream_t st = (hipStream_t)stream;
  if (Hp.act_fmt == CKV_F32)
    hipLaunchKernelGGL(k_hc_pre<CKV_F32>, grid, dim3(kHcThreads), 0, st, Hp, mix, h, x, coef);
  else
    hipLaunchKernelGGL(k_hc_pre<CKV_BF16>, grid, dim3(kHcThreads), 0, st, Hp, mix, h, x, coef);
  return (int)hipGetLastError();
}

int launch_hc_post(const HcParams& Hp, const float* coef, const void* h, const void* y, int T, void* hout,
                   void* stream) {
  dim3 grid(T, (Hp.hidden + kHcSlice - 1) / kHcSlice);
  hipStream_t st = (hipStream_t)stream;
  if (Hp.act_fmt == CKV_F32)
    hipLaunchKernelGGL(k_hc_post<CKV_F32>, grid, dim3(kHcThreads), 0, st, Hp, coef, h, y, hout);
  else
    hipLaunchKernelGGL(k_hc_post<CKV_BF16>, grid, dim3(kHcThreads), 0, st, Hp, coef, h, y, hout);
  return (int)hipGetLastError();
}

}  // namespace ckv
