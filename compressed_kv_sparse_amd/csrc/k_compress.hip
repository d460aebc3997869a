// Compressor state store, window pooling, RMSNorm, tail RoPE and cache
// insertion for one layer -- the per-token compressor of "ds4.c を読み解く
// (#3)" sections 4-5 (steps 3-8), fused into one kernel per step the way the
// vLLM DeepSeek V4 page fuses compressor + RMSNorm + RoPE + cache insertion.
//
// Window state: token t's (kappa, sigma) lives in slot t % W of a per-sequence
// ring (W = 8 for c4a, 128 for c128a; the vLLM page keeps the compressor state
// as a sliding window of the same sizes).  Compressed row i pools the tokens
// i*r - (W - r) + j, j = 0..W-1 (c4a: the previous stride block and its own;
// c128a: its own 128 tokens); slot j adds APE row j to its score, and
// positions before token 0 carry no weight.  The pooled row is RMS-normalised,
// its last n_rot channels are rotated at position i*r, and it is stored in
// the cache format.  The raw sliding-window row of token t is u_t rotated at t.
#include "ckv_device.h"

namespace ckv {

// ------------------------------------------------------------ row helpers

// Rotate the last `nrot` entries of z[0..width) (LDS) at position `pos`.
// Caller synchronises before and after.
__device__ __forceinline__ void rope_lds(float* z, int width, int nrot, double base, double pos) {
  const int dn = width - nrot;
  for (int j = threadIdx.x; j < nrot / 2; j += blockDim.x) {
    float c, s;
    rope_cs(base, nrot, j, pos, &c, &s);
    const float a = z[dn + 2 * j], b = z[dn + 2 * j + 1];
    z[dn + 2 * j] = a * c - b * s;
    z[dn + 2 * j + 1] = a * s + b * c;
  }
}

// z <- gamma * z / sqrt(mean(z^2) + eps), channels owned as c = tid + k*blockDim.
__device__ __forceinline__ void rmsnorm_lds(float* z, int width, const float* gamma, float eps,
                                            float* red) {
  float ss = 0.f;
  for (int c = threadIdx.x; c < width; c += blockDim.x) ss += z[c] * z[c];
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)width + eps);
  for (int c = threadIdx.x; c < width; c += blockDim.x) z[c] = gamma[c] * (z[c] * inv);
}

// Store z[0..d) (LDS) as one K=V row record of format KVF.  All threads call.
template <int KVF>
__device__ __forceinline__ void store_row(uint8_t* dst, const float* z, int d, int n_rot,
                                          float* red) {
  if constexpr (KVF == CKV_F32) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) ((float*)dst)[c] = z[c];
  } else if constexpr (KVF == CKV_BF16) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) ((uint16_t*)dst)[c] = (uint16_t)f32_to_bf16(z[c]);
  } else {
    const int dn = d - n_rot;
    float amax = 0.f;
    for (int c = threadIdx.x; c < dn; c += blockDim.x) amax = fmaxf(amax, fabsf(z[c]));
    amax = block_max(amax, red);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    for (int c = threadIdx.x; c < dn; c += blockDim.x) dst[c] = (uint8_t)f32_to_e4m3(z[c] / s);
    uint16_t* tail = (uint16_t*)(dst + dn);
    for (int c = threadIdx.x; c < n_rot; c += blockDim.x) tail[c] = (uint16_t)f32_to_bf16(z[dn + c]);
    if (threadIdx.x == 0) *(float*)(dst + dn + 2 * n_rot) = s;
  }
}

template <int F>
__device__ __forceinline__ void store_vals(void* dst, const float* z, int n) {
  for (int c = threadIdx.x; c < n; c += blockDim.x) store_val<F>(dst, c, z[c]);
}

// Online per-channel softmax pooling over one window (same result as the
// max / exp / normalise sequence of the pages, one pass).
struct PoolAcc {
  float m = -INFINITY, s = 0.f, acc = 0.f;
  __device__ __forceinline__ void add(float e, float kv) {
    if (e > m) {
      const float f = expf(m - e);
      s = s * f + 1.f;
      acc = acc * f + kv;
      m = e;
    } else {
      const float w = expf(e - m);
      s += w;
      acc += w * kv;
    }
  }
  __device__ __forceinline__ float value() const { return s > 0.f ? acc / s : 0.f; }
};

// ------------------------------------------------------------ decode

// One block per sequence.  part: projection partials [splits][B][ncol].
template <int KVF, int IDXF, int ACTF>
__global__ __launch_bounds__(256) void k_compress_decode(LayerParams P, Weights w, Cache cc,
                                                         const void* __restrict__ u,
                                                         const int32_t* __restrict__ pos,
                                                         const float* __restrict__ part,
                                                         int splits, int B) {
  __shared__ float zs[kMaxD];
  __shared__ float zi[kMaxDI];
  __shared__ float red[16];
  const int b = blockIdx.x;
  const int p = pos[b];
  if (p < 0) {
    if (threadIdx.x == 0 && cc.status) atomicOr(&cc.status[b], CKV_STATUS_BAD_POS);
    return;
  }
  const int d = P.d, r = P.ratio;

  // raw sliding-window row: u rotated at p, stored in slot p % swa
  for (int c = threadIdx.x; c < d; c += blockDim.x) zs[c] = load_val<ACTF>(u, (long)b * d + c);
  __syncthreads();
  rope_lds(zs, d, P.n_rot, P.base, (double)p);
  __syncthreads();
  store_row<KVF>(cc.raw + ((size_t)b * P.swa + p % P.swa) * P.row_bytes, zs, d, P.n_rot, red);
  if (r == 0) return;

  // this token's projections -> window state slot p % W
  const int W = P.W;
  const size_t pstride = (size_t)B * P.ncol;
  const float* pb = part + (size_t)b * P.ncol;
  float kap[2] = {0.f, 0.f}, sig[2] = {0.f, 0.f};
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int c = threadIdx.x + n * blockDim.x;
    if (c < d) {
      float a = 0.f, g = 0.f;
      for (int s = 0; s < splits; ++s) {
        a += pb[s * pstride + c];
        g += pb[s * pstride + d + c];
      }
      kap[n] = a;
      sig[n] = g;
      const size_t o = ((size_t)b * W + p % W) * d + c;
      cc.st_kv[o] = a;
      cc.st_sc[o] = g;
    }
  }
  float kapi = 0.f, sigi = 0.f;
  const int DI = P.DI;
  if (r == 4 && (int)threadIdx.x < DI) {
    const int c = threadIdx.x;
    for (int s = 0; s < splits; ++s) {
      kapi += pb[s * pstride + 2 * d + c];
      sigi += pb[s * pstride + 2 * d + DI + c];
    }
    const size_t o = ((size_t)b * 8 + p % 8) * DI + c;
    cc.ist_kv[o] = kapi;
    cc.ist_sc[o] = sigi;
  }
  if ((p + 1) % r != 0) return;
  const int i = (p + 1) / r - 1;
  if (i >= P.cap) {
    if (threadIdx.x == 0 && cc.status) atomicOr(&cc.status[b], CKV_STATUS_CAPACITY);
    return;
  }

  // pool row i of the attention lane
  const int t0 = i * r - (W - r);
  const float* skv = cc.st_kv + (size_t)b * W * d;
  const float* ssc = cc.st_sc + (size_t)b * W * d;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int c = threadIdx.x + n * blockDim.x;
    if (c < d) {
      PoolAcc pa;
      for (int j = 0; j < W; ++j) {
        const int t = t0 + j;
        if (t < 0) continue;
        float kv, sc;
        if (t == p) {
          kv = kap[n];
          sc = sig[n];
        } else {
          kv = skv[(t % W) * d + c];
          sc = ssc[(t % W) * d + c];
        }
        pa.add(sc + w.ape[j * d + c], kv);
      }
      zs[c] = pa.value();
    }
  }
  rmsnorm_lds(zs, d, w.gamma, P.eps, red);
  __syncthreads();
  rope_lds(zs, d, P.n_rot, P.base, (double)i * r);
  __syncthreads();
  store_row<KVF>(cc.comp + ((size_t)b * P.cap + i) * P.row_bytes, zs, d, P.n_rot, red);

  if (r == 4) {  // indexer lane: its own compressor of the same form
    const float* ikv = cc.ist_kv + (size_t)b * 8 * DI;
    const float* isc = cc.ist_sc + (size_t)b * 8 * DI;
    const int c = threadIdx.x;
    if (c < DI) {
      PoolAcc pa;
      for (int j = 0; j < 8; ++j) {
        const int t = t0 + j;
        if (t < 0) continue;
        float kv, sc;
        if (t == p) {
          kv = kapi;
          sc = sigi;
        } else {
          kv = ikv[(t % 8) * DI + c];
          sc = isc[(t % 8) * DI + c];
        }
        pa.add(sc + w.idx_ape[j * DI + c], kv);
      }
      zi[c] = pa.value();
    }
    rmsnorm_lds(zi, DI, w.idx_gamma, P.eps, red);
    __syncthreads();
    rope_lds(zi, DI, P.idx_rot, P.base, (double)i * r);
    __syncthreads();
    uint8_t* dst = (uint8_t*)cc.idx + ((size_t)b * P.cap + i) * DI * (IDXF == CKV_F32 ? 4 : 2);
    store_vals<IDXF>(dst, zi, DI);
  }
}

// ------------------------------------------------------------ prefill

// Stage the raw rows of positions pos0-swa+1 .. pos0+T-1: earlier positions
// are copied from the ring, chunk positions computed from u.  One block per
// stage row.
template <int KVF, int ACTF>
__global__ __launch_bounds__(256) void k_stage_raw(LayerParams P, Cache cc, const void* __restrict__ u,
                                                   int seq, int pos0) {
  __shared__ float zs[kMaxD];
  __shared__ float red[16];
  const int sr = blockIdx.x;
  const int t = pos0 - (P.swa - 1) + sr;
  if (t < 0) return;
  uint8_t* dst = cc.stage + (size_t)sr * P.row_bytes;
  if (t < pos0) {
    const uint32_t* src = (const uint32_t*)(cc.raw + ((size_t)seq * P.swa + t % P.swa) * P.row_bytes);
    for (int c = threadIdx.x; c < P.row_bytes / 4; c += blockDim.x) ((uint32_t*)dst)[c] = src[c];
    return;
  }
  const int d = P.d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) zs[c] = load_val<ACTF>(u, (long)(t - pos0) * d + c);
  __syncthreads();
  rope_lds(zs, d, P.n_rot, P.base, (double)t);
  __syncthreads();
  store_row<KVF>(dst, zs, d, P.n_rot, red);
}

// Pool every row whose window closes inside the chunk.  Window tokens before
// pos0 come from the state ring, chunk tokens from the projection part[n][col].
// One block per emitted row i = i_first + blockIdx.x.
template <int KVF, int IDXF>
__global__ __launch_bounds__(256) void k_pool_prefill(LayerParams P, Weights w, Cache cc,
                                                      const float* __restrict__ part, int seq,
                                                      int pos0, int i_first) {
  __shared__ float zs[kMaxD];
  __shared__ float zi[kMaxDI];
  __shared__ float red[16];
  const int i = i_first + blockIdx.x;
  const int d = P.d, r = P.ratio, W = P.W, DI = P.DI, nc = P.ncol;
  const int t0 = i * r - (W - r);
  const float* skv = cc.st_kv + (size_t)seq * W * d;
  const float* ssc = cc.st_sc + (size_t)seq * W * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    PoolAcc pa;
    for (int j = 0; j < W; ++j) {
      const int t = t0 + j;
      if (t < 0) continue;
      float kv, sc;
      if (t >= pos0) {
        const float* pr = part + (size_t)(t - pos0) * nc;
        kv = pr[c];
        sc = pr[d + c];
      } else {
        kv = skv[(t % W) * d + c];
        sc = ssc[(t % W) * d + c];
      }
      pa.add(sc + w.ape[j * d + c], kv);
    }
    zs[c] = pa.value();
  }
  rmsnorm_lds(zs, d, w.gamma, P.eps, red);
  __syncthreads();
  rope_lds(zs, d, P.n_rot, P.base, (double)i * r);
  __syncthreads();
  store_row<KVF>(cc.comp + ((size_t)seq * P.cap + i) * P.row_bytes, zs, d, P.n_rot, red);
  if (r != 4) return;
  const float* ikv = cc.ist_kv + (size_t)seq * 8 * DI;
  const float* isc = cc.ist_sc + (size_t)seq * 8 * DI;
  for (int c = threadIdx.x; c < DI; c += blockDim.x) {
    PoolAcc pa;
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + j;
      if (t < 0) continue;
      float kv, sc;
      if (t >= pos0) {
        const float* pr = part + (size_t)(t - pos0) * nc;
        kv = pr[2 * d + c];
        sc = pr[2 * d + DI + c];
      } else {
        kv = ikv[(t % 8) * DI + c];
        sc = isc[(t % 8) * DI + c];
      }
      pa.add(sc + w.idx_ape[j * DI + c], kv);
    }
    zi[c] = pa.value();
  }
  rmsnorm_lds(zi, DI, w.idx_gamma, P.eps, red);
  __syncthreads();
  rope_lds(zi, DI, P.idx_rot, P.base, (double)i * r);
  __syncthreads();
  uint8_t* dst = (uint8_t*)cc.idx + ((size_t)seq * P.cap + i) * DI * (IDXF == CKV_F32 ? 4 : 2);
  store_vals<IDXF>(dst, zi, DI);
}

// After the chunk: the last W tokens' projections go to the state rings and
// the last swa staged raw rows to the raw ring.  Block j handles the j-th of
// the last swa positions.
__global__ __launch_bounds__(256) void k_state_prefill(LayerParams P, Cache cc,
                                                       const float* __restrict__ part, int seq,
                                                       int pos0, int T) {
  const int j = blockIdx.x;
  const int d = P.d, nc = P.ncol, DI = P.DI;
  const int end = pos0 + T;
  const int traw = end - P.swa + j;
  if (traw >= pos0) {
    const uint32_t* src = (const uint32_t*)(cc.stage + (size_t)(traw - pos0 + P.swa - 1) * P.row_bytes);
    uint32_t* dst = (uint32_t*)(cc.raw + ((size_t)seq * P.swa + traw % P.swa) * P.row_bytes);
    for (int c = threadIdx.x; c < P.row_bytes / 4; c += blockDim.x) dst[c] = src[c];
  }
  if (P.ratio == 0 || j >= P.W) return;
  const int W = P.W;
  const int t = end - W + j;
  if (t < pos0) return;
  const float* pr = part + (size_t)(t - pos0) * nc;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    const size_t o = ((size_t)seq * W + t % W) * d + c;
    cc.st_kv[o] = pr[c];
    cc.st_sc[o] = pr[d + c];
  }
  if (P.ratio == 4) {
    for (int c = threadIdx.x; c < DI; c += blockDim.x) {
      const size_t o = ((size_t)seq * 8 + t % 8) * DI + c;
      cc.ist_kv[o] = pr[2 * d + c];
      cc.ist_sc[o] = pr[2 * d + DI + c];
    }
  }
}

// ------------------------------------------------------------ launchers

template <int KVF, int IDXF, int ACTF>
static void go_decode(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                      const int32_t* pos, int B, const float* part, int splits, hipStream_t st) {
  hipLaunchKernelGGL((k_compress_decode<KVF, IDXF, ACTF>), dim3(B), dim3(256), 0, st, P, w, c, u,
                     pos, part, splits, B);
}

#define CKV_DISPATCH_KV_IDX_ACT(FN, ...)                                               \
  do {                                                                                 \
    const bool idx32 = P.idx_fmt == CKV_F32, act32 = P.act_fmt == CKV_F32;            \
    if (P.kv_fmt == CKV_F32) {                                                         \
      if (idx32 && act32) FN<CKV_F32, CKV_F32, CKV_F32>(__VA_ARGS__);                  \
      else if (act32) FN<CKV_F32, CKV_BF16, CKV_F32>(__VA_ARGS__);                     \
      else FN<CKV_F32, CKV_BF16, CKV_BF16>(__VA_ARGS__);                               \
    } else if (P.kv_fmt == CKV_BF16) {                                                 \
      if (act32) FN<CKV_BF16, CKV_BF16, CKV_F32>(__VA_ARGS__);                         \
      else if (idx32) FN<CKV_BF16, CKV_F32, CKV_BF16>(__VA_ARGS__);                    \
      else FN<CKV_BF16, CKV_BF16, CKV_BF16>(__VA_ARGS__);                              \
    } else {                                                                           \
      if (idx32) FN<CKV_E4M3, CKV_F32, CKV_BF16>(__VA_ARGS__);                         \
      else FN<CKV_E4M3, CKV_BF16, CKV_BF16>(__VA_ARGS__);                              \
    }                                                                                  \
  } while (0)

int launch_compress_decode(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                           const int32_t* pos, int B, const float* part, int splits, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  CKV_DISPATCH_KV_IDX_ACT(go_decode, P, w, c, u, pos, B, part, splits, st);
  return (int)hipGetLastError();
}

template <int KVF, int IDXF, int ACTF>
static void go_prefill(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                       int seq, int pos0, int T, const float* part, hipStream_t st) {
  hipLaunchKernelGGL((k_stage_raw<KVF, ACTF>), dim3(T + P.swa - 1), dim3(256), 0, st, P, c, u, seq,
                     pos0);
  if (P.ratio) {
    const int i_first = pos0 / P.ratio, i_end = (pos0 + T) / P.ratio;
    if (i_end > i_first)
      hipLaunchKernelGGL((k_pool_prefill<KVF, IDXF>), dim3(i_end - i_first), dim3(256), 0, st, P, w,
                         c, part, seq, pos0, i_first);
  }
  hipLaunchKernelGGL(k_state_prefill, dim3(P.swa), dim3(256), 0, st, P, c, part, seq, pos0, T);
}

int launch_compress_prefill(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                            int seq, int pos0, int T, const float* part, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  CKV_DISPATCH_KV_IDX_ACT(go_prefill, P, w, c, u, seq, pos0, T, part, st);
  return (int)hipGetLastError();
}

}  // namespace ckv
