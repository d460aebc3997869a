// Concatenated compressor weights and the decode projection block shared by
// the projection kernel and the fused decode-step scan (steps 1-2 of the
// per-token compressor of "ds4.c を読み解く (#3)", section 4).
#pragma once

#include "ckv_device.h"

namespace ckv {

// The four weight matrices seen as one [ncol, hidden] matrix whose row blocks
// are wkv | wgate | idx_wkv | idx_wgate.
struct WCat {
  const void* p[4];
  int start[5];  // column ranges of the four blocks
};

__device__ __forceinline__ const void* wcat_row(const WCat& wc, int col, int K, int esz, int* local) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (col >= wc.start[i]) s = i;
  *local = col - wc.start[s];
  return (const char*)wc.p[s] + (size_t)(*local) * K * esz;
}

inline WCat make_wcat(const LayerParams& P, const Weights& w) {
  WCat wc;
  wc.p[0] = w.wkv;
  wc.p[1] = w.wgate;
  wc.p[2] = w.idx_wkv;
  wc.p[3] = w.idx_wgate;
  // (two-lane c4a: each matrix has both lanes' rows, lane A first)
  wc.start[0] = 0;
  wc.start[1] = P.lanes * P.d;
  wc.start[2] = P.ratio == 4 ? 2 * P.lanes * P.d : 1 << 30;
  wc.start[3] = P.ratio == 4 ? P.lanes * (2 * P.d + P.DI) : 1 << 30;
  wc.start[4] = P.ncol;
  return wc;
}

// bf16 x bf16 on MFMA: 16 columns (col0 ..) x 16 rows (m0 ..) over all of K,
// the NW waves of the block taking the k-steps w, w + NW, ... (SF of them in
// flight per round, loads unconditional with the step clamped); partial
// tiles summed through LDS in wave order.  Writes part[m][col].
// K slice `slice` of `nslice` (k-steps of 32, split evenly) when nslice > 1;
// the result goes to part + slice * M * ncol.
template <int NW, int SF = 8>
__device__ __forceinline__ void proj_tile(const uint16_t* __restrict__ X, int M, int K, const WCat& wc, int ncol,
                                          float* __restrict__ part, int col0, int m0, int slice = 0,
                                          int nslice = 1) {
  __shared__ f32x4 red[NW][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  int local;
  const uint16_t* wrow = (const uint16_t*)wcat_row(wc, col0 + r, K, 2, &local);
  const uint16_t* xrow = X + (size_t)min(m0 + r, M - 1) * K;
  const int ktot = K / 32, per = (ktot + nslice - 1) / nslice;
  const int sbeg = slice * per, nsteps = min(ktot, sbeg + per);
  part += (size_t)slice * M * ncol;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = sbeg + wave; s0 < nsteps; s0 += NW * SF) {
    u32x4 a[SF], b[SF];
#pragma unroll
    for (int e = 0; e < SF; ++e) {
      const int k = 32 * min(s0 + NW * e, nsteps - 1) + 8 * g;
      a[e] = *(const u32x4*)(xrow + k);
      b[e] = *(const u32x4*)(wrow + k);
    }
#pragma unroll
    for (int e = 0; e < SF; ++e)
      if (s0 + NW * e < nsteps) acc = mfma16x16x32(as_bf16x8(a[e]), as_bf16x8(b[e]), acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 t = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += red[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 4 * g + i;
      if (m < M) part[(size_t)m * ncol + col0 + r] = t[i];
    }
  }
}

}  // namespace ckv
