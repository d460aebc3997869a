// Compressor projections kappa = W_kv x, sigma = W_gate x (and the indexer
// lane's pair on ratio-4 layers) -- steps 1-2 of the per-token compressor of
// "ds4.c を読み解く (#3)", section 4.
//
// The four weight matrices are treated as one [ncol, hidden] matrix whose row
// blocks are wkv | wgate | idx_wkv | idx_wgate.  The result goes to
// part[split][m][col] in fp32; split-K partials are summed, in split order, by
// the compress kernels that consume them.
#include "proj_dec.h"

namespace ckv {

// bf16 activations x bf16 weights on MFMA.  One wave computes a 32 x 16 tile
// (two 16-row blocks of x against 16 weight rows) over one K range.
// grid: x = (cend - cbase) / 64 (4 waves of 16 columns), y = splits,
// z = ceil(M / 32); part rows have stride ncol.
__global__ __launch_bounds__(256) void k_proj_mfma(const uint16_t* __restrict__ X, int M, int K,
                                                   WCat wc, int ncol, int klen,
                                                   float* __restrict__ part, int cbase, int cend) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col0 = cbase + blockIdx.x * 64 + wave * 16;
  if (col0 >= cend) return;
  const int m0 = blockIdx.z * 32;
  const int k0 = blockIdx.y * klen, k1 = min(K, k0 + klen);
  const int r = lane & 15, g = lane >> 4;

  int local;
  const uint16_t* wrow = (const uint16_t*)wcat_row(wc, col0 + r, K, 2, &local);
  const bool ok0 = (m0 + r) < M, ok1 = (m0 + 16 + r) < M;
  const uint16_t* x0 = X + (size_t)(ok0 ? m0 + r : 0) * K;
  const uint16_t* x1 = X + (size_t)(ok1 ? m0 + 16 + r : 0) * K;

  f32x4 c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
  const u32x4 zero = {0, 0, 0, 0};
  int k = k0;
  for (; k + 256 <= k1; k += 256) {   // eight k-steps' loads in flight
    u32x4 a0[8], a1[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kk = k + 32 * s + 8 * g;
      b[s] = *(const u32x4*)(wrow + kk);
      a0[s] = ok0 ? *(const u32x4*)(x0 + kk) : zero;
      a1[s] = ok1 ? *(const u32x4*)(x1 + kk) : zero;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      c0 = mfma16x16x32(as_bf16x8(a0[s]), as_bf16x8(b[s]), c0);
      c1 = mfma16x16x32(as_bf16x8(a1[s]), as_bf16x8(b[s]), c1);
    }
  }
  for (; k < k1; k += 32) {
    const int kk = k + 8 * g;
    const u32x4 b = *(const u32x4*)(wrow + kk);
    const u32x4 a0 = ok0 ? *(const u32x4*)(x0 + kk) : zero;
    const u32x4 a1 = ok1 ? *(const u32x4*)(x1 + kk) : zero;
    c0 = mfma16x16x32(as_bf16x8(a0), as_bf16x8(b), c0);
    c1 = mfma16x16x32(as_bf16x8(a1), as_bf16x8(b), c1);
  }
  float* out = part + (size_t)blockIdx.y * M * ncol;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ma = m0 + 4 * g + i, mb = m0 + 16 + 4 * g + i;
    if (ma < M) out[(size_t)ma * ncol + col0 + r] = c0[i];
    if (mb < M) out[(size_t)mb * ncol + col0 + r] = c1[i];
  }
}

// Decode (few rows): bf16 x bf16 on MFMA, one block of 4 waves per 16
// columns x 16 rows x one of gridDim.z slices of K.  Wave w takes the
// slice's k-steps w, w + 4, ... (eight of them in flight per round, their
// loads unconditional with the step index clamped); the 4 partial tiles are
// summed through LDS in wave order, so the result is the same on every run.
// Splitting K over blocks puts the weight stream on more compute units (a
// unit keeps only a limited number of misses in flight).  grid: x = ncol / 16,
// y = ceil(M / 16), z = K slices; writes part[slice][m][col].
// (Measured, c128a layer, 16 rows, K = 4096 in 4 slices: 5.1 us with 4 waves
// of 8 k-steps each, 7.2 us with 8 waves, 10.7 us with 16 waves of 2 useful
// k-steps and 6 clamped repeats; 2 waves 5.4 us, 8 slices 5.2-7.3 us.)
constexpr int kProjDecWaves = 4;
__global__ __launch_bounds__(1024) void k_proj_dec(const uint16_t* __restrict__ X, int M, int K, WCat wc, int ncol,
                                                   float* __restrict__ part, int cbase) {
  proj_tile<kProjDecWaves>(X, M, K, wc, ncol, part, cbase + blockIdx.x * 16, blockIdx.y * 16, blockIdx.z,
                           gridDim.z);
}

// Chunk projection (M >= 128 rows): a tiled GEMM.  A block computes a 128 x 128
// tile of part[m][col] (128 rows of x against 128 weight rows, which all lie
// in one of the four weight matrices when d and D_I are multiples of 128);
// wave w takes the 64 x 64 quadrant (w / 2, w % 2) as 4 x 4 MFMA tiles.  K is
// walked in chunks of 64: both 128 x 64 operand tiles are staged in LDS
// (double-buffered; the next chunk's global loads are issued before the
// current chunk is multiplied).  A tile row is 128 bytes = 8 chunks of 16; row
// R keeps chunk c at position c ^ ((R >> 1) & 7), so the 16 rows of a fragment
// read spread over all banks.
constexpr int kGM = 128, kGN = 128, kGK = 64;

__device__ __forceinline__ int gsw(int R, int c) { return R * 128 + 16 * (c ^ ((R >> 1) & 7)); }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_proj_gemm(
    const uint16_t* __restrict__ X, int M, int K, WCat wc, int ncol, float* __restrict__ part, int cbase) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[2][kGM * 128], sb[2][kGN * 128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int col0 = cbase + blockIdx.x * kGN, m0 = blockIdx.y * kGM;
  int local;
  const uint16_t* W = (const uint16_t*)wcat_row(wc, col0, K, 2, &local);   // row col0 of its matrix
  // staging: thread t moves 16-byte chunks t + 256 e (e < 4) of each 128 x 64 tile: row ch >> 3, chunk ch & 7
  u32x4 pa[4], pb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch = tid + 256 * e, R = ch >> 3, c = ch & 7;
      pa[e] = *(const u32x4*)(X + (size_t)min(m0 + R, M - 1) * K + k0 + 8 * c);
      pb[e] = *(const u32x4*)(W + (size_t)R * K + k0 + 8 * c);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch = tid + 256 * e, R = ch >> 3, c = ch & 7;
      *(u32x4*)&sa[buf][gsw(R, c)] = pa[e];
      *(u32x4*)&sb[buf][gsw(R, c)] = pb[e];
    }
  };
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int nk = K / kGK;
  load(0);
  store(0);
  lds_barrier();
#pragma unroll 1
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) load((kc + 1) * kGK);   // in flight during this chunk
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *(const u32x4*)&sa[buf][gsw(wm + 16 * i + r, 4 * ks + g)];
        bf[i] = *(const u32x4*)&sb[buf][gsw(wn + 16 * i + r, 4 * ks + g)];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(as_bf16x8(af[i]), as_bf16x8(bf[j]), acc[i][j]);
    }
    if (kc + 1 < nk) store(buf ^ 1);
    lds_barrier();
  }
  // D[4 g + e][r] of tile (i, j): row m0 + wm + 16 i + 4 g + e, column col0 + wn + 16 j + r
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + wm + 16 * i + 4 * g + e;
      if (m < M) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part[(size_t)m * ncol + col0 + wn + 16 * j + r] = acc[i][j][e];
      }
    }
}

// Any formats, vector ALU: one wave per (column, 4 rows), lanes stride K.
// grid: x = ncol, y = ceil(M / 4).  Writes split 0.
template <int XF, int WF>
__global__ __launch_bounds__(64) void k_proj_vec(const void* __restrict__ X, int M, int K, WCat wc,
                                                 int ncol, float* __restrict__ part, int cbase) {
  const int col = cbase + blockIdx.x, m0 = blockIdx.y * 4, lane = threadIdx.x;
  int local;
  const void* wrow = wcat_row(wc, col, K, WF == CKV_F32 ? 4 : 2, &local);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = lane; k < K; k += 64) {
    const float wv = load_val<WF>(wrow, k);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + i < M) acc[i] += wv * load_val<XF>(X, (long)(m0 + i) * K + k);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = wave_sum(acc[i]);
    if (lane == 0 && m0 + i < M) part[(size_t)(m0 + i) * ncol + col] = s;
  }
}

int launch_proj(const LayerParams& P, const Weights& w, const void* x, int M, float* part,
                int splits, void* stream, int c_begin, int c_end) {
  hipStream_t st = (hipStream_t)stream;
  const WCat wc = make_wcat(P, w);
  const int K = P.hidden;
  if (c_end < 0) c_end = P.ncol;
  const int nc = c_end - c_begin;   // columns of this launch; part rows keep stride ncol
  if (P.act_fmt == CKV_BF16 && P.w_fmt == CKV_BF16 && M <= 64 && c_begin % 16 == 0 && nc % 16 == 0) {
    dim3 grid(nc / 16, (M + 15) / 16, splits);
    hipLaunchKernelGGL(k_proj_dec, grid, dim3(64 * kProjDecWaves), 0, st, (const uint16_t*)x, M, K, wc, P.ncol,
                       part, c_begin);
  } else if (P.act_fmt == CKV_BF16 && P.w_fmt == CKV_BF16 && splits == 1 && M >= kGM && P.d % kGN == 0 &&
             (P.ratio != 4 || P.DI % kGN == 0) && K % kGK == 0 && c_begin % kGN == 0 && nc % kGN == 0) {
    dim3 grid(nc / kGN, (M + kGM - 1) / kGM);
    hipLaunchKernelGGL(k_proj_gemm, grid, dim3(256), 0, st, (const uint16_t*)x, M, K, wc, P.ncol, part, c_begin);
  } else if (P.act_fmt == CKV_BF16 && P.w_fmt == CKV_BF16 && c_begin % 64 == 0) {
    const int klen = ((K / splits) + 31) / 32 * 32;
    dim3 grid((nc + 63) / 64, splits, (M + 31) / 32);
    hipLaunchKernelGGL(k_proj_mfma, grid, dim3(256), 0, st, (const uint16_t*)x, M, K, wc, P.ncol, klen, part,
                       c_begin, c_end);
  } else {
    dim3 grid(nc, (M + 3) / 4);
#define CKV_PV(XF, WF)                                                                          \
  hipLaunchKernelGGL((k_proj_vec<XF, WF>), grid, dim3(64), 0, st, x, M, K, wc, P.ncol, part, c_begin)
    if (P.act_fmt == CKV_F32 && P.w_fmt == CKV_F32) CKV_PV(CKV_F32, CKV_F32);
    else if (P.act_fmt == CKV_F32) CKV_PV(CKV_F32, CKV_BF16);
    else if (P.w_fmt == CKV_F32) CKV_PV(CKV_BF16, CKV_F32);
    else CKV_PV(CKV_BF16, CKV_BF16);
#undef CKV_PV
  }
  return (int)hipGetLastError();
}

}  // namespace ckv
