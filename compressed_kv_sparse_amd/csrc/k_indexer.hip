// Ratio-4 indexer: score every visible compressed row and keep the top k
// ("ds4.c を読み解く (#3)", section 6; DSA on the vLLM DeepSeek V4 page).
//
// Score of row s for a query at position p:
//   I(s) = sum_h w_h * relu(qI_h . kI_s),  qI rotated at p (tail) and cast to
//   the indexer-cache format, s < V = (p+1)/4.
// The score kernel writes an order-preserving 32-bit key per row and a
// histogram of the keys' top 12 bits per query.  The select kernel then finds
// the exact k-th largest key with two more histogram levels over the
// candidates (bits 19..8, then 7..0) and emits, in ascending index order,
// every row above it plus the lowest-index rows equal to it.
#include "ckv_device.h"

namespace ckv {

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

struct IdxQuery {
  int seq, p, V;
};

__device__ __forceinline__ IdxQuery idx_query(const LayerParams& P, const int32_t* pos, int seq_fixed,
                                              int pos0, int qn) {
  IdxQuery q;
  q.seq = pos ? qn : seq_fixed;
  q.p = pos ? pos[qn] : pos0 + qn;
  q.V = q.p < 0 ? 0 : min((q.p + 1) / 4, P.cap);
  return q;
}

// LDS histogram of the block's keys, flushed to the query's global histogram.
__device__ __forceinline__ void hist_flush(uint32_t* lh, uint32_t* gh) {
  __syncthreads();
  for (int e = threadIdx.x; e < kHistBins; e += blockDim.x) {
    const uint32_t v = lh[e];
    if (v) atomicAdd(&gh[e], v);
  }
}

// ---------------------------------------------------------------- MFMA score
// bf16 indexer rows; MT = ceil(H_I / 16) head tiles, KS = D_I / 32 k-steps.
// grid: x = row blocks of 256, y = queries.  Each wave scores 64 rows.
template <int MT, int KS, int QF>
__global__ __launch_bounds__(256) void k_idx_score_mfma(LayerParams P, const uint16_t* __restrict__ idx,
                                                        const void* __restrict__ qI,
                                                        const float* __restrict__ wt,
                                                        const int32_t* __restrict__ pos, int seq_fixed,
                                                        int pos0, uint32_t* __restrict__ keys,
                                                        uint32_t* __restrict__ hist) {
  constexpr int DI = KS * 32;
  constexpr int HP = MT * 16;
  __shared__ __attribute__((aligned(16))) uint16_t qh[HP * DI];
  __shared__ float wsh[HP];
  __shared__ float cs_[32], sn_[32];
  __shared__ uint32_t lh[kHistBins];
  const int qn = blockIdx.y;
  const IdxQuery Q = idx_query(P, pos, seq_fixed, pos0, qn);
  const int rb0 = blockIdx.x * 256;
  if (rb0 >= Q.V) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int HI = P.HI, nrot = P.idx_rot, dn = DI - nrot;

  if (tid < nrot / 2) rope_cs(P.base, nrot, tid, (double)Q.p, &cs_[tid], &sn_[tid]);
  for (int e = tid; e < kHistBins; e += 256) lh[e] = 0;
  if (tid < HP) wsh[tid] = tid < HI ? wt[(size_t)qn * HI + tid] : 0.f;
  __syncthreads();
  for (int pe = tid; pe < HP * DI / 2; pe += 256) {
    const int h = pe / (DI / 2), c = 2 * (pe % (DI / 2));
    float a = 0.f, b = 0.f;
    if (h < HI) {
      const size_t o = ((size_t)qn * HI + h) * DI + c;
      a = load_val<QF>(qI, o);
      b = load_val<QF>(qI, o + 1);
      if (c >= dn) {
        const int j = (c - dn) >> 1;
        const float x = a * cs_[j] - b * sn_[j], y = a * sn_[j] + b * cs_[j];
        a = x;
        b = y;
      }
    }
    ((uint32_t*)qh)[(h * DI + c) >> 1] = pack_bf16x2(a, b);
  }
  __syncthreads();

  u32x4 A[MT][KS];
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) A[mt][ks] = *(const u32x4*)&qh[(16 * mt + r) * DI + 32 * ks + 8 * g];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = wsh[16 * mt + 4 * g + i];
  }

  const int row0 = rb0 + wave * 64;
  const uint16_t* base = idx + (size_t)Q.seq * P.cap * DI;
  const u32x4 zero = {0, 0, 0, 0};
  u32x4 Bv[4][KS];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = row0 + 16 * t + r;
    const bool ok = row < Q.V;
    const uint16_t* rp = base + (size_t)(ok ? row : 0) * DI + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) Bv[t][ks] = ok ? *(const u32x4*)(rp + 32 * ks) : zero;
  }
  const bool relu = !(P.flags & CKV_FLAG_IDX_NO_RELU);
  float sc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float s = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(as_bf16x8(A[mt][ks]), as_bf16x8(Bv[t][ks]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) s += wv[mt][i] * (relu ? fmaxf(acc[i], 0.f) : acc[i]);
    }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    sc[t] = s;
  }
  const float mine = g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3];
  const int row = row0 + lane;
  if (row < Q.V) {
    const uint32_t key = float_key(mine);
    keys[(size_t)qn * P.cap + row] = key;
    atomicAdd(&lh[key >> 20], 1u);
  }
  hist_flush(lh, hist + (size_t)qn * kHistBins);
}

// ---------------------------------------------------------------- vector score
// Any formats.  One thread per row.  grid: x = row blocks of 256, y = queries.
template <int IDXF, int QF>
__global__ __launch_bounds__(256) void k_idx_score_vec(LayerParams P, const void* __restrict__ idx,
                                                       const void* __restrict__ qI,
                                                       const float* __restrict__ wt,
                                                       const int32_t* __restrict__ pos, int seq_fixed,
                                                       int pos0, uint32_t* __restrict__ keys,
                                                       uint32_t* __restrict__ hist) {
  __shared__ float qh[64 * kMaxDI];
  __shared__ float wsh[64];
  __shared__ float cs_[32], sn_[32];
  __shared__ uint32_t lh[kHistBins];
  const int qn = blockIdx.y;
  const IdxQuery Q = idx_query(P, pos, seq_fixed, pos0, qn);
  const int rb0 = blockIdx.x * 256;
  if (rb0 >= Q.V) return;
  const int tid = threadIdx.x;
  const int HI = P.HI, DI = P.DI, nrot = P.idx_rot, dn = DI - nrot;
  if (tid < nrot / 2) rope_cs(P.base, nrot, tid, (double)Q.p, &cs_[tid], &sn_[tid]);
  for (int e = tid; e < kHistBins; e += 256) lh[e] = 0;
  if (tid < HI) wsh[tid] = wt[(size_t)qn * HI + tid];
  __syncthreads();
  for (int pe = tid; pe < HI * DI / 2; pe += 256) {
    const int h = pe / (DI / 2), c = 2 * (pe % (DI / 2));
    const size_t o = ((size_t)qn * HI + h) * DI + c;
    float a = load_val<QF>(qI, o), b = load_val<QF>(qI, o + 1);
    if (c >= dn) {
      const int j = (c - dn) >> 1;
      const float x = a * cs_[j] - b * sn_[j], y = a * sn_[j] + b * cs_[j];
      a = x;
      b = y;
    }
    if (IDXF == CKV_BF16) {
      a = bf16_to_f32(f32_to_bf16(a));
      b = bf16_to_f32(f32_to_bf16(b));
    }
    qh[h * DI + c] = a;
    qh[h * DI + c + 1] = b;
  }
  __syncthreads();
  const bool relu = !(P.flags & CKV_FLAG_IDX_NO_RELU);
  const int row = rb0 + tid;
  if (row < Q.V) {
    const size_t ro = ((size_t)Q.seq * P.cap + row) * DI;
    float s = 0.f;
    for (int h = 0; h < HI; ++h) {
      float dot = 0.f;
      for (int c = 0; c < DI; ++c) dot += qh[h * DI + c] * load_val<IDXF>(idx, ro + c);
      s += wsh[h] * (relu ? fmaxf(dot, 0.f) : dot);
    }
    const uint32_t key = float_key(s);
    keys[(size_t)qn * P.cap + row] = key;
    atomicAdd(&lh[key >> 20], 1u);
  }
  hist_flush(lh, hist + (size_t)qn * kHistBins);
}

// ---------------------------------------------------------------- select

// Exclusive prefix sum over the block (1024 threads); returns the thread's
// exclusive sum, *total receives the block total.
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) before += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  return before + x - v;
}

// Histogram sh[0..nb) (nb a multiple of... any <= 4096): find the bin b where
// the count of keys in bins above b is < need and reaches need including b.
// Thread t owns the bins nb-(t+1)*per .. nb-t*per-1 (highest bins first).
__device__ __forceinline__ void find_bin(const uint32_t* sh, int nb, uint32_t need, uint32_t* wsum,
                                         uint32_t* bc) {
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int hi = nb - threadIdx.x * per;  // exclusive
  const int lo = max(0, hi - per);
  uint32_t local = 0;
  for (int b = lo; b < hi; ++b) local += sh[b];
  if (threadIdx.x == 0) {  // in-range fallback should the counts disagree
    bc[0] = 0;
    bc[1] = 0;
  }
  uint32_t tot;
  const uint32_t above = block_exscan(local, wsum, &tot);
  if (above < need && above + local >= need) {
    uint32_t cum = above;
    for (int b = hi - 1; b >= lo; --b) {
      if (cum + sh[b] >= need) {
        bc[0] = (uint32_t)b;
        bc[1] = cum;
        break;
      }
      cum += sh[b];
    }
  }
  __syncthreads();
}

// One block of 1024 threads per query.
__global__ __launch_bounds__(1024) void k_topk_select(LayerParams P, const uint32_t* __restrict__ keys,
                                                      const uint32_t* __restrict__ hist,
                                                      const int32_t* __restrict__ pos, int pos0,
                                                      int32_t* __restrict__ out) {
  __shared__ uint32_t sh[kHistBins];
  __shared__ uint32_t wsum[16], wgt[16], weq[16];
  __shared__ uint32_t bc[2];
  const int qn = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = P.topk;
  const IdxQuery Q = idx_query(P, pos, 0, pos0, qn);
  const int V = Q.V;
  int32_t* o = out + (size_t)qn * k;
  if (V <= k) {
    for (int j = tid; j < k; j += blockDim.x) o[j] = j < V ? j : -1;
    return;
  }
  const uint32_t* kq = keys + (size_t)qn * P.cap;

  // level 1: top 12 bits, histogram built by the score kernel
  for (int e = tid; e < kHistBins; e += blockDim.x) sh[e] = hist[(size_t)qn * kHistBins + e];
  __syncthreads();
  uint32_t need = (uint32_t)k;
  find_bin(sh, kHistBins, need, wsum, bc);
  uint32_t prefix = bc[0] << 20, mask = 0xfff00000u;
  need -= bc[1];
  // levels 2 and 3 over the keys that share the prefix
#pragma unroll 1
  for (int lvl = 0; lvl < 2; ++lvl) {
    const int shift = lvl == 0 ? 8 : 0;
    const int nb = lvl == 0 ? 4096 : 256;
    __syncthreads();
    for (int e = tid; e < nb; e += blockDim.x) sh[e] = 0;
    __syncthreads();
    for (int s = tid; s < V; s += blockDim.x) {
      const uint32_t key = kq[s];
      if ((key & mask) == prefix) atomicAdd(&sh[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(sh, nb, need, wsum, bc);
    prefix |= bc[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    need -= bc[1];
  }
  const uint32_t T = prefix;  // the k-th largest key; `need` keys equal to it are taken

  // ascending emission: each wave walks a contiguous chunk of indices
  const int nw = blockDim.x >> 6;
  const int CH = ((V + nw - 1) / nw + 63) / 64 * 64;
  const int c0 = wave * CH, c1 = min(V, c0 + CH);
  uint32_t ngt = 0, neq = 0;
  for (int b0 = c0; b0 < c1; b0 += 64) {
    const int s = b0 + lane;
    const uint32_t key = s < c1 ? kq[s] : 0u;
    ngt += __popcll(__ballot(s < c1 && key > T));
    neq += __popcll(__ballot(s < c1 && key == T));
  }
  if (lane == 0) {
    wgt[wave] = ngt;
    weq[wave] = neq;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += wgt[w];
    eq_before += weq[w];
  }
  uint32_t eq_run = eq_before;
  uint32_t sel_run = gt_before + min(eq_before, need);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = c0; b0 < c1; b0 += 64) {
    const int s = b0 + lane;
    const uint32_t key = s < c1 ? kq[s] : 0u;
    const bool gt = s < c1 && key > T, eq = s < c1 && key == T;
    const unsigned long long eqm = __ballot(eq);
    const uint32_t eq_rank = eq_run + (uint32_t)__popcll(eqm & lt);
    const bool sel = gt || (eq && eq_rank < need);
    const unsigned long long sm = __ballot(sel);
    const uint32_t slot = sel_run + (uint32_t)__popcll(sm & lt);
    if (sel && slot < (uint32_t)k) o[slot] = s;
    eq_run += (uint32_t)__popcll(eqm);
    sel_run += (uint32_t)__popcll(sm);
  }
}

// ---------------------------------------------------------------- launcher

int launch_indexer(const LayerParams& P, const Cache& c, const void* qI, const float* w,
                   const int32_t* pos, int seq, int pos0, int nq, uint32_t* keys, uint32_t* hist,
                   int32_t* topk, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const size_t nh = (size_t)nq * kHistBins;
  const size_t fb = (nh + 255) / 256;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)(fb < 1024 ? fb : 1024)), dim3(256), 0, st, hist, nh, 0u);
  launch_idx_score(P, c, qI, w, pos, seq, pos0, nq, keys, hist, stream);
  hipLaunchKernelGGL(k_topk_select, dim3(nq), dim3(1024), 0, st, P, keys, hist, pos, pos0, topk);
  return (int)hipGetLastError();
}

int launch_idx_score(const LayerParams& P, const Cache& c, const void* qI, const float* w,
                     const int32_t* pos, int seq, int pos0, int nq, uint32_t* keys, uint32_t* hist,
                     void* stream) {
  hipStream_t st = (hipStream_t)stream;
  // rows to cover: decode -> the whole capacity; prefill -> rows visible to the last query
  const int vlast = (pos0 + nq) / 4;
  const int vmax = pos ? P.cap : (vlast < P.cap ? vlast : P.cap);
  dim3 grid((unsigned)(vmax > 0 ? (vmax + 255) / 256 : 1), nq);
  const bool mf = P.idx_fmt == CKV_BF16 && P.DI == 128 && P.HI <= 64;
  if (mf) {
    const uint16_t* ix = (const uint16_t*)c.idx;
    const int MT = (P.HI + 15) / 16;
#define CKV_IS(MTV, QF)                                                                          \
  hipLaunchKernelGGL((k_idx_score_mfma<MTV, 4, QF>), grid, dim3(256), 0, st, P, ix, qI, w, pos, seq, \
                     pos0, keys, hist)
    if (P.act_fmt == CKV_BF16) {
      if (MT == 1) CKV_IS(1, CKV_BF16);
      else if (MT == 2) CKV_IS(2, CKV_BF16);
      else if (MT == 3) CKV_IS(3, CKV_BF16);
      else CKV_IS(4, CKV_BF16);
    } else {
      if (MT == 1) CKV_IS(1, CKV_F32);
      else if (MT == 2) CKV_IS(2, CKV_F32);
      else if (MT == 3) CKV_IS(3, CKV_F32);
      else CKV_IS(4, CKV_F32);
    }
#undef CKV_IS
  } else {
#define CKV_IV(IF, QF)                                                                               \
  hipLaunchKernelGGL((k_idx_score_vec<IF, QF>), grid, dim3(256), 0, st, P, c.idx, qI, w, pos, seq, pos0, \
                     keys, hist)
    if (P.idx_fmt == CKV_F32 && P.act_fmt == CKV_F32) CKV_IV(CKV_F32, CKV_F32);
    else if (P.idx_fmt == CKV_F32) CKV_IV(CKV_F32, CKV_BF16);
    else if (P.act_fmt == CKV_F32) CKV_IV(CKV_BF16, CKV_F32);
    else CKV_IV(CKV_BF16, CKV_BF16);
#undef CKV_IV
  }
  return (int)hipGetLastError();
}

}  // namespace ckv
