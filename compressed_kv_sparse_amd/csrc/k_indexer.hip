// Ratio-4 indexer: score every visible compressed row and keep the top k
// ("ds4.c を読み解く (#3)", section 6; DSA on the vLLM DeepSeek V4 page).
//
// Score of row s for a query at position p:
//   I(s) = sum_h w_h * relu(qI_h . kI_s),  qI rotated at p (tail) and cast to
//   the indexer-cache format, s < V = (p+1)/4.
// The score kernel writes an order-preserving 32-bit key per row.  The select
// kernel works on d = M - key, M the largest key of the query, and finds the
// k-th smallest d by radix levels of up to 10 bits, most significant first;
// each level counts only the keys that share the bits chosen so far.  The
// first level bins d >> 14 and counts only d < 2^24 (scores within about two
// octaves of the maximum), so the top rows spread over narrow bins instead of
// piling into a few; when fewer than k keys fall in that range it widens the
// range and counts again.  Every row above the k-th key is emitted, plus the
// lowest-index rows equal to it, in ascending index order.
#include <hip/hip_ext.h>

#include <type_traits>

#include "compress_dec.h"
#include "idx_fp4.h"
#include "proj_dec.h"

namespace ckv {

// Score-kernel timing: when armed, the next score launch of this thread goes
// through hipExtLaunchKernel, which stamps the two events at the kernel's own
// start and end (no launch gaps in between), then disarms.
static thread_local hipEvent_t t_score_ev[2] = {nullptr, nullptr};

void arm_score_timing(void* start_event, void* stop_event) {
  t_score_ev[0] = (hipEvent_t)start_event;
  t_score_ev[1] = (hipEvent_t)stop_event;
}

template <typename F, typename... Args>
static void launch_score(F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  if (t_score_ev[0] || t_score_ev[1]) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, t_score_ev[0], t_score_ev[1], 0, args...);
    t_score_ev[0] = t_score_ev[1] = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  }
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

// ---------------------------------------------------------------- MFMA score
// bf16 indexer rows; MT = ceil(H_I / 16) head tiles, KS = D_I / 32 k-steps.
// grid: x = row blocks of 256 * kScoreGroups, y = queries.  Per group each
// wave scores 64 rows; the next group's rows are loaded while the current one
// is multiplied.  Heads are the MFMA M dimension, rows the N dimension, so the
// weighted head sum is 4 in-lane adds per tile and two cross-lane adds.
//
// Every global load here is unconditional (indices clamped into range, the
// value replaced afterwards), the key stores are branch-free, and the group
// loop has a compile-time trip count: a load under a branch, or in a loop of
// unknown length, makes the compiler wait for all outstanding loads right
// after it, which turns the prefetch into a chain of full memory round trips.
// Each wave keeps kScoreBufs row groups in registers: while group i is
// multiplied, groups i+1 .. i+kScoreBufs-1 are in flight.  Two buffers and
// the query fragments fill 256 registers (VGPRs + MFMA accumulators), so the
// kernel runs two waves per SIMD -- two blocks per CU -- and four groups per
// block give the 128k-context batch 512 blocks, all resident at once.  Left
// to its default occupancy target the compiler reuses one buffer's
// registers for the next and every wave's loads and multiplies serialise;
// with more blocks than fit, a second round of blocks waits for the first.
// (Measured on the 16 x 32768-row batch, rows read from HBM: 26.3 us here,
// the time of a kernel that issues the same loads and no arithmetic; 27.7 us
// with two groups per block (two rounds of blocks); 29-30 us with one buffer
// at three or four waves per SIMD.)
constexpr int kScoreGroups = 4;
// The decode step's launch: scan blocks of 5 groups (416 for the 16 x 32768-
// row batch), then the 80 projection blocks, each wave keeping 16 of its
// k-steps' loads in flight: 496 blocks, all resident at two per compute unit
// from the start.  (Measured step scan: 34.4 us; 37.1 us with 4 groups, where
// the projection blocks wait for scan blocks to finish; 37.4 us with 6.)
constexpr int kStepGroups = 5;
// fp4 rows: groups per block of the score kernel and of the step scan, and
// groups in flight per wave
constexpr int kFp4Groups = 4;
constexpr int kFp4StepGroups = 5;
constexpr int kFp4Bufs = 8;
constexpr bool kStepProjLast = true;
constexpr int kStepProjSF = 16;
constexpr int kScoreBufs = 2;

// Destination of the key stores of rows at or past the cache capacity (the
// last row block of a query can run past it); written, never read.
__device__ uint32_t g_key_sink[64];

// Rows of a scan block: rows rb0 + 64 j + q (rb0 a multiple of 64, q < 64)
// of sequence seq, rows past V - 1 clamped to it (their keys are never read).
// Contiguous caches: the sequence's rows in order.  Paged caches (PAGED: 64
// indexer rows a page, NT * 64 pages a block): lane l keeps the addresses of
// pages l, 64 + l, .. of the block as the table names them (an entry outside
// the pool reads page 0), loaded once before any row; a wave takes a page's
// address from that lane with a lane read, so the row loads need no table
// access of their own.  j is the same in the whole wave.
template <bool PAGED, int NT = 1>
struct ScanRows;

template <int NT>
struct ScanRows<false, NT> {
  const uint8_t* base;
  int rb0, vlast;
  __device__ __forceinline__ ScanRows(const LayerParams& P, const void* idx, int seq, int rb0_, int vlast_,
                                      int row_bytes)
      : base((const uint8_t*)idx + (size_t)seq * P.cap * row_bytes), rb0(rb0_), vlast(vlast_) {}
  __device__ __forceinline__ const uint8_t* row(int j, int q, int row_bytes) const {
    return base + (size_t)min(rb0 + 64 * j + q, vlast) * row_bytes;
  }
};

template <int NT>
struct ScanRows<true, NT> {
  uint64_t pb[NT];   // this lane's page addresses
  int jlast, vin;    // page and in-page index of the last visible row (V - 1)
  __device__ __forceinline__ ScanRows(const LayerParams& P, const void* idx, int seq, int rb0, int vlast,
                                      int row_bytes) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int blk = min((rb0 >> 6) + 64 * t + (int)(threadIdx.x & 63), P.max_blocks - 1);
      int pg = P.blocks[(size_t)seq * P.max_blocks + blk];
      pg = (pg >= 0 && pg < P.n_pages) ? pg : 0;
      pb[t] = (uint64_t)((const uint8_t*)idx + (size_t)pg * 64 * row_bytes);
    }
    jlast = (vlast >> 6) - (rb0 >> 6);
    vin = vlast & 63;
  }
  __device__ __forceinline__ const uint8_t* row(int j, int q, int row_bytes) const {
    const int jj = __builtin_amdgcn_readfirstlane(min(j, jlast));
    uint64_t a = pb[0];
#pragma unroll
    for (int t = 1; t < NT; ++t)
      if (jj >= 64 * t) a = pb[t];
    const int l = jj & 63;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)a, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(a >> 32), l);
    const int qq = jj == jlast ? min(q, vin) : q;
    return (const uint8_t*)(((uint64_t)hi << 32) | lo) + (size_t)qq * row_bytes;
  }
};

// The body as a device function: block (bx, qn) of the grid above.
// old_only: the rows of the query's cache except the row its own token
// closes (a decode step whose compressor runs concurrently scores that row
// separately).
template <int MT, int KS, int QF, bool HIST, int NG = kScoreGroups, bool PAGED = false>
__device__ __forceinline__ void idx_score_block(const LayerParams& P, const uint16_t* idx, const void* __restrict__ qI,
                                                const float* __restrict__ wt, const int32_t* __restrict__ pos,
                                                int seq_fixed, int pos0, uint32_t* __restrict__ keys,
                                                uint32_t* __restrict__ hist, int bx, int qn, bool old_only) {
  constexpr int DI = KS * 32;
  constexpr int HP = MT * 16;
  constexpr int RB = 256 * NG;
  __shared__ __attribute__((aligned(16))) uint16_t qh[HP * DI];
  __shared__ float wsh[256];
  __shared__ float cs_[32], sn_[32];
  __shared__ uint32_t lh[kHistBins];
  IdxQuery Q = idx_query(P, pos, seq_fixed, pos0, qn);
  if (old_only && Q.p >= 0 && (Q.p + 1) % 4 == 0 && (Q.p + 1) / 4 <= P.cap) Q.V -= 1;
  const int rb0 = bx * RB;
  if (rb0 >= Q.V) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int HI = P.HI, nrot = P.idx_rot, dn = DI - nrot;
  const int vlast = Q.V - 1;
  const ScanRows<PAGED> rows(P, idx, Q.seq, rb0, vlast, 2 * DI);

  // the query: MT chunks of 8 channels per thread (chunk ci = tid + 256 e is
  // head ci / (DI/8), channels 8 (ci % (DI/8)) .. +7); heads past H_I read head
  // H_I - 1 and are zeroed below
  constexpr int CPH = DI / 8;
  u32x4 qraw[MT][QF == CKV_F32 ? 2 : 1];
#pragma unroll
  for (int e = 0; e < MT; ++e) {
    const int ci = tid + 256 * e, h = min(ci / CPH, HI - 1), c = 8 * (ci % CPH);
    const size_t o = ((size_t)qn * HI + h) * DI + c;
    if constexpr (QF == CKV_F32) {
      qraw[e][0] = *(const u32x4*)((const float*)qI + o);
      qraw[e][1] = *(const u32x4*)((const float*)qI + o + 4);
    } else {
      qraw[e][0] = *(const u32x4*)((const uint16_t*)qI + o);
    }
  }
  const float wl = wt[(size_t)qn * HI + min(tid, HI - 1)];
  // (the query and head weights stay ahead of the rows in the load queue:
  // waiting for them then does not wait for the rows)
  asm volatile("" ::: "memory");

  // rows of group gi for this wave -> B operands; rows past V re-read row V-1
  auto load = [&](u32x4(&Bv)[4][KS], int gi) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint16_t* rp = (const uint16_t*)rows.row(4 * gi + wave, 16 * t + r, 2 * DI) + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) Bv[t][ks] = *(const u32x4*)(rp + 32 * ks);
    }
  };
  u32x4 Bq[kScoreBufs][4][KS];
  constexpr int kAhead = kScoreBufs > 1 ? kScoreBufs - 1 : 1;   // groups issued before the prologue
#pragma unroll
  for (int b = 0; b < kAhead && b < NG; ++b) load(Bq[b % kScoreBufs], b);

  if (tid < nrot / 2) rope_cs_theta(theta_c_sel(P, tid), (double)Q.p, &cs_[tid], &sn_[tid]);
  wsh[tid] = tid < HI ? wl : 0.f;   // (unconditional: the load stays where it is issued)
  if constexpr (HIST)
    for (int e = tid; e < kHistBins; e += 256) lh[e] = 0;
  lds_barrier();   // cs_, sn_, wsh, lh (no wait for the rows in flight)
  // rotated query -> bf16 in LDS
#pragma unroll
  for (int e = 0; e < MT; ++e) {
    const int ci = tid + 256 * e, h = ci / CPH, c = 8 * (ci % CPH);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (QF == CKV_F32) v[i] = __uint_as_float(qraw[e][i >> 2][i & 3]);
      else v[i] = bf16_to_f32((qraw[e][0][i >> 1] >> (16 * (i & 1))) & 0xffffu);
      if (h >= HI) v[i] = 0.f;
    }
    u32x4 packed;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = v[2 * i], b = v[2 * i + 1];
      const int cc = c + 2 * i;
      if (cc >= dn) {
        const int j = (cc - dn) >> 1;
        const float x = a * cs_[j] - b * sn_[j], y = a * sn_[j] + b * cs_[j];
        a = x;
        b = y;
      }
      packed[i] = pack_bf16x2(a, b);
    }
    *(u32x4*)&qh[h * DI + c] = packed;
  }
  lds_barrier();   // qh

  u32x4 A[MT][KS];
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) A[mt][ks] = *(const u32x4*)&qh[(16 * mt + r) * DI + 32 * ks + 8 * g];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = wsh[16 * mt + 4 * g + i];
  }
  const bool relu = !(P.flags & CKV_FLAG_IDX_NO_RELU);
  uint32_t* kout = keys + (size_t)qn * P.cap;

  auto score = [&](const u32x4(&Bv)[4][KS], int gi) {
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
      sc[t] = rows4_sum(s);
    }
    const float mine = g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3];
    const int row = rb0 + 256 * gi + wave * 64 + lane;
    // branch-free: keys of rows in [V, cap) are written but never read; rows
    // past the capacity go to the sink; only rows below V enter the histogram
    const uint32_t key = float_key(mine);
    *(row < P.cap ? kout + row : g_key_sink + lane) = key;
    if constexpr (HIST) atomicAdd(&lh[key >> 20], row < Q.V ? 1u : 0u);
  };
  // An empty asm that takes the buffer about to be multiplied as in/out
  // operands and clobbers memory: the loads issued before it cannot sink
  // below it, and the multiplies (which read its outputs) cannot rise above
  // it.  Without it the compiler places each prefetch after the previous
  // group's multiplies.  (idx is deliberately not __restrict__: with it the
  // compiler may prove the clobber cannot touch the rows and move the loads
  // anyway.)
  auto pin = [&](u32x4(&Bv)[4][KS]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(Bv[t][ks]) : : "memory");
  };
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if constexpr (kScoreBufs > 1) {
      if (gi + kAhead < NG) load(Bq[(gi + kAhead) % kScoreBufs], gi + kAhead);
    }
    pin(Bq[gi % kScoreBufs]);
    score(Bq[gi % kScoreBufs], gi);
    if constexpr (kScoreBufs == 1) {
      if (gi + 1 < NG) load(Bq[0], gi + 1);
    }
  }
  if constexpr (HIST) {  // this block's key histogram (LDS, filled above) into the query's
    lds_barrier();
    uint32_t* gh = hist + (size_t)qn * kHistBins;
    for (int e = tid; e < kHistBins; e += 256) {
      const uint32_t v = lh[e];
      if (v) atomicAdd(&gh[e], v);
    }
  }
}

// ---------------------------------------------------------------- fp4 MFMA score
// fp4 indexer rows (68-byte MXFP4 records of the Hadamard-rotated rows, D_I =
// 128): one scaled fp4 MFMA (16 heads x 16 rows x all 128 channels) per head
// tile and row tile, 4x fewer bytes per row than bf16.  Same grid, groups and
// load pipeline as the bf16 block above.  Lane (r, g)'s share of a 16-row
// tile is the 16-byte code block g of row r and the row's scale dword (byte g
// is its block scale), both at 4-byte aligned addresses; a tile is 1088
// contiguous bytes.  The query: wave mt loads head tile mt (lane (r, g):
// head 16 mt + r, channels 32 g .. 32 g + 31), rotates its tail, applies the
// Hadamard transform and the MXFP4 rounding in registers and leaves the
// codes and scales in LDS in MFMA operand order; every wave then reads the
// MT tiles back.  The query's loads go out before the rows', so waiting for
// them does not wait for the rows (loads complete in order).

template <int MT, bool HIST, int NG = kScoreGroups, bool PAGED = false>
__device__ __forceinline__ void idx_score_block_fp4(const LayerParams& P, const uint8_t* idx,
                                                    const void* __restrict__ qI, const float* __restrict__ wt,
                                                    const int32_t* __restrict__ pos, int seq_fixed, int pos0,
                                                    uint32_t* __restrict__ keys, uint32_t* __restrict__ hist, int bx,
                                                    int qn, bool old_only, uint8_t* __restrict__ qout) {
  constexpr int HP = MT * 16;
  constexpr int RB = 256 * NG;
  __shared__ __attribute__((aligned(16))) u32x4 qc[MT * 64];
  __shared__ uint32_t qs[MT * 64];
  __shared__ float wsh[256];
  __shared__ __attribute__((aligned(16))) float cs_[64], sn_[64];   // per channel pair; 1, 0 before the tail
  __shared__ uint32_t lh[kHistBins];
  IdxQuery Q = idx_query(P, pos, seq_fixed, pos0, qn);
  if (old_only && Q.p >= 0 && (Q.p + 1) % 4 == 0 && (Q.p + 1) / 4 <= P.cap) Q.V -= 1;
  const int rb0 = bx * RB;
  if (rb0 >= Q.V) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int HI = P.HI;
  const int vlast = Q.V - 1;
  const ScanRows<PAGED> rows(P, idx, Q.seq, rb0, vlast, kFp4RowBytes);

  // the query first: head tile (wave % MT), 32 channels per lane; heads past
  // H_I read head H_I - 1 and are zeroed below
  const int qh = 16 * (wave % MT) + r;
  u32x4 qraw[4];
  {
    const uint16_t* qp = (const uint16_t*)qI + ((size_t)qn * HI + min(qh, HI - 1)) * 128 + 32 * g;
#pragma unroll
    for (int k = 0; k < 4; ++k) qraw[k] = *(const u32x4*)(qp + 8 * k);
  }
  const float wl = wt[(size_t)qn * HI + min(tid, HI - 1)];
  // (the query and head weights stay ahead of the rows in the load queue:
  // waiting for them then does not wait for the rows)
  asm volatile("" ::: "memory");

  auto load = [&](u32x4(&Bc)[4], uint32_t(&Bs)[4], int gi) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint8_t* rp = rows.row(4 * gi + wave, 16 * t + r, kFp4RowBytes);
      Bc[t] = *(const u32x4_a4*)(rp + 16 * g);
      Bs[t] = *(const uint32_t*)(rp + 64);
    }
  };
  // the first BUFS groups' loads go out before the prologue (20 registers a
  // group); each later group is issued into the buffer the scores just freed
  constexpr int BUFS = NG < kFp4Bufs ? NG : kFp4Bufs;
  u32x4 Bc[BUFS][4];
  uint32_t Bs[BUFS][4];
#pragma unroll
  for (int b = 0; b < BUFS; ++b) load(Bc[b], Bs[b], b);

  if (tid < 64) {   // pair tid of the 128 channels: the tail's pairs rotate, the others keep (1, 0)
    const int j = tid - (64 - P.idx_rot / 2);
    float c = 1.f, sn = 0.f;
    if (j >= 0) rope_cs_theta(theta_c_sel(P, j), (double)Q.p, &c, &sn);
    cs_[tid] = c;
    sn_[tid] = sn;
  }
  wsh[tid] = tid < HI ? wl : 0.f;   // (unconditional: the load stays where it is issued)
  if constexpr (HIST)
    for (int e = tid; e < kHistBins; e += 256) lh[e] = 0;
  lds_barrier();   // cs_, sn_, wsh, lh
  {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = bf16_to_f32((qraw[i >> 3][(i >> 1) & 3] >> (16 * (i & 1))) & 0xffffu);
      if (qh >= HI) v[i] = 0.f;
    }
    rope_block32(v, cs_ + 16 * g, sn_ + 16 * g);
    fwht128(v);
    uint32_t sb;
    const u32x4 codes = mxfp4_block(v, sb);
    if (wave < MT) {
      qc[wave * 64 + lane] = codes;
      qs[wave * 64 + lane] = sb;
    }
  }
  lds_barrier();   // qc, qs
  u32x4 A[MT];
  uint32_t sa[MT];
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    A[mt] = qc[mt * 64 + lane];
    sa[mt] = qs[mt * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = wsh[16 * mt + 4 * g + i];
  }
  const bool relu = !(P.flags & CKV_FLAG_IDX_NO_RELU);
  uint32_t* kout = keys + (size_t)qn * P.cap;

  auto score = [&](const u32x4(&Bc)[4], const uint32_t(&Bs)[4], int gi) {
    float sc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float s = 0.f;
      const uint32_t sb = Bs[t] >> (8 * g);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 acc = mfma_fp4(A[mt], sa[mt], Bc[t], sb, (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) s += wv[mt][i] * (relu ? fmaxf(acc[i], 0.f) : acc[i]);
      }
      sc[t] = rows4_sum(s);
    }
    const float mine = g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3];
    const int row = rb0 + 256 * gi + wave * 64 + lane;
    const uint32_t key = float_key(mine);
    *(row < P.cap ? kout + row : g_key_sink + lane) = key;
    if constexpr (HIST) atomicAdd(&lh[key >> 20], row < Q.V ? 1u : 0u);
  };
  // keeps the loads above the multiplies (as in the bf16 block)
  auto pin = [&](u32x4(&Bc)[4], uint32_t(&Bs)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      asm volatile("" : "+v"(Bc[t]) : : "memory");
      asm volatile("" : "+v"(Bs[t]) : : "memory");
    }
  };
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    pin(Bc[gi % BUFS], Bs[gi % BUFS]);
    score(Bc[gi % BUFS], Bs[gi % BUFS], gi);
    if (gi + BUFS < NG) load(Bc[gi % BUFS], Bs[gi % BUFS], gi + BUFS);
  }
  // the query's fp4 form for the selection block (record layout: head h at
  // qout + 68 (64 qn + h)), by the first row block, after its loads
  if (qout && bx == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt == wave) {
        uint8_t* rec = qout + (size_t)(64 * qn + 16 * mt + r) * kFp4RowBytes;
        *(u32x4_a4*)(rec + 16 * g) = A[mt];
        rec[64 + g] = (uint8_t)sa[mt];
      }
    }
  }
  if constexpr (HIST) {
    lds_barrier();
    uint32_t* gh = hist + (size_t)qn * kHistBins;
    for (int e = tid; e < kHistBins; e += 256) {
      const uint32_t v = lh[e];
      if (v) atomicAdd(&gh[e], v);
    }
  }
}

template <int MT, bool HIST, bool PAGED = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_idx_score_fp4(LayerParams P, const uint8_t* idx, const void* __restrict__ qI,
                                                       const float* __restrict__ wt, const int32_t* __restrict__ pos,
                                                       int seq_fixed, int pos0, uint32_t* __restrict__ keys,
                                                       uint32_t* __restrict__ hist) {
  idx_score_block_fp4<MT, HIST, kFp4Groups, PAGED>(P, idx, qI, wt, pos, seq_fixed, pos0, keys, hist, blockIdx.x,
                                                   blockIdx.y, false, nullptr);
}

template <int MT, int KS, int QF, bool HIST, bool PAGED = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_idx_score_mfma(
    LayerParams P, const uint16_t* idx, const void* __restrict__ qI, const float* __restrict__ wt,
    const int32_t* __restrict__ pos, int seq_fixed, int pos0, uint32_t* __restrict__ keys,
    uint32_t* __restrict__ hist) {
  idx_score_block<MT, KS, QF, HIST, kScoreGroups, PAGED>(P, idx, qI, wt, pos, seq_fixed, pos0, keys, hist, blockIdx.x,
                                                         blockIdx.y, false);
}

// ---------------------------------------------------------------- prefill score GEMM
// Chunked prefill scores every query of the chunk against every row it sees:
// a [T x H_I, D_I] x [D_I, V] product.  One block takes 8 consecutive
// queries (one per wave, its rotated query held as MFMA A fragments) and a run
// of kPfTiles row tiles of 128 rows; each tile is staged once in LDS and
// multiplied by all 8 queries, so a row is read from memory once per 8
// queries instead of once per query.  Rows at or past a query's V get keys
// that are never read (the select stops at V); rows past the group's last
// visible row re-read that row.  grid: x = row runs, y = query groups.
//
// Heads are the MFMA M dimension and rows N: a lane's accumulators hold 4
// heads of one row, so the weighted head sum is in-lane adds plus a sum over
// the 4 lane groups, done for four sub-tiles at once as a scattered sum
// (v_permlane32_swap / v_permlane16_swap, no LDS); relu is
// one integer max on the float's bits (negative floats have negative bit
// patterns, so max(bits, 0) is relu; a lower bound of INT_MIN keeps x), which
// needs no NaN-quieting step in front as a float max does.
//
// Tiles are double-buffered in LDS and filled by direct global-to-LDS loads
// (no registers: two blocks of 8 waves fit a compute unit).  A wave's load
// instruction fills 1 KB = 4 rows, lane l taking 16-byte position l % 16 of
// row l / 16; position q of row R holds the row's chunk q ^ (R % 16), so the
// 16 lanes of a B-fragment read (16 rows, one chunk each) hit 16 distinct
// bank groups.  The tile reads are inline asm: the compiler would otherwise
// wait for every direct load in flight -- including the next tile's -- before
// any LDS read.  The kernel therefore waits for the tile loads itself (all
// counters, then a barrier) at the top of each tile, and reads no other LDS
// in the tile loop.  Sub-tiles are addressed through the read's offset field.
//
// Measured on MI355X (4096 queries at position 61440): a loop of the same
// MFMA chains and epilogue with operands in registers runs at 73-80 % of
// the bf16 peak; this kernel reaches about half of it.  Without the
// epilogue it takes 88 % of its time, without three quarters of the LDS
// reads 89 %, without the tile loads 97 %.  Requesting the next sub-tile's
// fragments before the current epilogue (no spare registers for a second
// set) and 16 queries per block were both slower.
constexpr int kPfRows = 128, kPfQ = 8, kPfTiles = 64;
static_assert(kPfRows % (4 * kPfQ) == 0, "each wave fills whole 4-row slices of a tile");

__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// four 16-byte LDS reads at byte offset OFF from each address, waited for
template <int OFF>
__device__ __forceinline__ void lds_read4_b128_at(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, u32x4& r0,
                                                  u32x4& r1, u32x4& r2, u32x4& r3) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\tds_read_b128 %1, %5 offset:%8\n\tds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "i"(OFF)
      : "memory");
}
// Sums over the 4 lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48) of four values
// at once, scattered: row 0 of the result holds the total of s0, row 1 of s2,
// row 2 of s1, row 3 of s3 (three row swaps and three adds instead of four
// full two-step sums).
__device__ __forceinline__ float rows4_sum_scatter(float s0, float s1, float s2, float s3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
  const float A = __uint_as_float(a[0]) + __uint_as_float(a[1]);   // rows 0-1: s0, rows 2-3: s1
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s2), __float_as_uint(s3), false, false);
  const float B = __uint_as_float(b[0]) + __uint_as_float(b[1]);   // rows 0-1: s2, rows 2-3: s3
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(B), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

template <int MT, bool PAGED = false>
__global__ __launch_bounds__(64 * kPfQ) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_idx_score_prefill(
    LayerParams P, const uint16_t* idx, const uint16_t* __restrict__ qI, const float* __restrict__ wt, int seq,
    int pos0, int T, uint32_t* __restrict__ keys) {
  constexpr int DI = 128, KS = DI / 32;
  constexpr int TB = kPfRows * DI * 2;   // bytes per tile buffer
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[2 * TB];
  __shared__ float cs_[kPfQ][32], sn_[kPfQ][32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.y * kPfQ;
  const int nlast = min(n0 + kPfQ, T) - 1;
  const int vmax = min((pos0 + nlast + 1) / 4, P.cap);   // rows the group's last query sees
  const int row0 = blockIdx.x * kPfRows * kPfTiles;
  if (row0 >= vmax) return;
  const int ntile = min(kPfTiles, (vmax - row0 + kPfRows - 1) / kPfRows);
  const int HI = P.HI, dn = DI - P.idx_rot;
  const int n = min(n0 + wave, T - 1);   // waves past the chunk redo its last query
  const int vlast = vmax - 1;
  // the run's rows: 128 pages of 64 (two a tile)
  static_assert(kPfRows * kPfTiles == 128 * 64 && kPfRows == 128, "two lane tables of 64 pages");
  const ScanRows<PAGED, 2> rows(P, idx, seq, row0, vlast, 2 * DI);

  // direct loads of tile rb into buffer buf: instruction e of this wave fills
  // rows 4 (kPfQ e + wave) .. + 3, which lie in the tile's page e / 2 (a page
  // the whole wave shares)
  auto load_tile = [&](int buf, int rb) {
#pragma unroll
    for (int e = 0; e < kPfRows / (4 * kPfQ); ++e) {
      const int R = 4 * (kPfQ * e + wave) + (lane >> 4);
      const int q = (lane & 15) ^ (R & 15);
      const uint8_t* rp = rows.row(((rb - row0) >> 6) + (e >> 1), R & 63, 2 * DI);
      lds_dma16(rp + 16 * q, tiles + buf * TB + 1024 * (kPfQ * e + wave));
    }
  };
  load_tile(0, row0);
  // this lane's query fragments: head 16 mt + r, channels 32 ks + 8 g .. + 7
  u32x4 Qf[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      Qf[mt][ks] = *(const u32x4*)(qI + ((size_t)n * HI + min(16 * mt + r, HI - 1)) * DI + 32 * ks + 8 * g);
  // weights of the heads this lane's accumulators hold: head 16 mt + 4 g + i
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * mt + 4 * g + i;
      wv[mt][i] = h < HI ? wt[(size_t)n * HI + min(h, HI - 1)] : 0.f;
    }
  if (tid < kPfQ * 32) {
    const int qq = tid >> 5, j = tid & 31;
    rope_cs_c(P, j, (double)(pos0 + min(n0 + qq, T - 1)), &cs_[qq][j], &sn_[qq][j]);
  }
  lds_barrier();
  // rotated query -> bf16 A fragments (heads past H_I are zero)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = bf16_to_f32(Qf[mt][ks][i] & 0xffffu), b = bf16_to_f32(Qf[mt][ks][i] >> 16);
        const int c = 32 * ks + 8 * g + 2 * i;
        if (c >= dn) {
          const int j = (c - dn) >> 1;
          const float x = a * cs_[wave][j] - b * sn_[wave][j], y = a * sn_[wave][j] + b * cs_[wave][j];
          a = x;
          b = y;
        }
        Qf[mt][ks][i] = 16 * mt + r < HI ? pack_bf16x2(a, b) : 0u;
      }
    }
  const int lo = (P.flags & CKV_FLAG_IDX_NO_RELU) ? INT_MIN : 0;   // relu on the bits: max(bits, lo)
  uint32_t* kout = keys + (size_t)n * P.cap;
  // this lane's B-fragment byte offsets within a buffer, k-step ks: row r of
  // a sixteen-row sub-tile, chunk 4 ks + g at position (4 ks + g) ^ r
  uint32_t boff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) boff[ks] = lds_addr(tiles) + r * 256 + 16 * ((4 * ks + g) ^ r);

#pragma unroll 1
  for (int t = 0; t < ntile; ++t) {
    const int rb = row0 + t * kPfRows;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's share of tile t has landed
    lds_barrier();                    // ... everyone's, and buffer (t + 1) % 2 is free
    if (t + 1 < ntile) load_tile((t + 1) & 1, rb + kPfRows);
    uint32_t ba[KS];   // sub-tile 0 of the buffer; later sub-tiles by offset fields
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ba[ks] = boff[ks] + (uint32_t)((t & 1) * TB);
#pragma unroll 1
    for (int sq = 0; sq < kPfRows / 64; ++sq) {   // groups of 4 sixteen-row sub-tiles
      float sc[4];
      auto sub = [&](auto uc) {
        constexpr int u = decltype(uc)::value;
        u32x4 Rv[KS];
        lds_read4_b128_at<u * 16 * 256>(ba[0], ba[1], ba[2], ba[3], Rv[0], Rv[1], Rv[2], Rv[3]);
        float sv = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(as_bf16x8(Qf[mt][ks]), as_bf16x8(Rv[ks]), acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) sv = fmaf(wv[mt][i], __int_as_float(max(__float_as_int(acc[i]), lo)), sv);
        }
        sc[u] = sv;   // this lane's heads; rows r of the other lane groups hold the rest
      };
      sub(std::integral_constant<int, 0>{});
      sub(std::integral_constant<int, 1>{});
      sub(std::integral_constant<int, 2>{});
      sub(std::integral_constant<int, 3>{});
      // lane group g receives the total of sub-tile (g & 1) * 2 + (g >> 1)
      const float mine = rows4_sum_scatter(sc[0], sc[1], sc[2], sc[3]);
      const int row = rb + 64 * sq + 16 * ((g & 1) * 2 + (g >> 1)) + r;
      *(row < P.cap ? kout + row : g_key_sink + lane) = float_key(mine);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ba[ks] += 64 * 256;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // no direct load outlives the block
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
  if (tid < nrot / 2) rope_cs_c(P, tid, (double)Q.p, &cs_[tid], &sn_[tid]);
  if (tid < HI) wsh[tid] = wt[(size_t)qn * HI + tid];
  if (hist)
    for (int e = tid; e < kHistBins; e += 256) lh[e] = 0;
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
    const size_t ro = (size_t)row_slot_rd(P, Q.seq, row) * DI;
    float s = 0.f;
    for (int h = 0; h < HI; ++h) {
      float dot = 0.f;
      for (int c = 0; c < DI; ++c) dot += qh[h * DI + c] * load_val<IDXF>(idx, ro + c);
      s += wsh[h] * (relu ? fmaxf(dot, 0.f) : dot);
    }
    const uint32_t key = float_key(s);
    keys[(size_t)qn * P.cap + row] = key;
    if (hist) atomicAdd(&lh[key >> 20], 1u);
  }
  if (hist) {
    __syncthreads();
    uint32_t* gh = hist + (size_t)qn * kHistBins;
    for (int e = tid; e < kHistBins; e += 256) {
      const uint32_t v = lh[e];
      if (v) atomicAdd(&gh[e], v);
    }
  }
}

// ---------------------------------------------------------------- select
// The block-wide helpers below synchronise with LDS-only barriers: their data
// lives in registers and LDS, and a full barrier would also wait for every
// global store the caller still has in flight.

// Exclusive prefix sum over the block (1024 threads); returns the thread's
// exclusive sum, *total receives the block total.
// NW > 0: the block has exactly NW waves (wsum 16-byte aligned); the wave
// totals are then read with a few vector reads issued together instead of a
// loop of dependent reads.
template <int NW = 0>
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  lds_barrier();
  if (lane == 63) wsum[wave] = x;
  lds_barrier();
  uint32_t before = 0, tot = 0;
  if constexpr (NW > 0) {
    u32x4 q[NW / 4];
#pragma unroll
    for (int j = 0; j < NW / 4; ++j) q[j] = *(const u32x4*)&wsum[4 * j];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += w < wave ? q[w >> 2][w & 3] : 0u;
      tot += q[w >> 2][w & 3];
    }
  } else {
    for (int w = 0; w < nw; ++w) {
      if (w < wave) before += wsum[w];
      tot += wsum[w];
    }
  }
  *total = tot;
  return before + x - v;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* wsum) {
  v = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  lds_barrier();
  if (lane == 0) wsum[wave] = v;
  lds_barrier();
  uint32_t t = 0;
  for (int w = 0; w < nw; ++w) t += wsum[w];
  lds_barrier();
  return t;
}

// Histogram sh[0..nb) ascending: find the bin b where the count of keys in
// bins below b is < need and reaches need including b.  Thread t owns bins
// t*per .. (t+1)*per-1.  bc[0] = b, bc[1] = count below b.
__device__ __forceinline__ void find_bin_asc(const uint32_t* sh, int nb, uint32_t need, uint32_t* wsum,
                                             uint32_t* bc) {
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int lo = min(nb, (int)threadIdx.x * per), hi = min(nb, lo + per);
  uint32_t local = 0;
  for (int b = lo; b < hi; ++b) local += sh[b];
  if (threadIdx.x == 0) {  // in-range fallback should the counts disagree
    bc[0] = 0;
    bc[1] = 0;
  }
  uint32_t tot;
  const uint32_t below = block_exscan(local, wsum, &tot);
  if (below < need && below + local >= need) {
    uint32_t cum = below;
    for (int b = lo; b < hi; ++b) {
      if (cum + sh[b] >= need) {
        bc[0] = (uint32_t)b;
        bc[1] = cum;
        break;
      }
      cum += sh[b];
    }
  }
  lds_barrier();
}

// Radix select over d = M - key.  count_level(shift, nbits, pfx, pmask, sh)
// must histogram (d >> shift) & ((1 << nbits) - 1) into sh for the keys whose
// d agrees with pfx on the bits in pmask.  Returns T (the k-th largest key) and
// sets *need to the number of keys equal to T that are selected.
template <typename CountLevel>
__device__ __forceinline__ uint32_t radix_select(uint32_t M, uint32_t k, CountLevel count_level, uint32_t* sh,
                                                 uint32_t* wsum, uint32_t* bc, uint32_t* need_out) {
  uint32_t need = k;
  // level 1: d >> s over d < 2^(s + 10); widen until at least k keys are in range
  int shift = 14;
  for (;;) {
    count_level(shift, 10, 0u, shift + 10 >= 32 ? 0u : ~((1u << (shift + 10)) - 1u), sh);
    uint32_t tot = 0;
    {
      uint32_t part = 0;
      for (int e = threadIdx.x; e < 1024; e += blockDim.x) part += sh[e];
      tot = (uint32_t)block_sum_u32(part, wsum);
    }
    if (tot >= need || shift >= 22) break;
    shift += 8;
  }
  // bins are ascending in d: bin 0 holds the largest keys; find the bin where
  // the running count (from bin 0 up) reaches `need`
  find_bin_asc(sh, 1024, need, wsum, bc);
  uint32_t pfx = bc[0] << shift;
  uint32_t pmask = ~((1u << shift) - 1u);
  need -= bc[1];
  while (shift > 0) {
    const int nbits = shift < 10 ? shift : 10;
    shift -= nbits;
    count_level(shift, nbits, pfx, pmask, sh);
    find_bin_asc(sh, 1 << nbits, need, wsum, bc);
    pfx |= bc[0] << shift;
    pmask |= ((1u << nbits) - 1u) << shift;
    need -= bc[1];
  }
  *need_out = need;
  return M - pfx;
}

// The selection once the k-th largest key T is known and `need` keys equal to
// T are to be taken: wave w walks its contiguous chunk [c0, c1) in steps of
// 64, so indices come out ascending.  key_at(j) returns the key of step j of
// this lane (index c0 + 64 j + lane).  NS > 0 fixes the step count at compile
// time (register-resident keys); NS == 0 walks the chunk at run time.
template <int NS, typename KeyAt>
__device__ __forceinline__ void emit_selected(KeyAt key_at, int c0, int c1, uint32_t T, uint32_t need,
                                              int k, int32_t* o, uint32_t* wgt, uint32_t* weq) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nstep = NS > 0 ? NS : (c1 - c0 + 63) / 64;
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < (NS > 0 ? NS : 1 << 30); ++j) {
    if (NS == 0 && j >= nstep) break;
    const int s = c0 + 64 * j + lane;
    const uint32_t key = s < c1 ? key_at(j) : 0u;
    ngt += __popcll(__ballot(s < c1 && key > T));
    neq += __popcll(__ballot(s < c1 && key == T));
  }
  if (lane == 0) {
    wgt[wave] = ngt;
    weq[wave] = neq;
  }
  lds_barrier();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += wgt[w];
    eq_before += weq[w];
  }
  uint32_t eq_run = eq_before;
  uint32_t sel_run = gt_before + min(eq_before, need);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < (NS > 0 ? NS : 1 << 30); ++j) {
    if (NS == 0 && j >= nstep) break;
    const int s = c0 + 64 * j + lane;
    const uint32_t key = s < c1 ? key_at(j) : 0u;
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

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* wsum) {
  v = max(v, dpp_u32<0xb1>(0u, v));
  v = max(v, dpp_u32<0x4e>(0u, v));
  v = max(v, dpp_u32<0x141>(0u, v));
  v = max(v, dpp_u32<0x140>(0u, v));
  v = max(v, dpp_u32<0x142, 0xa>(0u, v));
  v = max(v, dpp_u32<0x143, 0xc>(0u, v));
  v = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  lds_barrier();
  if (lane == 0) wsum[wave] = v;
  lds_barrier();
  uint32_t t = 0;
  for (int w = 0; w < nw; ++w) t = max(t, wsum[w]);
  lds_barrier();
  return t;
}

// Keys of one query held in registers: wave w owns indices [64 KPT w,
// 64 KPT (w + 1)), step j of lane l holding index 64 KPT w + 64 j + l.
// V <= NT KPT.  One block of NT threads per query.
// Prefill chunks (V <= 16384 at the 4096-token chunk of a 64k context): 512
// threads of 32 keys (several blocks share a compute unit, and each block's
// radix levels synchronise 8 waves instead of 16: 0.214 -> 0.155 ms per
// chunk against 1024 threads of 16 keys).
constexpr int kSelRegKPT = 32, kSelRegNT = 512;
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void k_topk_select_reg(LayerParams P, const uint32_t* __restrict__ keys,
                                                          const int32_t* __restrict__ pos, int pos0,
                                                          int32_t* __restrict__ out) {
  __shared__ uint32_t sh[1024];
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
  const int c0 = wave * (KPT * 64);
  uint32_t kr[KPT];
  uint32_t mloc = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int s = c0 + 64 * j + lane;
    kr[j] = s < V ? kq[s] : 0u;
    mloc = max(mloc, kr[j]);
  }
  const uint32_t M = block_max_u32(mloc, wsum);
  auto count_level = [&](int shift, int nbits, uint32_t pfx, uint32_t pmask, uint32_t* h) {
    const uint32_t nb = 1u << nbits;
    for (int e = tid; e < (int)nb; e += blockDim.x) h[e] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t d = M - kr[j];
      if (c0 + 64 * j + lane < V && (d & pmask) == pfx) atomicAdd(&h[(d >> shift) & (nb - 1u)], 1u);
    }
    __syncthreads();
  };
  uint32_t need;
  const uint32_t T = radix_select(M, (uint32_t)k, count_level, sh, wsum, bc, &need);
  const int c1 = min(V, c0 + KPT * 64);
  emit_selected<KPT>([&](int j) -> uint32_t { return kr[j]; }, c0, max(c0, c1), T, need, k, o, wgt, weq);
}

// Any V: the same selection streaming the keys from memory.  Wave w owns the
// contiguous chunk [c0, c1).  One block of 1024 threads per query.
__global__ __launch_bounds__(1024) void k_topk_select(LayerParams P, const uint32_t* __restrict__ keys,
                                                      const int32_t* __restrict__ pos, int pos0,
                                                      int32_t* __restrict__ out) {
  __shared__ uint32_t sh[1024];
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
  const int CH = ((V + 15) / 16 + 63) / 64 * 64;
  const int c0 = min(V, wave * CH), c1 = min(V, c0 + CH);
  uint32_t mloc = 0;
  for (int s = c0 + lane; s < c1; s += 64) mloc = max(mloc, kq[s]);
  const uint32_t M = block_max_u32(mloc, wsum);
  auto count_level = [&](int shift, int nbits, uint32_t pfx, uint32_t pmask, uint32_t* h) {
    const uint32_t nb = 1u << nbits;
    for (int e = tid; e < (int)nb; e += blockDim.x) h[e] = 0;
    __syncthreads();
    for (int s = c0 + lane; s < c1; s += 64) {
      const uint32_t d = M - kq[s];
      if ((d & pmask) == pfx) atomicAdd(&h[(d >> shift) & (nb - 1u)], 1u);
    }
    __syncthreads();
  };
  uint32_t need;
  const uint32_t T = radix_select(M, (uint32_t)k, count_level, sh, wsum, bc, &need);
  emit_selected<0>([&](int j) -> uint32_t { return kq[c0 + 64 * j + lane]; }, c0, c1, T, need, k, o, wgt,
                   weq);
}

// Decode selection spread over many blocks, driven by the score kernel's
// histogram of the keys' top 12 bits, in two kernels.
//
// k_topk_classify (grid: x = chunks of kSelChunk keys, y = queries): every
// block reads the query's histogram and finds the bin b1 holding the k-th
// largest key (A keys lie in higher bins, A < k).  It classifies its chunk:
// keys above b1 are selected outright and appended to the query's "sure"
// list, keys in b1 are appended to its candidate list (offsets from atomics
// on per-query counters).
//
// k_topk_finish (one block per query) resolves the candidates: two radix
// levels over their low 20 bits give the k-th key T exactly and how many keys
// equal to T are taken (the lowest-index ones); the k selected indices are
// sorted ascending in LDS (bitonic) and written out, and the histogram and
// counters are returned to zero.  Should the candidate bin hold more keys
// than the list takes (heavily tied scores), it runs the exact streaming
// radix select over all keys of the query instead.
//
// The lists cross from one kernel to the next: within one kernel, making one
// block's stores visible to a block on another XCD takes a device-scope
// fence, which writes back and invalidates the L2 (tens of microseconds when
// every block issues one); the kernel boundary does it once.
constexpr int kSelChunk = 2048;

// bitonic sort of sh[0..n) ascending, n a power of two, all threads
__device__ __forceinline__ void bitonic_sort_lds(uint32_t* sh, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t a = sh[lo], b = sh[hi];
        if ((a > b) == up) {
          sh[lo] = b;
          sh[hi] = a;
        }
      }
      lds_barrier();
    }
  }
}

// In a histogram of nb bins held as `per` consecutive bins per thread
// (thread t: bins t*per .. t*per+per-1, values v[]), find the bin where the
// count of keys in higher bins first reaches `need`: out[0] = bin, out[1] =
// count in bins above it, out[2] = count in the bin.  All threads.
template <int PER, int NW = 0>
__device__ __forceinline__ void find_from_top(const uint32_t (&v)[PER], uint32_t need, uint32_t* wsum,
                                              uint32_t* out) {
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += v[i];
  uint32_t tot;
  const uint32_t before = block_exscan<NW>(local, wsum, &tot);   // bins below this thread's
  const uint32_t above = tot - before - local;                // bins above this thread's
  if (above < need && above + local >= need) {
    uint32_t cum = above;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (cum < need && cum + v[i] >= need) {
        out[0] = (uint32_t)(threadIdx.x * PER + i);
        out[1] = cum;
        out[2] = v[i];
      }
      cum += v[i];
    }
  }
  lds_barrier();
}

// The query's histogram, 16 consecutive bins per thread -> b1 and A.
__device__ __forceinline__ void hist_threshold(const uint32_t* gh, uint32_t k, uint32_t* wsum, uint32_t* res,
                                               uint32_t (&hv)[16]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const u32x4 t4 = *(const u32x4*)(gh + 16 * threadIdx.x + 4 * e);
    hv[4 * e] = t4.x;
    hv[4 * e + 1] = t4.y;
    hv[4 * e + 2] = t4.z;
    hv[4 * e + 3] = t4.w;
  }
  if (threadIdx.x == 0) {
    res[0] = 0;
    res[1] = 0;
  }
  find_from_top<16>(hv, k, wsum, res);
}

__global__ __launch_bounds__(256) void k_topk_classify(LayerParams P, const uint32_t* __restrict__ keys,
                                                       SelWs S, const int32_t* __restrict__ pos) {
  constexpr int KPT = kSelChunk / 256;
  __shared__ uint32_t wsum[8], res[4], wcnt[2][4], base[2];
  const int qn = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = P.topk;
  const IdxQuery Q = idx_query(P, pos, 0, 0, qn);
  const int V = Q.V;
  const int c0 = blockIdx.x * kSelChunk;
  if (V <= k || c0 >= V) return;   // nothing to select, or no key of this query here
  const uint32_t* gh = S.hist + (size_t)qn * kHistBins;
  uint32_t* ctr = S.ctr + (size_t)qn * 4;
  const uint32_t* kq = keys + (size_t)qn * P.cap;
  // this block's keys (indices clamped, rows past V masked below), issued
  // together with the histogram loads
  uint32_t kr[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) kr[j] = kq[min(c0 + 256 * j + tid, V - 1)];
  uint32_t hv[16];
  hist_threshold(gh, (uint32_t)k, wsum, res, hv);
  const uint32_t b1 = res[0];

  // classify: counts per wave, one global append per list per block
  uint32_t ns = 0, nc = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool ok = c0 + 256 * j + tid < V;
    const uint32_t bin = kr[j] >> 20;
    ns += __popcll(__ballot(ok && bin > b1));
    nc += __popcll(__ballot(ok && bin == b1));
  }
  if (lane == 0) {
    wcnt[0][wave] = ns;
    wcnt[1][wave] = nc;
  }
  __syncthreads();
  if (tid < 2) {   // the two appends' offsets, one thread each (in parallel)
    const uint32_t t = wcnt[tid][0] + wcnt[tid][1] + wcnt[tid][2] + wcnt[tid][3];
    base[tid] = t ? atomicAdd(&ctr[1 + tid], t) : 0u;
  }
  __syncthreads();
  {
    uint32_t os = base[0], oc = base[1];
    for (int w = 0; w < wave; ++w) {
      os += wcnt[0][w];
      oc += wcnt[1][w];
    }
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t* sure = S.sure + (size_t)qn * k;
    uint32_t* cnk = S.cand_key + (size_t)qn * kCandCap;
    uint32_t* cni = S.cand_idx + (size_t)qn * kCandCap;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int sidx = c0 + 256 * j + tid;
      const bool ok = sidx < V;
      const uint32_t bin = kr[j] >> 20;
      const bool is_s = ok && bin > b1, is_c = ok && bin == b1;
      const unsigned long long ms = __ballot(is_s), mc = __ballot(is_c);
      const uint32_t ps = os + (uint32_t)__popcll(ms & lt), pc = oc + (uint32_t)__popcll(mc & lt);
      if (is_s && ps < (uint32_t)k) sure[ps] = (uint32_t)sidx;
      if (is_c && pc < (uint32_t)kCandCap) {
        cnk[pc] = kr[j];
        cni[pc] = (uint32_t)sidx;
      }
      os += (uint32_t)__popcll(ms);
      oc += (uint32_t)__popcll(mc);
    }
  }
}

__global__ __launch_bounds__(256) void k_topk_finish(LayerParams P, const uint32_t* __restrict__ keys,
                                                     SelWs S, const int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ out) {
  __shared__ uint32_t sh[kHistBins];
  __shared__ uint32_t ck[kCandCap], ci[kCandCap];
  __shared__ uint32_t fin[4096];
  __shared__ uint32_t wsum[8], res[4], wcnt[2][4], nfin, neq;
  const int qn = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = P.topk;
  const IdxQuery Q = idx_query(P, pos, 0, 0, qn);
  const int V = Q.V;
  int32_t* o = out + (size_t)qn * k;
  uint32_t* gh = S.hist + (size_t)qn * kHistBins;
  uint32_t* ctr = S.ctr + (size_t)qn * 4;
  if (V <= k) {   // every visible row is taken; the histogram is cleared all the same
    for (int j = tid; j < k; j += 256) o[j] = j < V ? j : -1;
    for (int e = tid; e < kHistBins; e += 256) gh[e] = 0;
    return;
  }
  const uint32_t* kq = keys + (size_t)qn * P.cap;
  // the whole candidate and sure lists are read together with the histogram
  // (one memory round trip; their lengths are known only after it)
  const uint32_t* cnk = S.cand_key + (size_t)qn * kCandCap;
  const uint32_t* cni = S.cand_idx + (size_t)qn * kCandCap;
  const uint32_t* sure = S.sure + (size_t)qn * k;
  uint32_t rk[kCandCap / 256], ri[kCandCap / 256], rs[16];
#pragma unroll
  for (int e = 0; e < kCandCap / 256; ++e) {
    rk[e] = cnk[tid + 256 * e];
    ri[e] = cni[tid + 256 * e];
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) rs[e] = sure[min(tid + 256 * e, k - 1)];   // k <= 4096
  uint32_t hv[16];
  hist_threshold(gh, (uint32_t)k, wsum, res, hv);
  const uint32_t b1 = res[0], A = res[1], nb1 = res[2];   // nb1: keys in b1 = candidates appended
  if (nb1 <= (uint32_t)kCandCap) {
    const uint32_t nc_all = nb1;
#pragma unroll
    for (int e = 0; e < kCandCap / 256; ++e) {
      const int i = tid + 256 * e;
      if (i < (int)nc_all) {
        ck[i] = rk[e];
        ci[i] = ri[e];
      }
    }
    uint32_t need = (uint32_t)k - A;
    uint32_t prefix = b1 << 20, mask = 0xfff00000u;
    // two levels over the candidates: bits 19..8 (4096 bins), then 7..0
#pragma unroll 1
    for (int lvl = 0; lvl < 2; ++lvl) {
      const int shift = lvl == 0 ? 8 : 0;
      const int nb = lvl == 0 ? 4096 : 256;
      for (int e = tid; e < kHistBins; e += 256) sh[e] = 0;
      __syncthreads();
      for (int i = tid; i < (int)nc_all; i += 256) {
        const uint32_t key = ck[i];
        if ((key & mask) == prefix) atomicAdd(&sh[(key >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      uint32_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (lvl == 0 || tid < 16) ? sh[(16 * tid + i) & (kHistBins - 1)] : 0u;
      if (tid == 0) {
        res[0] = 0;
        res[1] = 0;
      }
      find_from_top<16>(v, need, wsum, res);
      prefix |= res[0] << shift;
      mask |= (uint32_t)(nb - 1) << shift;
      need -= res[1];
    }
    const uint32_t T = prefix;   // the k-th largest key; `need` keys equal to it are taken
    // The selected rows, marked in a bitmap over [0, V): the sure list, the
    // candidates above T and the `need` lowest-index candidates equal to T.
    // (Rows beyond the bitmap's reach go through a bitonic sort instead.)
    const bool use_bm = V <= 32 * 4096;
    const int nw = (V + 31) / 32;
    uint32_t* bm = fin;                 // bitmap words (V <= 131072)
    uint32_t* eql = sh;                 // candidates equal to T (sh is free now)
    if (use_bm)
      for (int e = tid; e < nw; e += 256) bm[e] = 0;
    if (tid == 0) {
      nfin = 0;
      neq = 0;
    }
    __syncthreads();
    auto mark = [&](uint32_t idx) {
      if (use_bm) atomicOr(&bm[idx >> 5], 1u << (idx & 31));
      else fin[atomicAdd(&nfin, 1u)] = idx;
    };
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (tid + 256 * e < (int)A) mark(rs[e]);
    for (int i = tid; i < (int)nc_all; i += 256) {
      const uint32_t key = ck[i];
      if (key > T) mark(ci[i]);
      else if (key == T) eql[atomicAdd(&neq, 1u)] = ci[i];
    }
    __syncthreads();
    const int ne = (int)neq;
    if (ne > (int)need) {   // more ties than taken: keep the lowest indices
      int n2 = 1;
      while (n2 < ne) n2 <<= 1;
      for (int i = ne + tid; i < n2; i += 256) eql[i] = 0xffffffffu;
      __syncthreads();
      bitonic_sort_lds(eql, n2);
    }
    for (int i = tid; i < (int)need; i += 256) mark(eql[i]);
    __syncthreads();
    if (use_bm) {
      // ascending emission: each thread owns a run of words; block prefix of
      // their popcounts gives its first output slot
      const int per = (nw + 255) / 256;
      const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
      uint32_t cnt = 0;
      for (int e = w0; e < w1; ++e) cnt += __popc(bm[e]);
      uint32_t tot;
      uint32_t slot = block_exscan(cnt, wsum, &tot);
      for (int e = w0; e < w1; ++e) {
        uint32_t bits = bm[e];
        while (bits) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          if (slot < (uint32_t)k) o[slot] = 32 * e + b;
          ++slot;
        }
      }
    } else {
      int n2 = 1;
      while (n2 < k) n2 <<= 1;
      for (int i = k + tid; i < n2; i += 256) fin[i] = 0xffffffffu;
      __syncthreads();
      bitonic_sort_lds(fin, n2);
      for (int j = tid; j < k; j += 256) o[j] = (int32_t)fin[j];
    }
  } else {
    // heavily tied scores: exact streaming radix select over all V keys
    const int CH = ((V + 3) / 4 + 63) / 64 * 64;
    const int w0 = min(V, wave * CH), w1 = min(V, w0 + CH);
    uint32_t mloc = 0;
    for (int s = w0 + lane; s < w1; s += 64) mloc = max(mloc, kq[s]);
    const uint32_t M = block_max_u32(mloc, wsum);
    auto count_level = [&](int shift, int nbits, uint32_t pfx, uint32_t pmask, uint32_t* h) {
      const uint32_t nb = 1u << nbits;
      for (int e = tid; e < (int)nb; e += 256) h[e] = 0;
      __syncthreads();
      for (int s = w0 + lane; s < w1; s += 64) {
        const uint32_t d = M - kq[s];
        if ((d & pmask) == pfx) atomicAdd(&h[(d >> shift) & (nb - 1u)], 1u);
      }
      __syncthreads();
    };
    uint32_t need;
    const uint32_t T = radix_select(M, (uint32_t)k, count_level, sh, wsum, res, &need);
    emit_selected<0>([&](int j) -> uint32_t { return kq[w0 + 64 * j + lane]; }, w0, w1, T, need, k, o,
                     wcnt[0], wcnt[1]);
  }
  // leave the histogram and counters zeroed for the next call
  for (int e = tid; e < kHistBins; e += 256) gh[e] = 0;
  if (tid < 4) ctr[tid] = 0;
}

// Decode selection of one query in one block (1024 threads, V <= 32768).
// Thread t holds the keys of rows t + 1024 e (e < 32) in registers.  The
// score kernel's histogram of the keys' top 12 bits gives the bin b1 holding
// the k-th largest key: rows in higher bins are selected outright; the rows
// of bin b1 are candidates, resolved exactly with two more radix levels (bits
// 19..8, then 7..0) in LDS, giving the k-th largest key T.  Rows above T are
// selected, and of the rows equal to T the lowest-index ones, ranked through
// a block scan of an equal-key bitmap.  The selection is a bitmap over the
// rows, emitted in ascending order from a block scan of its word popcounts.
// The histogram is returned to zero as it is read.  Should bin b1 hold more
// keys than the candidate list takes (heavily tied scores), the threshold is
// found by a radix select over all the keys instead.
constexpr int kSelKPT = 32;   // keys per thread of the one-block decode selection

// Key e of thread t in the one-block selection is row t + 1024 e: a wave's
// ballot over key e covers rows 1024 e + 64 w .. +63, i.e. bitmap words
// 32 e + 2 w and 32 e + 2 w + 1, so bitmaps come straight from ballots.
__device__ __forceinline__ void sel_load_keys(const uint32_t* kq, int cap, int t, uint32_t (&kr)[kSelKPT]) {
#pragma unroll
  for (int e = 0; e < kSelKPT; ++e) kr[e] = kq[min(t + 1024 * e, cap - 1)];
}

// One wave: in the LDS histogram h[0..64 PER) (lane l owns bins PER l ..
// PER l + PER - 1, PER 1 or a multiple of 4), the bin where the count of
// keys in higher bins first reaches need (1 <= need <= the total): returns
// the bin; *above = the count in higher bins, *cnt = the count in the bin.
// Every lane of the wave receives the results; no block barrier.
template <int PER>
__device__ __forceinline__ uint32_t wave_find_from_top(const uint32_t* h, uint32_t need, uint32_t* above,
                                                       uint32_t* cnt) {
  const int lane = threadIdx.x & 63;
  uint32_t v[PER];
  if constexpr (PER == 1) {
    v[0] = h[lane];
  } else {
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const u32x4 t = *(const u32x4*)(h + PER * lane + i);
      v[i] = t[0];
      v[i + 1] = t[1];
      v[i + 2] = t[2];
      v[i + 3] = t[3];
    }
  }
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += v[i];
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t abv = total - incl;   // bins of higher lanes
  const bool mine = abv < need && abv + local >= need;
  const int owner = (int)__builtin_ctzll(__ballot(mine));
  uint32_t bin = 0, ab = 0, c = 0, cum = abv;
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    if (cum < need && cum + v[i] >= need) {
      bin = (uint32_t)(PER * lane + i);
      ab = cum;
      c = v[i];
    }
    cum += v[i];
  }
  *above = (uint32_t)__builtin_amdgcn_readlane((int)ab, owner);
  *cnt = (uint32_t)__builtin_amdgcn_readlane((int)c, owner);
  return (uint32_t)__builtin_amdgcn_readlane((int)bin, owner);
}

// The selection itself, from keys kr (row tid + 1024 e) and histogram bins
// hv (bins 4 tid .. 4 tid + 3) held by the 1024 threads of the block, V > k.
//   1. b1 = the 12-bit key bin holding the k-th largest key (histogram scan);
//   2. the keys in b1 are appended to a candidate list (per-thread counts, one
//      block scan, no atomics) and refined by two radix levels (12 + 8 bits)
//      to the k-th largest key T and the number of keys equal to T to take;
//      with more candidates than the list holds, a radix select over all keys;
//   3. bitmaps of the rows with key > T and key == T from ballots; one block
//      scan of the words' packed popcounts gives every 32-row word its output
//      slot, rows equal to T being taken lowest index first; rows are written
//      ascending.
// With one block per query the selection runs on one compute unit, so its
// cost is the instructions per key: a few vector operations, and scalar ones
// (shared by the unit's 16 waves) only where a ballot is the product.
__device__ __forceinline__ void topk_decode_select(const LayerParams& P, int V, uint32_t (&kr)[kSelKPT],
                                                   uint32_t (&hv)[4], int32_t* __restrict__ o) {
  constexpr int KPT = kSelKPT;
  __shared__ uint32_t gtw[1024];   // rows with key > T
  __shared__ uint32_t eqw[1024];   // rows with key == T
  __shared__ uint32_t sh[kHistBins];
  __shared__ __attribute__((aligned(16))) uint32_t hl0[256], hl1[256], hl2[64];   // candidate radix levels
  __shared__ uint32_t ck[kCandCap], ci[kCandCap];
  __shared__ __attribute__((aligned(16))) uint32_t wsum[16];
  __shared__ uint32_t res[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = P.topk;
  const int nv = (V - tid + 1023) >> 10;   // this thread's keys e < nv are visible rows
  if (tid == 0) {
    res[0] = 0;
    res[1] = 0;
    res[2] = 0;
    res[3] = 0;
  }
  find_from_top<4, 16>(hv, (uint32_t)k, wsum, res);   // ends with a barrier
  const uint32_t b1 = res[0], A = res[1], nb1 = res[2];
  uint32_t T, need_eq, n_eq = 0u;
  if (nb1 <= (uint32_t)kCandCap) {
    // candidates: the keys of bin b1, appended at offsets from a wave scan of
    // the per-thread counts and one LDS atomic per wave (their order does not
    // matter: each carries its row)
    if (tid < 256) hl0[tid] = 0u;
    else if (tid < 512) hl1[tid - 256] = 0u;
    else if (tid < 576) hl2[tid - 512] = 0u;
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) cnt += (e < nv && (kr[e] >> 20) == b1) ? 1u : 0u;
    {
      const uint32_t incl = wave_incl_scan(cnt);
      const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      uint32_t wbase = 0u;
      if (lane == 0 && wtot) wbase = atomicAdd(&res[3], wtot);
      uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)wbase, 0) + incl - cnt;
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        if (e < nv && (kr[e] >> 20) == b1) {
          if (at < (uint32_t)kCandCap) {
            ck[at] = kr[e];
            ci[at] = (uint32_t)(tid + 1024 * e);
          }
          ++at;
        }
      }
    }
    lds_barrier();
    // wave 0 resolves the k-th key among them with three radix levels of
    // the candidates' low 20 bits (8, 8 and 4 bits), no block barrier
    if (wave == 0) {
      const int nc = (int)min(nb1, (uint32_t)kCandCap);
      uint32_t need = (uint32_t)k - A, ab, cn;
      for (int c = lane; c < nc; c += 64) atomicAdd(&hl0[(ck[c] >> 12) & 255u], 1u);
      const uint32_t d0 = wave_find_from_top<4>(hl0, need, &ab, &cn);
      need -= ab;
      const uint32_t p0 = (b1 << 20) | (d0 << 12);
      for (int c = lane; c < nc; c += 64)
        if ((ck[c] & 0xfffff000u) == p0) atomicAdd(&hl1[(ck[c] >> 4) & 255u], 1u);
      const uint32_t d1 = wave_find_from_top<4>(hl1, need, &ab, &cn);
      need -= ab;
      const uint32_t p1 = p0 | (d1 << 4);
      for (int c = lane; c < nc; c += 64)
        if ((ck[c] & 0xfffffff0u) == p1) atomicAdd(&hl2[ck[c] & 15u], 1u);
      const uint32_t d2 = wave_find_from_top<1>(hl2, need, &ab, &cn);
      if (lane == 0) {
        res[0] = p1 | d2;
        res[1] = need - ab;   // keys equal to T taken
        res[2] = cn;          // keys equal to T
      }
    }
    lds_barrier();
    T = res[0];
    need_eq = res[1];
    n_eq = res[2];
  } else {
    // heavily tied scores: radix select over all keys (d = M - key)
    uint32_t mloc = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) mloc = max(mloc, tid + 1024 * e < V ? kr[e] : 0u);
    const uint32_t M = block_max_u32(mloc, wsum);
    auto count_level = [&](int shift, int nbits, uint32_t pfx, uint32_t pmask, uint32_t* h) {
      const uint32_t nbn = 1u << nbits;
      for (int e = tid; e < (int)nbn; e += 1024) h[e] = 0;
      lds_barrier();
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const uint32_t dd = M - kr[e];
        if (tid + 1024 * e < V && (dd & pmask) == pfx) atomicAdd(&h[(dd >> shift) & (nbn - 1u)], 1u);
      }
      lds_barrier();
    };
    T = radix_select(M, (uint32_t)k, count_level, sh, wsum, res, &need_eq);
  }
  // bitmaps of key > T (gtw) and key == T (eqw); when every key equal to T
  // is taken (no tie at the k-th place) one bitmap of key >= T (gtw) does.
  // Lanes 0 and 1 write the low and high words of each ballot.
  const bool all_eq = n_eq == need_eq;
  if (all_eq) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const unsigned long long bg = __ballot(e < nv && kr[e] >= T);
      if (lane < 2) gtw[32 * e + 2 * wave + lane] = (uint32_t)(lane ? bg >> 32 : bg);
    }
  } else {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const unsigned long long bg = __ballot(e < nv && kr[e] > T), be = __ballot(e < nv && kr[e] == T);
      if (lane < 2) {
        const int wd = 32 * e + 2 * wave + lane;
        gtw[wd] = (uint32_t)(lane ? bg >> 32 : bg);
        eqw[wd] = (uint32_t)(lane ? be >> 32 : be);
      }
    }
  }
  lds_barrier();
  // word tid covers rows 32 tid .. 32 tid + 31: its slot from the counts of
  // the words before it (key > T in the high half, key == T in the low half)
  {
    const uint32_t g = gtw[tid], q = all_eq ? 0u : eqw[tid];
    uint32_t tot;
    const uint32_t before = block_exscan<16>(((uint32_t)__popc(g) << 16) | (uint32_t)__popc(q), wsum, &tot);
    const uint32_t gt_before = before >> 16, eq_before = before & 0xffffu;
    uint32_t keep = 0u, bits = q, r = eq_before;
    while (bits && r < need_eq) {
      const uint32_t lowest = bits & (~bits + 1u);
      keep |= lowest;
      bits ^= lowest;
      ++r;
    }
    uint32_t sel = g | keep;
    uint32_t slot = gt_before + min(eq_before, need_eq);
    while (sel) {
      const int bpos = __ffs(sel) - 1;
      sel &= sel - 1;
      if (slot < (uint32_t)k) o[slot] = 32 * tid + bpos;
      ++slot;
    }
    const uint32_t total = (tot >> 16) + min(tot & 0xffffu, need_eq);
    for (int j = (int)total + tid; j < k; j += 1024) o[j] = -1;
  }
}

__global__ __launch_bounds__(1024) void k_topk_decode(LayerParams P, const uint32_t* __restrict__ keys, SelWs S,
                                                      const int32_t* __restrict__ pos, int32_t* __restrict__ out) {
  const int qn = blockIdx.x, tid = threadIdx.x;
  const int k = P.topk;
  const IdxQuery Q = idx_query(P, pos, 0, 0, qn);
  const int V = Q.V;
  int32_t* o = out + (size_t)qn * k;
  uint32_t* gh = S.hist + (size_t)qn * kHistBins;
  // histogram bins 4 t .. 4 t + 3 and this thread's keys, one round of loads
  const u32x4 h4 = *(const u32x4*)(gh + 4 * tid);
  const uint32_t* kq = keys + (size_t)qn * P.cap;
  uint32_t kr[kSelKPT];
  sel_load_keys(kq, P.cap, tid, kr);
  *(u32x4*)(gh + 4 * tid) = (u32x4){0u, 0u, 0u, 0u};
  if (V <= k) {   // every visible row is taken
    for (int j = tid; j < k; j += 1024) o[j] = j < V ? j : -1;
    return;
  }
  uint32_t hv[4] = {h4[0], h4[1], h4[2], h4[3]};
  topk_decode_select(P, V, kr, hv, o);
}

// ---------------------------------------------------------------- fused decode step
// One decode step of a ratio-4 layer in three launches (plus the attention
// merge): the compressor's projection runs inside the score scan's launch
// (the rows the scan reads do not depend on it), and one block per sequence
// then runs the compressor, scores the row its token closed and selects.
//
// k_step_scan: the last nproj blocks compute the projection tiles (16
// columns x 16 rows each, 4 waves over one of kProjSlices K slices); the
// others score the query's cache rows except the row its own token closes,
// building the key histogram.
template <int MT, int QF, int IDXF, bool PAGED = false, int NG = kStepGroups>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_step_scan(
    LayerParams P, const void* idx, const void* __restrict__ qI, const float* __restrict__ wt,
    const int32_t* __restrict__ pos, uint32_t* __restrict__ keys, uint32_t* __restrict__ hist,
    const uint16_t* __restrict__ X, int M, WCat wc, float* __restrict__ proj, int nproj, int nrb,
    uint8_t* __restrict__ qf4) {
  const int nscan = (int)gridDim.x - nproj;
  const int bid = blockIdx.x;
  if (kStepProjLast ? bid >= nscan : bid < nproj) {
    const int t = kStepProjLast ? bid - nscan : bid;
    const int ntile = nproj / kProjSlices, tile = t % ntile;
    const int ncb = P.ncol / 16;
    proj_tile<4, kStepProjSF>(X, M, P.hidden, wc, P.ncol, proj, 16 * (tile % ncb), 16 * (tile / ncb), t / ntile,
                              kProjSlices);
    return;
  }
  const int i = kStepProjLast ? bid : bid - nproj;
  if constexpr (IDXF == CKV_FP4)
    idx_score_block_fp4<MT, true, NG, PAGED>(P, (const uint8_t*)idx, qI, wt, pos, 0, 0, keys, hist, i % nrb,
                                             i / nrb, true, qf4);
  else
    idx_score_block<MT, 4, QF, true, NG, PAGED>(P, (const uint16_t*)idx, qI, wt, pos, 0, 0, keys, hist, i % nrb,
                                                i / nrb, true);
}

// k_step_select: one block of 1024 threads per sequence.  The indexer query
// and the histogram are loaded first, then the compressor's inputs, then the
// query's keys, which stay in flight while the compressor (state store, raw
// row, pooling, RMSNorm, RoPE, cache insertion) runs on the block; when the
// token closed a row, its indexer score is computed here (the rotated query
// cast to the indexer format, dotted with the row's stored values, relu,
// weighted head sum) and joins the keys and the histogram; then the selection.
// With fp4 indexer rows the scan has already rotated and transformed the
// query (Hadamard, MXFP4) and left it in S.qf4: the block reads those codes
// instead of the bf16 query, so both kernels score with the same fp4 query.
template <int KVF, int IDXF, int ACTF, int NL = 1>
__global__ __launch_bounds__(1024) void k_step_select(LayerParams P, Weights w, Cache cc, const void* __restrict__ u,
                                                      const int32_t* __restrict__ pos, const float* __restrict__ proj,
                                                      int B, const void* __restrict__ qI,
                                                      const float* __restrict__ wt, const uint32_t* __restrict__ keys,
                                                      SelWs S, int32_t* __restrict__ out) {
  static_assert(ACTF == CKV_BF16 && (IDXF == CKV_BF16 || IDXF == CKV_FP4),
                "the fused step takes bf16 activations and bf16 or fp4 indexer rows");
  constexpr int DI = 128, CPT = DI / 16;
  __shared__ __attribute__((aligned(16))) float red[64];
  __shared__ __attribute__((aligned(16))) float idx_row[kMaxDI];
  __shared__ __attribute__((aligned(16))) float hsum[64];
  __shared__ float rtab[192];
  __shared__ __attribute__((aligned(16))) uint32_t h_lds[kHistBins];
  __shared__ __attribute__((aligned(16))) uint32_t q_lds[64 * DI / 2];
  const int qn = blockIdx.x, tid = threadIdx.x;
  const int k = P.topk, HI = P.HI;
  const IdxQuery Q = idx_query(P, pos, 0, 0, qn);
  const int V = Q.V;
  int32_t* o = out + (size_t)qn * k;
  // this thread's 8 channels of one indexer head (heads past H_I read the
  // last one) and histogram bins 4 tid .. 4 tid + 3
  uint32_t* gh = S.hist + (size_t)qn * kHistBins;
  const int hh = tid >> 4, c0 = (tid & 15) * CPT;
  u32x4 q4;
  if constexpr (IDXF == CKV_FP4) {
    // the scan's fp4 form of the query: this thread's 8 codes and their block scale
    const uint8_t* rec = S.qf4 + (size_t)(64 * qn + min(hh, HI - 1)) * kFp4RowBytes;
    q4 = (u32x4){*(const uint32_t*)(rec + 4 * (tid & 15)), (uint32_t)rec[64 + ((tid & 15) >> 2)], 0u, 0u};
  } else {
    q4 = *(const u32x4*)((const uint16_t*)qI + ((size_t)qn * HI + min(hh, HI - 1)) * DI + c0);
  }
  const u32x4 h4 = *(const u32x4*)(gh + 4 * tid);
  const float wv = wt[(size_t)qn * HI + min(hh, HI - 1)];
  // the compressor; the keys are issued after its own loads, so its waits
  // for them do not wait for the keys (no store is issued before those
  // waits: with loads and stores both in flight, every wait is a wait for all)
  uint32_t kr[kSelKPT];
  // (the query and the histogram, the first loads issued, are parked in LDS
  // once the keys are on their way: registers are short while the compressor
  // holds its window)
  const int st = compress_c4a_seq<KVF, IDXF, ACTF, NL>(P, w, cc, u, pos, proj, kProjSlices, B, qn, red, rtab, idx_row, [&] {
    sel_load_keys(keys + (size_t)qn * P.cap, P.cap, tid, kr);
    *(u32x4*)(h_lds + 4 * tid) = h4;
    *(u32x4*)(q_lds + 4 * tid) = q4;
  });
  // the histogram is left zero for the next call (its load has completed)
  *(u32x4*)(gh + 4 * tid) = (u32x4){0u, 0u, 0u, 0u};
  if (st < 0 || V <= k) {   // bad position (V = 0), or every visible row is taken
    for (int j = tid; j < k; j += 1024) o[j] = j < V ? j : -1;
    advance_tokens(cc, qn, Q.p, st);
    return;
  }
  lds_barrier();   // idx_row complete
  const u32x4 h4s = *(const u32x4*)(h_lds + 4 * tid);
  uint32_t hv[4] = {h4s[0], h4s[1], h4s[2], h4s[3]};
  if (st == 1 && V == (Q.p + 1) / 4) {
    // score of row V - 1: query tail rotated at p, cast to the indexer
    // format, dotted with the row's stored values
    float dot = 0.f;
    if constexpr (IDXF == CKV_FP4) {
      // the query's fp4 values (left by the scan, which rotated and
      // transformed it) dotted with the row's stored values
      const u32x4 q4s = *(const u32x4*)(q_lds + 4 * tid);
      float v[8];
      fp4_decode8(q4s[0], q4s[1], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += v[i] * idx_row[c0 + i];
      dot = row16_sum(dot);
    } else {
      const int dn = DI - P.idx_rot;
      const u32x4 q4s = *(const u32x4*)(q_lds + 4 * tid);
#pragma unroll
      for (int i = 0; i < CPT / 2; ++i) {
        float a = bf16_to_f32(q4s[i] & 0xffffu), b2 = bf16_to_f32(q4s[i] >> 16);
        const int c = c0 + 2 * i;
        if (c >= dn) {   // the query's tail at p, in the compressed class's frame
          const int j = (c - dn) >> 1;
          const float x = a * rtab[128 + j] - b2 * rtab[160 + j], y = a * rtab[160 + j] + b2 * rtab[128 + j];
          a = x;
          b2 = y;
        }
        a = bf16_to_f32(f32_to_bf16(a));
        b2 = bf16_to_f32(f32_to_bf16(b2));
        dot += a * idx_row[c] + b2 * idx_row[c + 1];
      }
      dot = row16_sum(dot);
    }
    const bool relu = !(P.flags & CKV_FLAG_IDX_NO_RELU);
    if ((tid & 15) == 0) hsum[hh] = hh < HI ? wv * (relu ? fmaxf(dot, 0.f) : dot) : 0.f;
    lds_barrier();
    float sc = 0.f;   // heads past H_I hold 0
#pragma unroll
    for (int h4 = 0; h4 < 64; h4 += 4) {
      const float4 q = *(const float4*)&hsum[h4];
      sc += (q.x + q.y) + (q.z + q.w);
    }
    const uint32_t key = float_key(sc);
    const int x = V - 1;   // row t + 1024 e is key e of thread t
#pragma unroll
    for (int e = 0; e < kSelKPT; ++e)
      if (e == (x >> 10) && tid == (x & 1023)) kr[e] = key;
    const uint32_t bin = key >> 20;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (tid == (int)(bin >> 2) && i == (int)(bin & 3)) hv[i] += 1u;
  }
  topk_decode_select(P, V, kr, hv, o);
  advance_tokens(cc, qn, Q.p, st);
}

int launch_indexer(const LayerParams& P, const Cache& c, const void* qI, const float* w,
                   const int32_t* pos, int seq, int pos0, int nq, uint32_t* keys, const SelWs* sel,
                   int32_t* topk, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int vlast = (pos0 + nq) / 4;
  const int vmax = pos ? P.cap : (vlast < P.cap ? vlast : P.cap);
  // decode: the score kernel fills the workspace histogram, the chunked
  // select consumes it and leaves it (and its counters) zero
  const bool use_hist = pos && sel;
  launch_idx_score(P, c, qI, w, pos, seq, pos0, nq, keys, use_hist ? sel->hist : nullptr, stream);
  if (use_hist && P.cap <= 32768) {
    hipLaunchKernelGGL(k_topk_decode, dim3(nq), dim3(1024), 0, st, P, keys, *sel, pos, topk);
  } else if (use_hist) {
    dim3 grid((unsigned)((vmax + kSelChunk - 1) / kSelChunk), nq);
    hipLaunchKernelGGL(k_topk_classify, grid, dim3(256), 0, st, P, keys, *sel, pos);
    hipLaunchKernelGGL(k_topk_finish, dim3(nq), dim3(256), 0, st, P, keys, *sel, pos, topk);
  } else if (vmax <= kSelRegNT * kSelRegKPT)
    hipLaunchKernelGGL((k_topk_select_reg<kSelRegKPT, kSelRegNT>), dim3(nq), dim3(kSelRegNT), 0, st, P, keys, pos,
                       pos0, topk);
  else if (vmax <= 32768)
    hipLaunchKernelGGL((k_topk_select_reg<32, 1024>), dim3(nq), dim3(1024), 0, st, P, keys, pos, pos0, topk);
  else
    hipLaunchKernelGGL(k_topk_select, dim3(nq), dim3(1024), 0, st, P, keys, pos, pos0, topk);
  return (int)hipGetLastError();
}

bool step_fusable(const LayerParams& P, int B) {
  return P.ratio == 4 && (P.lanes == 1 || P.lanes == 2) && (P.idx_fmt == CKV_BF16 || P.idx_fmt == CKV_FP4) &&
         P.DI == 128 &&
         P.HI <= 64 &&
         P.cap <= 32768 &&
         P.idx_rot == P.n_rot && P.n_rot == 64 &&
         P.act_fmt == CKV_BF16 && P.w_fmt == CKV_BF16 && B <= 64 && P.d <= 512;
}

int launch_step_scan_select(const LayerParams& P, const Weights& w, const Cache& c, const void* x,
                            const void* u, const void* qI, const float* wt, const int32_t* pos, int B,
                            float* proj, uint32_t* keys, const SelWs& sel, int32_t* topk, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const WCat wc = make_wcat(P, w);
  const int nproj = (P.ncol / 16) * ((B + 15) / 16) * kProjSlices;
  // two-lane layers have twice the projection blocks: their scan blocks take
  // one row group more, so that every block is resident from the start
  constexpr int kTwoLaneGroups = kStepGroups + 1;
  const bool wide = P.lanes == 2;
  const bool fp4 = P.idx_fmt == CKV_FP4;
  const int RB = 256 * (wide ? kTwoLaneGroups : fp4 ? kFp4StepGroups : kStepGroups);
  const int nrb = (P.cap + RB - 1) / RB;
  const int MT = (P.HI + 15) / 16;
  dim3 grid(nproj + nrb * B);
#define CKV_SS_NG(MTV, IF, NGV)                                                                                  \
  if (P.blocks)                                                                                                   \
    launch_score((k_step_scan<MTV, CKV_BF16, IF, true, NGV>), grid, dim3(256), st, P, (const void*)c.idx, qI, wt, \
                 pos, keys, sel.hist, (const uint16_t*)x, B, wc, proj, nproj, nrb, sel.qf4);                      \
  else                                                                                                            \
    launch_score((k_step_scan<MTV, CKV_BF16, IF, false, NGV>), grid, dim3(256), st, P, (const void*)c.idx, qI,    \
                 wt, pos, keys, sel.hist, (const uint16_t*)x, B, wc, proj, nproj, nrb, sel.qf4)
#define CKV_SS(MTV, IF)                                              \
  if (wide) CKV_SS_NG(MTV, IF, kTwoLaneGroups);                       \
  else CKV_SS_NG(MTV, IF, (IF == CKV_FP4 ? kFp4StepGroups : kStepGroups))
#define CKV_SS_MT(IF)      \
  if (MT == 1) CKV_SS(1, IF); \
  else if (MT == 2) CKV_SS(2, IF); \
  else if (MT == 3) CKV_SS(3, IF); \
  else CKV_SS(4, IF)
  if (fp4) CKV_SS_MT(CKV_FP4);
  else CKV_SS_MT(CKV_BF16);
#undef CKV_SS_MT
#undef CKV_SS
#undef CKV_SS_NG
#define CKV_SEL(KF, IF)                                                                                         \
  if (P.lanes == 2)                                                                                              \
    hipLaunchKernelGGL((k_step_select<KF, IF, CKV_BF16, 2>), dim3(B), dim3(1024), 0, st, P, w, c, u, pos, proj, B, \
                       qI, wt, keys, sel, topk);                                                                 \
  else                                                                                                           \
    hipLaunchKernelGGL((k_step_select<KF, IF, CKV_BF16>), dim3(B), dim3(1024), 0, st, P, w, c, u, pos, proj, B, qI, \
                       wt, keys, sel, topk)
  if (P.kv_fmt == CKV_E4M3) {
    if (fp4) CKV_SEL(CKV_E4M3, CKV_FP4);
    else CKV_SEL(CKV_E4M3, CKV_BF16);
  } else if (P.kv_fmt == CKV_BF16) {
    if (fp4) CKV_SEL(CKV_BF16, CKV_FP4);
    else CKV_SEL(CKV_BF16, CKV_BF16);
  } else {
    if (fp4) CKV_SEL(CKV_F32, CKV_FP4);
    else CKV_SEL(CKV_F32, CKV_BF16);
  }
#undef CKV_SEL
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
  if (P.idx_fmt == CKV_FP4) {   // validated: D_I 128, H_I <= 64, bf16 queries
    const uint8_t* ix = (const uint8_t*)c.idx;
    const int MT = (P.HI + 15) / 16;
    constexpr int RB = 256 * kFp4Groups;
    dim3 mgrid((unsigned)(vmax > 0 ? (vmax + RB - 1) / RB : 1), nq);
#define CKV_F4P(MTV, PG)                                                                                          \
  if (hist)                                                                                                       \
    launch_score(k_idx_score_fp4<MTV, true, PG>, mgrid, dim3(256), st, P, ix, qI, w, pos, seq, pos0, keys, hist); \
  else                                                                                                            \
    launch_score(k_idx_score_fp4<MTV, false, PG>, mgrid, dim3(256), st, P, ix, qI, w, pos, seq, pos0, keys, hist)
#define CKV_F4(MTV)         \
  do {                      \
    if (P.blocks) {         \
      CKV_F4P(MTV, true);   \
    } else {                \
      CKV_F4P(MTV, false);  \
    }                       \
  } while (0)
    if (MT == 1) CKV_F4(1);
    else if (MT == 2) CKV_F4(2);
    else if (MT == 3) CKV_F4(3);
    else CKV_F4(4);
#undef CKV_F4
#undef CKV_F4P
  } else if (mf && !pos && !hist && P.act_fmt == CKV_BF16) {
    const uint16_t* ix = (const uint16_t*)c.idx;
    const int MT = (P.HI + 15) / 16;
    constexpr int RUN = kPfRows * kPfTiles;
    dim3 pgrid((unsigned)(vmax > 0 ? (vmax + RUN - 1) / RUN : 1), (unsigned)((nq + kPfQ - 1) / kPfQ));
#define CKV_PF(MTV)                                                                                              \
  if (P.blocks)                                                                                                   \
    launch_score(k_idx_score_prefill<MTV, true>, pgrid, dim3(64 * kPfQ), st, P, ix, (const uint16_t*)qI, w, seq,  \
                 pos0, nq, keys);                                                                                 \
  else                                                                                                            \
    launch_score(k_idx_score_prefill<MTV>, pgrid, dim3(64 * kPfQ), st, P, ix, (const uint16_t*)qI, w, seq, pos0, \
                 nq, keys)
    if (MT == 1) CKV_PF(1);
    else if (MT == 2) CKV_PF(2);
    else if (MT == 3) CKV_PF(3);
    else CKV_PF(4);
#undef CKV_PF
  } else if (mf) {
    const uint16_t* ix = (const uint16_t*)c.idx;
    const int MT = (P.HI + 15) / 16;
    constexpr int RB = 256 * kScoreGroups;
    dim3 mgrid((unsigned)(vmax > 0 ? (vmax + RB - 1) / RB : 1), nq);
#define CKV_ISP(MTV, QF, PG)                                                                                  \
  if (hist)                                                                                                   \
    launch_score(k_idx_score_mfma<MTV, 4, QF, true, PG>, mgrid, dim3(256), st, P, ix, qI, w, pos, seq, pos0, \
                 keys, hist);                                                                                 \
  else                                                                                                        \
    launch_score(k_idx_score_mfma<MTV, 4, QF, false, PG>, mgrid, dim3(256), st, P, ix, qI, w, pos, seq, pos0, \
                 keys, hist)
#define CKV_IS(MTV, QF)         \
  do {                          \
    if (P.blocks) {             \
      CKV_ISP(MTV, QF, true);   \
    } else {                    \
      CKV_ISP(MTV, QF, false);  \
    }                           \
  } while (0)
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
#undef CKV_ISP
  } else {
#define CKV_IV(IF, QF) \
  launch_score(k_idx_score_vec<IF, QF>, grid, dim3(256), st, P, c.idx, qI, w, pos, seq, pos0, keys, hist)
    if (P.idx_fmt == CKV_F32 && P.act_fmt == CKV_F32) CKV_IV(CKV_F32, CKV_F32);
    else if (P.idx_fmt == CKV_F32) CKV_IV(CKV_F32, CKV_BF16);
    else if (P.act_fmt == CKV_F32) CKV_IV(CKV_BF16, CKV_F32);
    else CKV_IV(CKV_BF16, CKV_BF16);
#undef CKV_IV
  }
  return (int)hipGetLastError();
}

}  // namespace ckv
