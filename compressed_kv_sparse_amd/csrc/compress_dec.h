// Device code of the per-token compressor shared by the decode kernels:
// row helpers, the online pooling accumulator and the per-sequence decode
// body (state store, window pooling, RMSNorm, tail RoPE and cache insertion,
// "ds4.c を読み解く (#3)" sections 4-5; fused the way the vLLM DeepSeek V4
// page fuses compressor + RMSNorm + RoPE + cache insertion).
#pragma once

#include <type_traits>

#include "ckv_device.h"
#include "idx_fp4.h"

namespace ckv {

// ------------------------------------------------------------ row helpers

// Rotate the last `nrot` entries of z[0..width) (LDS) at position `pos`, in
// the compressed class's frame (`comp`) or the raw rows' frame.
// Caller synchronises before and after.
__device__ __forceinline__ void rope_lds(const LayerParams& P, float* z, int width, int nrot, double pos,
                                         bool comp) {
  const int dn = width - nrot;
  for (int j = threadIdx.x; j < nrot / 2; j += blockDim.x) {
    float c, s;
    if (comp) rope_cs_c(P, j, pos, &c, &s);
    else rope_cs(P, j, pos, &c, &s);
    const float a = z[dn + 2 * j], b = z[dn + 2 * j + 1];
    z[dn + 2 * j] = a * c - b * s;
    z[dn + 2 * j + 1] = a * s + b * c;
  }
}

// 1 / rms of a row whose squares sum to ss over `width` channels, or 1 under
// CKV_FLAG_SKIP_NORM (the gamma weight is then 1 too: norm_gamma).
__device__ __forceinline__ float norm_inv(const LayerParams& P, float ss, int width) {
  return (P.flags & CKV_FLAG_SKIP_NORM) ? 1.f : 1.0f / sqrtf(ss / (float)width + P.eps);
}
__device__ __forceinline__ float norm_gamma(const LayerParams& P, float g) {
  return (P.flags & CKV_FLAG_SKIP_NORM) ? 1.f : g;
}
__device__ __forceinline__ float2 norm_gamma(const LayerParams& P, float2 g) {
  return (P.flags & CKV_FLAG_SKIP_NORM) ? make_float2(1.f, 1.f) : g;
}

// z <- gamma * z / sqrt(mean(z^2) + eps), channels owned as c = tid + k*blockDim.
__device__ __forceinline__ void rmsnorm_lds(const LayerParams& P, float* z, int width, const float* gamma,
                                            float* red) {
  float ss = 0.f;
  for (int c = threadIdx.x; c < width; c += blockDim.x) ss += z[c] * z[c];
  ss = block_sum(ss, red);
  const float inv = norm_inv(P, ss, width);
  for (int c = threadIdx.x; c < width; c += blockDim.x) z[c] = norm_gamma(P, gamma[c]) * (z[c] * inv);
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
  // N entries at once: one rescale to the round's new maximum, then N
  // weights exp(e - m) by the hardware exp2, no branch
  template <int N>
  __device__ __forceinline__ void add_round(const float (&e)[N], const float (&kv)[N]) {
    constexpr float kL2e = 1.4426950408889634f;
    float mr = e[0];
#pragma unroll
    for (int i = 1; i < N; ++i) mr = fmaxf(mr, e[i]);
    const float nm = fmaxf(m, mr);
    const float f = __builtin_amdgcn_exp2f((m - nm) * kL2e);   // m = -inf: 0, and s, acc are 0
    s *= f;
    acc *= f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float w = __builtin_amdgcn_exp2f((e[i] - nm) * kL2e);
      s += w;
      acc = fmaf(w, kv[i], acc);
    }
    m = nm;
  }
  __device__ __forceinline__ float value() const { return s > 0.f ? acc / s : 0.f; }
};

// ------------------------------------------------------------ decode

template <int F>
__device__ __forceinline__ float2 load2(const void* p, long i) {  // i even
  if constexpr (F == CKV_F32) return *(const float2*)((const float*)p + i);
  else {
    const uint32_t w = *(const uint32_t*)((const uint16_t*)p + i);
    return make_float2(bf16_to_f32(w & 0xffffu), bf16_to_f32(w >> 16));
  }
}

__device__ __forceinline__ float2 ld2(const float* p) { return *(const float2*)p; }

namespace cmp {
// block-wide sum and max (every thread returns the totals); red: 2 * 32 floats
__device__ __forceinline__ float2 block_sum_max(float s, float m, float* red) {
  s = wave_sum(s);
  m = wave_max(m);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  lds_barrier();
  if ((threadIdx.x & 63) == 0) {
    red[w] = s;
    red[32 + w] = m;
  }
  lds_barrier();
  float ts = 0.f, tm = 0.f;
  for (int i = 0; i < nw; ++i) {
    ts += red[i];
    tm = fmaxf(tm, red[32 + i]);
  }
  return make_float2(ts, tm);
}
}  // namespace cmp

// Store one row from per-thread channel pairs (c, c+1) in format KVF.  Every
// thread of the block calls (the E4M3 row scale is a block-wide max).
template <int KVF>
__device__ __forceinline__ void store_row2(uint8_t* dst, float2 z, int c, bool act, int d, int n_rot,
                                           float* red) {
  if constexpr (KVF == CKV_F32) {
    if (act) *(float2*)(dst + 4 * c) = z;
  } else if constexpr (KVF == CKV_BF16) {
    if (act) *(uint32_t*)(dst + 2 * c) = pack_bf16x2(z.x, z.y);
  } else {
    const int dn = d - n_rot;
    const float amax = cmp::block_sum_max(0.f, act && c < dn ? fmaxf(fabsf(z.x), fabsf(z.y)) : 0.f, red).y;
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    if (act) {
      if (c < dn) *(uint16_t*)(dst + c) = (uint16_t)(f32_to_e4m3(z.x / s) | (f32_to_e4m3(z.y / s) << 8));
      else *(uint32_t*)(dst + dn + 2 * (c - dn)) = pack_bf16x2(z.x, z.y);
    }
    if (threadIdx.x == 0) *(float*)(dst + dn + 2 * n_rot) = s;
  }
}

// Rotate the pair (c, c+1) if it lies in the last n_rot channels of `width`.
__device__ __forceinline__ float2 rope2(const LayerParams& P, float2 z, int c, int width, int nrot, double pos) {
  const int dn = width - nrot;
  if (c < dn) return z;
  float cs, sn;
  rope_cs(P, (c - dn) >> 1, pos, &cs, &sn);
  return make_float2(z.x * cs - z.y * sn, z.x * sn + z.y * cs);
}
// The same with cos / sin of pair j taken from tables cs[j], sn[j] (LDS).
__device__ __forceinline__ float2 rope2t(float2 z, int c, int width, int nrot, const float* cs, const float* sn) {
  const int dn = width - nrot;
  if (c < dn) return z;
  const int j = (c - dn) >> 1;
  return make_float2(z.x * cs[j] - z.y * sn[j], z.x * sn[j] + z.y * cs[j]);
}

// Sequence check of a decode step (cache->n_tokens): the token at p is stored
// when p is the sequence's next position or its last one (a re-run of that
// step).  `nt` is n_tokens[b]; every thread has read it before the barrier
// after which thread 0 writes p + 1 (the check itself decides a return that
// precedes that barrier, or pin_tokens holds the value there).
__device__ __forceinline__ int seq_tokens(const Cache& cc, int b, int p) {
  return cc.n_tokens ? cc.n_tokens[b] : p;
}
__device__ __forceinline__ void pin_tokens(int nt) { asm volatile("" : : "s"(nt) : "memory"); }
// After a body returned st >= 0 (the token was stored): the sequence's count
// becomes p + 1.  Called by the kernel at its end (a store placed before the
// body's waits would make them wait for it too); every thread read the count
// before the body's barriers.
__device__ __forceinline__ void advance_tokens(const Cache& cc, int b, int p, int st) {
  if (st >= 0 && threadIdx.x == 0 && cc.n_tokens) cc.n_tokens[b] = p + 1;
}
__device__ __forceinline__ bool seq_ok(const Cache& cc, int p, int nt) {
  return !cc.n_tokens || p == nt || p == nt - 1;
}

// Pool channels (c, c+1) of row i over its window.  Token p's own values come
// from registers; the other W-1 tokens from the state ring.  Loads go out in
// groups of 8 slots before the group is accumulated.
__device__ __forceinline__ float2 pool2(const float* skv, const float* ssc, const float* ape, int width, int W,
                                        int r, int i, int p, float2 kcur, float2 scur, int c) {
  PoolAcc a0, a1;
  const int t0 = i * r - (W - r);
  for (int j0 = 0; j0 < W; j0 += 8) {
    float2 kv[8], sc[8], ap[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int t = t0 + j0 + jj;
      kv[jj] = sc[jj] = make_float2(0.f, 0.f);
      if (t >= 0 && t != p) {
        kv[jj] = ld2(skv + (size_t)(t % W) * width + c);
        sc[jj] = ld2(ssc + (size_t)(t % W) * width + c);
      }
      ap[jj] = ld2(ape + (size_t)(j0 + jj) * width + c);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int t = t0 + j0 + jj;
      if (t < 0) continue;
      const float2 k = t == p ? kcur : kv[jj];
      const float2 e = t == p ? scur : sc[jj];
      a0.add(e.x + ap[jj].x, k.x);
      a1.add(e.y + ap[jj].y, k.y);
    }
  }
  return make_float2(a0.value(), a1.value());
}

// Decode: one block per sequence; thread t works on the channel pair
// c = 2 (t % NP) (NP = d / 2 pairs) and, on ratio 4, on the indexer pair of
// the same index (t % NP < D_I / 2).  TPC threads share a pair: part
// t / NP pools W / TPC of the window's slots, and the parts' online-softmax
// states are merged through LDS.
//
// The window state is a ring: token t sits in slot t % W, and the row closed
// by token p = i r + r - 1 pools tokens t0 .. t0 + W - 1 with t0 = i r - (W - r),
// i.e. every slot of the ring, token t0 + j in slot (t0 + j) % W.  So the ring
// loads do not depend on p and go out together with this token's inputs; p
// only decides which window position j (and APE row) each slot takes, which
// slot is the current token (taken from registers, its ring slot still holds
// token p - W), and which positions precede token 0 (no weight).
//   c4a  (W 8,   r 4):   t0 % 8 is 0 or 4, so j = s ^ (t0 & 4)
//   c128a (W 128, r 128): t0 % 128 = 0, so j = s
// Every load is unconditional (clamped indices, values selected afterwards);
// on c128a the ring is read only on a boundary step (a block-uniform branch),
// in rounds of 8 slots per thread.  On c4a with TPC parts, part q holds slots
// q + TPC e: flipping by 4 maps that set onto itself (slot q + TPC e takes the
// APE row of local index e ^ (4 / TPC)), so its loads do not depend on p.

// The per-sequence body, called by every thread of a block of at least
// TPC * d / 2 threads (threads past that take part in the reductions only).
// Returns 1 when the token closed a row (on ratio 4 the indexer row's stored
// values are left in idx_row[0 .. D_I) when idx_row is non-NULL), 0 when it
// did not, -1 for a negative position.  red: 64 floats of LDS; mrg: the
// parts' merge area (TPC > 1): TPC * d / 2 * 6 floats, plus TPC * D_I / 2 * 6
// on c4a.  rtab: 128 floats of LDS, left holding cos (rtab[j]) and sin
// (rtab[64 + j]) of pair j at p, and at the row position i r in
// rtab[32 + j], rtab[96 + j] (n_rot = 64).  issue() is called once every load
// of the body has been issued and before any is waited for: a caller's own
// loads placed there overlap the body (the vector memory counter completes in
// issue order).  Every load of the body is issued before its first store, and
// no barrier here waits for global memory after that, so stores stay in
// flight while the body and the caller go on.
template <int KVF, int IDXF, int ACTF, int W, int TPC, int MAXS = 4, typename Issue>
__device__ __forceinline__ int compress_decode_seq(const LayerParams& P, const Weights& w, const Cache& cc,
                                                   const void* __restrict__ u, const int32_t* __restrict__ pos,
                                                   const float* __restrict__ proj, int splits, int B, int b,
                                                   float* red, float* mrg, float* idx_row, float* rtab,
                                                   Issue&& issue) {
  static_assert(IDXF != CKV_FP4, "fp4 indexer rows are written by compress_c4a_seq");
  constexpr int SPT = W / TPC;                 // slots per thread
  constexpr int RND = SPT < 8 ? SPT : 8;       // slots per load round
  constexpr int r = W == 8 ? 4 : 128;
  const int d = P.d, DI = P.DI, NP = d / 2;
  const int tid = threadIdx.x;
  const int pair = tid % NP, part = min(tid / NP, TPC);
  const int c = 2 * pair;
  const bool ilane = W == 8 && pair < DI / 2;  // indexer channels (ratio 4)
  const int ci = 2 * min(pair, max(DI / 2 - 1, 0));

  // this token's inputs and, on c4a, the whole ring: one round of loads
  const int p = pos[b];
  const int nt = seq_tokens(cc, b, p);
  const float2 uu = load2<ACTF>(u, (long)b * d + c);
  // projection partials (at most MAXS K slices), summed in slice order
  float2 ka = make_float2(0.f, 0.f), sa = ka, kia = ka, sia = ka;
  {
    float2 pk[MAXS], psg[MAXS], pki[MAXS], psi[MAXS];
#pragma unroll
    for (int q = 0; q < MAXS; ++q) {
      const float* pj = proj + ((size_t)min(q, splits - 1) * B + b) * P.ncol;
      pk[q] = ld2(pj + c);
      psg[q] = ld2(pj + d + c);
      if (W == 8) {
        pki[q] = ld2(pj + 2 * d + ci);
        psi[q] = ld2(pj + 2 * d + DI + ci);
      }
    }
#pragma unroll
    for (int q = 0; q < MAXS; ++q) {
      if (q < splits) {
        ka.x += pk[q].x; ka.y += pk[q].y;
        sa.x += psg[q].x; sa.y += psg[q].y;
        if (W == 8) {
          kia.x += pki[q].x; kia.y += pki[q].y;
          sia.x += psi[q].x; sia.y += psi[q].y;
        }
      }
    }
  }
  const float* skv = cc.st_kv + (size_t)b * W * d;
  const float* ssc = cc.st_sc + (size_t)b * W * d;
  static_assert(W != 8 || (TPC == 1 || TPC == 2 || TPC == 4), "c4a parts must divide the flip");
  constexpr int S8 = W == 8 ? 8 / TPC : 1;   // c4a ring slots per thread
  const int q8 = min(part, TPC - 1);         // threads past the parts mirror the last one's loads
  float2 rk[S8], rs[S8], ap[S8], irk[S8], irs[S8], iap[S8];
  float2 gm = make_float2(1.f, 1.f), gmi = gm;
  if (W == 8) {
    const float* ikv = cc.ist_kv + (size_t)b * 8 * DI;
    const float* isc = cc.ist_sc + (size_t)b * 8 * DI;
#pragma unroll
    for (int e = 0; e < S8; ++e) {
      const int sl = q8 + TPC * e;
      rk[e] = ld2(skv + sl * d + c);
      rs[e] = ld2(ssc + sl * d + c);
      ap[e] = ld2(w.ape + sl * d + c);
      irk[e] = ld2(ikv + sl * DI + ci);
      irs[e] = ld2(isc + sl * DI + ci);
      iap[e] = ld2(w.idx_ape + sl * DI + ci);
    }
    gmi = norm_gamma(P, ld2(w.idx_gamma + ci));
  }
  gm = norm_gamma(P, ld2(w.gamma + c));
  // compiler fences: the loads above stay above, the caller's stay in between
  asm volatile("" ::: "memory");
  issue();
  asm volatile("" ::: "memory");

  const bool emit = (p + 1) % r == 0;
  const int i = (p + 1) / r - 1;
  const bool pool = emit && i < P.cap;
  const int t0 = i * r - (W - r);
  const int cur = p & (W - 1);

  // ---- pooling: online softmax per channel over this thread's slots
  PoolAcc a0, a1, b0, b1;
  if (pool) {
    if (W == 8) {
      // the flip (t0 & 4) is block-uniform; both forms are instantiated with
      // compile-time slot indices so the register arrays stay in registers
      auto pool8 = [&](auto flip) {
        constexpr int F = decltype(flip)::value;
        constexpr int FE = F / TPC;   // the flip in local slot indices
#pragma unroll
        for (int e = 0; e < S8; ++e) {
          const int sl = q8 + TPC * e;
          const int j = sl ^ F;
          const bool valid = t0 + j >= 0 && part < TPC;
          const bool self = sl == cur;
          const float2 kk = self ? ka : rk[e], ss = self ? sa : rs[e];
          const float2 ikk = self ? kia : irk[e], iss = self ? sia : irs[e];
          if (valid) {
            a0.add(ss.x + ap[e ^ FE].x, kk.x);
            a1.add(ss.y + ap[e ^ FE].y, kk.y);
            b0.add(iss.x + iap[e ^ FE].x, ikk.x);
            b1.add(iss.y + iap[e ^ FE].y, ikk.y);
          }
        }
      };
      if (t0 & 4) pool8(std::integral_constant<int, 4>{});
      else pool8(std::integral_constant<int, 0>{});
    } else {
      // c128a: j = slot; the window starts at t0 = 128 i >= 0.  The thread's
      // SPT slots in rounds of RND, the next round's loads issued before the
      // current round is pooled (parts past TPC re-read the last part's slots
      // and are dropped by the merge)
      constexpr int NR = SPT / RND;
      const int sb = min(part, TPC - 1) * SPT;
      float2 kk[2][RND], ss[2][RND], aa[2][RND];
      auto load_round = [&](int rr) {
#pragma unroll
        for (int e = 0; e < RND; ++e) {
          const int sl = sb + rr * RND + e;
          kk[rr & 1][e] = ld2(skv + sl * d + c);
          ss[rr & 1][e] = ld2(ssc + sl * d + c);
          aa[rr & 1][e] = ld2(w.ape + sl * d + c);
        }
      };
      load_round(0);
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        if (rr + 1 < NR) load_round(rr + 1);
        float e0[RND], e1[RND], v0[RND], v1[RND];
#pragma unroll
        for (int e = 0; e < RND; ++e) {
          const int sl = sb + rr * RND + e;
          const bool self = sl == cur;
          const float2 k2 = self ? ka : kk[rr & 1][e], s2 = self ? sa : ss[rr & 1][e];
          e0[e] = s2.x + aa[rr & 1][e].x;
          e1[e] = s2.y + aa[rr & 1][e].y;
          v0[e] = k2.x;
          v1[e] = k2.y;
        }
        a0.add_round(e0, v0);
        a1.add_round(e1, v1);
      }
    }
  }
  float2 y = make_float2(a0.value(), a1.value());
  float2 yi = make_float2(b0.value(), b1.value());
  if (TPC > 1) {
    // merge the parts' (max, sum, acc) per channel; part 0 ends with the row.
    // mrg: attention pairs [TPC][NP][6], then (c4a) indexer pairs [TPC][DI/2][6]
    float* mi = mrg + TPC * NP * 6;
    if (pool && part < TPC) {
      float* mm = mrg + (part * NP + pair) * 6;
      mm[0] = a0.m; mm[1] = a0.s; mm[2] = a0.acc;
      mm[3] = a1.m; mm[4] = a1.s; mm[5] = a1.acc;
      if (W == 8 && ilane) {
        float* mb = mi + (part * (DI / 2) + pair) * 6;
        mb[0] = b0.m; mb[1] = b0.s; mb[2] = b0.acc;
        mb[3] = b1.m; mb[4] = b1.s; mb[5] = b1.acc;
      }
    }
    __syncthreads();
    if (pool && part == 0) {
      auto merge = [](PoolAcc& x, float m, float s, float acc) {
        if (s == 0.f) return;
        if (x.s == 0.f) { x.m = m; x.s = s; x.acc = acc; return; }
        const float mx = fmaxf(x.m, m);
        const float fa = expf(x.m - mx), fb = expf(m - mx);
        x.s = x.s * fa + s * fb;
        x.acc = x.acc * fa + acc * fb;
        x.m = mx;
      };
      PoolAcc t0a = a0, t1a = a1;
      for (int q = 1; q < TPC; ++q) {
        const float* mm = mrg + (q * NP + pair) * 6;
        merge(t0a, mm[0], mm[1], mm[2]);
        merge(t1a, mm[3], mm[4], mm[5]);
      }
      y = make_float2(t0a.value(), t1a.value());
      if (W == 8 && ilane) {
        PoolAcc t0b = b0, t1b = b1;
        for (int q = 1; q < TPC; ++q) {
          const float* mb = mi + (q * (DI / 2) + pair) * 6;
          merge(t0b, mb[0], mb[1], mb[2]);
          merge(t1b, mb[3], mb[4], mb[5]);
        }
        yi = make_float2(t0b.value(), t1b.value());
      }
    }
  }
  const bool own = part == 0;   // the thread that stores this pair
  // A negative position stores nothing.  The check sits here, after the
  // pooling (whose arithmetic is harmless for p < 0), not before the loads:
  // a branch there lets the compiler sink loads below it, and the wait for a
  // late load is a wait for everything issued before it.
  if (p < 0 || !seq_ok(cc, p, nt)) {
    if (tid == 0 && cc.status) atomicOr(&cc.status[b], p < 0 ? CKV_STATUS_BAD_POS : CKV_STATUS_SEQUENCE);
    return -1;
  }
  // RoPE tables: wave 0 computes pair tid % 32 at p in the raw frame (lanes
  // 0-31) and at i r in the compressed frame (lanes 32-63); read after the
  // barrier below
  if (__builtin_amdgcn_readfirstlane(tid >> 6) == 0) {
    // theta of pair tid % 32 selected from scalar loads of the whole tables (a
    // per-lane load would be one more vector load to wait for)
    double theta = 0.0;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) theta = (tid & 31) == jj ? (tid < 32 ? P.theta[jj] : P.theta_c[jj]) : theta;
    float cs, sn;
    rope_cs_theta(theta, tid < 32 ? (double)p : (double)((p + 1) / r * r - r), &cs, &sn);
    if (tid < 64) {
      rtab[tid] = cs;
      rtab[64 + tid] = sn;
    }
  }
  lds_barrier();                // rtab complete

  // ---- raw sliding-window row: u rotated at p into slot p % swa
  {
    const float2 z = rope2t(uu, c, d, P.n_rot, rtab, rtab + 64);
    store_row2<KVF>(cc.raw + ((size_t)b * P.swa + (p & (P.swa - 1))) * P.row_bytes, z, c, own, d, P.n_rot, red);
  }
  // ---- this token's projections -> state slot p % W
  if (own) {
    const size_t o = ((size_t)b * W + cur) * d + c;
    *(float2*)(cc.st_kv + o) = ka;
    *(float2*)(cc.st_sc + o) = sa;
  }
  if (W == 8 && own && ilane) {
    const size_t o = ((size_t)b * 8 + cur) * DI + c;
    *(float2*)(cc.ist_kv + o) = kia;
    *(float2*)(cc.ist_sc + o) = sia;
  }
  // (the status atomic sits after every load of the body has been waited for:
  // a memory operation under a branch before those waits makes the compiler
  // wait for every outstanding load instead of the ones it needs)
  if (emit && i >= P.cap && tid == 0 && cc.status) atomicOr(&cc.status[b], CKV_STATUS_CAPACITY);
  if (!pool) return 0;

  // ---- attention lane: RMSNorm, tail RoPE at i r, store row i
  {
    const float ss = cmp::block_sum_max(own ? y.x * y.x + y.y * y.y : 0.f, 0.f, red).x;
    const float inv = norm_inv(P, ss, d);
    const float2 z = rope2t(make_float2(gm.x * (y.x * inv), gm.y * (y.y * inv)), c, d, P.n_rot, rtab + 32, rtab + 96);
    const long long slot = row_slot_wr(P, tid == 0 ? cc.status : nullptr, b, i);
    if (slot >= 0) store_row2<KVF>(cc.comp + slot * P.row_bytes, z, c, own, d, P.n_rot, red);
  }
  if (W == 8) {  // indexer lane: its own compressor of the same form
    const float ss = cmp::block_sum_max(own && ilane ? yi.x * yi.x + yi.y * yi.y : 0.f, 0.f, red).x;
    const float inv = norm_inv(P, ss, DI);
    if (own && ilane) {
      const float2 z = rope2t(make_float2(gmi.x * (yi.x * inv), gmi.y * (yi.y * inv)), c, DI, P.idx_rot, rtab + 32,
                              rtab + 96);
      const long long slot = row_slot_wr(P, c == 0 ? cc.status : nullptr, b, i);
      uint8_t* dst = (uint8_t*)cc.idx + (slot < 0 ? 0 : slot) * P.idx_row_bytes;
      if (slot < 0) {
        // (a block-table entry outside the pool: the row is not stored)
      } else if (IDXF == CKV_F32) {
        *(float2*)(dst + 4 * c) = z;
        if (idx_row) {
          idx_row[c] = z.x;
          idx_row[c + 1] = z.y;
        }
      } else {
        const uint32_t pz = pack_bf16x2(z.x, z.y);
        *(uint32_t*)(dst + 2 * c) = pz;
        if (idx_row) {
          idx_row[c] = bf16_to_f32(pz & 0xffffu);
          idx_row[c + 1] = bf16_to_f32(pz >> 16);
        }
      }
    }
  }
  return 1;
}

// ------------------------------------------------------------ c4a decode

// One stored-row channel c in format KVF (E4M3 codes are z / s with s the row
// scale, written separately; the RoPE tail stays bf16).
template <int KVF>
__device__ __forceinline__ void put_chan(uint8_t* dst, float z, int c, int dn, float s) {
  if constexpr (KVF == CKV_F32) {
    ((float*)dst)[c] = z;
  } else if constexpr (KVF == CKV_BF16) {
    ((uint16_t*)dst)[c] = (uint16_t)f32_to_bf16(z);
  } else {
    if (c < dn) dst[c] = (uint8_t)f32_to_e4m3(z / s);
    else ((uint16_t*)(dst + dn))[c - dn] = (uint16_t)f32_to_bf16(z);
  }
}

// Rotate channel c of a row whose pairs (2j, 2j+1) sit in adjacent lanes, if c
// is one of the last nrot channels; cs / sn: tables of pair j (LDS).  Every
// lane calls (the partner value comes from lane ^ 1).
__device__ __forceinline__ float rope1t(float v, int c, int width, int nrot, const float* cs, const float* sn) {
  const float o = dpp_f32<0xb1>(0.f, v);   // lane ^ 1
  const int dn = width - nrot;
  if (c < dn) return v;
  const int j = (c - dn) >> 1;
  return (c & 1) ? fmaf(o, sn[j], v * cs[j]) : fmaf(-o, sn[j], v * cs[j]);
}

// Softmax pooling of one channel over the 8 window positions of row i
// (window token t0 + j sits in ring slot (t0 + j) % 8 = j ^ F, F = t0 & 4),
// two passes: the maximum of the valid scores, then exp-weighted sums.  The
// current token's slot is taken from (kcur, scur).  Window positions 0-3 take
// the ring values (rkA, rsA), positions 4-7 (rkB, rsB): the same arrays for a
// one-lane compressor, lane A and lane B for a two-lane one (the current
// token, position 7, is lane B).
template <int F>
__device__ __forceinline__ float pool_c4a(const float (&rkA)[8], const float (&rsA)[8], const float (&rkB)[8],
                                          const float (&rsB)[8], const float (&ap)[8], float kcur, float scur,
                                          int t0, int cur) {
  float e[8];
  float mx = -INFINITY;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) {
    const bool valid = t0 + (sl ^ F) >= 0;
    const float rs = (sl ^ F) < 4 ? rsA[sl] : rsB[sl];
    e[sl] = valid ? (sl == cur ? scur : rs) + ap[sl ^ F] : -INFINITY;
    mx = fmaxf(mx, e[sl]);
  }
  constexpr float kLog2e = 1.4426950408889634f;
  float sw = 0.f, acc = 0.f;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) {
    const float wgt = __builtin_amdgcn_exp2f((e[sl] - mx) * kLog2e);
    sw += wgt;
    const float rk = (sl ^ F) < 4 ? rkA[sl] : rkB[sl];
    acc = fmaf(wgt, sl == cur ? kcur : rk, acc);
  }
  return acc / sw;
}

// The c4a per-sequence body (window 8, stride 4, with the indexer lane),
// for a block of at least d + D_I threads.  Thread t < d owns channel t of
// the attention row (and of the raw row); thread d + t' owns channel t' of
// the indexer row; the rest only join the barriers.  Every thread issues the
// same loads (idle threads at clamped addresses), and the work of idle waves
// is skipped by wave-uniform branches.  One block reduction serves the
// RMSNorm of both rows and the E4M3 scales of the raw and compressed rows:
// the compressed row is (gamma y) * inv with inv > 0 a constant, so its
// largest magnitude is inv times the largest |gamma y| (rounding is
// monotonic).
// Returns 1 when the token closed a row (idx_row, when non-NULL, receives the
// indexer row's stored values), 0 when not, -1 for a negative position.
// red: 64 floats of LDS (16-byte aligned); rtab: 128 floats of LDS (RoPE cos
// and sin at p and at the row position, as for compress_decode_seq); issue()
// as there.
// rtab: 192 floats (cos / sin of pair j at p raw, at 4 i compressed, at p
// compressed: [j], [64 + j]; [32 + j], [96 + j]; [128 + j], [160 + j]).
// NL: compressor lanes (2: CKV_FLAG_TWO_LANE, each token's projections and
// ring slot hold lane A then lane B, ape row s holds lane A's slot s then lane
// B's slot 4 + s).
template <int KVF, int IDXF, int ACTF, int NL = 1, typename Issue>
__device__ __forceinline__ int compress_c4a_seq(const LayerParams& P, const Weights& w, const Cache& cc,
                                                const void* __restrict__ u, const int32_t* __restrict__ pos,
                                                const float* __restrict__ proj, int splits, int B, int b,
                                                float* red, float* rtab, float* idx_row, Issue&& issue) {
  const int d = P.d, DI = P.DI;
  const int dn = d - P.n_rot;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nact = (d + DI + 63) / 64;   // waves holding channels
  const bool roleA = tid < d, roleI = !roleA && tid < d + DI;
  const int col = roleA ? tid : min(tid - d, DI - 1);
  const int width = roleA ? d : DI;
  const int sw = NL * width;   // ring slot (and APE row) stride
  float* const skv = roleA ? cc.st_kv + (size_t)b * 8 * NL * d : cc.ist_kv + (size_t)b * 8 * NL * DI;
  float* const ssc = roleA ? cc.st_sc + (size_t)b * 8 * NL * d : cc.ist_sc + (size_t)b * 8 * NL * DI;
  const float* ape = (roleA ? w.ape : w.idx_ape) + col;
  const float* pj = proj + (size_t)b * P.ncol;
  const int kb = roleA ? 0 : 2 * NL * d;   // this compressor's kappa columns; sigma from kb + NL * width

  // one round of loads: this token's projections (the sum of up to 4 K-slice
  // partials, in slice order; slices past `splits` re-read the last and
  // count zero) and raw input, the ring, the APE rows and the RMSNorm gain
  const int p = pos[b];
  const int nt = seq_tokens(cc, b, p);
  float ka = 0.f, sa = 0.f, kb2 = 0.f, sb2 = 0.f;   // lane A (the only lane at NL = 1), lane B
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* pq = pj + (size_t)min(q, splits - 1) * B * P.ncol;
    const float kq = pq[kb + col], sq = pq[kb + sw + col];
    ka += q < splits ? kq : 0.f;
    sa += q < splits ? sq : 0.f;
    if constexpr (NL == 2) {
      const float kq2 = pq[kb + width + col], sq2 = pq[kb + sw + width + col];
      kb2 += q < splits ? kq2 : 0.f;
      sb2 += q < splits ? sq2 : 0.f;
    }
  }
  const float uu = load_val<ACTF>(u, (long)b * d + (roleA ? col : 0));
  float rk[8], rs[8], ap[8];
  float rkB[NL == 2 ? 8 : 1], rsB[NL == 2 ? 8 : 1];
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) {
    rk[sl] = skv[sl * sw + col];
    rs[sl] = ssc[sl * sw + col];
    if constexpr (NL == 2) {
      rkB[sl] = skv[sl * sw + width + col];
      rsB[sl] = ssc[sl * sw + width + col];
      ap[sl] = ape[(sl & 3) * sw + (sl < 4 ? 0 : width)];   // window position sl
    } else {
      ap[sl] = ape[sl * width];
    }
  }
  const float gm = norm_gamma(P, (roleA ? w.gamma : w.idx_gamma)[col]);
  // this lane's RoPE frequency for the tables below (wave 0: the raw frame in
  // lanes 0-31, the compressed frame in lanes 32-63; wave 1: the compressed
  // frame): a per-lane index into the kernel-argument arrays is a vector
  // load, so it is waited for here, before the caller's loads -- waited for
  // after them, the wait would cover them all
  double th_lane = wave == 0 && lane < 32 ? P.theta[lane & 31] : P.theta_c[lane & 31];
  asm volatile("" : "+v"(th_lane));
  asm volatile("" ::: "memory");
  issue();
  asm volatile("" ::: "memory");

  const bool emit = p >= 0 && (p + 1) % 4 == 0;
  const int i = (p + 1) / 4 - 1;
  const bool pool = emit && i < P.cap;
  const int t0 = 4 * i - 4, cur = p & 7;
  // RoPE tables (wave 0): pair j at p (raw frame) and at the row position
  // 4 i (compressed frame)
  if (wave == 0) {
    float cs, sn;
    rope_cs_theta(th_lane, tid < 32 ? (double)p : (double)(4 * i), &cs, &sn);
    rtab[tid] = cs;
    rtab[64 + tid] = sn;
  } else if (wave == 1 && lane < 32) {   // pair j at p in the compressed frame (the indexer query)
    float cs, sn;
    rope_cs_theta(th_lane, (double)p, &cs, &sn);
    rtab[128 + lane] = cs;
    rtab[160 + lane] = sn;
  }
  float y = 0.f;
  if (wave < nact) {
    if (pool) {
      if constexpr (NL == 2)
        y = (t0 & 4) ? pool_c4a<4>(rk, rs, rkB, rsB, ap, kb2, sb2, t0, cur)
                     : pool_c4a<0>(rk, rs, rkB, rsB, ap, kb2, sb2, t0, cur);
      else
        y = (t0 & 4) ? pool_c4a<4>(rk, rs, rk, rs, ap, ka, sa, t0, cur) : pool_c4a<0>(rk, rs, rk, rs, ap, ka, sa, t0, cur);
    }
    const float gy = gm * y;
    float v0 = roleA ? y * y : 0.f;
    float v1 = roleI ? y * y : 0.f;
    float v2 = roleA && col < dn ? fabsf(gy) : 0.f;
    float v3 = roleA && col < dn ? fabsf(uu) : 0.f;
    v0 = wave_sum(v0);
    v1 = wave_sum(v1);
    v2 = wave_max(v2);
    v3 = wave_max(v3);
    if (lane == 0) *(float4*)(red + 4 * wave) = make_float4(v0, v1, v2, v3);
  }
  pin_tokens(nt);  // read before the barrier that precedes its update
  lds_barrier();   // red, rtab
  float sA = 0.f, sI = 0.f, mA = 0.f, mU = 0.f;
  {
    float4 t[16];   // the 16 reads go out together (red holds 16 waves' entries)
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) t[w2] = *(const float4*)(red + 4 * w2);
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) {
      if (w2 < nact) {
        sA += t[w2].x;
        sI += t[w2].y;
        mA = fmaxf(mA, t[w2].z);
        mU = fmaxf(mU, t[w2].w);
      }
    }
  }
  if (p < 0 || !seq_ok(cc, p, nt)) {
    if (tid == 0 && cc.status) atomicOr(&cc.status[b], p < 0 ? CKV_STATUS_BAD_POS : CKV_STATUS_SEQUENCE);
    return -1;
  }
  if (emit && i >= P.cap && tid == 0 && cc.status) atomicOr(&cc.status[b], CKV_STATUS_CAPACITY);
  if (wave < nact) {
    // raw sliding-window row: u rotated at p, slot p % swa (attention waves)
    const float zr = rope1t(uu, col, d, P.n_rot, rtab, rtab + 64);
    if (roleA) {
      uint8_t* dst = cc.raw + ((size_t)b * P.swa + (p & (P.swa - 1))) * P.row_bytes;
      const float sc = mU > 0.f ? mU / 448.0f : 1.0f;
      put_chan<KVF>(dst, zr, col, dn, sc);
      if (KVF == CKV_E4M3 && tid == 0) *(float*)(dst + dn + 2 * P.n_rot) = sc;
    }
    if (roleA || roleI) {   // this token's projections -> state slot p % 8
      skv[cur * sw + col] = ka;
      ssc[cur * sw + col] = sa;
      if constexpr (NL == 2) {
        skv[cur * sw + width + col] = kb2;
        ssc[cur * sw + width + col] = sb2;
      }
    }
    if (pool) {   // RMSNorm, tail RoPE at 4 i, row i of the attention or indexer cache
      const float inv = roleA ? norm_inv(P, sA, d) : norm_inv(P, sI, DI);
      const float z = rope1t(gm * y * inv, col, width, roleA ? P.n_rot : P.idx_rot, rtab + 32, rtab + 96);
      if (roleA) {
        const long long slot = row_slot_wr(P, tid == 0 ? cc.status : nullptr, b, i);
        const float amax = mA * inv;
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
        if (slot >= 0) {
          uint8_t* dst = cc.comp + slot * P.row_bytes;
          put_chan<KVF>(dst, z, col, dn, sc);
          if (KVF == CKV_E4M3 && tid == 0) *(float*)(dst + dn + 2 * P.n_rot) = sc;
        }
      } else if (roleI) {
        if constexpr (IDXF == CKV_FP4) {
          idx_row[col] = z;   // encoded below
        } else {
          const long long slot = row_slot(P, b, i);   // (the attention role reports a bad entry)
          float zs = z;
          if constexpr (IDXF == CKV_F32) {
            zs = z;
          } else {
            zs = bf16_to_f32(f32_to_bf16(z));
          }
          if (slot >= 0) {
            uint8_t* dst = (uint8_t*)cc.idx + slot * P.idx_row_bytes;
            if constexpr (IDXF == CKV_F32) ((float*)dst)[col] = z;
            else ((uint16_t*)dst)[col] = (uint16_t)f32_to_bf16(z);
          }
          if (idx_row) idx_row[col] = zs;
        }
      }
    }
  }
  if constexpr (IDXF == CKV_FP4) {
    // fp4 indexer row: Hadamard + MXFP4 by wave 0 from the RoPE'd row in LDS;
    // idx_row then holds the stored (decoded) values
    if (pool) {
      lds_barrier();
      const long long slot = row_slot(P, b, i);
      if (wave == 0) fp4_store_row(idx_row, (uint8_t*)cc.idx + (slot < 0 ? 0 : slot) * kFp4RowBytes, idx_row,
                                   slot >= 0);
    }
  }
  return pool ? 1 : 0;
}

}  // namespace ckv
