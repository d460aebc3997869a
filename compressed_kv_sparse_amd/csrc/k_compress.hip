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
#include "compress_dec.h"

namespace ckv {

template <int KVF, int IDXF, int ACTF, int W, int TPC>
__global__ __launch_bounds__(256 * TPC) void k_compress_decode(LayerParams P, Weights w, Cache cc,
                                                               const void* __restrict__ u,
                                                               const int32_t* __restrict__ pos,
                                                               const float* __restrict__ proj, int splits, int B) {
  __shared__ float red[64];
  __shared__ float mrg[TPC > 1 ? TPC * (kMaxD / 2 + (W == 8 ? kMaxDI / 2 : 0)) * 6 : 1];
  __shared__ float rtab[128];
  const int st = compress_decode_seq<KVF, IDXF, ACTF, W, TPC>(P, w, cc, u, pos, proj, splits, B, blockIdx.x, red,
                                                              mrg, nullptr, rtab, [] {});
  advance_tokens(cc, blockIdx.x, pos[blockIdx.x], st);
}

// c4a: the role-split body, one block of d + D_I threads (rounded up
// to whole waves) per sequence; up to 4 projection slices; NL compressor lanes.
template <int KVF, int IDXF, int ACTF, int NL = 1>
__global__ __launch_bounds__(1024) void k_compress_c4a(LayerParams P, Weights w, Cache cc, const void* __restrict__ u,
                                                       const int32_t* __restrict__ pos,
                                                       const float* __restrict__ proj, int splits, int B) {
  __shared__ __attribute__((aligned(16))) float red[64];
  __shared__ float rtab[192];
  __shared__ __attribute__((aligned(16))) float idx_lds[IDXF == CKV_FP4 ? kMaxDI : 1];   // fp4 row staging
  const int st = compress_c4a_seq<KVF, IDXF, ACTF, NL>(P, w, cc, u, pos, proj, splits, B, blockIdx.x, red, rtab,
                                                       IDXF == CKV_FP4 ? idx_lds : nullptr, [] {});
  advance_tokens(cc, blockIdx.x, pos[blockIdx.x], st);
}

// Ratio 0: only the raw sliding-window row.
template <int KVF, int ACTF>
__global__ __launch_bounds__(256) void k_raw_insert_decode(LayerParams P, Cache cc, const void* __restrict__ u,
                                                           const int32_t* __restrict__ pos) {
  __shared__ float red[64];
  const int b = blockIdx.x, c = 2 * threadIdx.x, d = P.d;
  const bool act = c < d;
  const int p = pos[b];
  const int nt = seq_tokens(cc, b, p);
  const float2 uu = load2<ACTF>(u, (long)b * d + min(c, d - 2));
  if (p < 0 || !seq_ok(cc, p, nt)) {
    if (threadIdx.x == 0 && cc.status) atomicOr(&cc.status[b], p < 0 ? CKV_STATUS_BAD_POS : CKV_STATUS_SEQUENCE);
    return;
  }
  const float2 z = rope2(P, uu, c, d, P.n_rot, p);
  store_row2<KVF>(cc.raw + ((size_t)b * P.swa + (p & (P.swa - 1))) * P.row_bytes, z, c, act, d, P.n_rot, red);
  lds_barrier();
  if (threadIdx.x == 0 && cc.n_tokens) cc.n_tokens[b] = p + 1;
}

// ------------------------------------------------------------ c128a decode
// The 128-slot window of a c128a row pooled channel slice by channel slice:
// the per-channel softmax of the pages' compressor needs no other channel, so
// slice g (64 channels) of sequence b is one block, and only the row's
// RMSNorm sum and the E4M3 scale need all channels -- a second, per-sequence
// kernel takes the slices' partial sums and finishes the row.  (One block per
// sequence would pull the whole 512 KB window state and 256 KB of APE through
// one compute unit.)
//
// k_c128a_slices: grid (B, d / 64), 256 threads: thread t pools channel pair
// 64 g + 2 (t % 32) over window slots 16 (t / 32) .. +15 (on a boundary step;
// the 8 parts merged through LDS), writes y and the slice's (sum y^2,
// max |gamma y| of the non-RoPE channels) to the workspace, and stores this
// token's (kappa, sigma) of the slice in slot p % 128.  Slice 0 also stores
// the raw row (u rotated at p).
constexpr int kC128Parts = 8, kC128SlotsPer = 128 / kC128Parts;

template <int KVF, int ACTF>
__global__ __launch_bounds__(256) void k_c128a_slices(LayerParams P, Weights w, Cache cc, const void* __restrict__ u,
                                                      const int32_t* __restrict__ pos, const float* __restrict__ proj,
                                                      int splits, int B, float* __restrict__ pool_ws) {
  __shared__ float mrg[kC128Parts][32][6];
  __shared__ float red[64];
  const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int q = tid & 31, part = tid >> 5;
  const int d = P.d, dn = d - P.n_rot, c = 64 * g + 2 * q;
  const int p = pos[b];
  const int nt = seq_tokens(cc, b, p);
  float2 ka = make_float2(0.f, 0.f), sa = ka;
#pragma unroll
  for (int s = 0; s < 4; ++s) {   // this token's projections, the K slices summed in order
    const float* pj = proj + ((size_t)min(s, splits - 1) * B + b) * P.ncol;
    const float2 k2 = ld2(pj + c), s2 = ld2(pj + d + c);
    if (s < splits) {
      ka.x += k2.x; ka.y += k2.y;
      sa.x += s2.x; sa.y += s2.y;
    }
  }
  const bool ok = p >= 0 && seq_ok(cc, p, nt);
  const bool emit = ok && (p + 1) % 128 == 0;
  const float* skv = cc.st_kv + (size_t)b * 128 * d;
  const float* ssc = cc.st_sc + (size_t)b * 128 * d;
  if (emit) {   // block-uniform: the window of row (p + 1) / 128 - 1 is the whole ring, slot = position j
    PoolAcc a0, a1;
    float2 kv[kC128SlotsPer], sc[kC128SlotsPer], ap[kC128SlotsPer];
#pragma unroll
    for (int jj = 0; jj < kC128SlotsPer; ++jj) {
      const int j = kC128SlotsPer * part + jj;
      kv[jj] = ld2(skv + (size_t)j * d + c);
      sc[jj] = ld2(ssc + (size_t)j * d + c);
      ap[jj] = ld2(w.ape + (size_t)j * d + c);
    }
    const int jc = p & 127;   // this token's slot holds the previous window's token: take the registers
    float e0[kC128SlotsPer], e1[kC128SlotsPer], k0[kC128SlotsPer], k1[kC128SlotsPer];
#pragma unroll
    for (int jj = 0; jj < kC128SlotsPer; ++jj) {
      const bool cur = kC128SlotsPer * part + jj == jc;
      const float2 k = cur ? ka : kv[jj], e = cur ? sa : sc[jj];
      e0[jj] = e.x + ap[jj].x;
      e1[jj] = e.y + ap[jj].y;
      k0[jj] = k.x;
      k1[jj] = k.y;
    }
    a0.add_round(e0, k0);
    a1.add_round(e1, k1);
    float* mm = mrg[part][q];
    mm[0] = a0.m; mm[1] = a0.s; mm[2] = a0.acc;
    mm[3] = a1.m; mm[4] = a1.s; mm[5] = a1.acc;
    lds_barrier();
    float ss = 0.f, mx = 0.f;
    if (part == 0) {   // merge the parts' online-softmax states
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int r = 0; r < kC128Parts; ++r) {
        m0 = fmaxf(m0, mrg[r][q][0]);
        m1 = fmaxf(m1, mrg[r][q][3]);
      }
      float s0 = 0.f, c0 = 0.f, s1 = 0.f, c1 = 0.f;
#pragma unroll
      for (int r = 0; r < kC128Parts; ++r) {
        const float f0 = __expf(mrg[r][q][0] - m0), f1 = __expf(mrg[r][q][3] - m1);
        s0 += mrg[r][q][1] * f0;
        c0 += mrg[r][q][2] * f0;
        s1 += mrg[r][q][4] * f1;
        c1 += mrg[r][q][5] * f1;
      }
      const float2 y = make_float2(s0 > 0.f ? c0 / s0 : 0.f, s1 > 0.f ? c1 / s1 : 0.f);
      *(float2*)(pool_ws + (size_t)b * d + c) = y;
      const float2 gm = norm_gamma(P, ld2(w.gamma + c));
      ss = y.x * y.x + y.y * y.y;
      mx = c < dn ? fmaxf(fabsf(gm.x * y.x), fabsf(gm.y * y.y)) : 0.f;
    }
    const float2 t = cmp::block_sum_max(ss, mx, red);
    if (tid == 0) *(float2*)(pool_ws + (size_t)B * d + ((size_t)b * 8 + g) * 2) = t;
  }
  if (ok && part == 0) {   // this token's projections -> state slot p % 128
    const size_t o = ((size_t)b * 128 + (p & 127)) * d + c;
    *(float2*)(cc.st_kv + o) = ka;
    *(float2*)(cc.st_sc + o) = sa;
  }
  if (g == 0 && ok) {      // raw sliding-window row: u rotated at p (raw frame), slot p % swa
    const int cr = 2 * tid;
    const float2 uu = load2<ACTF>(u, (long)b * d + min(cr, d - 2));
    const float2 z = rope2(P, uu, cr, d, P.n_rot, p);
    store_row2<KVF>(cc.raw + ((size_t)b * P.swa + (p & (P.swa - 1))) * P.row_bytes, z, cr, cr < d, d, P.n_rot, red);
  }
}

// k_c128a_finish: grid (B), 256 threads (channel pair 2 t): on a boundary
// step, RMSNorm with the slices' sums, RoPE at i * 128 (compressed frame), the
// E4M3 scale inv * max |gamma y| (the row is (gamma y) inv with inv > 0), and
// row i stored; the sequence's status bits and token count.
template <int KVF>
__global__ __launch_bounds__(256) void k_c128a_finish(LayerParams P, Weights w, Cache cc,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ pool_ws, int B) {
  __shared__ float red[64];
  const int b = blockIdx.x, tid = threadIdx.x, c = 2 * tid;
  const int d = P.d, dn = d - P.n_rot, nsl = d / 64;
  const int p = pos[b];
  const int nt = seq_tokens(cc, b, p);
  if (p < 0 || !seq_ok(cc, p, nt)) {
    if (tid == 0 && cc.status) atomicOr(&cc.status[b], p < 0 ? CKV_STATUS_BAD_POS : CKV_STATUS_SEQUENCE);
    return;
  }
  const bool emit = (p + 1) % 128 == 0;
  const int i = (p + 1) / 128 - 1;
  if (emit && i >= P.cap && tid == 0 && cc.status) atomicOr(&cc.status[b], CKV_STATUS_CAPACITY);
  if (emit && i < P.cap) {
    float ss = 0.f, mx = 0.f;
    for (int g = 0; g < nsl; ++g) {
      const float2 t = ld2(pool_ws + (size_t)B * d + ((size_t)b * 8 + g) * 2);
      ss += t.x;
      mx = fmaxf(mx, t.y);
    }
    const float inv = norm_inv(P, ss, d);
    const bool act = c < d;
    const float2 y = ld2(pool_ws + (size_t)b * d + min(c, d - 2));
    const float2 gm = norm_gamma(P, ld2(w.gamma + min(c, d - 2)));
    float2 z = make_float2(gm.x * (y.x * inv), gm.y * (y.y * inv));
    if (c >= dn && act) {
      float cs, sn;
      rope_cs_c(P, (c - dn) >> 1, (double)i * 128, &cs, &sn);
      z = make_float2(z.x * cs - z.y * sn, z.x * sn + z.y * cs);
    }
    const long long slot = row_slot_wr(P, tid == 0 ? cc.status : nullptr, b, i);
    uint8_t* dst = cc.comp + (slot < 0 ? 0 : slot) * P.row_bytes;
    if (slot < 0) {
      // (a block-table entry outside the pool: the row is not stored)
    } else if constexpr (KVF == CKV_E4M3) {
      const float amax = mx * inv;
      const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
      if (act) {
        if (c < dn) *(uint16_t*)(dst + c) = (uint16_t)(f32_to_e4m3(z.x / sc) | (f32_to_e4m3(z.y / sc) << 8));
        else *(uint32_t*)(dst + dn + 2 * (c - dn)) = pack_bf16x2(z.x, z.y);
      }
      if (tid == 0) *(float*)(dst + dn + 2 * P.n_rot) = sc;
    } else {
      store_row2<KVF>(dst, z, c, act, d, P.n_rot, red);
    }
  }
  lds_barrier();
  advance_tokens(cc, b, p, 0);
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
  rope_lds(P, zs, d, P.n_rot, (double)t, false);
  __syncthreads();
  store_row<KVF>(dst, zs, d, P.n_rot, red);
}

// Pool every row whose window closes inside the chunk.  Window tokens before
// pos0 come from the state ring, chunk tokens from the projection part[n][col].
// One block per emitted row i = i_first + blockIdx.x; lanes: bit 0 the
// attention row, bit 1 the indexer row (ratio 4).
template <int KVF, int IDXF>
__global__ __launch_bounds__(256) void k_pool_prefill(LayerParams P, Weights w, Cache cc,
                                                      const float* __restrict__ part, int seq,
                                                      int pos0, int i_first, int lanes) {
  __shared__ float zs[kMaxD];
  __shared__ __attribute__((aligned(16))) float zi[kMaxDI];
  __shared__ float red[16];
  const int i = i_first + blockIdx.x;
  const int d = P.d, r = P.ratio, W = P.W, DI = P.DI, nc = P.ncol, NL = P.lanes;
  if (cc.n_tokens && cc.n_tokens[seq] != pos0) return;   // out of sequence: the cache stays as it is
  const int t0 = i * r - (W - r);
  // two lanes (ratio 4): window positions 0-3 take lane A (offset 0) of
  // their token's projections / ring slot / APE row j, positions 4-7 lane B
  // (offset w) of APE row j - 4; one lane: APE row j
  const float* skv = cc.st_kv + (size_t)seq * W * NL * d;
  const float* ssc = cc.st_sc + (size_t)seq * W * NL * d;
  if (lanes & 1) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
      PoolAcc pa;
      for (int j = 0; j < W; ++j) {
        const int t = t0 + j;
        if (t < 0) continue;
        const int lo = NL == 2 && j >= 4 ? d : 0;   // lane offset
        float kv, sc;
        if (t >= pos0) {
          const float* pr = part + (size_t)(t - pos0) * nc;
          kv = pr[lo + c];
          sc = pr[NL * d + lo + c];
        } else {
          kv = skv[(t % W) * NL * d + lo + c];
          sc = ssc[(t % W) * NL * d + lo + c];
        }
        pa.add(sc + w.ape[(NL == 2 ? (j & 3) * 2 * d : j * d) + lo + c], kv);
      }
      zs[c] = pa.value();
    }
    rmsnorm_lds(P, zs, d, w.gamma, red);
    __syncthreads();
    rope_lds(P, zs, d, P.n_rot, (double)i * r, true);
    __syncthreads();
    const long long slot = row_slot_wr(P, threadIdx.x == 0 ? cc.status : nullptr, seq, i);
    if (slot >= 0) store_row<KVF>(cc.comp + slot * P.row_bytes, zs, d, P.n_rot, red);
  }
  if (r != 4 || !(lanes & 2)) return;
  const float* ikv = cc.ist_kv + (size_t)seq * 8 * NL * DI;
  const float* isc = cc.ist_sc + (size_t)seq * 8 * NL * DI;
  for (int c = threadIdx.x; c < DI; c += blockDim.x) {
    PoolAcc pa;
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + j;
      if (t < 0) continue;
      const int lo = NL == 2 && j >= 4 ? DI : 0;
      float kv, sc;
      if (t >= pos0) {
        const float* pr = part + (size_t)(t - pos0) * nc + 2 * NL * d;
        kv = pr[lo + c];
        sc = pr[NL * DI + lo + c];
      } else {
        kv = ikv[(t % 8) * NL * DI + lo + c];
        sc = isc[(t % 8) * NL * DI + lo + c];
      }
      pa.add(sc + w.idx_ape[(NL == 2 ? (j & 3) * 2 * DI : j * DI) + lo + c], kv);
    }
    zi[c] = pa.value();
  }
  rmsnorm_lds(P, zi, DI, w.idx_gamma, red);
  __syncthreads();
  rope_lds(P, zi, DI, P.idx_rot, (double)i * r, true);
  __syncthreads();
  const long long slot = row_slot_wr(P, threadIdx.x == 0 ? cc.status : nullptr, seq, i);
  if (slot < 0) return;
  uint8_t* dst = (uint8_t*)cc.idx + slot * P.idx_row_bytes;
  if constexpr (IDXF == CKV_FP4) {
    if (threadIdx.x < 64) fp4_store_row(zi, dst, nullptr);
  } else {
    store_vals<IDXF>(dst, zi, DI);
  }
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
  if (cc.n_tokens && cc.n_tokens[seq] != pos0) return;   // out of sequence: the cache stays as it is
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
  const int wa = P.lanes * d, wi = P.lanes * DI;   // a ring slot holds every lane of its token
  for (int c = threadIdx.x; c < wa; c += blockDim.x) {
    const size_t o = ((size_t)seq * W + t % W) * wa + c;
    cc.st_kv[o] = pr[c];
    cc.st_sc[o] = pr[wa + c];
  }
  if (P.ratio == 4) {
    for (int c = threadIdx.x; c < wi; c += blockDim.x) {
      const size_t o = ((size_t)seq * 8 + t % 8) * wi + c;
      cc.ist_kv[o] = pr[2 * wa + c];
      cc.ist_sc[o] = pr[2 * wa + wi + c];
    }
  }
}

// The chunk's sequence check and token count (cache->n_tokens): launched after
// every kernel of the chunk has read the count.
__global__ void k_advance_tokens(Cache cc, int seq, int pos0, int T) {
  if (cc.n_tokens[seq] == pos0) cc.n_tokens[seq] = pos0 + T;
  else if (cc.status) atomicOr(&cc.status[seq], CKV_STATUS_SEQUENCE);
}

// ------------------------------------------------------------ launchers

template <int KVF, int IDXF, int ACTF>
static void go_decode(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                      const int32_t* pos, int B, const float* part, int splits, float* pool_ws, hipStream_t st) {
  const int np = P.d / 2;
  if (P.ratio == 128 && c128a_sliced(P) && splits <= 4) {
    hipLaunchKernelGGL((k_c128a_slices<KVF, ACTF>), dim3(B, P.d / 64), dim3(256), 0, st, P, w, c, u, pos, part,
                       splits, B, pool_ws);
    hipLaunchKernelGGL((k_c128a_finish<KVF>), dim3(B), dim3(256), 0, st, P, w, c, pos, pool_ws, B);
  } else if (P.ratio == 4 && P.lanes == 2) {   // (decode projections have at most 4 slices)
    hipLaunchKernelGGL((k_compress_c4a<KVF, IDXF, ACTF, 2>), dim3(B), dim3((P.d + P.DI + 63) / 64 * 64), 0, st, P,
                       w, c, u, pos, part, splits, B);
  } else if (P.ratio == 4 && (splits <= 4 || IDXF == CKV_FP4))   // (fp4: splits is at most 4)
    hipLaunchKernelGGL((k_compress_c4a<KVF, IDXF, ACTF>), dim3(B), dim3((P.d + P.DI + 63) / 64 * 64), 0, st, P, w,
                       c, u, pos, part, splits, B);
  else if constexpr (IDXF == CKV_FP4)
    return;   // fp4 indexer rows are ratio 4 only
  else if (P.ratio == 4)
    hipLaunchKernelGGL((k_compress_decode<KVF, IDXF, ACTF, 8, 1>), dim3(B), dim3(np), 0, st, P, w, c, u, pos,
                       part, splits, B);
  else if (P.ratio == 128)
    hipLaunchKernelGGL((k_compress_decode<KVF, IDXF, ACTF, 128, 4>), dim3(B), dim3(4 * np), 0, st, P, w, c, u,
                       pos, part, splits, B);
  else
    hipLaunchKernelGGL((k_raw_insert_decode<KVF, ACTF>), dim3(B), dim3(np), 0, st, P, c, u, pos);
}

#define CKV_DISPATCH_KV_IDX_ACT(FN, ...)                                               \
  do {                                                                                 \
    const bool idx32 = P.idx_fmt == CKV_F32, act32 = P.act_fmt == CKV_F32;            \
    if (P.idx_fmt == CKV_FP4) {   /* validated: bf16 activations */                  \
      if (P.kv_fmt == CKV_F32) FN<CKV_F32, CKV_FP4, CKV_BF16>(__VA_ARGS__);            \
      else if (P.kv_fmt == CKV_BF16) FN<CKV_BF16, CKV_FP4, CKV_BF16>(__VA_ARGS__);     \
      else FN<CKV_E4M3, CKV_FP4, CKV_BF16>(__VA_ARGS__);                               \
    } else if (P.kv_fmt == CKV_F32) {                                                  \
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
                           const int32_t* pos, int B, const float* part, int splits, float* pool_ws,
                           void* stream) {
  hipStream_t st = (hipStream_t)stream;
  CKV_DISPATCH_KV_IDX_ACT(go_decode, P, w, c, u, pos, B, part, splits, pool_ws, st);
  return (int)hipGetLastError();
}

template <int KVF, int IDXF, int ACTF>
static void go_prefill(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                       int seq, int pos0, int T, const float* part, hipStream_t st, int parts) {
  if (parts & kPfStage)
    hipLaunchKernelGGL((k_stage_raw<KVF, ACTF>), dim3(T + P.swa - 1), dim3(256), 0, st, P, c, u, seq, pos0);
  const int lanes = ((parts & kPfPoolAttn) ? 1 : 0) | ((parts & kPfPoolIdx) && P.ratio == 4 ? 2 : 0);
  if (P.ratio && lanes) {
    const int i_first = pos0 / P.ratio, i_end = (pos0 + T) / P.ratio;
    if (i_end > i_first)
      hipLaunchKernelGGL((k_pool_prefill<KVF, IDXF>), dim3(i_end - i_first), dim3(256), 0, st, P, w,
                         c, part, seq, pos0, i_first, lanes);
  }
  if (parts & kPfState) {
    hipLaunchKernelGGL(k_state_prefill, dim3(P.swa), dim3(256), 0, st, P, c, part, seq, pos0, T);
    if (c.n_tokens) hipLaunchKernelGGL(k_advance_tokens, dim3(1), dim3(1), 0, st, c, seq, pos0, T);
  }
}

int launch_compress_prefill(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                            int seq, int pos0, int T, const float* part, void* stream, int parts) {
  hipStream_t st = (hipStream_t)stream;
  CKV_DISPATCH_KV_IDX_ACT(go_prefill, P, w, c, u, seq, pos0, T, part, st, parts);
  return (int)hipGetLastError();
}

}  // namespace ckv
