// Sliding-window + sparse compressed attention with shared K = V
// ("ds4.c を読み解く (#3)", section 7: one online softmax over the raw window
// rows and the selected compressed rows; vLLM DeepSeek V4 page: the same
// vector is key and value, and the output tail is rotated back by -p).
//
// Row list of a query at p: raw positions max(0, p-swa+1) .. p, then
//   ratio 4   : the top-k list (entries < 0 skipped, the list ends at the first
//               entry >= V),
//   ratio 128 : rows 0 .. V-1,
//   ratio 0   : nothing.
// The list is cut into splits; each block runs the online softmax over its
// split and either finishes the output (one split) or leaves (max, sum,
// unnormalised output) for the merge kernel.
#include "ckv_device.h"

namespace ckv {

struct AttnQuery {
  int seq, p, V, n_raw, n_list;
};

__device__ __forceinline__ AttnQuery attn_query(const LayerParams& P, const int32_t* pos, int seq_fixed,
                                                int pos0, int qn) {
  AttnQuery a;
  a.seq = pos ? qn : seq_fixed;
  a.p = pos ? pos[qn] : pos0 + qn;
  if (a.p < 0) {
    a.V = a.n_raw = a.n_list = 0;
    return a;
  }
  a.V = P.ratio ? min((a.p + 1) / P.ratio, P.cap) : 0;
  a.n_raw = min(P.swa, a.p + 1);
  a.n_list = a.n_raw + (P.ratio == 4 ? P.topk : P.ratio == 128 ? a.V : 0);
  return a;
}

// Pointer to list entry j's stored row, or NULL when the entry is skipped.
__device__ __forceinline__ const uint8_t* attn_row(const LayerParams& P, const Cache& c, const AttnQuery& a,
                                                   bool decode, int pos0, const int32_t* tk, int tk_end,
                                                   int j) {
  if (j < a.n_raw) {
    const int t = a.p - a.n_raw + 1 + j;
    if (decode) return c.raw + ((size_t)a.seq * P.swa + t % P.swa) * P.row_bytes;
    return c.stage + (size_t)(t - pos0 + P.swa - 1) * P.row_bytes;
  }
  const int jj = j - a.n_raw;
  int row;
  if (P.ratio == 4) {
    if (jj >= tk_end) return nullptr;
    row = tk[jj];
    if (row < 0) return nullptr;
  } else {
    row = jj;
  }
  return c.comp + ((size_t)a.seq * P.cap + row) * P.row_bytes;
}

// First index of the top-k list holding a row >= V (the list ends there).
__device__ __forceinline__ int topk_end(const int32_t* tk, int k, int V, int* smem) {
  if (threadIdx.x == 0) *smem = k;
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += blockDim.x)
    if (tk[j] >= V) atomicMin(smem, j);
  __syncthreads();
  return *smem;
}

// ----------------------------------------------------------------- MFMA
// bf16 activations; rows bf16 or E4M3 (+ bf16 tail, fp32 scale).  Block of 4
// waves, each owning 16 heads; grid (queries, splits, H / 64).  The K = V row
// tile sits in LDS twice: row-major for the QK^T operand and channel-major for
// the PV operand.  An E4M3 row enters the products exactly (codes are exact in
// bf16); its scale multiplies the non-RoPE logit part and the non-RoPE
// probability operand.  The rotated query and the probabilities are fp32
// values split into a bf16 pair hi + lo, each product taking two MFMAs, so
// both contractions run at close to fp32 operand precision; the rows
// themselves are exact in bf16.
template <int KVF, int D>
__global__ __launch_bounds__(256) void k_attn_mfma(LayerParams P, Cache cc, const uint16_t* __restrict__ q,
                                                   const int32_t* __restrict__ pos, int seq_fixed, int pos0,
                                                   const int32_t* __restrict__ topk, int rows_per_split,
                                                   int nsplit, float* __restrict__ part_o,
                                                   float* __restrict__ part_ml, uint16_t* __restrict__ out) {
  constexpr int R = 32;          // rows per tile
  constexpr int KP = D + 8;      // K row stride (bf16 elements)
  constexpr int VP = R + 8;      // Vt channel stride
  constexpr int KS = D / 32;     // k-steps of QK^T
  constexpr int NO = D / 16;     // output channel tiles
  constexpr int DN = D - 64;     // non-RoPE channels
  constexpr int C8 = D / 8;      // 8-channel chunks per row
  constexpr int IT = (R / 2) * C8 / 256;  // staging items per thread per tile
  constexpr int MAXK = 4096;     // top-k list held in LDS
  __shared__ __attribute__((aligned(16))) uint16_t Ks[R * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
  // per wave: probabilities hi / lo, and (E4M3) scaled probabilities hi / lo
  __shared__ __attribute__((aligned(16))) uint16_t Ps[4][4][16 * VP];
  __shared__ int32_t tks[MAXK];
  __shared__ float rsc[R];
  __shared__ float cs_[32], sn_[32];
  __shared__ int tk_lim;

  const int qn = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int H = P.H;
  const int h0 = blockIdx.z * 64 + wave * 16;
  const bool decode = pos != nullptr;
  const AttnQuery A = attn_query(P, pos, seq_fixed, pos0, qn);
  const int j0 = split * rows_per_split;
  const int j1 = min(A.n_list, j0 + rows_per_split);
  const int32_t* tkg = (P.ratio == 4 && topk) ? topk + (size_t)qn * P.topk : nullptr;
  // top-k list into LDS; the list ends at its first entry >= V
  if (tid == 0) tk_lim = tkg ? P.topk : 0;
  __syncthreads();
  if (tkg) {
    for (int j0 = 0; j0 < P.topk; j0 += 256 * 4) {   // four loads per thread in flight
      int v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + tid + 256 * e;
        v[e] = j < P.topk ? tkg[j] : -1;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + tid + 256 * e;
        if (j < P.topk) {
          tks[j] = v[e];
          if (v[e] >= A.V) atomicMin(&tk_lim, j);
        }
      }
    }
  }
  if (tid < 32) rope_cs(P, tid, (double)A.p, &cs_[tid], &sn_[tid]);
  __syncthreads();
  const int tk_end = tk_lim;

  // address of list entry j's stored row (NULL: skipped entry or past the split)
  auto row_ptr = [&](int j) -> const uint8_t* {
    if (j >= j1) return nullptr;
    if (j < A.n_raw) {
      const int t = A.p - A.n_raw + 1 + j;
      if (decode) return cc.raw + ((size_t)A.seq * P.swa + t % P.swa) * P.row_bytes;
      return cc.stage + (size_t)(t - pos0 + P.swa - 1) * P.row_bytes;
    }
    const int jj = j - A.n_raw;
    int row = jj;
    if (P.ratio == 4) {
      if (jj >= tk_end) return nullptr;
      row = tks[jj];
      if (row < 0) return nullptr;
    }
    return cc.comp + ((size_t)A.seq * P.cap + row) * P.row_bytes;
  };

  // staged global loads of one tile: item e covers rows (2pr, 2pr+1), channels
  // 8*c8..; the row pair varies fastest across lanes so that the channel-major
  // Vt stores of 16 lanes land in 16 consecutive LDS words
  u32x4 stg[IT][2];
  float ssc[IT][2];
  auto issue = [&](int jt) {
#pragma unroll
    for (int e = 0; e < IT; ++e) {
      const int it = tid + 256 * e, pr = it & 15, c8 = it >> 4;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint8_t* rp = row_ptr(jt + 2 * pr + h);
        u32x4 v = {0u, 0u, 0u, 0u};
        float sc = -1.f;
        if (rp) {
          if (KVF == CKV_BF16) {
            v = *(const u32x4*)(rp + 16 * c8);
          } else if (8 * c8 >= DN) {
            v = *(const u32x4*)(rp + DN + 16 * (c8 - DN / 8));
          } else {
            const u32x2 cw = *(const u32x2*)(rp + 8 * c8);
            v[0] = cw[0];
            v[1] = cw[1];
          }
          if (c8 == 0) sc = KVF == CKV_E4M3 ? *(const float*)(rp + DN + 128) : 1.f;
        }
        stg[e][h] = v;
        ssc[e][h] = sc;
      }
    }
  };
  // staged registers -> LDS (row-major K, channel-major V); E4M3 codes become
  // their exact bf16 values
  auto commit = [&]() {
#pragma unroll
    for (int e = 0; e < IT; ++e) {
      const int it = tid + 256 * e, pr = it & 15, c8 = it >> 4;
      u32x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v[h] = stg[e][h];
        if (KVF == CKV_E4M3 && 8 * c8 < DN) {
          // OCP E4M3 codes -> their exact bf16 values, two per conversion
          const uint32_t w0 = v[h][0], w1 = v[h][1];
          u32x4 t;
          t[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
          t[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
          t[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
          t[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
          v[h] = t;
        }
        *(u32x4*)&Ks[(2 * pr + h) * KP + 8 * c8] = v[h];
        if (c8 == 0) rsc[2 * pr + h] = ssc[e][h];
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        *(uint32_t*)&Vt[(8 * c8 + 2 * f) * VP + 2 * pr] = (v[0][f] & 0xffffu) | (v[1][f] << 16);
        *(uint32_t*)&Vt[(8 * c8 + 2 * f + 1) * VP + 2 * pr] = (v[0][f] >> 16) | (v[1][f] & 0xffff0000u);
      }
    }
  };

  if (j0 < j1) issue(j0);

  // rotated query of head h0 + r as the A operand (hi, lo), one bf16x8 per k-step;
  // the non-RoPE channels are bf16 inputs, exact in hi with lo = 0
  u32x4 Aq[KS], Aql[KS];
  {
    const uint16_t* qr = q + ((size_t)qn * H + h0 + r) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 32 * ks + 8 * g;
      u32x4 v = *(const u32x4*)(qr + c0);
      u32x4 lo = {0u, 0u, 0u, 0u};
      if (c0 >= DN) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = bf16_to_f32(v[e] & 0xffffu), b = bf16_to_f32(v[e] >> 16);
          const int jp = (c0 - DN) / 2 + e;
          const float x = a * cs_[jp] - b * sn_[jp], y = a * sn_[jp] + b * cs_[jp];
          v[e] = pack_bf16x2(x, y);
          lo[e] = pack_bf16x2(x - bf16_to_f32(v[e] & 0xffffu), y - bf16_to_f32(v[e] >> 16));
        }
      }
      Aq[ks] = v;
      Aql[ks] = lo;
    }
  }

  float m_i[4], l_i[4];
  f32x4 O[NO];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_i[i] = -INFINITY;
    l_i[i] = 0.f;
  }
#pragma unroll
  for (int n = 0; n < NO; ++n) O[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float scale = P.scale;

  for (int jt = j0; jt < j1; jt += R) {
    __syncthreads();              // the previous tile's readers are done
    commit();
    __syncthreads();
    if (jt + R < j1) issue(jt + R);   // next tile's loads fly during this tile's math

    // logits for 2 row tiles of 16
    float S[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 b = *(const u32x4*)&Ks[(16 * nt + r) * KP + 32 * ks + 8 * g];
        if (32 * ks < DN) {
          a1 = mfma16x16x32(as_bf16x8(Aq[ks]), as_bf16x8(b), a1);
        } else {
          a2 = mfma16x16x32(as_bf16x8(Aq[ks]), as_bf16x8(b), a2);
          a2 = mfma16x16x32(as_bf16x8(Aql[ks]), as_bf16x8(b), a2);
        }
      }
      const float rs = rsc[16 * nt + r];
#pragma unroll
      for (int i = 0; i < 4; ++i) S[nt][i] = rs < 0.f ? -INFINITY : (a1[i] * rs + a2[i]) * scale;
    }
    // online softmax per head 4g+i (rows spread over the 16 lanes of group g).
    // The reference max m_i moves only when a tile's max exceeds it by more
    // than 8 (probabilities stay below e^8, safe in fp32 and bf16), so the
    // rescale of the 128 accumulators is rare; the result does not depend on
    // the reference chosen.
    float alpha[4];
    bool moved = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = fmaxf(S[0][i], S[1][i]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const bool move = mx > m_i[i] + 8.f;
      const float mn = move ? mx : m_i[i];
      const bool none = mn == -INFINITY;
      alpha[i] = (none || !move) ? 1.f : __expf(m_i[i] - mn);
      moved |= move && !none;
      float ps = 0.f;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float pv = none ? 0.f : __expf(S[nt][i] - mn);
        S[nt][i] = pv;
        ps += pv;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o, 64);
      l_i[i] = l_i[i] * alpha[i] + ps;
      m_i[i] = mn;
    }
    if (__ballot(moved)) {
#pragma unroll
      for (int n = 0; n < NO; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[n][i] *= alpha[i];
    }
    // probabilities -> LDS as the A operand [16 heads][32 rows], split hi + lo
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float rs = rsc[16 * nt + r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (4 * g + i) * VP + 16 * nt + r;
        const float pv = S[nt][i];
        const uint32_t hb = f32_to_bf16(pv);
        Ps[wave][0][o] = (uint16_t)hb;
        Ps[wave][1][o] = (uint16_t)f32_to_bf16(pv - bf16_to_f32(hb));
        if (KVF == CKV_E4M3) {
          const float ps = pv * fmaxf(rs, 0.f);
          const uint32_t hs = f32_to_bf16(ps);
          Ps[wave][2][o] = (uint16_t)hs;
          Ps[wave][3][o] = (uint16_t)f32_to_bf16(ps - bf16_to_f32(hs));
        }
      }
    }
    __syncthreads();
    const int pa = r * VP + 8 * g;
    const u32x4 aph = *(const u32x4*)&Ps[wave][0][pa];
    const u32x4 apl = *(const u32x4*)&Ps[wave][1][pa];
    const u32x4 ash = KVF == CKV_E4M3 ? *(const u32x4*)&Ps[wave][2][pa] : aph;
    const u32x4 asl = KVF == CKV_E4M3 ? *(const u32x4*)&Ps[wave][3][pa] : apl;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const u32x4 b = *(const u32x4*)&Vt[(16 * n + r) * VP + 8 * g];
      const bool nope = 16 * n < DN;
      O[n] = mfma16x16x32(as_bf16x8(nope ? ash : aph), as_bf16x8(b), O[n]);
      O[n] = mfma16x16x32(as_bf16x8(nope ? asl : apl), as_bf16x8(b), O[n]);
    }
  }

  if (nsplit == 1) {
    // finish: normalise, rotate the tail back by -p, store bf16
#pragma unroll
    for (int n = 0; n < NO; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float inv = l_i[i] > 0.f ? 1.f / l_i[i] : 0.f;
        float v = O[n][i] * inv;
        const int ch = 16 * n + r;
        if (ch >= DN && !(P.flags & CKV_FLAG_NO_INV_ROPE)) {
          const float other = __shfl_xor(v, 1, 64);
          const int jp = (ch - DN) >> 1;
          // rotation by -p: (a, b) -> (a cos + b sin, -a sin + b cos)
          v = (ch & 1) ? (-other * sn_[jp] + v * cs_[jp]) : (v * cs_[jp] + other * sn_[jp]);
        }
        out[((size_t)qn * H + h0 + 4 * g + i) * D + ch] = (uint16_t)f32_to_bf16(v);
      }
    }
    return;
  }
  const size_t pb = ((size_t)qn * nsplit + split) * H;
#pragma unroll
  for (int n = 0; n < NO; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) part_o[(pb + h0 + 4 * g + i) * D + 16 * n + r] = O[n][i];
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part_ml[(pb + h0 + 4 * g + i) * 2] = m_i[i];
      part_ml[(pb + h0 + 4 * g + i) * 2 + 1] = l_i[i];
    }
  }
}

// ----------------------------------------------------------------- vector
// Any formats.  Block of 256 = 16 heads x 16 lanes; lane `sub` owns channels
// [sub*dpt, (sub+1)*dpt).  grid (queries, splits, H / 16).
template <int KVF, int ACTF>
__global__ __launch_bounds__(256) void k_attn_vec(LayerParams P, Cache cc, const void* __restrict__ q,
                                                  const int32_t* __restrict__ pos, int seq_fixed, int pos0,
                                                  const int32_t* __restrict__ topk, int rows_per_split,
                                                  int nsplit, float* __restrict__ part_o,
                                                  float* __restrict__ part_ml) {
  __shared__ int tk_lim;
  const int qn = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, hl = tid >> 4, sub = tid & 15;
  const int d = P.d, H = P.H, h = blockIdx.z * 16 + hl;
  const int dpt = d / 16, dn = d - P.n_rot;
  const bool decode = pos != nullptr;
  const AttnQuery A = attn_query(P, pos, seq_fixed, pos0, qn);
  const int j0 = split * rows_per_split, j1 = min(A.n_list, j0 + rows_per_split);
  const int32_t* tk = (P.ratio == 4 && topk) ? topk + (size_t)qn * P.topk : nullptr;
  int tk_end = 0;
  if (tk) tk_end = topk_end(tk, P.topk, A.V, &tk_lim);

  float qv[32], acc[32];
  const int c0 = sub * dpt;
  for (int e = 0; e < dpt; e += 2) {
    const size_t o = ((size_t)qn * H + h) * d + c0 + e;
    float a = load_val<ACTF>(q, o), b = load_val<ACTF>(q, o + 1);
    if (c0 + e >= dn) {
      float cs, sn;
      rope_cs(P, (c0 + e - dn) / 2, (double)A.p, &cs, &sn);
      const float x = a * cs - b * sn, y = a * sn + b * cs;
      a = x;
      b = y;
    }
    qv[e] = a * P.scale;
    qv[e + 1] = b * P.scale;
    acc[e] = acc[e + 1] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = j0; j < j1; ++j) {
    const uint8_t* rp = attn_row(P, cc, A, decode, pos0, tk, tk_end, j);
    if (!rp) continue;
    float rv[32];
    float dot = 0.f;
    for (int e = 0; e < dpt; ++e) {
      const int ch = c0 + e;
      float v;
      if (KVF == CKV_F32) v = ((const float*)rp)[ch];
      else if (KVF == CKV_BF16) v = bf16_to_f32(((const uint16_t*)rp)[ch]);
      else v = ch < dn ? e4m3_to_f32(rp[ch]) * *(const float*)(rp + dn + 2 * P.n_rot)
                       : bf16_to_f32(((const uint16_t*)(rp + dn))[ch - dn]);
      rv[e] = v;
      dot += qv[e] * v;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dot += __shfl_xor(dot, o, 64);
    const float mn = fmaxf(m, dot);
    const float f = __expf(m - mn), pw = __expf(dot - mn);
    l = l * f + pw;
    for (int e = 0; e < dpt; ++e) acc[e] = acc[e] * f + pw * rv[e];
    m = mn;
  }
  const size_t pb = ((size_t)qn * nsplit + split) * H + h;
  for (int e = 0; e < dpt; ++e) part_o[pb * d + c0 + e] = acc[e];
  if (sub == 0) {
    part_ml[pb * 2] = m;
    part_ml[pb * 2 + 1] = l;
  }
}

// ----------------------------------------------------------------- merge
// grid (queries, H); block d/4 threads, each four adjacent channels.  The
// splits' (max, sum) pairs are read once into LDS.
template <int ACTF>
__global__ __launch_bounds__(128) void k_attn_merge(LayerParams P, const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ pos, int pos0, int nsplit,
                                                    void* __restrict__ out) {
  __shared__ float wsh[kMaxSplits];
  __shared__ float Lsh;
  const int qn = blockIdx.x, h = blockIdx.y, H = P.H, d = P.d;
  const int c = 4 * threadIdx.x;
  const int p = pos ? pos[qn] : pos0 + qn;
  const size_t b0 = (size_t)qn * nsplit * H + h;
  if (threadIdx.x < 64) {
    // max over splits with rows, then each split's weight exp(m_s - M)
    float m[4], l[4];
    float M = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sidx = threadIdx.x + 64 * e;
      m[e] = -INFINITY;
      l[e] = 0.f;
      if (sidx < nsplit) {
        const float2 ml = *(const float2*)(part_ml + (b0 + (size_t)sidx * H) * 2);
        m[e] = ml.x;
        l[e] = ml.y;
        if (l[e] > 0.f) M = fmaxf(M, m[e]);
      }
    }
    M = wave_max(M);
    float L = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sidx = threadIdx.x + 64 * e;
      const float wgt = l[e] > 0.f ? __expf(m[e] - M) : 0.f;
      if (sidx < nsplit) wsh[sidx] = wgt;
      L += l[e] * wgt;
    }
    L = wave_sum(L);
    if (threadIdx.x == 0) Lsh = L;
  }
  __syncthreads();
  if (c >= d) return;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < nsplit; s0 += 8) {   // eight splits' loads in flight at a time
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s0 + j < nsplit && wsh[s0 + j] != 0.f) v[j] = *(const float4*)(part_o + (b0 + (size_t)(s0 + j) * H) * d + c);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wgt = s0 + j < nsplit ? wsh[s0 + j] : 0.f;
      a.x += v[j].x * wgt;
      a.y += v[j].y * wgt;
      a.z += v[j].z * wgt;
      a.w += v[j].w * wgt;
    }
  }
  const float inv = Lsh > 0.f ? 1.f / Lsh : 0.f;
  float o[4] = {a.x * inv, a.y * inv, a.z * inv, a.w * inv};
  const int dn = d - P.n_rot;
  if (c >= dn && !(P.flags & CKV_FLAG_NO_INV_ROPE) && p >= 0) {
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      float cs, sn;
      rope_cs(P, (c + e - dn) / 2, (double)p, &cs, &sn);
      const float x = o[e] * cs + o[e + 1] * sn, y = -o[e] * sn + o[e + 1] * cs;
      o[e] = x;
      o[e + 1] = y;
    }
  }
  const size_t oo = ((size_t)qn * H + h) * d + c;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_val<ACTF>(out, oo + e, o[e]);
}

// ----------------------------------------------------------------- launcher

int launch_attn(const LayerParams& P, const Cache& c, const void* q, const int32_t* pos, int seq,
                int pos0, int nq, const int32_t* topk, void* out, const WsLayout& L, uint8_t* ws,
                void* stream) {
  hipStream_t st = (hipStream_t)stream;
  float* po = (float*)(ws + L.part_o);
  float* pml = (float*)(ws + L.part_ml);
  const int ns = L.attn_splits, rps = L.attn_rows_per_split;
  const bool mf = P.act_fmt == CKV_BF16 && P.kv_fmt != CKV_F32 && P.H % 64 == 0 &&
                  (P.d == 512 || P.d == 128) && P.n_rot == 64;
  if (mf) {
    dim3 grid(nq, ns, P.H / 64);
    const uint16_t* qq = (const uint16_t*)q;
    uint16_t* oo = (uint16_t*)out;
#define CKV_AM(KF, DD)                                                                              \
  hipLaunchKernelGGL((k_attn_mfma<KF, DD>), grid, dim3(256), 0, st, P, c, qq, pos, seq, pos0, topk, rps, \
                     ns, po, pml, oo)
    if (P.kv_fmt == CKV_BF16) {
      if (P.d == 512) CKV_AM(CKV_BF16, 512);
      else CKV_AM(CKV_BF16, 128);
    } else {
      if (P.d == 512) CKV_AM(CKV_E4M3, 512);
      else CKV_AM(CKV_E4M3, 128);
    }
#undef CKV_AM
    if (ns == 1) return (int)hipGetLastError();
  } else {
    dim3 grid(nq, ns, P.H / 16);
#define CKV_AV(KF, AF)                                                                                  \
  hipLaunchKernelGGL((k_attn_vec<KF, AF>), grid, dim3(256), 0, st, P, c, q, pos, seq, pos0, topk, rps, ns, \
                     po, pml)
    if (P.act_fmt == CKV_F32) {
      if (P.kv_fmt == CKV_F32) CKV_AV(CKV_F32, CKV_F32);
      else if (P.kv_fmt == CKV_BF16) CKV_AV(CKV_BF16, CKV_F32);
      else CKV_AV(CKV_E4M3, CKV_F32);
    } else {
      if (P.kv_fmt == CKV_F32) CKV_AV(CKV_F32, CKV_BF16);
      else if (P.kv_fmt == CKV_BF16) CKV_AV(CKV_BF16, CKV_BF16);
      else CKV_AV(CKV_E4M3, CKV_BF16);
    }
#undef CKV_AV
  }
  dim3 mg(nq, P.H);
  if (P.act_fmt == CKV_F32)
    hipLaunchKernelGGL(k_attn_merge<CKV_F32>, mg, dim3(128), 0, st, P, po, pml, pos, pos0, ns, out);
  else
    hipLaunchKernelGGL(k_attn_merge<CKV_BF16>, mg, dim3(128), 0, st, P, po, pml, pos, pos0, ns, out);
  return (int)hipGetLastError();
}

}  // namespace ckv
