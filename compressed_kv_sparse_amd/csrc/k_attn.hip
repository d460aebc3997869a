// Sliding-window + sparse compressed attention with shared K = V
// ("ds4.c を読み解く (#3)", section 7: one online softmax over the raw window
// rows and the selected compressed rows; vLLM DeepSeek V4 page: the same
// vector is key and value, and the output tail is rotated back by -p).
//
// Row list of a query at p: swa (= 128) raw slots first, slot j holding
// position t = p - swa + 1 + j (skipped while t < 0, so that every 32-row tile
// holds one row class only), then
//   ratio 4   : the top-k list (entries < 0 skipped, the list ends at the first
//               entry >= V),
//   ratio 128 : rows 0 .. V-1,
//   ratio 0   : nothing.
// The list is cut into splits; each block runs the online softmax over its
// split and either finishes the output (one split) or leaves (max, sum,
// normalised output) for the merge kernel.
//
// Rotation frames.  Raw rows carry their position in the raw class's frame
// (base theta), compressed rows in the compressed class's frame (theta_c;
// the same when the layer has one base).  The query is rotated at p into the
// frame of the split's first row class; when a split crosses from the raw
// slots into the compressed entries, the query tail and the accumulated output
// tail are both turned by p (theta_c - theta), which moves them into the
// compressed frame (the output is linear in the rows, and a rotation commutes
// with the softmax rescaling).  Each split rotates its output back by -p in
// the frame it ended in, so the merge only adds.
#include "ckv_device.h"

namespace ckv {

struct AttnQuery {
  int seq, p, V, n_list;
};

__device__ __forceinline__ AttnQuery attn_query(const LayerParams& P, const int32_t* pos, int seq_fixed,
                                                int pos0, int qn) {
  AttnQuery a;
  a.seq = pos ? qn : seq_fixed;
  a.p = pos ? pos[qn] : pos0 + qn;
  if (a.p < 0) {
    a.V = a.n_list = 0;
    return a;
  }
  a.V = P.ratio ? min((a.p + 1) / P.ratio, P.cap) : 0;
  a.n_list = P.swa + (P.ratio == 4 ? P.topk : P.ratio == 128 ? a.V : 0);
  return a;
}

// Pointer to list entry j's stored row, or NULL when the entry is skipped.
__device__ __forceinline__ const uint8_t* attn_row(const LayerParams& P, const Cache& c, const AttnQuery& a,
                                                   bool decode, int pos0, const int32_t* tk, int tk_end,
                                                   int j) {
  if (j < P.swa) {
    const int t = a.p - P.swa + 1 + j;
    if (t < 0) return nullptr;
    if (decode) return c.raw + ((size_t)a.seq * P.swa + t % P.swa) * P.row_bytes;
    return c.stage + (size_t)(t - pos0 + P.swa - 1) * P.row_bytes;
  }
  const int jj = j - P.swa;
  int row;
  if (P.ratio == 4) {
    if (jj >= tk_end) return nullptr;
    row = tk[jj];
    if (row < 0) return nullptr;
  } else {
    row = jj;
  }
  return c.comp + row_slot_rd(P, a.seq, row) * P.row_bytes;
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

// (a, b) <- rotation of the pair by the angle whose cos / sin are (c, s);
// s < 0 turns backwards.
__device__ __forceinline__ void rot2(float& a, float& b, float c, float s) {
  const float x = a * c - b * s, y = a * s + b * c;
  a = x;
  b = y;
}

// ----------------------------------------------------------------- MFMA
// bf16 activations, head_dim 512, rows bf16 or E4M3 (+ bf16 tail, fp32 row
// scale).  One block of 8 waves per (query, split, 64 heads); grid x =
// queries * splits (split fastest), y = H / 64.
//
// Wave (hg, cg) = (w & 3, w >> 2) owns heads 16 hg .. +15 and channels
// 256 cg .. +255.  Both products are taken transposed, so that everything a
// head needs sits in that head's lanes: lane (r, g) = (l & 15, l >> 4) works
// for head 16 hg + r.
//   * logits S^T = K Q^T: A = 16 rows of the tile (row-major copy in LDS),
//     B = the rotated query; lane (r, g) receives rows 16 nt + 4 g + i.  Each
//     wave covers its 256-channel half; the two halves of a head group are
//     summed through LDS in a fixed order, so both waves hold identical logits
//     and run identical online-softmax updates (one head, 8 rows per lane).
//   * output O^T = V^T P^T: A = 16 channels x 32 rows, read from the same
//     row-major tile with the LDS transpose read (ds_read_b64_tr_b16: within
//     each 16-lane group, lane 4 a + e receives element e of the 8-byte rows
//     addressed by lanes a, a + 4, a + 8, a + 12), so lane (r, g) gathers
//     channel r of rows 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3 -- the
//     order in which it holds its probabilities, which therefore go into PV
//     straight from the registers as the B operand.  Lane (r, g) accumulates
//     channels 16 n + 4 g + i of its head.
// Operand precision: the tile, the rotated query and the probabilities are
// fp16 (MFMA f16 x f16 -> fp32).  E4M3 codes are exact in fp16 and a row's
// scale multiplies the non-RoPE logit part and, for PV, the probability
// operand of the non-RoPE channels; bf16 values convert to fp16 with 2^-11
// relative rounding, and so do the rotated query tail and the probabilities
// (bf16 probabilities, 2^-9, would be 4x coarser: visible where rows of
// opposite sign cancel).  Logits are kept in base-2 units (times scale
// log2 e), so that a probability is one exp2; a skipped entry's logit is -inf
// through a per-row bias.
// Range guard: a bf16 value at or above 65520 in magnitude has no fp16 image
// (it becomes infinite).  An infinite operand makes the split's softmax sum
// not finite (a +inf or NaN logit), or zero although the split has rows
// (every logit -inf), or its output not finite (inf times a zero
// probability); the block checks these once, at the end of the split, and
// then recomputes the split in fp32 (k_attn_tile's second half), which also
// takes a split whose normalised output exceeds fp16's range when it leaves
// a partial (written then as two fp16 halves under a power-of-two scale).  So
// such inputs cost time, not accuracy.  Small values need no guard: below
// 2^-14 fp16 keeps an absolute error under 2^-25, far inside the
// comparison's absolute tolerance.
//
// The block first lays out its split's row list in LDS as 64-bit row
// addresses (bit 0 set: skipped entry, an all-zero row stands in); on ratio
// 128 (CMP) the compressed entries are computed instead (row jj at index jj),
// so the table holds at most the raw slots and a top-k list.  Staging is
// coalesced: consecutive lanes load consecutive 16-byte chunks of one stored
// row and convert them into the row-major tile.  The tile is double-buffered: tile t is
// multiplied from one buffer while tile t + 1 is written into the other, two
// barriers per tile.  Global loads are unconditional and sit outside any
// branch, so the compiler waits only for the tile being committed; two
// tiles' loads are in flight while a tile is multiplied.  The wave index comes
// from readfirstlane, so branches on the wave's role (around MFMAs) are
// scalar branches, and the barriers inside the loop order LDS only
// (lds_barrier).
namespace attn {
constexpr int D = 512, DN = 448, R = 32, SWA = 128;
constexpr int NT = 512;     // threads per block
constexpr int KP = D + 16;  // row-major row stride (16-bit elements)
// Element e of tile row R: row stride 528 elements (1056 bytes, 8 banks of
// shift per row), and the 16-byte chunk e / 8 XORed with bit 2 of R.  The
// transposed PV reads (4 rows x 32 bytes per 16 lanes) then hit 32 distinct
// banks, and so do the 16-byte logit reads (8 lanes = rows r .. r + 7 of
// one chunk; rows r and r + 4, 32 banks apart by the stride, differ by the
// XOR).
__device__ __forceinline__ int tix(int R, int e) { return R * KP + ((((e >> 3) ^ (R >> 2)) & 1) | (e >> 3 & ~1)) * 8 + (e & 7); }
constexpr int MAXK = 2048;                   // top-k entries (the layer check caps top_k here)
constexpr int MAXL = SWA + MAXK + 4 * R;     // row-table entries of one split (+ padding tiles)
constexpr int RAW_TILES = SWA / R;           // the raw slots fill the first four tiles
constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
constexpr float MOVE2 = 8.f * LOG2E;         // the running max moves by more than e^8 only
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
// two floats -> packed fp16 pair (hardware conversion, round to nearest even)
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}
__device__ __forceinline__ float lo_f16(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
__device__ __forceinline__ float hi_f16(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// 8 bf16 values -> 8 fp16 values
__device__ __forceinline__ u32x4 bf16x8_to_f16(u32x4 v) {
  u32x4 t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = pk_f16(lo_bf16(v[i]), hi_bf16(v[i]));
  return t;
}
// 8 E4M3 codes -> their exact fp16 values
__device__ __forceinline__ u32x4 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  u32x4 t;
  t[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
  t[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
  t[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
  t[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
  return t;
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ u32x2 ds_tr16(const uint16_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) i16x4_t*)(p)));
}
// Position of channel c in a split's fp16 partial row: channels
// 256 cg + 16 n + 4 g + i sit at 256 cg + 64 g + 4 n + i, so that the lane
// that accumulated them (lane 16 g + r of a cg wave) writes 128 contiguous
// bytes; groups of four channels stay contiguous.
__device__ __forceinline__ int part_pos(int c) {
  return (c & ~255) | ((c >> 2 & 3) << 6) | ((c >> 4 & 15) << 2) | (c & 3);
}
// 16 bytes from a global address held as an integer
__device__ __forceinline__ u32x4 ldg16(uint64_t a) {
  return *(const __attribute__((address_space(1))) u32x4*)(a);
}
__device__ __forceinline__ float ldg_f32(uint64_t a) {
  return *(const __attribute__((address_space(1))) float*)(a);
}
// fp8 output records (CKV_FLAG_OUT_FP8): a row's d E4M3 codes, then one fp32
// scale per group of 128 channels
__device__ __forceinline__ int out8_bytes(int d) { return d + 4 * (d >> 7); }
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float e) {
  return f32_to_e4m3(a) | (f32_to_e4m3(b) << 8) | (f32_to_e4m3(c) << 16) | (f32_to_e4m3(e) << 24);
}
}  // namespace attn

// The row skipped list entries point at: zeros, so that a skipped row adds
// nothing to PV (its logit is -inf through its bias slot) without a select
// per staged value.  Written never.
__device__ __attribute__((aligned(256))) uint8_t g_attn_zero_row[2048];

// CMP: ratio-128 layers, whose compressed entries are computed from their
// index instead of read from the row table.
template <int KVF, bool CMP>
__global__ __launch_bounds__(512) void k_attn_tile(LayerParams P, Cache cc, const uint16_t* __restrict__ q,
                                                   const int32_t* __restrict__ pos, int seq_fixed, int pos0,
                                                   const int32_t* __restrict__ topk, int rows_per_split,
                                                   int nsplit, float* __restrict__ part_o,
                                                   float* __restrict__ part_ml, uint16_t* __restrict__ out) {
  using namespace attn;
  constexpr bool F8 = KVF == CKV_E4M3;
  // staging items per thread: bf16 rows are 64 chunks of 16 bytes; E4M3 rows
  // 28 code chunks + 8 tail chunks
  constexpr int CPR = F8 ? 36 : 64;                 // chunks per row
  constexpr int IT = (R * CPR + NT - 1) / NT;       // 4 (bf16) or 3 (E4M3)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][R * KP];
  __shared__ __attribute__((aligned(16))) float Sp[8][2][4][64];            // partial logits per wave
  __shared__ __attribute__((aligned(16))) float St[F8 ? 4 : 1][2][4][64];   // E4M3: RoPE-tail logits per head group
  __shared__ uint64_t rtab[MAXL];                                           // row addresses of the split
  __shared__ __attribute__((aligned(16))) float rsc[2][R];                  // E4M3 row scales
  __shared__ __attribute__((aligned(16))) float rbi[2][R];                  // logit bias: 0, or -inf (skipped)
  // cos / sin tables of pair j: [0] at p in the raw frame, [1] at p in the
  // compressed frame, [2] the frame switch (angle p (theta_c - theta))
  __shared__ float cs_[3][32], sn_[3][32];
  __shared__ u32x4 qt_[4][2][64];   // the tail waves' stored query tails, for the frame switch
  __shared__ float qss[2][64];      // query norm: each channel half's sum of squares per head
  __shared__ int tk_lim, any_bad, any_row;   // any_row: the split has an entry that is not skipped

  const int qn = blockIdx.x / nsplit, split = blockIdx.x - qn * nsplit;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 3, cg = wave >> 2;
  const bool tailw = cg == 1;   // this wave's half holds the RoPE tail (channels 448..511)
  const int r = lane & 15, g = lane >> 4;
  const int H = P.H;
  const int head = blockIdx.y * 64 + 16 * hg + r;
  const bool decode = pos != nullptr;
  const int j0 = split * rows_per_split;
  // splits of raw slots need no list.  Neither this test nor the loads below
  // involve the query's position, so they go out before its load returns.
  const int K = (P.ratio == 4 && topk && j0 + rows_per_split > SWA) ? P.topk : 0;

  // ---- the split's row list -> rtab.  The top-k list ends at its first
  // entry >= V; entries < 0 are skipped.  The list's loads go out first, then
  // the query's (which depend on nothing), so that waiting for the list does
  // not wait for the query; the prologue's barriers order LDS only.
  int tkv[MAXK / NT];
  if (K) {
    const int32_t* tkg = topk + (size_t)qn * P.topk;
#pragma unroll
    for (int e = 0; e < MAXK / NT; ++e) tkv[e] = tkg[min(tid + NT * e, K - 1)];
  }
  u32x4 Bq[8];
  {
    const uint16_t* qr = q + ((size_t)qn * H + head) * D + 256 * cg + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) Bq[ks] = *(const u32x4*)(qr + 32 * ks);
  }
  if (tid == 0) {
    tk_lim = K;
    any_bad = 0;
    any_row = 0;
  }
  const AttnQuery A = attn_query(P, pos, seq_fixed, pos0, qn);
  const int j1 = min(A.n_list, j0 + rows_per_split);
  const int ntiles = j1 > j0 ? (j1 - j0 + R - 1) / R : 0;
  const int nent = (ntiles + 4) * R;   // table entries incl. the padding tiles the loop issues
  const uint8_t* dummy = g_attn_zero_row;
  const int tile0 = j0 / R;                                  // list tile of the split's first tile
  const bool start_comp = tile0 >= RAW_TILES;
  const bool switches = P.two_bases && !start_comp && tile0 + ntiles > RAW_TILES;
  const bool end_comp = tile0 + ntiles > RAW_TILES;          // frame of the split's output
  const bool inv = !(P.flags & CKV_FLAG_NO_INV_ROPE);
  const float c2 = P.scale * LOG2E;                          // logit -> base-2 units
  lds_barrier();
  if (K) {
    int first = K;
#pragma unroll
    for (int e = 0; e < MAXK / NT; ++e)
      if (tid + NT * e < K && tkv[e] >= A.V) first = min(first, tid + NT * e);
    if (first < K) atomicMin(&tk_lim, first);
  }
  if (tid < 96) {
    const int j = tid & 31, f = tid >> 5;
    float c, sn;
    if (f == 0) rope_cs(P, j, (double)max(A.p, 0), &c, &sn);
    else if (f == 1) rope_cs_c(P, j, (double)max(A.p, 0), &c, &sn);
    else rope_cs_switch(P, j, (double)max(A.p, 0), &c, &sn);
    cs_[f][j] = c;
    sn_[f][j] = sn;
  }
  lds_barrier();
  const int tk_end = tk_lim;
  for (int x = tid; x < min(nent, MAXL); x += NT) {   // raw slots, padding
    const int j = j0 + x;
    const int t = A.p - SWA + 1 + j;
    uint64_t v = (uint64_t)dummy | 1u;
    if (j < j1 && j < SWA && t >= 0) {
      v = (uint64_t)(decode ? cc.raw + ((size_t)A.seq * P.swa + (t & (P.swa - 1))) * P.row_bytes
                            : cc.stage + (size_t)(t - pos0 + P.swa - 1) * P.row_bytes);
      any_row = 1;
    }
    if (!(j < j1 && j >= SWA && P.ratio == 4)) rtab[x] = v;
  }
  if (CMP && tid == 0 && min(j1, SWA + A.V) > max(j0, SWA)) any_row = 1;   // computed entries
  if (K) {   // top-k entries of this split, from the registers that hold them
#pragma unroll
    for (int e = 0; e < MAXK / NT; ++e) {
      const int jj = tid + NT * e;
      const int x = SWA + jj - j0;
      if (jj < K && x >= 0 && SWA + jj < j1) {
        const int row = tkv[e];
        const bool ok = jj < tk_end && row >= 0 && row < A.V;
        if (ok) any_row = 1;
        rtab[x] = ok ? (uint64_t)(cc.comp + row_slot_rd(P, A.seq, row) * P.row_bytes) : ((uint64_t)dummy | 1u);
      }
    }
  }
  // query norm: this lane's 64 channels' squares, summed over the head's four
  // lanes here and over the two channel halves through LDS
  const bool qnorm = P.flags & CKV_FLAG_Q_NORM;
  if (qnorm) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = lo_bf16(Bq[ks][e]), b = hi_bf16(Bq[ks][e]);
        ss = fmaf(a, a, fmaf(b, b, ss));
      }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (g == 0) qss[cg][16 * hg + r] = ss;
  }
  lds_barrier();
  // 1 without the norm (an exact multiply)
  const float qsc = qnorm ? 1.f / sqrtf((qss[0][16 * hg + r] + qss[1][16 * hg + r]) * (1.f / D) + P.eps) : 1.f;
  // address of ratio-128 compressed entry j (list index)
  auto comp_addr = [&](int j) -> uint64_t {
    const int jj = j - SWA;
    return (j < j1 && jj < A.V) ? (uint64_t)(cc.comp + row_slot_rd(P, A.seq, jj) * P.row_bytes)
                                : ((uint64_t)dummy | 1u);
  };
  // address of split entry x (any x, for the fp32 recompute)
  auto addr_of = [&](int x) -> uint64_t {
    if (CMP && j0 + x >= SWA) return comp_addr(j0 + x);
    return rtab[min(x, MAXL - 1)];
  };

  // staging: item e of this thread is chunk it % CPR of tile row it / CPR,
  // it = tid + NT e; items past the tile read the zero row and are dropped.
  // Thread t < 32 also loads the scale of row t (E4M3) and its skip bit.
  struct Stg {
    u32x4 v[IT];
    float s;
    bool sok;
  };
  auto issue = [&](Stg& S, int tile) {
    // tiles hold one row class; on CMP layers a compressed tile's addresses
    // are computed (a uniform branch)
    const bool ctile = CMP && __builtin_amdgcn_readfirstlane(j0 + tile * R) >= SWA;
#pragma unroll
    for (int e = 0; e < IT; ++e) {
      const int it = tid + NT * e;
      const int row = min(it / CPR, R - 1), ch = it % CPR;
      const int x = tile * R + row;
      const uint64_t ra = ctile ? comp_addr(j0 + x) : rtab[min(x, MAXL - 1)];
      const int off = !F8 ? 16 * ch : (ch < 28 ? 16 * ch : DN + 16 * (ch - 28));
      S.v[e] = ldg16((ra & ~(uint64_t)1) + off);
    }
    const int xs = tile * R + (tid & 31);
    const uint64_t rs = ctile ? comp_addr(j0 + xs) : rtab[min(xs, MAXL - 1)];
    S.s = F8 ? ldg_f32((rs & ~(uint64_t)1) + DN + 128) : 1.f;
    S.sok = !(rs & 1u);
  };
  auto pin = [&](Stg& S) {
#pragma unroll
    for (int e = 0; e < IT; ++e) asm volatile("" : "+v"(S.v[e]) : : "memory");
    asm volatile("" : "+v"(S.s) : : "memory");
  };
  auto commit = [&](const Stg& S, int buf) {
    uint16_t* kb = Ks[buf];
#pragma unroll
    for (int e = 0; e < IT; ++e) {
      const int it = tid + NT * e;
      const int row = it / CPR, ch = it % CPR;
      if (it < R * CPR) {
        const u32x4 v = S.v[e];   // skipped entries read the zero row
        if (!F8) {
          *(u32x4*)&kb[tix(row, 8 * ch)] = bf16x8_to_f16(v);
        } else if (ch < 28) {   // 16 codes -> 16 fp16 channels
          *(u32x4*)&kb[tix(row, 16 * ch)] = e4m3x8_to_f16(v[0], v[1]);
          *(u32x4*)&kb[tix(row, 16 * ch + 8)] = e4m3x8_to_f16(v[2], v[3]);
        } else {                // 8 bf16 tail channels
          *(u32x4*)&kb[tix(row, DN + 8 * (ch - 28))] = bf16x8_to_f16(v);
        }
      }
    }
    if (tid < 32) {
      rbi[buf][tid] = S.sok ? 0.f : -INFINITY;
      if (F8) rsc[buf][tid] = S.s;
    }
  };

  // query of this lane's head in fp16, channels 256 cg + 32 ks + 8 g .. +7
  // (B operand); the tail rotated at p in the frame of the split's first row
  // class.  LDS keeps the stored tail for the frame switch.
  Stg S0, S1;
  {
    const int f0 = start_comp ? 1 : 0;
    // the first tiles' loads go out behind the query's
    issue(S0, 0);
    if (!F8) issue(S1, 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 v = Bq[ks];
      if (tailw && ks >= 6) {
        if (switches) qt_[hg][ks - 6][lane] = v;
        const int jb = (32 * ks + 8 * g + 256 - DN) / 2;   // first pair index of this chunk
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float a = lo_bf16(v[e]) * qsc, b = hi_bf16(v[e]) * qsc;
          rot2(a, b, cs_[f0][jb + e], sn_[f0][jb + e]);
          Bq[ks][e] = pk_f16(a, b);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) Bq[ks][e] = pk_f16(lo_bf16(v[e]) * qsc, hi_bf16(v[e]) * qsc);
      }
    }
  }

  float m_i = -INFINITY, l_i = 0.f;   // running max (base-2 units) and sum of this lane's head
  f32x4 O[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) O[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // transpose-read addresses: lane 16 g + 4 j + a reads row base + j,
  // channels ch0 + 4 a .. + 3 (base 4 g, then 16 + 4 g)
  const int tr_row = 4 * g + ((lane & 15) >> 2), tr_col = 4 * (lane & 3);
  // per-lane tile offsets of the logit and PV reads; each access adds a
  // compile-time offset
  const int s_lane = tix(r, 256 * cg + 8 * g);
  const int p_lane = tix(tr_row, 256 * cg + tr_col);

  // raw slots -> compressed entries: the query tail is rotated afresh in the
  // compressed frame, and the output tail turns by p (theta_c - theta) (tail
  // waves only; channels 448 + 16 (n - 12) + 4 g + i of O[n] are pairs
  // 8 (n - 12) + 2 g + i / 2)
  auto frame_switch = [&]() {
    if (!tailw) return;
#pragma unroll
    for (int ks = 6; ks < 8; ++ks) {
      const int jb = (32 * ks + 8 * g + 256 - DN) / 2;
      const u32x4 qs = qt_[hg][ks - 6][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = lo_bf16(qs[e]) * qsc, b = hi_bf16(qs[e]) * qsc;
        rot2(a, b, cs_[1][jb + e], sn_[1][jb + e]);
        Bq[ks][e] = pk_f16(a, b);
      }
    }
    if (inv) {
#pragma unroll
      for (int n = 12; n < 16; ++n)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int jp = 8 * (n - 12) + 2 * g + i / 2;
          float a = O[n][i], b = O[n][i + 1];
          rot2(a, b, cs_[2][jp], sn_[2][jp]);
          O[n][i] = a;
          O[n][i + 1] = b;
        }
    }
  };

  auto tile_math = [&](int buf) {
    const uint16_t* kb = Ks[buf];
    // partial logits S^T over this wave's channel half: rows 16 nt + 4 g + i;
    // with E4M3 rows the tail wave keeps its RoPE channels (k-steps 6, 7)
    // apart (the row scale multiplies the code channels only).  Element
    // tix(16 nt + r, 256 cg + 32 ks + 8 g) is s_lane + 16 nt KP + 32 ks (the
    // swizzle flips bit 0 of the chunk, which ks does not touch).
    const uint16_t* ks_ = kb + s_lane;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 an = {0.f, 0.f, 0.f, 0.f}, at = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const u32x4 a = *(const u32x4*)(ks_ + 16 * nt * KP + 32 * ks);
        an = mfma_f16(a, Bq[ks], an);
      }
      const u32x4 a6 = *(const u32x4*)(ks_ + 16 * nt * KP + 192);
      const u32x4 a7 = *(const u32x4*)(ks_ + 16 * nt * KP + 224);
      if (F8 && tailw) {
        at = mfma_f16(a6, Bq[6], at);
        at = mfma_f16(a7, Bq[7], at);
        *(f32x4*)&St[F8 ? hg : 0][nt][0][4 * lane] = at;
      } else {
        an = mfma_f16(a6, Bq[6], an);
        an = mfma_f16(a7, Bq[7], an);
      }
      *(f32x4*)&Sp[wave][nt][0][4 * lane] = an;
    }
    lds_barrier();
    // logits of this lane's head for its 8 rows, in base-2 units; online
    // softmax with one head per lane: the tile max and sum reduce 8 values in
    // the lane and across the 4 lanes of the head (lanes r, r + 16, r + 32,
    // r + 48).  The reference max moves only when a tile's max exceeds it by
    // more than e^8, so the rescale of the accumulators is rare.
    float Sv[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const f32x4 n0 = *(const f32x4*)&Sp[hg][nt][0][4 * lane];
      const f32x4 n1 = *(const f32x4*)&Sp[hg + 4][nt][0][4 * lane];
      const f32x4 bi = *(const f32x4*)&rbi[buf][16 * nt + 4 * g];
      f32x4 tl = {0.f, 0.f, 0.f, 0.f}, sc = {1.f, 1.f, 1.f, 1.f};
      if (F8) {
        tl = *(const f32x4*)&St[F8 ? hg : 0][nt][0][4 * lane];
        sc = *(const f32x4*)&rsc[buf][16 * nt + 4 * g];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s = n0[i] + n1[i];
        if (F8) s = fmaf(s, sc[i], tl[i]);
        Sv[nt][i] = fmaf(s, c2, bi[i]);
        mx = fmaxf(mx, Sv[nt][i]);
      }
    }
    mx = rows4_max(mx);
    const bool move = mx > m_i + MOVE2;
    const float mn = move ? mx : m_i;
    const float mref = mn == -INFINITY ? 0.f : mn;   // nothing seen yet: every logit is -inf
    const float alpha = move ? __builtin_amdgcn_exp2f(m_i - mn) : 1.f;
    float ps = 0.f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(Sv[nt][i] - mref);
        Sv[nt][i] = pv;
        ps += pv;
      }
    ps = rows4_sum(ps);
    l_i = l_i * alpha + ps;
    m_i = mn;
    if (__builtin_amdgcn_readfirstlane(__ballot(alpha != 1.f) != 0ull)) {
#pragma unroll
      for (int n = 0; n < 16; ++n) O[n] *= alpha;
    }
    // PV B operands: k = 8 g + e holds rows 4 g + e (e < 4) and 16 + 4 g + e - 4
    // (e >= 4), i.e. Sv[0][e] and Sv[1][e - 4].  bpp: plain probabilities;
    // bps (E4M3): times the row scale, for the non-RoPE channels
    u32x4 bpp, bps;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int nt = e2 >> 1, i = 2 * (e2 & 1);
      const float a = Sv[nt][i], b = Sv[nt][i + 1];
      bpp[e2] = pk_f16(a, b);
      if (F8) {
        const f32x2_t sc = *(const f32x2_t*)&rsc[buf][16 * nt + 4 * g + i];
        bps[e2] = pk_f16(a * sc[0], b * sc[1]);
      } else {
        bps[e2] = bpp[e2];
      }
    }
    // channels 256 cg + 16 n + (0..15): n < 12 non-RoPE on both waves; n >= 12
    // non-RoPE on cg 0, RoPE tail on the tail wave
    const u32x4 bhi = tailw ? bpp : bps;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      // element tix(tr_row, 256 cg + 16 n + tr_col) = p_lane + 16 n; rows
      // tr_row and tr_row + 16 share bit 2, so one swizzled offset serves both
      const uint16_t* tp = kb + p_lane + 16 * n;
      const u32x2 lo4 = ds_tr16(tp), hi4 = ds_tr16(tp + 16 * KP);
      const u32x4 a = {lo4[0], lo4[1], hi4[0], hi4[1]};
      O[n] = mfma_f16(a, n < 12 ? bps : bhi, O[n]);
    }
  };

  // tile loop in pairs, both halves always commit and issue (see above).
  // Iteration t: tile t sits in LDS buffer 0 (committed earlier); multiply
  // it, commit tile t + 1 into buffer 1 and issue the next loads; then the
  // same with the buffers swapped.  Each tile_math has its own barrier (logit
  // halves), and one barrier per tile publishes the next buffer.  bf16 rows
  // keep two tiles' loads in flight in registers (S0, S1); E4M3 rows one
  // (S0 only: measured slower with two, 29 -> 32 us on the window-only
  // decode step).  The frame switch runs before the first compressed tile (a
  // scalar branch).
  constexpr bool TWO = !F8;
  pin(S0);
  commit(S0, 0);
  if (TWO) issue(S0, 2);
  else issue(S0, 1);
  lds_barrier();
  for (int t = 0; t < ntiles; t += 2) {
    if (switches && tile0 + t == RAW_TILES) frame_switch();
    tile_math(0);
    if (TWO) {
      pin(S1);
      commit(S1, 1);
      issue(S1, t + 3);
    } else {
      pin(S0);
      commit(S0, 1);
      issue(S0, t + 2);
    }
    lds_barrier();
    if (t + 1 < ntiles) {
      if (switches && tile0 + t + 1 == RAW_TILES) frame_switch();
      tile_math(1);
    }
    pin(S0);
    commit(S0, 0);
    issue(S0, TWO ? t + 4 : t + 3);
    lds_barrier();
  }

  const int fe = end_comp ? 1 : 0;   // frame the output ended in
  // the range guard's checks (see above): a sum that is not finite, or zero
  // although the split has rows, an output that is not finite (the sum of its
  // values is then inf or NaN), or a normalised output beyond the fp16
  // partial's range, sends the split to the fp32 recompute
  const float il = l_i > 0.f ? __builtin_amdgcn_rcpf(l_i) : 0.f;
  float om = 0.f, os = 0.f;
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    om = fmaxf(om, fmaxf(fmaxf(fabsf(O[n][0]), fabsf(O[n][1])), fmaxf(fabsf(O[n][2]), fabsf(O[n][3]))));
    os += (O[n][0] + O[n][1]) + (O[n][2] + O[n][3]);
  }
  bool bad = !(l_i < INFINITY) || (l_i == 0.f && any_row) || !(os - os == 0.f);
  if (nsplit > 1) bad |= !(om * il < 65504.f);
  if (__ballot(bad) != 0ull && lane == 0) any_bad = 1;
  lds_barrier();
  if (any_bad) {
    const float scale = P.scale;
    // ---- range guard: the split again, in fp32, from the stored rows.  Four
    // passes of 16 heads, 32 threads per head, thread `sub` holding channels
    // 16 sub .. +15 (subs 28..31 hold the RoPE tail, pairs 8 (sub - 28) ..).
    const int hh = tid >> 5, sub = tid & 31, c0 = 16 * sub;
    const bool tl = c0 >= DN;
    const int jq = tl ? (c0 - DN) / 2 : 0;
    const int f0 = start_comp ? 1 : 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int hd = blockIdx.y * 64 + 16 * pass + hh;
      float qv[16], acc[16];
      {
        const u32x4* qr = (const u32x4*)(q + ((size_t)qn * H + hd) * D + c0);
        const u32x4 w0 = qr[0], w1 = qr[1];
        float gsc = 1.f;   // query norm over the head's 32 threads
        if (qnorm) {
          float ss = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a0 = lo_bf16(w0[i]), b0 = hi_bf16(w0[i]), a1 = lo_bf16(w1[i]), b1 = hi_bf16(w1[i]);
            ss = fmaf(a0, a0, fmaf(b0, b0, fmaf(a1, a1, fmaf(b1, b1, ss))));
          }
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o, 64);
          gsc = 1.f / sqrtf(ss * (1.f / D) + P.eps);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x4 w = h2 ? w1 : w0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float a = lo_bf16(w[i]) * gsc, b = hi_bf16(w[i]) * gsc;
            if (tl) rot2(a, b, cs_[f0][jq + 4 * h2 + i], sn_[f0][jq + 4 * h2 + i]);
            qv[8 * h2 + 2 * i] = a * scale;
            qv[8 * h2 + 2 * i + 1] = b * scale;
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = 0.f;
      float m = -INFINITY, l = 0.f;
      for (int x = 0; x < ntiles * R; ++x) {
        if (switches && x == (RAW_TILES - tile0) * R && tl) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            rot2(qv[2 * e], qv[2 * e + 1], cs_[2][jq + e], sn_[2][jq + e]);
            if (inv) rot2(acc[2 * e], acc[2 * e + 1], cs_[2][jq + e], sn_[2][jq + e]);
          }
        }
        const uint64_t ra = addr_of(x);
        if (ra & 1u) continue;
        const uint8_t* rp = (const uint8_t*)ra;
        float v[16];
        if (!F8 || tl) {
          const u32x4* src = (const u32x4*)(F8 ? rp + DN + 2 * (c0 - DN) : rp + 2 * c0);
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const u32x4 w = src[h2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[8 * h2 + 2 * i] = lo_bf16(w[i]);
              v[8 * h2 + 2 * i + 1] = hi_bf16(w[i]);
            }
          }
        } else {
          const float sr = *(const float*)(rp + DN + 128);
          const u32x4 w = *(const u32x4*)(rp + c0);
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = e4m3_to_f32((w[i >> 2] >> (8 * (i & 3))) & 0xffu) * sr;
        }
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) dot += qv[i] * v[i];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) dot += __shfl_xor(dot, o, 64);
        const float mn = fmaxf(m, dot);
        const float f = __expf(m - mn), pw = __expf(dot - mn);
        l = l * f + pw;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = acc[i] * f + pw * v[i];
        m = mn;
      }
      const float il = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] *= il;
      if (tl && inv) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rot2(acc[2 * e], acc[2 * e + 1], cs_[fe][jq + e], -sn_[fe][jq + e]);
      }
      if (nsplit == 1) {
        if (P.flags & CKV_FLAG_OUT_FP8) {   // fp8 record: group sub / 8 = 8 lanes
          float am = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) am = fmaxf(am, fabsf(acc[c]));
#pragma unroll
          for (int o = 1; o < 8; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
          const float sc = am > 0.f ? am / 448.f : 1.f;
          uint8_t* rec = (uint8_t*)out + ((size_t)qn * H + hd) * out8_bytes(D);
          const u32x4 w = {e4m3x4(acc[0] / sc, acc[1] / sc, acc[2] / sc, acc[3] / sc),
                           e4m3x4(acc[4] / sc, acc[5] / sc, acc[6] / sc, acc[7] / sc),
                           e4m3x4(acc[8] / sc, acc[9] / sc, acc[10] / sc, acc[11] / sc),
                           e4m3x4(acc[12] / sc, acc[13] / sc, acc[14] / sc, acc[15] / sc)};
          *(u32x4*)(rec + c0) = w;
          if ((sub & 7) == 0) *(float*)(rec + D + 4 * (sub >> 3)) = sc;
          continue;
        }
#pragma unroll
        for (int c = 0; c < 16; c += 2)
          *(uint32_t*)&out[((size_t)qn * H + hd) * D + c0 + c] = pack_bf16x2(acc[c], acc[c + 1]);
        continue;
      }
      // partial: the normalised output times 2^-e (e chosen so that the
      // head's largest magnitude stays below 2^15) as two fp16 halves, the
      // high one in the usual place and the low-order remainder in the second
      // half of the partial buffer (about 22 significant bits: values this
      // large can cancel in the merge); the merge multiplies by 2^e
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(acc[c]));
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      int ex = 0;
      if (amax >= 16384.f) {   // amax = m 2^f, m in [0.5, 1): scaled to m 2^14
        (void)frexpf(amax, &ex);
        ex -= 14;
      }
      const float down = ldexpf(1.f, -ex);
      const size_t pb = ((size_t)qn * nsplit + split) * H + hd;
      const size_t lo_half = (size_t)gridDim.x * H * D;   // fp16 entries of the high halves
      uint16_t* ph = (uint16_t*)part_o;
#pragma unroll
      for (int c = 0; c < 16; c += 2) {
        const float a = acc[c] * down, b = acc[c + 1] * down;
        const uint32_t hi = pk_f16(a, b);
        *(uint32_t*)&ph[pb * D + part_pos(c0 + c)] = hi;
        *(uint32_t*)&ph[lo_half + pb * D + part_pos(c0 + c)] = pk_f16(a - lo_f16(hi), b - hi_f16(hi));
      }
      if (sub == 0) *(float4*)(part_ml + pb * 4) = make_float4(m, l, ldexpf(1.f, ex), 1.f);
    }
    return;
  }

  // lane (r, g) holds channels 256 cg + 16 n + 4 g + i of head `head`;
  // normalise and rotate the tail back by -p in the frame the split ended in
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    O[n] *= il;
    if (tailw && n >= 12 && inv) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int jp = 8 * (n - 12) + 2 * g + i / 2;
        float a = O[n][i], b = O[n][i + 1];
        rot2(a, b, cs_[fe][jp], -sn_[fe][jp]);
        O[n][i] = a;
        O[n][i + 1] = b;
      }
    }
  }
  if (nsplit == 1) {
    if (P.flags & CKV_FLAG_OUT_FP8) {
      // fp8 record: this wave's channels are groups 2 cg (n < 8) and 2 cg + 1,
      // each spread over the head's four lanes (l ^ 16, l ^ 32)
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const float m = fmaxf(fmaxf(fabsf(O[n][0]), fabsf(O[n][1])), fmaxf(fabsf(O[n][2]), fabsf(O[n][3])));
        if (n < 8) a0 = fmaxf(a0, m);
        else a1 = fmaxf(a1, m);
      }
      a0 = rows4_max(a0);
      a1 = rows4_max(a1);
      const float s0 = a0 > 0.f ? a0 / 448.f : 1.f, s1 = a1 > 0.f ? a1 / 448.f : 1.f;
      uint8_t* rec = (uint8_t*)out + ((size_t)qn * H + head) * out8_bytes(D);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const float sc = n < 8 ? s0 : s1;
        *(uint32_t*)(rec + 256 * cg + 16 * n + 4 * g) =
            e4m3x4(O[n][0] / sc, O[n][1] / sc, O[n][2] / sc, O[n][3] / sc);
      }
      if (g == 0) *(float2*)(rec + D + 8 * cg) = make_float2(s0, s1);
      return;
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int ch = 256 * cg + 16 * n + 4 * g;
      u32x2 w = {pack_bf16x2(O[n][0], O[n][1]), pack_bf16x2(O[n][2], O[n][3])};
      *(u32x2*)&out[((size_t)qn * H + head) * D + ch] = w;
    }
    return;
  }
  // partial: this split's normalised output O / l in fp16 (half the bytes of
  // fp32 to write here and to read in the merge), in the order of part_pos
  // (this lane's 64 channels contiguous), plus (m, l, 1) with m in
  // natural-log units
  const size_t pb = ((size_t)qn * nsplit + split) * H + head;
  uint16_t* ph = (uint16_t*)part_o;
#pragma unroll
  for (int n = 0; n < 16; n += 2) {
    const u32x4 w = {pk_f16(O[n][0], O[n][1]), pk_f16(O[n][2], O[n][3]), pk_f16(O[n + 1][0], O[n + 1][1]),
                     pk_f16(O[n + 1][2], O[n + 1][3])};
    *(u32x4*)&ph[pb * D + 256 * cg + 64 * g + 4 * n] = w;
  }
  if (g == 0 && cg == 0) *(float4*)(part_ml + pb * 4) = make_float4(m_i * LN2, l_i, 1.f, 0.f);
}


// ----------------------------------------------------------------- vector
// Any formats.  Block of 256 = 16 heads x 16 lanes; lane `sub` owns channels
// [sub*dpt, (sub+1)*dpt).  grid (queries, splits, H / 16).  Leaves the
// split's unnormalised output, rotated back by -p in the frame it ended in,
// and (max, sum, 1).
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
  const bool start_comp = j0 >= P.swa, end_comp = j1 > P.swa;
  const bool switches = P.two_bases && !start_comp && end_comp;
  const bool inv = !(P.flags & CKV_FLAG_NO_INV_ROPE);
  const double pp = (double)max(A.p, 0);

  float qv[32], acc[32];
  const int c0 = sub * dpt;
  float qsc = 1.f;   // query norm: the head's sum of squares over its 16 lanes
  if (P.flags & CKV_FLAG_Q_NORM) {
    float ss = 0.f;
    for (int e = 0; e < dpt; ++e) {
      const float a = load_val<ACTF>(q, ((size_t)qn * H + h) * d + c0 + e);
      ss = fmaf(a, a, ss);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
    qsc = 1.f / sqrtf(ss / (float)d + P.eps);
  }
  for (int e = 0; e < dpt; e += 2) {
    const size_t o = ((size_t)qn * H + h) * d + c0 + e;
    float a = load_val<ACTF>(q, o) * qsc, b = load_val<ACTF>(q, o + 1) * qsc;
    if (c0 + e >= dn) {
      float cs, sn;
      if (start_comp) rope_cs_c(P, (c0 + e - dn) / 2, pp, &cs, &sn);
      else rope_cs(P, (c0 + e - dn) / 2, pp, &cs, &sn);
      rot2(a, b, cs, sn);
    }
    qv[e] = a * P.scale;
    qv[e + 1] = b * P.scale;
    acc[e] = acc[e + 1] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = j0; j < j1; ++j) {
    if (switches && j == P.swa) {   // raw slots -> compressed entries: change frame
      for (int e = 0; e < dpt; e += 2) {
        if (c0 + e < dn) continue;
        float cs, sn;
        rope_cs_switch(P, (c0 + e - dn) / 2, pp, &cs, &sn);
        rot2(qv[e], qv[e + 1], cs, sn);
        if (inv) rot2(acc[e], acc[e + 1], cs, sn);
      }
    }
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
  if (inv) {   // rotate back by -p in the frame the split ended in
    for (int e = 0; e < dpt; e += 2) {
      if (c0 + e < dn) continue;
      float cs, sn;
      if (end_comp) rope_cs_c(P, (c0 + e - dn) / 2, pp, &cs, &sn);
      else rope_cs(P, (c0 + e - dn) / 2, pp, &cs, &sn);
      rot2(acc[e], acc[e + 1], cs, -sn);
    }
  }
  const size_t pb = ((size_t)qn * nsplit + split) * H + h;
  for (int e = 0; e < dpt; ++e) part_o[pb * d + c0 + e] = acc[e];
  if (sub == 0) *(float4*)(part_ml + pb * 4) = make_float4(m, l, 1.f, 0.f);
}

// ----------------------------------------------------------------- merge
// grid (queries, H); block d/4 threads, each four adjacent channels.  The
// splits' (max, sum, scale) entries are read once into LDS.  HALF: the
// partials are fp16 normalised outputs O_s / l_s times 1 / scale_s (tile
// kernel), combined with weights l_s scale_s exp(m_s - M); otherwise fp32
// unnormalised O_s with weights exp(m_s - M).  The splits have already
// rotated their outputs back, so the merge only adds.
template <int ACTF, bool HALF, bool OUT8 = false>
__global__ __launch_bounds__(128) void k_attn_merge(LayerParams P, const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml, int nsplit,
                                                    void* __restrict__ out) {
  __shared__ float wsh[kMaxSplits];
  __shared__ float lsh[kMaxSplits];   // 1: the split also left a low-order half (fp16 partials)
  __shared__ float Lsh;
  __shared__ int any_lo;
  const int qn = blockIdx.x, h = blockIdx.y, H = P.H, d = P.d;
  const int c = 4 * threadIdx.x;
  const size_t b0 = (size_t)qn * nsplit * H + h;
  // Loads first, all unconditional (indices clamped): the splits' (max, sum,
  // scale) entries (lane l of each wave: splits l + 64 e), then this thread's
  // four channels of the first kPF splits' partials, so that one memory round
  // trip serves both (the weights wait only for the entries, issued first).
  constexpr int kPF = 16;
  const int cl = min(c, d - 4);
  float4 mlv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int sidx = (threadIdx.x & 63) + 64 * e;
    mlv[e] = *(const float4*)(part_ml + (b0 + (size_t)min(sidx, nsplit - 1) * H) * 4);
  }
  // fp16 partials (the tile kernel's) hold channel c at attn::part_pos(c)
  const int pcl = HALF ? attn::part_pos(cl) : cl;
  auto load_part = [&](int sp) -> float4 {
    const size_t o = (b0 + (size_t)min(sp, nsplit - 1) * H) * d + pcl;
    if constexpr (HALF) {
      const _Float16* hp = (const _Float16*)part_o + o;
      return make_float4((float)hp[0], (float)hp[1], (float)hp[2], (float)hp[3]);
    } else {
      return *(const float4*)(part_o + o);
    }
  };
  __builtin_amdgcn_sched_barrier(0);   // (keeps the entries' loads ahead of the partials')
  float4 v0[kPF];
#pragma unroll
  for (int j = 0; j < kPF; ++j) v0[j] = load_part(j);
  {
    // max over splits with rows, then each split's weight exp(m_s - M)
    float m[4], l[4], sc[4];
    float M = -INFINITY, lo_any = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // splits past nsplit weigh 0
      const int sidx = (threadIdx.x & 63) + 64 * e;
      const bool in = sidx < nsplit;
      m[e] = in ? mlv[e].x : -INFINITY;
      l[e] = in ? mlv[e].y : 0.f;
      sc[e] = mlv[e].z;
      if (l[e] > 0.f) M = fmaxf(M, m[e]);
      if (in) lo_any = fmaxf(lo_any, mlv[e].w);
    }
    M = wave_max(M);
    lo_any = wave_max(lo_any);
    float L = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sidx = (threadIdx.x & 63) + 64 * e;
      const float wgt = l[e] > 0.f ? __expf(m[e] - M) : 0.f;
      if (threadIdx.x < 64 && sidx < nsplit) {
        wsh[sidx] = HALF ? l[e] * wgt * sc[e] : wgt;
        lsh[sidx] = mlv[e].w;
      }
      L += l[e] * wgt;
    }
    L = wave_sum(L);
    if (threadIdx.x == 0) {
      Lsh = L;
      any_lo = HALF && lo_any > 0.f;
    }
  }
  __syncthreads();
  if (c >= d) return;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  auto accum = [&](const float4& x, int sp) {
    const float wgt = sp < nsplit ? wsh[sp] : 0.f;
    a.x += x.x * wgt;
    a.y += x.y * wgt;
    a.z += x.z * wgt;
    a.w += x.w * wgt;
  };
#pragma unroll
  for (int j = 0; j < kPF; ++j) accum(v0[j], j);
  for (int s0 = kPF; s0 < nsplit; s0 += 8) {   // further splits, eight loads in flight at a time
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = load_part(s0 + j);
#pragma unroll
    for (int j = 0; j < 8; ++j) accum(v[j], s0 + j);
  }
  if (any_lo) {   // splits recomputed by the range guard: their low-order halves
    const size_t lo_half = (size_t)gridDim.x * nsplit * H * d;
    for (int sp = 0; sp < nsplit; ++sp) {
      if (lsh[sp] == 0.f) continue;
      const _Float16* hp = (const _Float16*)part_o + lo_half + (b0 + (size_t)sp * H) * d + pcl;
      const float wgt = wsh[sp];
      a.x += (float)hp[0] * wgt;
      a.y += (float)hp[1] * wgt;
      a.z += (float)hp[2] * wgt;
      a.w += (float)hp[3] * wgt;
    }
  }
  const float inv = Lsh > 0.f ? 1.f / Lsh : 0.f;
  const float o[4] = {a.x * inv, a.y * inv, a.z * inv, a.w * inv};
  if constexpr (OUT8) {
    // fp8 record of this (query, head): group c / 128 = the 32 lanes of this
    // half-wave; its scale max|o| / 448, written by the group's first lane
    float am = fmaxf(fmaxf(fabsf(o[0]), fabsf(o[1])), fmaxf(fabsf(o[2]), fabsf(o[3])));
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
    const float sc = am > 0.f ? am / 448.f : 1.f;
    uint8_t* rec = (uint8_t*)out + ((size_t)qn * H + h) * attn::out8_bytes(d);
    *(uint32_t*)(rec + c) = attn::e4m3x4(o[0] / sc, o[1] / sc, o[2] / sc, o[3] / sc);
    if ((c & 127) == 0) *(float*)(rec + d + 4 * (c >> 7)) = sc;
  } else {
    const size_t oo = ((size_t)qn * H + h) * d + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_val<ACTF>(out, oo + e, o[e]);
  }
}

// ----------------------------------------------------------------- launcher

int launch_attn(const LayerParams& P, const Cache& c, const void* q, const int32_t* pos, int seq,
                int pos0, int nq, const int32_t* topk, void* out, const WsLayout& L, uint8_t* ws,
                void* stream) {
  hipStream_t st = (hipStream_t)stream;
  float* po = (float*)(ws + L.part_o);
  float* pml = (float*)(ws + L.part_ml);
  const int ns = L.attn_splits, rps = L.attn_rows_per_split;
  if (attn_uses_tiles(P)) {
    dim3 grid(nq * ns, P.H / 64);
    const uint16_t* qq = (const uint16_t*)q;
    uint16_t* oo = (uint16_t*)out;
    const bool cmp = P.ratio == 128;
#define CKV_AT(KF, CM) \
  hipLaunchKernelGGL((k_attn_tile<KF, CM>), grid, dim3(512), 0, st, P, c, qq, pos, seq, pos0, topk, rps, ns, po, pml, oo)
    if (P.kv_fmt == CKV_BF16 && cmp) CKV_AT(CKV_BF16, true);
    else if (P.kv_fmt == CKV_BF16) CKV_AT(CKV_BF16, false);
    else if (cmp) CKV_AT(CKV_E4M3, true);
    else CKV_AT(CKV_E4M3, false);
#undef CKV_AT
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
  const bool half = attn_uses_tiles(P);
  if (P.flags & CKV_FLAG_OUT_FP8)   // (validated: the tiled path, bf16 activations)
    hipLaunchKernelGGL((k_attn_merge<CKV_BF16, true, true>), mg, dim3(128), 0, st, P, po, pml, ns, out);
  else if (P.act_fmt == CKV_F32 && half)
    hipLaunchKernelGGL((k_attn_merge<CKV_F32, true>), mg, dim3(128), 0, st, P, po, pml, ns, out);
  else if (P.act_fmt == CKV_F32)
    hipLaunchKernelGGL((k_attn_merge<CKV_F32, false>), mg, dim3(128), 0, st, P, po, pml, ns, out);
  else if (half)
    hipLaunchKernelGGL((k_attn_merge<CKV_BF16, true>), mg, dim3(128), 0, st, P, po, pml, ns, out);
  else
    hipLaunchKernelGGL((k_attn_merge<CKV_BF16, false>), mg, dim3(128), 0, st, P, po, pml, ns, out);
  return (int)hipGetLastError();
}

}  // namespace ckv
