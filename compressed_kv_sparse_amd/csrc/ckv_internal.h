// Internal declarations of libckv: the normalised layer parameters the kernels
// take, the workspace layout, and the kernel launchers the C ABI dispatches to.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/ckv.h"

namespace ckv {

constexpr int kMaxD = 512;
constexpr int kHistBins = 4096;   // top-k histogram of the keys' top 12 bits
constexpr int kCandCap = 4096;    // decode top-k: keys of the threshold bin resolved in LDS
constexpr int kMaxSplits = 256;   // attention partial results merged per query
constexpr int kMaxDI = 128;
constexpr int kMaxTopK = 2048;    // top-k entries a query may keep (attention row table)

// Layer parameters as the kernels see them (built from ckv_layer_desc after
// validation; plain values, passed by value to every kernel).
struct LayerParams {
  int ratio, hidden, d, n_rot, H, swa, HI, DI, topk, cap, batch;
  int kv_fmt, idx_fmt, act_fmt, w_fmt;
  unsigned flags;
  double base;
  float eps, scale;
  int W;          // compressor window: 8 (ratio 4), 128 (ratio 128), 0
  int row_bytes;  // stored K=V row size
  int ncol;       // projection columns: 2d (+ 2 DI on ratio 4)
  int idx_rot;    // RoPE channels of indexer rows / queries: min(n_rot, DI)
  int idx_row_bytes;   // stored indexer row size (ckv_idx_row_bytes)
  double theta[32];    // RoPE frequencies of the raw class: base^(-2j/n_rot), j < n_rot/2
  double theta_c[32];  // the compressed class (compressed rows, indexer rows, indexer query)
  int two_bases;       // theta_c differs from theta (one frame per row class)
  // paged layout (cache->block_table): page table, pages per pool, table
  // columns per sequence, log2 of the compressed rows a page holds; blocks
  // NULL: contiguous [batch, cap] rows
  const int32_t* blocks;
  int n_pages, max_blocks, rpb_shift;
  int lanes;   // compressor lanes: 2 on two-lane c4a layers (CKV_FLAG_TWO_LANE), else 1
};

struct Weights {
  const void* wkv;
  const void* wgate;
  const float* ape;
  const float* gamma;
  const void* idx_wkv;
  const void* idx_wgate;
  const float* idx_ape;
  const float* idx_gamma;
};

struct Cache {
  uint8_t* raw;
  uint8_t* comp;
  void* idx;
  float* st_kv;
  float* st_sc;
  float* ist_kv;
  float* ist_sc;
  uint8_t* stage;
  int stage_rows;
  uint32_t* status;
  int32_t* n_tokens;   // per-sequence token count (NULL: no sequence check)
};

// Workspace carve-up (all offsets 256-byte aligned).  The sync region comes
// first in every mode: counters and histograms that must hold zeros before a
// call and that every call leaves at zero.
// Decode top-k scratch.  hist [n][kHistBins] and ctr [n][4] (finished
// blocks, sure count, candidate count) live in the zero-kept sync region;
// sure [n][top_k] and cand_key / cand_idx [n][kCandCap] are plain scratch.
struct SelWs {
  uint32_t* hist;
  uint32_t* ctr;
  uint32_t* sure;
  uint32_t* cand_key;
  uint32_t* cand_idx;
  uint8_t* qf4;   // fp4 indexer: each query's rotated, transformed query as [n][64 heads] 68-byte records
};

struct WsLayout {
  size_t sync;      // zero-kept region: hist and ctr (ratio 4)
  size_t sync_bytes;
  size_t hist;      // uint32 [batch][kHistBins]
  size_t ctr;       // uint32 [batch][4]
  size_t sure;      // uint32 [n][top_k]
  size_t cand_key;  // uint32 [n][kCandCap]
  size_t cand_idx;  // uint32 [n][kCandCap]
  size_t qf4;       // uint8 [n][64][68]   fp4 indexer decode: the queries in fp4 record form
  size_t proj;      // float [proj_splits][n][ncol]
  size_t keys;      // uint32 [n][cap]   indexer keys
  size_t pool;      // float [n][d] + [n][8][2]   c128a decode: pooled rows and slice sums
  size_t part_o;    // float [n][splits][H][d]  attention partial outputs
  size_t part_ml;   // float [n][splits][H][4]  attention partial (max, sum, scale of the stored output, 0)
  size_t total;
  int proj_splits;
  int attn_splits;
  int attn_rows_per_split;
};

// Hyper-Connection mixer parameters (validated ckv_hc_desc)
struct HcParams {
  int hidden, iters, act_fmt;
  float eps;
};

bool make_params(const ckv_layer_desc* desc, LayerParams* P);
WsLayout ws_layout(const LayerParams& P, int mode, int n);
int attn_max_rows(const LayerParams& P);
// the tiled MFMA attention kernel serves this layer (bf16 activations, bf16 or
// E4M3 rows, head_dim 512, heads a multiple of 64)
bool attn_uses_tiles(const LayerParams& P);

// ---- launchers (return 0 or a hipError_t value) ----------------------------
// projection: part[s][m][c] for columns c_begin <= c < c_end (-1: ncol) of
// the concatenated weights
int launch_proj(const LayerParams& P, const Weights& w, const void* x, int M, float* part,
                int splits, void* stream, int c_begin = 0, int c_end = -1);
// c128a decode pools channel slices of 64 in parallel blocks (head_dim a
// multiple of 64, at most 512); pool_ws: the workspace's pool region
bool c128a_sliced(const LayerParams& P);
int launch_compress_decode(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                           const int32_t* pos, int B, const float* part, int splits, float* pool_ws,
                           void* stream);
// the chunk's compressor pieces: raw staging, attention-lane rows,
// indexer-lane rows, then the state rings and the token count (in that order
// when several are asked for)
constexpr int kPfStage = 1, kPfPoolAttn = 2, kPfPoolIdx = 4, kPfState = 8, kPfAll = 15;
int launch_compress_prefill(const LayerParams& P, const Weights& w, const Cache& c, const void* u,
                            int seq, int pos0, int T, const float* part, void* stream, int parts = kPfAll);
// indexer: decode (pos != NULL, query b of sequence b) or prefill (pos == NULL,
// query n of sequence seq at position pos0 + n)
int launch_indexer(const LayerParams& P, const Cache& c, const void* qI, const float* w,
                   const int32_t* pos, int seq, int pos0, int nq, uint32_t* keys, const SelWs* sel,
                   int32_t* topk, void* stream);
// hist may be NULL: scores only
int launch_idx_score(const LayerParams& P, const Cache& c, const void* qI, const float* w,
                     const int32_t* pos, int seq, int pos0, int nq, uint32_t* keys, uint32_t* hist,
                     void* stream);
// K slices of the decode projection (partial sums added by the compressor)
constexpr int kProjSlices = 1;
// events that bracket the calling thread's next launch of an indexer score
// kernel (start, stop; either may be NULL), consumed by that launch
void arm_score_timing(void* start_event, void* stop_event);
int launch_attn(const LayerParams& P, const Cache& c, const void* q, const int32_t* pos, int seq,
                int pos0, int nq, const int32_t* topk, void* out, const WsLayout& L, uint8_t* ws,
                void* stream);
// fused decode step of a ratio-4 layer: projection + scan of the existing rows
// in one launch, then per-sequence compressor + new-row score + selection
bool step_fusable(const LayerParams& P, int B);
// every host check of ckv_decode_step, nothing enqueued (CKV_OK or the code
// ckv_decode_step would return)
int decode_step_checks(const ckv_layer_desc* desc, const ckv_layer_weights* w, const ckv_layer_cache* cache,
                       const void* x, const void* u, const void* q, const void* qI, const float* iw,
                       const int32_t* pos, int32_t B, int32_t* topk, void* out, void* ws, size_t ws_bytes,
                       LayerParams* P, WsLayout* L);
// Hyper-Connection mixer: split + Sinkhorn + pre mix, and the post mix
int launch_hc_pre(const HcParams& Hp, const float* mix, const void* h, int T, void* x, float* coef, void* stream);
int launch_hc_post(const HcParams& Hp, const float* coef, const void* h, const void* y, int T, void* hout,
                   void* stream);
int launch_step_scan_select(const LayerParams& P, const Weights& w, const Cache& c, const void* x,
                            const void* u, const void* qI, const float* wt, const int32_t* pos, int B,
                            float* proj, uint32_t* keys, const SelWs& sel, int32_t* topk, void* stream);

}  // namespace ckv
