/*
 * ckv.h -- C ABI of the MI355X compressed-KV sparse attention library (libckv.so).
 *
 * One attention layer of the DeepSeek-V4 design described in
 *   [P1] "【#3】ds4.c を読み解く" (compressor s4-s5, indexer s6, mixed attention
 *        s7, tail-only RoPE s8, FP8 cache s9, prefill chunks s3), and
 *   [P4] "vLLM DeepSeek V4 サポート" (shared K=V with inverse RoPE, c4a / c128a,
 *        DSA top-k, sliding window of 128, fused cache insertion), and
 *   [P5] "【#6】ds4.c を読み解く" (s10: KV state whose token prefix does not
 *        match the request is refused before any layer work).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer is a DEVICE pointer unless its comment says "host".
 * - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *   Every call only enqueues work on that stream and returns; nothing
 *   synchronises.  The caller keeps every buffer alive until that work ends.
 * - The caller owns every buffer.  The library allocates no device memory and
 *   keeps no pointer after a call returns, so calls on different streams over
 *   disjoint caches may overlap.  Its only mutable state is the per-thread
 *   arming of ckv_time_next_score (a profiling hook, off unless armed).
 * - Errors: each call returns CKV_OK (0) or a negative CKV_E_* code.  All
 *   argument, shape, capacity and workspace checks run on the host BEFORE any
 *   work is enqueued, so a failed call leaves every buffer untouched.
 *   Conditions only the device can see (a per-sequence position beyond the
 *   cache capacity, a negative position, a position that is not the
 *   sequence's next token) skip that sequence and OR a bit into
 *   cache->status[b] (when status is non-NULL); the caller reads it at its own
 *   synchronisation point.  No call aborts, prints or throws.
 * - A layer is described by ckv_layer_desc; ckv_validate() checks it.  The
 *   compiled kernels support: ratio 0, 4 or 128; n_rot 64; swa 128;
 *   head_dim 128 or 512 (a multiple of 64, at most 512); idx_dim 64 or 128;
 *   n_heads a multiple of 16, at most 128; idx_heads 1..64; top_k 1..2048;
 *   hidden a multiple of 64, at most 65536.
 *
 * Stored row formats (one K=V row of head_dim channels)
 * -----------------------------------------------------
 *   CKV_F32  : head_dim float32                          (4*head_dim bytes)
 *   CKV_BF16 : head_dim bfloat16                         (2*head_dim bytes)
 *   CKV_E4M3 : head_dim-n_rot OCP E4M3FN codes of z_c/s, then the n_rot RoPE
 *              channels as bfloat16, then the float32 row scale
 *              s = max|z_c|/448 over the non-RoPE channels (1 if all zero),
 *              padded to a multiple of 128 bytes (640 bytes at head_dim 512).
 *              The FP8 round trip covers the non-RoPE part only [P1 s9].
 * ckv_row_bytes() returns the size.
 *
 * Indexer rows (idx_fmt; ckv_idx_row_bytes() returns the size)
 * ------------------------------------------------------------
 *   CKV_F32  : idx_dim float32
 *   CKV_BF16 : idx_dim bfloat16
 *   CKV_FP4  : the indexer's quantisation-aware form [P1 s9]: the row, after
 *              its tail RoPE, multiplied by the orthonormal Walsh-Hadamard
 *              matrix of order idx_dim (Sylvester order, entries
 *              +-1/sqrt(idx_dim)), then stored as OCP MXFP4: per block of 32
 *              consecutive channels one E8M0 scale 2^e, e = floor(log2 of the
 *              block's max |x|) - 2 clamped to [-127, 127] (-127 for an
 *              all-zero block), and 32 E2M1 codes of x / 2^e (grid 0, 0.5, 1,
 *              1.5, 2, 3, 4, 6; nearest, ties to the even code, saturated at
 *              6; bit 3 the sign, kept only for a nonzero magnitude).  Record:
 *              idx_dim/2 code bytes (channel 2j in the low nibble of byte j,
 *              2j+1 in the high one), then idx_dim/32 bytes e + 127 -- 68
 *              bytes at idx_dim 128.  The indexer query gets the same
 *              transform (RoPE, Hadamard, MXFP4 round trip) before the dot
 *              products, so scores are exact products of the two fp4 vectors.
 *              The pages name the transform and the 4-bit width but not the
 *              block size, scale rule or bit layout: these are the OCP
 *              microscaling format's.  Built for ratio 4, idx_dim 128,
 *              idx_heads <= 64 and act_fmt BF16.
 */
#ifndef CKV_H
#define CKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define CKV_OK 0
#define CKV_E_INVAL (-1)       /* NULL pointer, bad size, misaligned pointer   */
#define CKV_E_UNSUPPORTED (-2) /* shape / format / ratio not built, or indexer on r != 4 */
#define CKV_E_CAPACITY (-3)    /* B > batch, T > chunk cap, rows beyond comp_cap, stage too small */
#define CKV_E_WORKSPACE (-4)   /* ws NULL or ws_bytes < ckv_workspace_bytes()  */
#define CKV_E_HIP (-5)         /* a kernel launch failed                       */
#define CKV_E_SEQUENCE (-6)    /* pos0 is not the sequence's token count in
                                  cache->n_tokens_host                          */

/* ---- cache->status bits (device-detected, sticky) ------------------------ */
#define CKV_STATUS_BAD_POS 1u   /* pos < 0                                      */
#define CKV_STATUS_CAPACITY 2u  /* the row a token closes lies beyond comp_cap  */
#define CKV_STATUS_SEQUENCE 4u  /* position is not the sequence's next token
                                   (cache->n_tokens); the token was not stored */
#define CKV_STATUS_PAGE 8u      /* a compressed row's block-table entry lies
                                   outside the page pool; the row was not
                                   stored                                      */

/* ---- formats -------------------------------------------------------------- */
#define CKV_F32 0
#define CKV_BF16 1
#define CKV_E4M3 2
#define CKV_FP4 3   /* indexer rows only */

/* ---- desc.flags ------------------------------------------------------------ */
#define CKV_FLAG_NO_INV_ROPE 1u  /* skip the inverse RoPE on the output [P4]   */
#define CKV_FLAG_IDX_NO_RELU 2u  /* indexer sums raw dots instead of relu(dots) */
/* Debug stage skips, for tests that isolate one stage of the compressor or
 * the attention [P1 s4 steps 6-8]:
 *   SKIP_NORM  compressed rows of both lanes are stored without RMSNorm
 *              (neither the 1/rms factor nor the gamma weight);
 *   SKIP_ROPE  no tail rotation anywhere: raw, compressed and indexer rows,
 *              both queries and the output (every angle is zero);
 *   KEEP_F32   every cast is the identity: accepted only with f32 caches,
 *              activations and weights (else CKV_E_UNSUPPORTED). */
#define CKV_FLAG_SKIP_NORM 4u
#define CKV_FLAG_SKIP_ROPE 8u
#define CKV_FLAG_KEEP_F32 16u
/* Attention output in fp8, fused with its inverse RoPE [P4 "GPU compute
 * saturation": inverse RoPE + fp8 quantisation of the attention output]:
 * every (query, head) row of `out` is a record of head_dim OCP E4M3FN codes,
 * then head_dim/128 float32 scales, one per group of 128 consecutive channels
 * (s = max|o| / 448 over the group, 1 when all zero; code = RNE(o / s),
 * saturated) -- 528 bytes at head_dim 512; out is [n, n_heads, 528] bytes.
 * The page names the fusion, not the format: the group size and scale rule
 * are this library's reading.  Built for the tiled attention (bf16
 * activations, bf16 or E4M3 caches, head_dim 512, n_heads a multiple of 64),
 * else CKV_E_UNSUPPORTED. */
#define CKV_FLAG_OUT_FP8 32u
/* Query norm inside the attention [P4 "GPU compute saturation": the query
 * norm fused with the raw keys' RoPE and insertion]: before its RoPE, each
 * head's attention query is divided by its RMS over head_dim channels,
 * q_h / sqrt(mean(q_h^2) + norm_eps), in float32 with no learned weight (the
 * page names the step, not its form: this is the library's reading).  The
 * attention kernels apply it as they load the query, so the normalised query
 * is never stored.  Any layer shape; affects sparse_swa_attn (and the decode
 * step's attention) only, not the indexer query. */
#define CKV_FLAG_Q_NORM 64u
/* Two-lane c4a compressors [P1 s5: a ratio-4 compressor's state is twice as
 * wide as its rows, a first and a second half]: ratio-4 layers only (else
 * CKV_E_UNSUPPORTED).  Every token projects to two lanes of width w (w = d for
 * the attention compressor, D_I for the indexer's): wkv, wgate [2d, hidden]
 * and idx_wkv, idx_wgate [2 D_I, hidden], lane A the first w rows.  Row i
 * pools lane A of tokens 4i-4 .. 4i-1 (window slots 0-3) and lane B of tokens
 * 4i .. 4i+3 (slots 4-7); ape [4, 2d] (idx_ape [4, 2 D_I]) holds lane A's
 * bias of slot s in row s, columns 0..w-1, and lane B's (slot 4 + s) in
 * columns w..2w-1.  The state rings keep both lanes of each token: st_kv,
 * st_sc [batch, 8, 2d], ist_kv, ist_sc [batch, 8, 2 D_I].  The page names the
 * two lanes, not what each holds: this is the library's reading (without the
 * flag one lane serves both windows). */
#define CKV_FLAG_TWO_LANE 128u

/* ---- modes for ckv_workspace_bytes ---------------------------------------- */
#define CKV_MODE_DECODE 0
#define CKV_MODE_PREFILL 1

/* Largest chunk one prefill call accepts [P1 s3: prompts are prefilled in
 * chunks of at most 4096 tokens]. */
#define CKV_MAX_CHUNK 4096

/* Layer description (host memory).
 *   ratio       0 (sliding window only), 4 (c4a: rows pool 8 tokens at stride
 *               4, with indexer) or 128 (c128a: 128 tokens at stride 128, every
 *               visible row attended) [P4 "KV Cache Compression"; P1 s1]
 *   hidden      D, width of the compressor input x
 *   head_dim    d, width of q, of the shared K=V rows and of the output
 *   n_rot       RoPE channels at the end of each head (64) [P1 s8]
 *   n_heads     H query heads sharing one K=V head [P4]
 *   swa         raw sliding-window rows (128) [P1 s2; P4]
 *   idx_heads, idx_dim, top_k   indexer shape (ratio 4 only) [P1 s6]
 *   comp_cap    compressed rows per sequence the cache holds
 *   batch       sequences the cache holds
 *   kv_fmt      CKV_F32 / CKV_BF16 / CKV_E4M3 for raw and compressed rows
 *   idx_fmt     CKV_F32 / CKV_BF16 / CKV_FP4 for indexer rows
 *   act_fmt     CKV_F32 / CKV_BF16 for x, u, q, qI and out
 *   w_fmt       CKV_F32 / CKV_BF16 for wkv / wgate / idx_wkv / idx_wgate
 *   rope_base   the layer's RoPE base [P1 s8]: it serves the raw rows and the
 *               query's rotation against them, and, unless rope_base_comp is
 *               set, everything else as well
 *   rope_base_comp  0, or a separate base for the compressed class:
 *               compressed rows, indexer rows and the indexer query, and the
 *               query's rotation against compressed rows.  Attention then
 *               takes one softmax over both classes and rotates each class's
 *               share of the output back by -p in its own frame [P4 "Shared
 *               Key and Value": inverse RoPE]
 *   norm_eps    RMSNorm epsilon of the compressor [P1 s4 step 6]
 *   softmax_scale  logit scale; 0 means 1/sqrt(head_dim)
 *   flags       CKV_FLAG_* */
typedef struct ckv_layer_desc {
  int32_t ratio;
  int32_t hidden;
  int32_t head_dim;
  int32_t n_rot;
  int32_t n_heads;
  int32_t swa;
  int32_t idx_heads;
  int32_t idx_dim;
  int32_t top_k;
  int32_t comp_cap;
  int32_t batch;
  int32_t kv_fmt;
  int32_t idx_fmt;
  int32_t act_fmt;
  int32_t w_fmt;
  uint32_t flags;
  double rope_base;
  float norm_eps;
  float softmax_scale;
  double rope_base_comp;
} ckv_layer_desc;

/* Compressor weights (device pointers, read only).
 *   wkv, wgate          [head_dim, hidden] row-major, w_fmt   [P1 s4 steps 1-2]
 *                       (CKV_FLAG_TWO_LANE: [2 head_dim, hidden]; the indexer's
 *                       and both APEs change alike, see there)
 *   ape                 [W, head_dim] float32, W = 8 (r=4) / 128 (r=128): the
 *                       learned position bias added to the score of window slot j
 *   gamma               [head_dim] float32 RMSNorm weight
 *   idx_wkv, idx_wgate  [idx_dim, hidden] (ratio 4 only)   [P1 s6]
 *   idx_ape             [8, idx_dim] float32
 *   idx_gamma           [idx_dim] float32 */
typedef struct ckv_layer_weights {
  const void* wkv;
  const void* wgate;
  const float* ape;
  const float* gamma;
  const void* idx_wkv;
  const void* idx_wgate;
  const float* idx_ape;
  const float* idx_gamma;
} ckv_layer_weights;

/* Per-layer cache (device pointers; the struct itself is host memory).
 *   raw        [batch, swa, row_bytes]      raw rows, token t in slot t % swa,
 *                                           stored RoPE'd at t      [P1 s2, s7]
 *   comp       [batch, comp_cap, row_bytes] compressed row i at index i
 *              (paged: see block_table)
 *   idx        [batch, comp_cap, idx row]   indexer rows (ratio 4; paged: see
 *                                           block_table)
 *   st_kv, st_sc   [batch, W, head_dim] float32: compressor window state,
 *                  token t's (kappa, sigma) in slot t % W          [P1 s5; P4]
 *                  (CKV_FLAG_TWO_LANE: [batch, 8, 2 head_dim], lane A then B)
 *   ist_kv, ist_sc [batch, 8, idx_dim] float32: indexer compressor state
 *                  (CKV_FLAG_TWO_LANE: [batch, 8, 2 idx_dim])
 *   raw_stage  [stage_rows, row_bytes]: prefill staging of the raw rows of
 *              positions pos0-swa+1 .. pos0+T-1 (stage_rows >= T + swa - 1)
 *   status     [batch] uint32 sticky device error bits, or NULL
 *   n_tokens   [batch] int32 (device), or NULL: tokens of each sequence stored
 *              so far, i.e. its next position [P1 s1: the engine refuses
 *              state that does not match rather than guessing; ds4 rejects a
 *              KV checkpoint whose prefix does not match, P5 s10].  When given,
 *              compress_append stores a token only at position n_tokens[b]
 *              (then sets n_tokens[b] = pos + 1) or again at n_tokens[b] - 1
 *              (a re-run of the last step, which rewrites the same slots); any
 *              other position sets CKV_STATUS_SEQUENCE and leaves that
 *              sequence's cache untouched.  Prefill accepts pos0 = n_tokens[seq]
 *              only and advances it by T.
 *   n_tokens_host  [batch] int32 (HOST), or NULL: the caller's mirror of
 *              n_tokens.  When given, a prefill call whose pos0 differs from
 *              n_tokens_host[seq] returns CKV_E_SEQUENCE before any enqueue.
 *              The library reads it and never writes it.
 *   block_table  [batch, comp_cap / rpb] int32 (device), or NULL: the paged
 *              layout [P4 "KV cache memory management": one logical block
 *              of 256 token positions for every compressed layer, so rpb =
 *              256 / ratio rows a block -- 64 on c4a, 2 on c128a].  With a
 *              table, comp and idx are page pools, comp [n_pages, rpb,
 *              row_bytes] and idx [n_pages, 64, idx row] (ratio 4: the
 *              indexer rows use the same page index as the K=V rows), and
 *              compressed row i of sequence b lives in page block_table[b *
 *              comp_cap / rpb + i / rpb], slot i % rpb.  comp_cap must be a
 *              multiple of rpb.  A store to a row whose entry lies outside
 *              [0, n_pages) is dropped and sets CKV_STATUS_PAGE; a read through
 *              such an entry reads page 0.  Pages are the caller's to hand out
 *              (a block needs its page before a call stores or reads its rows);
 *              the raw window and the compressor state stay per-sequence rings
 *              keyed by position (the page's sliding-window form of them).
 *   n_pages    pages in each pool (>= 1 with a table, else ignored).
 * Pointers a layer does not use (comp/state for ratio 0, idx/ist_* unless
 * ratio 4, raw_stage for decode) may be NULL. */
typedef struct ckv_layer_cache {
  void* raw;
  void* comp;
  void* idx;
  float* st_kv;
  float* st_sc;
  float* ist_kv;
  float* ist_sc;
  void* raw_stage;
  int32_t stage_rows;
  uint32_t* status;
  int32_t* n_tokens;
  const int32_t* n_tokens_host;
  const int32_t* block_table;
  int32_t n_pages;
} ckv_layer_cache;

/* ---- utilities (host only, never touch the GPU) --------------------------- */

/* Bytes of one stored K=V row in format fmt; 0 for an unknown format. */
size_t ckv_row_bytes(int32_t fmt, int32_t head_dim, int32_t n_rot);

/* Bytes of one stored indexer row of idx_dim channels in format fmt
 * (CKV_F32 4 idx_dim, CKV_BF16 2 idx_dim, CKV_FP4 idx_dim/2 + idx_dim/32 for a
 * multiple of 32); 0 for an unknown format or a size the format cannot hold.
 * The indexer cache is [batch][comp_cap] such rows, back to back. */
size_t ckv_idx_row_bytes(int32_t fmt, int32_t idx_dim);

/* Fail-fast check of a layer description against what the library is built
 * for [P1 s1: the engine refuses a layout it was not built for rather than
 * guessing].  Returns CKV_OK, CKV_E_INVAL or CKV_E_UNSUPPORTED. */
int ckv_validate(const ckv_layer_desc* desc);

/* Static string for a return code. */
const char* ckv_strerror(int code);

/* Name of the HIP error behind the calling thread's most recent CKV_E_HIP
 * ("none" if there was none).  Static string. */
const char* ckv_last_hip_error(void);

/* Kernel timing for profiling callers.  start_event / stop_event: hipEvent_t
 * handles created by the caller (timing enabled), or NULL.  Arms the calling
 * thread's next launch of an indexer score kernel (made by
 * ckv_indexer_score_decode, ckv_indexer_topk_decode or
 * ckv_indexer_topk_prefill, or the fused projection + scan launch of
 * ckv_decode_step) to stamp start_event when the kernel starts and stop_event
 * when it ends, so that hipEventElapsedTime gives the kernel's own duration,
 * without the launch gaps around it.  The events stay owned by the caller;
 * the arming is consumed by that one launch; two NULLs disarm.  Returns
 * CKV_OK. */
int ckv_time_next_score(void* start_event, void* stop_event);

/* Workspace bytes a call of `mode` with n = B (decode) or T (prefill) tokens
 * needs; the same figure serves all entry points of that mode.
 * 0 when desc is invalid.
 *
 * Workspace contract: the first ckv_workspace_sync_bytes(desc, mode, n) bytes
 * of the workspace hold counters and histograms that kernels accumulate into.
 * They must be zero before the workspace is first used (allocate it zeroed);
 * every call that completes leaves them zero again, so a workspace can be
 * reused across calls, modes and graph replays.  Calls sharing one workspace
 * must not overlap. */
size_t ckv_workspace_bytes(const ckv_layer_desc* desc, int32_t mode, int32_t n);
size_t ckv_workspace_sync_bytes(const ckv_layer_desc* desc, int32_t mode, int32_t n);

/* ---- compress_append: compressor + cache insertion [P1 s4-s5, s8-s9; P4 fused
 * compressor + RMSNorm + RoPE + cache insertion] ----------------------------
 *
 * Decode: one token per sequence b < B at position pos[b] (device int32).
 *   - kappa = wkv.x, sigma = wgate.x (and the indexer lane on ratio 4) are
 *     stored in state slot pos % W;
 *   - u[b] is RoPE'd at pos (tail only) and stored in raw slot pos % swa;
 *   - when (pos+1) % ratio == 0 the window of row i = (pos+1)/ratio - 1
 *     (tokens 4i-4..4i+3 for c4a, 128i..128i+127 for c128a) is pooled per
 *     channel with softmax(sigma + ape[slot]), RMS-normalised, RoPE'd at i*ratio
 *     and stored as comp row i (and idx row i).
 * x [B, hidden] act_fmt, u [B, head_dim] act_fmt.
 * ratio 0 stores the raw row only (weights may be NULL).
 * Re-running a step at the same positions rewrites identical values. */
int ckv_compress_append_decode(const ckv_layer_desc* desc, const ckv_layer_weights* w,
                               const ckv_layer_cache* cache, const void* x, const void* u,
                               const int32_t* pos, int32_t B, void* ws, size_t ws_bytes,
                               void* stream);

/* Prefill: tokens pos0 .. pos0+T-1 of sequence `seq` (host ints), 1 <= T <=
 * CKV_MAX_CHUNK; x [T, hidden], u [T, head_dim].  Equivalent to T decode
 * steps; compressor windows that straddle pos0 take their earlier tokens from
 * the state, so boundaries stay at absolute positions [P1 s3].  Also fills
 * cache->raw_stage with the raw rows of pos0-swa+1 .. pos0+T-1 (stage row
 * t - pos0 + swa - 1) for the prefill attention, then refreshes the raw ring. */
int ckv_compress_append_prefill(const ckv_layer_desc* desc, const ckv_layer_weights* w,
                                const ckv_layer_cache* cache, const void* x, const void* u,
                                int32_t seq, int32_t pos0, int32_t T, void* ws, size_t ws_bytes,
                                void* stream);

/* ---- indexer_topk: score every visible compressed row, keep the top k
 * [P1 s6; P4 DSA] (ratio 4 only, else CKV_E_UNSUPPORTED) ------------------------
 *
 * For query position p, V = (p+1)/4 rows are visible.  The indexer query
 * qI[h] is RoPE'd at p (tail) and cast to idx_fmt (for CKV_FP4: Hadamard,
 * then the MXFP4 round trip); row s scores
 * I(s) = sum_h w[h] * relu(qI[h] . idx[s]).  topk[0..k) receives the k best
 * rows (ties to the lower index) in ascending index order, -1 padded; when
 * V <= k it receives 0..V-1 then -1s.
 * Decode: qI [B, idx_heads, idx_dim] act_fmt, w [B, idx_heads] float32,
 *         pos [B] device, topk [B, top_k] int32.
 * Prefill: qI [T, ...], w [T, ...], topk [T, top_k] for queries pos0..pos0+T-1
 *         of sequence seq (run after compress_append_prefill of the chunk). */
int ckv_indexer_topk_decode(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                            const void* qI, const float* w, const int32_t* pos, int32_t B,
                            int32_t* topk, void* ws, size_t ws_bytes, void* stream);
/* The scoring stage of ckv_indexer_topk_decode on its own.  For every row
 * s < V of sequence b, keys[b * comp_cap + s] receives the order-preserving
 * 32-bit image of I(s): a non-negative score's float bits with the top bit
 * set, a negative score's bits inverted (-0 counts as +0), so keys compare
 * like the scores.  keys [B, comp_cap] uint32; other arguments as for the
 * decode call.  Entries V <= s < comp_cap may receive unspecified values;
 * nothing outside [B, comp_cap] is written. */
int ckv_indexer_score_decode(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                             const void* qI, const float* w, const int32_t* pos, int32_t B,
                             uint32_t* keys, void* stream);
int ckv_indexer_topk_prefill(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                             const void* qI, const float* w, int32_t seq, int32_t pos0, int32_t T,
                             int32_t* topk, void* ws, size_t ws_bytes, void* stream);

/* ---- sparse_swa_attn: one softmax over the raw window and the compressed rows,
 * shared K=V, inverse RoPE on the output [P1 s7; P4] -------------------------
 *
 * For query p, head h: q[h] RoPE'd at p; rows = raw positions
 * max(0, p-swa+1)..p, plus topk rows (ratio 4; entries < 0 skipped, entries
 * >= V end the list) or rows 0..V-1 (ratio 128) or none (ratio 0);
 * l_j = scale * q.row_j, o = sum_j softmax(l)_j row_j, then the output tail is
 * rotated by -p, and o is cast to act_fmt (with CKV_FLAG_OUT_FP8: written as
 * the fp8 records described there).
 * Decode: q [B, n_heads, head_dim], pos [B] device, topk [B, top_k] (ratio 4,
 *         else NULL), out [B, n_heads, head_dim].
 * Prefill: q [T, ...], topk [T, top_k] or NULL, out [T, ...] for queries
 *         pos0..pos0+T-1 of sequence seq; reads cache->raw_stage written by
 *         compress_append_prefill of the same chunk. */
int ckv_sparse_swa_attn_decode(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                               const void* q, const int32_t* pos, const int32_t* topk, int32_t B,
                               void* out, void* ws, size_t ws_bytes, void* stream);
int ckv_sparse_swa_attn_prefill(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                                const void* q, int32_t seq, int32_t pos0, int32_t T,
                                const int32_t* topk, void* out, void* ws, size_t ws_bytes,
                                void* stream);

/* ---- decode_step: compress_append + indexer_topk + sparse_swa_attn of one
 * decode token per sequence, in that order [P1 s4-s9; P4 decode path] -----------
 *
 * The result equals ckv_compress_append_decode, then (ratio 4)
 * ckv_indexer_topk_decode, then ckv_sparse_swa_attn_decode, with the same
 * arguments: x, u as for compress_append; q, out as for sparse_swa_attn;
 * qI, iw (the indexer head weights) and topk as for indexer_topk (ratio 4;
 * ignored and may be NULL otherwise).  topk receives the selection on ratio 4.
 * On ratio-4 layers with bf16 activations and weights, bf16 or fp4 indexer
 * rows, one or two compressor lanes, D_I = 128, at most 64 indexer heads,
 * comp_cap <= 32768 and B <= 64, the step runs as
 * three launches: the compressor projection shares a launch with the scoring
 * of the rows that precede this token's own row; one block per sequence then
 * runs the compressor, scores the row this token closed (if any) and selects;
 * then the attention.  The selection is the same; the score of the new row
 * may differ from the separate call's in the last bits (another summation
 * order).  Other layers run the three calls.  Error returns as for those
 * calls; on an error nothing after the failing stage is enqueued. */
int ckv_decode_step(const ckv_layer_desc* desc, const ckv_layer_weights* w, const ckv_layer_cache* cache,
                    const void* x, const void* u, const void* q, const void* qI, const float* iw,
                    const int32_t* pos, int32_t B, int32_t* topk, void* out, void* ws, size_t ws_bytes,
                    void* stream);

/* ---- prefill_chunk: the three prefill calls of one chunk, the indexer
 * branch on a second stream [P4 "GPU compute saturation": the indexer
 * pipeline on its own stream beside the main KV compression and the SWA
 * token insertion] -----------------------------------------------------------
 *
 * The result equals ckv_compress_append_prefill, then (ratio 4)
 * ckv_indexer_topk_prefill, then ckv_sparse_swa_attn_prefill with the same
 * arguments (x, u as for compress_append; q, out as for sparse_swa_attn; qI,
 * iw and topk as for indexer_topk, ratio 4 only, else ignored and may be
 * NULL), bit for bit.  With side_stream NULL or equal to stream, or on a
 * layer without an indexer, everything runs in that order on `stream`.
 * Otherwise the side stream (after the work already on `stream`) projects
 * and pools the indexer lane, then scores and selects, while `stream`
 * projects and pools the attention lane and stages the raw rows; `stream`
 * then updates the compressor state and the token count and runs the
 * attention once the selection is done.  When the call returns, every piece
 * of the chunk is ordered before later work on `stream`.  The side stream
 * must not be used to reuse this workspace or cache before `stream` has
 * passed this call.  The call creates its three ordering events itself (no
 * device memory).  Error returns as for the three calls. */
int ckv_prefill_chunk(const ckv_layer_desc* desc, const ckv_layer_weights* w, const ckv_layer_cache* cache,
                      const void* x, const void* u, const void* q, const void* qI, const float* iw, int32_t seq,
                      int32_t pos0, int32_t T, int32_t* topk, void* out, void* ws, size_t ws_bytes, void* stream,
                      void* side_stream);

/* ---- decode_step without a workspace argument ------------------------------
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation).  The same step as
 * ckv_decode_step, same arguments without ws / ws_bytes: the workspace is a
 * device array of CKV_STATIC_WORKSPACE_BYTES inside the library, one per GPU,
 * held until the process ends.  A layer / batch whose
 * ckv_workspace_bytes(desc, CKV_MODE_DECODE, B) exceeds that size returns
 * CKV_E_WORKSPACE before any work is enqueued (the 64k-context batch of 32
 * sequences needs 44 MiB).  The call clears the array's counter region with a
 * kernel, allocates nothing and records no memset.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams,
 * or threads) race and must not be issued. */
#define CKV_STATIC_WORKSPACE_BYTES ((size_t)48 << 20)
int ckv_decode_step_static(const ckv_layer_desc* desc, const ckv_layer_weights* w, const ckv_layer_cache* cache,
                           const void* x, const void* u, const void* q, const void* qI, const float* iw,
                           const int32_t* pos, int32_t B, int32_t* topk, void* out, void* stream);

/* ---- Hyper-Connection mixer around the attention block [P1 s10] ------------
 *
 * The hidden state is carried as n_hc = 4 residual streams h_0..h_3 of
 * `hidden` channels.  A per-token mixer row of 24 float32 values
 * m = [pre (4) | post (4) | coupling (16, row-major)] is split into
 *   pre_i  = sigmoid(m[i]),  post_j = sigmoid(m[4 + j]),
 *   C      = Sinkhorn(m[8..23]): a softmax along each row, a column
 *            normalisation, then (sinkhorn_iters - 1) times a row and a column
 *            normalisation, each dividing by (sum + eps)  (C rows j, columns i);
 * the block reads x = sum_i pre_i h_i, and after it (output y) the streams
 * become h'_j = sum_i C[j][i] h_i + post_j y.  The page fixes n_hc, the
 * iteration count (20 at the Flash shape), the split and the alternating
 * normalisation with eps; the row layout, the logistic gates and the first
 * iteration's form are this library's reading.  Arithmetic in float32. */
typedef struct ckv_hc_desc {
  int32_t hidden;          /* channels per stream: a multiple of 8, at most 65536 */
  int32_t n_hc;            /* streams: 4 */
  int32_t sinkhorn_iters;  /* 1..100 (20 at the Flash shape) */
  float eps;               /* Sinkhorn eps, >= 0 and finite (1e-6) */
  int32_t act_fmt;         /* CKV_F32 / CKV_BF16 for h, x, y and h_out */
} ckv_hc_desc;

/* CKV_OK, CKV_E_INVAL (NULL) or CKV_E_UNSUPPORTED. */
int ckv_hc_validate(const ckv_hc_desc* desc);

/* Split + Sinkhorn + pre mix of T tokens (T >= 1): mix [T, 24] float32,
 * h [T, 4, hidden] act_fmt -> x [T, hidden] act_fmt and coef [T, 24] float32
 * (pre 4, post 4, C 16 row-major), the input of ckv_hc_post.  Every pointer
 * 16-byte aligned (else CKV_E_INVAL); x must not overlap h. */
int ckv_hc_pre(const ckv_hc_desc* desc, const float* mix, const void* h, int32_t T, void* x, float* coef,
               void* stream);

/* Post mix: coef [T, 24] from ckv_hc_pre, h [T, 4, hidden], y [T, hidden]
 * (the block output) -> h_out [T, 4, hidden], all act_fmt but coef; h_out
 * must not overlap h or y. */
int ckv_hc_post(const ckv_hc_desc* desc, const float* coef, const void* h, const void* y, int32_t T,
                void* h_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CKV_H */
