// C ABI entry points of libckv: argument checks on the host, then kernel
// enqueues on the caller's stream.  Nothing here synchronises or allocates.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ckv_internal.h"

using namespace ckv;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptr(const void* p) { return (p && aligned16(p)) ? CKV_OK : CKV_E_INVAL; }

Weights to_weights(const ckv_layer_weights* w) {
  Weights x;
  x.wkv = w->wkv;
  x.wgate = w->wgate;
  x.ape = w->ape;
  x.gamma = w->gamma;
  x.idx_wkv = w->idx_wkv;
  x.idx_wgate = w->idx_wgate;
  x.idx_ape = w->idx_ape;
  x.idx_gamma = w->idx_gamma;
  return x;
}

Cache to_cache(const ckv_layer_cache* c) {
  Cache x;
  x.raw = (uint8_t*)c->raw;
  x.comp = (uint8_t*)c->comp;
  x.idx = c->idx;
  x.st_kv = c->st_kv;
  x.st_sc = c->st_sc;
  x.ist_kv = c->ist_kv;
  x.ist_sc = c->ist_sc;
  x.stage = (uint8_t*)c->raw_stage;
  x.stage_rows = c->stage_rows;
  x.status = c->status;
  x.n_tokens = c->n_tokens;
  return x;
}

// Common prologue: validate the description and the cache pointers a layer of
// this ratio uses.
int prologue(const ckv_layer_desc* d, const ckv_layer_cache* c, LayerParams* P) {
  int rc = ckv_validate(d);
  if (rc) return rc;
  if (!c) return CKV_E_INVAL;
  make_params(d, P);
  if (check_ptr(c->raw)) return CKV_E_INVAL;
  if (c->n_tokens && ((uintptr_t)c->n_tokens & 3u)) return CKV_E_INVAL;
  if (c->status && ((uintptr_t)c->status & 3u)) return CKV_E_INVAL;
  if (P->ratio) {
    if (check_ptr(c->comp) || check_ptr(c->st_kv) || check_ptr(c->st_sc)) return CKV_E_INVAL;
  }
  if (P->ratio == 4) {
    if (check_ptr(c->idx) || check_ptr(c->ist_kv) || check_ptr(c->ist_sc)) return CKV_E_INVAL;
  }
  P->blocks = nullptr;
  if (P->ratio && c->block_table) {   // paged: 256 token positions a block
    const int rpb = 256 / P->ratio;
    if ((uintptr_t)c->block_table & 3u || c->n_pages < 1) return CKV_E_INVAL;
    if (P->cap % rpb) return CKV_E_UNSUPPORTED;
    P->blocks = c->block_table;
    P->n_pages = c->n_pages;
    P->max_blocks = P->cap / rpb;
    P->rpb_shift = P->ratio == 4 ? 6 : 1;
  }
  return CKV_OK;
}

int check_ws(const LayerParams& P, int mode, int n, void* ws, size_t ws_bytes, WsLayout* L) {
  *L = ws_layout(P, mode, n);
  if (!ws || !aligned16(ws) || ws_bytes < L->total) return CKV_E_WORKSPACE;
  return CKV_OK;
}

int weights_ok(const LayerParams& P, const ckv_layer_weights* w) {
  if (P.ratio == 0) return CKV_OK;
  if (!w) return CKV_E_INVAL;
  if (check_ptr(w->wkv) || check_ptr(w->wgate) || check_ptr(w->ape) || check_ptr(w->gamma))
    return CKV_E_INVAL;
  if (P.ratio == 4 && (check_ptr(w->idx_wkv) || check_ptr(w->idx_wgate) || check_ptr(w->idx_ape) ||
                       check_ptr(w->idx_gamma)))
    return CKV_E_INVAL;
  return CKV_OK;
}

int prefill_range_ok(const LayerParams& P, const ckv_layer_cache* c, int32_t seq, int32_t pos0,
                     int32_t T) {
  if (T < 1 || pos0 < 0 || seq < 0) return CKV_E_INVAL;
  if (T > CKV_MAX_CHUNK || seq >= P.batch) return CKV_E_CAPACITY;
  if ((long long)pos0 + T > (1ll << 30)) return CKV_E_CAPACITY;
  if (P.ratio && (pos0 + T) / P.ratio > P.cap) return CKV_E_CAPACITY;
  if (!c->raw_stage || !aligned16(c->raw_stage)) return CKV_E_INVAL;
  if (c->stage_rows < T + P.swa - 1) return CKV_E_CAPACITY;
  return CKV_OK;
}

// The host mirror of the token counts, when the caller keeps one: a chunk
// must start at its sequence's next position.
int prefill_sequence_ok(const ckv_layer_cache* c, int32_t seq, int32_t pos0) {
  if (c->n_tokens_host && c->n_tokens_host[seq] != pos0) return CKV_E_SEQUENCE;
  return CKV_OK;
}

thread_local int t_last_hip = 0;

// An error left behind by an earlier, unrelated runtime call would otherwise be
// reported as this call's launch failure: read it off before enqueueing.
void clear_stale() { (void)hipGetLastError(); }

int launched(int hip_rc) {
  if (hip_rc) {
    t_last_hip = hip_rc;
    return CKV_E_HIP;
  }
  return CKV_OK;
}

}  // namespace

extern "C" int ckv_compress_append_decode(const ckv_layer_desc* desc, const ckv_layer_weights* w,
                                          const ckv_layer_cache* cache, const void* x, const void* u,
                                          const int32_t* pos, int32_t B, void* ws, size_t ws_bytes,
                                          void* stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if (B < 1) return CKV_E_INVAL;
  if (B > P.batch) return CKV_E_CAPACITY;
  if ((rc = weights_ok(P, w))) return rc;
  if (check_ptr(u) || check_ptr(pos) || (P.ratio && check_ptr(x))) return CKV_E_INVAL;
  WsLayout L;
  if ((rc = check_ws(P, CKV_MODE_DECODE, B, ws, ws_bytes, &L))) return rc;
  clear_stale();
  const Weights W = P.ratio ? to_weights(w) : Weights{};
  const Cache C = to_cache(cache);
  float* part = (float*)((uint8_t*)ws + L.proj);
  if (P.ratio) {
    if ((rc = launch_proj(P, W, x, B, part, L.proj_splits, stream))) return launched(rc);
  }
  return launched(launch_compress_decode(P, W, C, u, pos, B, part, L.proj_splits,
                                        (float*)((uint8_t*)ws + L.pool), stream));
}

extern "C" int ckv_compress_append_prefill(const ckv_layer_desc* desc, const ckv_layer_weights* w,
                                           const ckv_layer_cache* cache, const void* x, const void* u,
                                           int32_t seq, int32_t pos0, int32_t T, void* ws,
                                           size_t ws_bytes, void* stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if ((rc = prefill_range_ok(P, cache, seq, pos0, T))) return rc;
  if ((rc = prefill_sequence_ok(cache, seq, pos0))) return rc;
  if ((rc = weights_ok(P, w))) return rc;
  if (check_ptr(u) || (P.ratio && check_ptr(x))) return CKV_E_INVAL;
  WsLayout L;
  if ((rc = check_ws(P, CKV_MODE_PREFILL, T, ws, ws_bytes, &L))) return rc;
  clear_stale();
  const Weights W = P.ratio ? to_weights(w) : Weights{};
  const Cache C = to_cache(cache);
  float* part = (float*)((uint8_t*)ws + L.proj);
  if (P.ratio) {
    if ((rc = launch_proj(P, W, x, T, part, 1, stream))) return launched(rc);
  }
  return launched(launch_compress_prefill(P, W, C, u, seq, pos0, T, part, stream));
}

extern "C" int ckv_indexer_topk_decode(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                                       const void* qI, const float* w, const int32_t* pos, int32_t B,
                                       int32_t* topk, void* ws, size_t ws_bytes, void* stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if (P.ratio != 4) return CKV_E_UNSUPPORTED;
  if (B < 1) return CKV_E_INVAL;
  if (B > P.batch) return CKV_E_CAPACITY;
  if (check_ptr(qI) || check_ptr(w) || check_ptr(pos) || check_ptr(topk)) return CKV_E_INVAL;
  WsLayout L;
  if ((rc = check_ws(P, CKV_MODE_DECODE, B, ws, ws_bytes, &L))) return rc;
  clear_stale();
  uint8_t* wb = (uint8_t*)ws;
  SelWs sel;
  sel.hist = (uint32_t*)(wb + L.hist);
  sel.ctr = (uint32_t*)(wb + L.ctr);
  sel.sure = (uint32_t*)(wb + L.sure);
  sel.cand_key = (uint32_t*)(wb + L.cand_key);
  sel.cand_idx = (uint32_t*)(wb + L.cand_idx);
  sel.qf4 = wb + L.qf4;
  return launched(launch_indexer(P, to_cache(cache), qI, w, pos, 0, 0, B, (uint32_t*)(wb + L.keys), &sel,
                                 topk, stream));
}

extern "C" int ckv_indexer_score_decode(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                                        const void* qI, const float* w, const int32_t* pos, int32_t B,
                                        uint32_t* keys, void* stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if (P.ratio != 4) return CKV_E_UNSUPPORTED;
  if (B < 1) return CKV_E_INVAL;
  if (B > P.batch) return CKV_E_CAPACITY;
  if (check_ptr(qI) || check_ptr(w) || check_ptr(pos) || check_ptr(keys)) return CKV_E_INVAL;
  clear_stale();
  return launched(launch_idx_score(P, to_cache(cache), qI, w, pos, 0, 0, B, keys, nullptr, stream));
}

extern "C" int ckv_indexer_topk_prefill(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                                        const void* qI, const float* w, int32_t seq, int32_t pos0,
                                        int32_t T, int32_t* topk, void* ws, size_t ws_bytes,
                                        void* stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if (P.ratio != 4) return CKV_E_UNSUPPORTED;
  if (T < 1 || pos0 < 0 || seq < 0) return CKV_E_INVAL;
  if (T > CKV_MAX_CHUNK || seq >= P.batch || (pos0 + T) / 4 > P.cap) return CKV_E_CAPACITY;
  if (check_ptr(qI) || check_ptr(w) || check_ptr(topk)) return CKV_E_INVAL;
  WsLayout L;
  if ((rc = check_ws(P, CKV_MODE_PREFILL, T, ws, ws_bytes, &L))) return rc;
  clear_stale();
  uint8_t* wb = (uint8_t*)ws;
  return launched(launch_indexer(P, to_cache(cache), qI, w, nullptr, seq, pos0, T,
                                 (uint32_t*)(wb + L.keys), nullptr, topk, stream));
}

extern "C" int ckv_sparse_swa_attn_decode(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                                          const void* q, const int32_t* pos, const int32_t* topk,
                                          int32_t B, void* out, void* ws, size_t ws_bytes,
                                          void* stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if (B < 1) return CKV_E_INVAL;
  if (B > P.batch) return CKV_E_CAPACITY;
  if (check_ptr(q) || check_ptr(pos) || check_ptr(out)) return CKV_E_INVAL;
  if ((P.ratio == 4) != (topk != nullptr)) return CKV_E_INVAL;
  if (topk && !aligned16(topk)) return CKV_E_INVAL;
  WsLayout L;
  if ((rc = check_ws(P, CKV_MODE_DECODE, B, ws, ws_bytes, &L))) return rc;
  clear_stale();
  return launched(launch_attn(P, to_cache(cache), q, pos, 0, 0, B, topk, out, L, (uint8_t*)ws, stream));
}

extern "C" int ckv_sparse_swa_attn_prefill(const ckv_layer_desc* desc, const ckv_layer_cache* cache,
                                           const void* q, int32_t seq, int32_t pos0, int32_t T,
                                           const int32_t* topk, void* out, void* ws, size_t ws_bytes,
                                           void* stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if ((rc = prefill_range_ok(P, cache, seq, pos0, T))) return rc;
  if (check_ptr(q) || check_ptr(out)) return CKV_E_INVAL;
  if ((P.ratio == 4) != (topk != nullptr)) return CKV_E_INVAL;
  if (topk && !aligned16(topk)) return CKV_E_INVAL;
  WsLayout L;
  if ((rc = check_ws(P, CKV_MODE_PREFILL, T, ws, ws_bytes, &L))) return rc;
  clear_stale();
  return launched(
      launch_attn(P, to_cache(cache), q, nullptr, seq, pos0, T, topk, out, L, (uint8_t*)ws, stream));
}

namespace ckv {
int decode_step_checks(const ckv_layer_desc* desc, const ckv_layer_weights* w, const ckv_layer_cache* cache,
                       const void* x, const void* u, const void* q, const void* qI, const float* iw,
                       const int32_t* pos, int32_t B, int32_t* topk, void* out, void* ws, size_t ws_bytes,
                       LayerParams* P, WsLayout* L) {
  int rc = prologue(desc, cache, P);
  if (rc) return rc;
  if (B < 1) return CKV_E_INVAL;
  if (B > P->batch) return CKV_E_CAPACITY;
  if ((rc = weights_ok(*P, w))) return rc;
  if (check_ptr(u) || check_ptr(q) || check_ptr(pos) || check_ptr(out) || (P->ratio && check_ptr(x)))
    return CKV_E_INVAL;
  if (P->ratio == 4 && (check_ptr(qI) || check_ptr(iw) || check_ptr(topk))) return CKV_E_INVAL;
  return check_ws(*P, CKV_MODE_DECODE, B, ws, ws_bytes, L);
}
}  // namespace ckv

extern "C" int ckv_decode_step(const ckv_layer_desc* desc, const ckv_layer_weights* w,
                               const ckv_layer_cache* cache, const void* x, const void* u, const void* q,
                               const void* qI, const float* iw, const int32_t* pos, int32_t B, int32_t* topk,
                               void* out, void* ws, size_t ws_bytes, void* stream) {
  LayerParams P;
  WsLayout L;
  int rc = decode_step_checks(desc, w, cache, x, u, q, qI, iw, pos, B, topk, out, ws, ws_bytes, &P, &L);
  if (rc) return rc;
  if (P.ratio != 4 || !step_fusable(P, B)) {
    if ((rc = ckv_compress_append_decode(desc, w, cache, x, u, pos, B, ws, ws_bytes, stream))) return rc;
    if (P.ratio == 4 && (rc = ckv_indexer_topk_decode(desc, cache, qI, iw, pos, B, topk, ws, ws_bytes, stream)))
      return rc;
    return ckv_sparse_swa_attn_decode(desc, cache, q, pos, P.ratio == 4 ? topk : nullptr, B, out, ws, ws_bytes,
                                      stream);
  }
  clear_stale();
  uint8_t* wb = (uint8_t*)ws;
  SelWs sel;
  sel.hist = (uint32_t*)(wb + L.hist);
  sel.ctr = (uint32_t*)(wb + L.ctr);
  sel.sure = (uint32_t*)(wb + L.sure);
  sel.cand_key = (uint32_t*)(wb + L.cand_key);
  sel.cand_idx = (uint32_t*)(wb + L.cand_idx);
  sel.qf4 = wb + L.qf4;
  const Cache C = to_cache(cache);
  if ((rc = launch_step_scan_select(P, to_weights(w), C, x, u, qI, iw, pos, B, (float*)(wb + L.proj),
                                    (uint32_t*)(wb + L.keys), sel, topk, stream)))
    return launched(rc);
  return launched(launch_attn(P, C, q, pos, 0, 0, B, topk, out, L, wb, stream));
}

// ---- prefill chunk with the indexer on a second stream ----------------------

namespace {
// events of one call: created here, destroyed once enqueued (the runtime
// releases an event that is still pending when its work completes)
struct Events {
  hipEvent_t e[3] = {};
  int n = 0;
  int get(hipEvent_t* ev) {   // a hipError_t
    const hipError_t r = hipEventCreateWithFlags(&e[n], hipEventDisableTiming);
    if (r == hipSuccess) *ev = e[n++];
    return (int)r;
  }
  ~Events() {
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(e[i]);
  }
};
}  // namespace

extern "C" int ckv_prefill_chunk(const ckv_layer_desc* desc, const ckv_layer_weights* w,
                                 const ckv_layer_cache* cache, const void* x, const void* u, const void* q,
                                 const void* qI, const float* iw, int32_t seq, int32_t pos0, int32_t T,
                                 int32_t* topk, void* out, void* ws, size_t ws_bytes, void* stream,
                                 void* side_stream) {
  LayerParams P;
  int rc = prologue(desc, cache, &P);
  if (rc) return rc;
  if ((rc = prefill_range_ok(P, cache, seq, pos0, T))) return rc;
  if ((rc = prefill_sequence_ok(cache, seq, pos0))) return rc;
  if ((rc = weights_ok(P, w))) return rc;
  if (check_ptr(u) || check_ptr(q) || check_ptr(out) || (P.ratio && check_ptr(x))) return CKV_E_INVAL;
  if (P.ratio == 4 && (check_ptr(qI) || check_ptr(iw) || check_ptr(topk) || !aligned16(topk))) return CKV_E_INVAL;
  WsLayout L;
  if ((rc = check_ws(P, CKV_MODE_PREFILL, T, ws, ws_bytes, &L))) return rc;
  clear_stale();
  const Weights W = P.ratio ? to_weights(w) : Weights{};
  const Cache C = to_cache(cache);
  uint8_t* wb = (uint8_t*)ws;
  float* part = (float*)(wb + L.proj);
  uint32_t* keys = (uint32_t*)(wb + L.keys);
  int32_t* tk = P.ratio == 4 ? topk : nullptr;
  if (P.ratio != 4 || !side_stream || side_stream == stream) {
    if (P.ratio && (rc = launch_proj(P, W, x, T, part, 1, stream))) return launched(rc);
    if ((rc = launch_compress_prefill(P, W, C, u, seq, pos0, T, part, stream))) return launched(rc);
    if (P.ratio == 4 && (rc = launch_indexer(P, C, qI, iw, nullptr, seq, pos0, T, keys, nullptr, topk, stream)))
      return launched(rc);
    return launched(launch_attn(P, C, q, nullptr, seq, pos0, T, tk, out, L, wb, stream));
  }
  // Two streams.  Main: the attention lane's projection columns, the raw
  // staging and the attention rows.  Side: the indexer lane's projection
  // columns and rows (event `pooled`), then the scores and the selection
  // (event `selected`).  Main then moves the state rings and the token count
  // (which the indexer rows' pooling reads: after `pooled`) and runs the
  // attention after `selected`.
  hipStream_t main_st = (hipStream_t)stream, side = (hipStream_t)side_stream;
  const int ca = 2 * P.lanes * P.d;   // attention compressor's columns [0, ca), the indexer's [ca, ncol)
  Events ev;
  hipEvent_t fork, pooled, selected;
  if ((rc = ev.get(&fork)) || (rc = ev.get(&pooled)) || (rc = ev.get(&selected))) return launched(rc);
  if ((rc = (int)hipEventRecord(fork, main_st)) || (rc = (int)hipStreamWaitEvent(side, fork, 0)))
    return launched(rc);
  if ((rc = launch_proj(P, W, x, T, part, 1, side, ca, P.ncol)) ||
      (rc = launch_compress_prefill(P, W, C, u, seq, pos0, T, part, side, kPfPoolIdx)) ||
      (rc = (int)hipEventRecord(pooled, side)) ||
      (rc = launch_indexer(P, C, qI, iw, nullptr, seq, pos0, T, keys, nullptr, topk, side)) ||
      (rc = (int)hipEventRecord(selected, side)))
    return launched(rc);
  if ((rc = launch_proj(P, W, x, T, part, 1, main_st, 0, ca)) ||
      (rc = launch_compress_prefill(P, W, C, u, seq, pos0, T, part, main_st, kPfStage | kPfPoolAttn)) ||
      (rc = (int)hipStreamWaitEvent(main_st, pooled, 0)) ||
      (rc = launch_compress_prefill(P, W, C, u, seq, pos0, T, part, main_st, kPfState)) ||
      (rc = (int)hipStreamWaitEvent(main_st, selected, 0)))
    return launched(rc);
  return launched(launch_attn(P, C, q, nullptr, seq, pos0, T, tk, out, L, wb, stream));
}

extern "C" int ckv_time_next_score(void* start_event, void* stop_event) {
  arm_score_timing(start_event, stop_event);
  return CKV_OK;
}

extern "C" const char* ckv_last_hip_error(void) {
  return t_last_hip ? hipGetErrorName((hipError_t)t_last_hip) : "none";
}

// ---- Hyper-Connection mixer -------------------------------------------------

static HcParams hc_params(const ckv_hc_desc* d) {
  HcParams Hp;
  Hp.hidden = d->hidden;
  Hp.iters = d->sinkhorn_iters;
  Hp.eps = d->eps;
  Hp.act_fmt = d->act_fmt;
  return Hp;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

extern "C" int ckv_hc_pre(const ckv_hc_desc* d, const float* mix, const void* h, int32_t T, void* x, float* coef,
                          void* stream) {
  int rc = ckv_hc_validate(d);
  if (rc) return rc;
  if (T < 1 || check_ptr(mix) || check_ptr(h) || check_ptr(x) || check_ptr(coef)) return CKV_E_INVAL;
  const size_t es = d->act_fmt == CKV_F32 ? 4 : 2;
  if (overlap(x, (size_t)T * d->hidden * es, h, (size_t)T * 4 * d->hidden * es)) return CKV_E_INVAL;
  clear_stale();
  return launched(launch_hc_pre(hc_params(d), mix, h, T, x, coef, stream));
}

extern "C" int ckv_hc_post(const ckv_hc_desc* d, const float* coef, const void* h, const void* y, int32_t T,
                           void* h_out, void* stream) {
  int rc = ckv_hc_validate(d);
  if (rc) return rc;
  if (T < 1 || check_ptr(coef) || check_ptr(h) || check_ptr(y) || check_ptr(h_out)) return CKV_E_INVAL;
  const size_t es = d->act_fmt == CKV_F32 ? 4 : 2;
  const size_t nh = (size_t)T * 4 * d->hidden * es;
  if (overlap(h_out, nh, h, nh) || overlap(h_out, nh, y, (size_t)T * d->hidden * es)) return CKV_E_INVAL;
  clear_stale();
  return launched(launch_hc_post(hc_params(d), coef, h, y, T, h_out, stream));
}
