// Host-only, HIP-free part of libckv: layer-description checks, row sizes,
// workspace sizing and error strings.  Compiles with a plain C++ compiler so
// that its checks can be exercised on a machine without a GPU.
//
// The engine described in "ds4.c を読み解く (#3)" (section 1) refuses a model
// whose layout differs from the one it was built for instead of guessing;
// ckv_validate applies the same rule to a layer description.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "ckv_internal.h"

namespace ckv {

static bool fmt_ok(int f, bool allow_e4m3) {
  return f == CKV_F32 || f == CKV_BF16 || (allow_e4m3 && f == CKV_E4M3);
}

bool make_params(const ckv_layer_desc* d, LayerParams* P) {
  memset(P, 0, sizeof(*P));
  P->ratio = d->ratio;
  P->hidden = d->hidden;
  P->d = d->head_dim;
  P->n_rot = d->n_rot;
  P->H = d->n_heads;
  P->swa = d->swa;
  P->HI = d->ratio == 4 ? d->idx_heads : 0;
  P->DI = d->ratio == 4 ? d->idx_dim : 0;
  P->topk = d->ratio == 4 ? d->top_k : 0;
  P->cap = d->ratio ? d->comp_cap : 0;
  P->batch = d->batch;
  P->kv_fmt = d->kv_fmt;
  P->idx_fmt = d->idx_fmt;
  P->act_fmt = d->act_fmt;
  P->w_fmt = d->w_fmt;
  P->flags = d->flags;
  P->base = d->rope_base;
  P->eps = d->norm_eps;
  P->scale = d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / sqrt((double)d->head_dim));
  P->W = d->ratio == 4 ? 8 : d->ratio == 128 ? 128 : 0;
  P->row_bytes = (int)ckv_row_bytes(d->kv_fmt, d->head_dim, d->n_rot);
  P->lanes = d->ratio == 4 && (d->flags & CKV_FLAG_TWO_LANE) ? 2 : 1;
  P->ncol = d->ratio == 0 ? 0 : P->lanes * (2 * d->head_dim + (d->ratio == 4 ? 2 * d->idx_dim : 0));
  P->idx_rot = d->ratio == 4 ? (d->idx_dim < d->n_rot ? d->idx_dim : d->n_rot) : 0;
  P->idx_row_bytes = d->ratio == 4 ? (int)ckv_idx_row_bytes(d->idx_fmt, d->idx_dim) : 0;
  const double base_c = d->rope_base_comp > 0.0 ? d->rope_base_comp : d->rope_base;
  // CKV_FLAG_SKIP_ROPE: every frequency 0, so every rotation is the identity
  const bool rope = !(d->flags & CKV_FLAG_SKIP_ROPE);
  for (int j = 0; j < 32; ++j) {
    P->theta[j] = rope && 2 * j < d->n_rot ? pow(d->rope_base, -2.0 * j / (double)d->n_rot) : 0.0;
    P->theta_c[j] = rope && 2 * j < d->n_rot ? pow(base_c, -2.0 * j / (double)d->n_rot) : 0.0;
  }
  P->two_bases = rope && base_c != d->rope_base;
  return true;
}

int attn_max_rows(const LayerParams& P) {
  return P.swa + (P.ratio == 4 ? P.topk : P.ratio == 128 ? P.cap : 0);
}

bool c128a_sliced(const LayerParams& P) { return P.ratio == 128 && P.d % 64 == 0 && P.d <= kMaxD; }

bool attn_uses_tiles(const LayerParams& P) {
  return P.act_fmt == CKV_BF16 && P.kv_fmt != CKV_F32 && P.H % 64 == 0 && P.d == 512 && P.n_rot == 64;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const LayerParams& P, int mode, int n) {
  WsLayout L;
  memset(&L, 0, sizeof(L));
  const bool prefill = mode == CKV_MODE_PREFILL;
  const bool proj_mfma = P.act_fmt == CKV_BF16 && P.w_fmt == CKV_BF16;
  // a decode projection launched on its own (c128a layers, and the
  // separate-call c4a path) splits K over 4 blocks per tile (partial sums,
  // added by the compressor in slice order): 4 x 64 blocks instead of 64
  // latency-bound ones.  The single-call c4a step projects inside its scan
  // launch with kProjSlices slices, which this region also holds.
  L.proj_splits = (!prefill && proj_mfma) ? (kProjSlices > 4 ? kProjSlices : 4) : 1;
  const int rows = attn_max_rows(P);
  int rps;
  if (attn_uses_tiles(P)) {
    if (prefill || P.ratio == 0) {
      // (a window-only layer's 128 rows: one split per query -- four tiles in
      // one block, then the output, instead of two blocks and the merge launch)
      rps = rows;
    } else {
      // about 192 blocks over the batch, each split 2 to 10 tiles of 32 rows
      // (measured at 128k: 16 queries x 10 splits, 32 x 5 and 8 x 26 run
      // fastest; half or twice the blocks are 3-30 % slower)
      const int target = (192 + n / 2) / n > 1 ? (192 + n / 2) / n : 1;
      rps = (rows + target - 1) / target;
      rps = rps < 64 ? 64 : rps > 320 ? 320 : rps;
    }
  } else {
    rps = 32;
  }
  rps = (rps + 31) / 32 * 32;
  // the merge kernel combines at most kMaxSplits partial results per query
  const int min_rps = ((rows + kMaxSplits - 1) / kMaxSplits + 31) / 32 * 32;
  if (rps < min_rps) rps = min_rps;
  L.attn_rows_per_split = rps;
  L.attn_splits = (rows + rps - 1) / rps;
  size_t off = 0;
  // sync region: per-sequence top-k histograms of decode calls, sized by the
  // cache batch so that the same bytes are reserved in every mode
  L.sync = 0;
  L.hist = 0;
  if (P.ratio == 4) off += align256((size_t)P.batch * kHistBins * sizeof(uint32_t));
  L.ctr = off;
  if (P.ratio == 4) off += align256((size_t)P.batch * 4 * sizeof(uint32_t));
  L.sync_bytes = off;
  L.sure = off;
  L.cand_key = off;
  L.cand_idx = off;
  if (P.ratio == 4 && !prefill) {
    off += align256((size_t)n * P.topk * sizeof(uint32_t));
    L.cand_key = off;
    off += align256((size_t)n * kCandCap * sizeof(uint32_t));
    L.cand_idx = off;
    off += align256((size_t)n * kCandCap * sizeof(uint32_t));
  }
  L.qf4 = off;
  if (P.ratio == 4 && !prefill && P.idx_fmt == CKV_FP4) off += align256((size_t)n * 64 * 68);
  L.proj = off;
  off += align256((size_t)L.proj_splits * n * P.ncol * sizeof(float));
  L.keys = off;
  if (P.ratio == 4) off += align256((size_t)n * P.cap * sizeof(uint32_t));
  L.pool = off;
  if (P.ratio == 128 && !prefill) off += align256((size_t)n * (P.d + 16) * sizeof(float));
  const bool need_part = !(attn_uses_tiles(P) && L.attn_splits == 1);
  L.part_o = off;
  if (need_part) off += align256((size_t)n * L.attn_splits * P.H * P.d * sizeof(float));
  L.part_ml = off;
  if (need_part) off += align256((size_t)n * L.attn_splits * P.H * 4 * sizeof(float));
  L.total = off ? off : 256;
  return L;
}

}  // namespace ckv

using namespace ckv;

extern "C" size_t ckv_row_bytes(int32_t fmt, int32_t head_dim, int32_t n_rot) {
  if (head_dim <= 0 || n_rot < 0 || n_rot > head_dim) return 0;
  if (fmt == CKV_F32) return (size_t)4 * head_dim;
  if (fmt == CKV_BF16) return (size_t)2 * head_dim;
  if (fmt == CKV_E4M3) {
    const size_t raw = (size_t)(head_dim - n_rot) + 2 * (size_t)n_rot + 4;
    return (raw + 127) / 128 * 128;
  }
  return 0;
}

extern "C" size_t ckv_idx_row_bytes(int32_t fmt, int32_t idx_dim) {
  if (idx_dim <= 0) return 0;
  if (fmt == CKV_F32) return (size_t)4 * idx_dim;
  if (fmt == CKV_BF16) return (size_t)2 * idx_dim;
  if (fmt == CKV_FP4 && idx_dim % 32 == 0) return (size_t)idx_dim / 2 + (size_t)idx_dim / 32;
  return 0;
}

extern "C" int ckv_validate(const ckv_layer_desc* d) {
  if (!d) return CKV_E_INVAL;
  if (d->batch <= 0 || d->hidden <= 0 || d->head_dim <= 0 || d->n_heads <= 0) return CKV_E_INVAL;
  if (!(d->rope_base > 0.0) || !(d->rope_base_comp >= 0.0) || !(d->norm_eps >= 0.f) ||
      !(d->softmax_scale >= 0.f))
    return CKV_E_INVAL;
  if (d->ratio != 0 && d->ratio != 4 && d->ratio != 128) return CKV_E_UNSUPPORTED;
  if (d->n_rot != 64 || d->swa != 128) return CKV_E_UNSUPPORTED;
  if (d->head_dim < 64 || d->head_dim > kMaxD || d->head_dim % 32) return CKV_E_UNSUPPORTED;
  if (d->n_heads % 16 || d->n_heads > 128) return CKV_E_UNSUPPORTED;
  if (d->hidden % 64 || d->hidden > 65536) return CKV_E_UNSUPPORTED;
  if (!fmt_ok(d->kv_fmt, true) || !fmt_ok(d->act_fmt, false) || !fmt_ok(d->w_fmt, false))
    return CKV_E_UNSUPPORTED;
  if (d->kv_fmt == CKV_E4M3 && d->head_dim <= d->n_rot) return CKV_E_UNSUPPORTED;
  if (d->flags & ~(CKV_FLAG_NO_INV_ROPE | CKV_FLAG_IDX_NO_RELU | CKV_FLAG_SKIP_NORM | CKV_FLAG_SKIP_ROPE |
                   CKV_FLAG_KEEP_F32 | CKV_FLAG_OUT_FP8 | CKV_FLAG_Q_NORM | CKV_FLAG_TWO_LANE))
    return CKV_E_UNSUPPORTED;
  if ((d->flags & CKV_FLAG_TWO_LANE) && d->ratio != 4) return CKV_E_UNSUPPORTED;
  // fp8 output: the tiled attention's epilogues only
  if ((d->flags & CKV_FLAG_OUT_FP8) && !(d->act_fmt == CKV_BF16 && d->kv_fmt != CKV_F32 && d->n_heads % 64 == 0 &&
                                          d->head_dim == 512 && d->n_rot == 64))
    return CKV_E_UNSUPPORTED;
  if ((d->flags & CKV_FLAG_KEEP_F32) &&
      (d->kv_fmt != CKV_F32 || d->act_fmt != CKV_F32 || d->w_fmt != CKV_F32 || (d->ratio == 4 && d->idx_fmt != CKV_F32)))
    return CKV_E_UNSUPPORTED;
  if (d->ratio != 0) {
    if (d->comp_cap <= 0) return CKV_E_INVAL;
    if ((long long)d->comp_cap * d->ratio > (1ll << 30)) return CKV_E_UNSUPPORTED;
  }
  if (d->ratio == 4) {
    if (!fmt_ok(d->idx_fmt, false) && d->idx_fmt != CKV_FP4) return CKV_E_UNSUPPORTED;
    if (d->idx_dim != 64 && d->idx_dim != 128) return CKV_E_UNSUPPORTED;
    // fp4 rows: one 16 x 16 x 128 scaled MFMA per head tile and row tile
    if (d->idx_fmt == CKV_FP4 && (d->idx_dim != 128 || d->act_fmt != CKV_BF16)) return CKV_E_UNSUPPORTED;
    if (d->idx_heads < 1 || d->idx_heads > 64) return CKV_E_UNSUPPORTED;
    if (d->top_k < 1 || d->top_k > kMaxTopK) return CKV_E_UNSUPPORTED;
  }
  return CKV_OK;
}

extern "C" const char* ckv_strerror(int code) {
  switch (code) {
    case CKV_OK: return "ok";
    case CKV_E_INVAL: return "invalid argument (NULL pointer, bad size or misaligned pointer)";
    case CKV_E_UNSUPPORTED: return "unsupported layer shape, format or ratio";
    case CKV_E_CAPACITY: return "capacity exceeded (batch, chunk, compressed rows or stage)";
    case CKV_E_WORKSPACE: return "workspace missing or too small";
    case CKV_E_HIP: return "HIP kernel launch failed";
    case CKV_E_SEQUENCE: return "position is not the sequence's next token (host token count)";
    default: return "unknown error";
  }
}

extern "C" size_t ckv_workspace_sync_bytes(const ckv_layer_desc* d, int32_t mode, int32_t n) {
  if (ckv_validate(d) != CKV_OK || n <= 0) return 0;
  if (mode != CKV_MODE_DECODE && mode != CKV_MODE_PREFILL) return 0;
  LayerParams P;
  make_params(d, &P);
  return ws_layout(P, mode, n).sync_bytes;
}

extern "C" size_t ckv_workspace_bytes(const ckv_layer_desc* d, int32_t mode, int32_t n) {
  if (ckv_validate(d) != CKV_OK || n <= 0) return 0;
  if (mode != CKV_MODE_DECODE && mode != CKV_MODE_PREFILL) return 0;
  LayerParams P;
  make_params(d, &P);
  return ws_layout(P, mode, n).total;
}

extern "C" int ckv_hc_validate(const ckv_hc_desc* d) {
  if (!d) return CKV_E_INVAL;
  if (d->n_hc != 4) return CKV_E_UNSUPPORTED;
  if (d->hidden <= 0 || d->hidden % 8 || d->hidden > 65536) return CKV_E_UNSUPPORTED;
  if (d->sinkhorn_iters < 1 || d->sinkhorn_iters > 100) return CKV_E_UNSUPPORTED;
  if (!(d->eps >= 0.f) || !(d->eps < 1e30f)) return CKV_E_UNSUPPORTED;
  if (d->act_fmt != CKV_F32 && d->act_fmt != CKV_BF16) return CKV_E_UNSUPPORTED;
  return CKV_OK;
}
