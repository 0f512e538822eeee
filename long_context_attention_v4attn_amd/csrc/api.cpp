// C ABI of libv4attn: argument validation (before anything is enqueued),
// launch planning, workspace carving and HIP error mapping.  Semantics of each
// call are documented in include/v4attn.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/v4attn.h"
#include "kernels.hpp"

using namespace v4a;

namespace {

thread_local int32_t g_last_hip = 0;

// Launch-plan log: with V4ATTN_LOG=1 in the environment (read on every call)
// each call prints the plan it enqueues, one line on stderr.
bool plan_log() {
  const char* e = getenv("V4ATTN_LOG");
  return e && e[0] == '1';
}

void log_compress(const char* what, const CompressArgs& a) {
  if (!plan_log()) return;
  fprintf(stderr,
          "v4attn: %s B=%d T=%d d=%d m=%d t0=%lld out=%s fmt=%d overlap=%d paged=%d append=%d "
          "norm_rope=%d\n",
          what, a.B, a.T, a.d, a.m, (long long)a.t0, a.out_kind ? "keys" : "kv", a.out_fmt,
          a.kv_prev ? 1 : 0, a.pg.tab ? 1 : 0, a.apos ? 1 : 0, (a.nr_gamma || a.nr_inv) ? 1 : 0);
}

void log_index(const char* what, const IndexArgs& a) {
  if (!plan_log()) return;
  const char* path = a.samp ? "sampled (sample scan, thresholds, collect scan, select)"
                     : a.elist ? "filters, emit in the attention"
                               : "filters + emit";
  fprintf(stderr,
          "v4attn: %s B=%d Q=%d H_I=%d d=%d cap=%lld m=%d k=%d keys=%s scores=%s path=%s "
          "scan_wgs=%d scan_iters=%d partial_rows=%d paged=%d\n",
          what, a.B, a.Q, a.H, a.d, (long long)a.cap, a.m, a.k, a.key_mx ? "mxfp4" : "f32",
          a.score_bf16 ? "bf16" : "f32", path, a.score_wgs, a.score_iters, a.hp_ld,
          a.pg.tab ? 1 : 0);
}

void log_attend(const char* what, const AttendArgs& a) {
  if (!plan_log()) return;
  fprintf(stderr,
          "v4attn: %s B=%d Q=%d H=%d D=%d %s entries=%s splits=%d x %d partials=%s path=%s "
          "loads=%s norm_rope=%d paged=%d fused_select=%d\n",
          what, a.B, a.Q, a.H, a.d_nope + a.d_rope, a.csa ? "csa" : "hca",
          a.csa ? "top-k + window" : "all visible + window", a.n_split, a.split_size,
          a.n_split > 1 ? (a.part_bf16 ? "bf16" : "f32") : "none", a.fp8 ? "fp8 mfma" : "f32 valu",
          a.fp8 ? (a.csa && a.Q == 1 ? "streaming" : "plain") : "plain",
          (a.nr_gamma || a.nr_inv) ? 1 : 0, a.c_pg.tab ? 1 : 0, a.sel_ctr ? 1 : 0);
}
// events for the calling thread's next index / attend call (kernel timing)
thread_local KernelEvents g_time_next = {nullptr, nullptr};

// Takes the pending timing events, if any (one call consumes them).
const KernelEvents* take_events(KernelEvents* slot) {
  if (!g_time_next.start || !g_time_next.stop) return nullptr;
  *slot = g_time_next;
  g_time_next = {nullptr, nullptr};
  return slot;
}

v4a_status hip_status(hipError_t e) {
  if (e == hipSuccess) return V4A_OK;
  g_last_hip = (int32_t)e;
  return V4A_ERR_HIP;
}

bool is_pow2_le(int m, int hi) { return m >= 1 && m <= hi && (m & (m - 1)) == 0; }

bool valid_kv(const v4a_kv* kv) {
  if (!kv || !kv->nope || !kv->rope || kv->cap < 1 || kv->d_nope < 1 || kv->d_rope < 0) return false;
  if (kv->fmt == V4A_KV_FP8_BF16ROPE && !kv->scale) return false;
  return kv->fmt == V4A_F32 || kv->fmt == V4A_KV_FP8_BF16ROPE;
}

// Shared validation of the two attend calls.
// V4A_OK with *empty set: B == 0 or Q == 0, nothing to read or write.
v4a_status check_attend(const void* q, int32_t q_dtype, const v4a_kv* comp, const v4a_kv* win,
                        int32_t n_win, const int64_t* pos, int32_t B, int32_t Q, int32_t H,
                        void* out, int32_t out_dtype, bool* empty) {
  *empty = false;
  if (B < 0 || Q < 0) return V4A_ERR_INVALID;
  if (B == 0 || Q == 0) {
    *empty = true;
    return V4A_OK;
  }
  if (!q || !pos || !out || !comp || !win || B < 0 || Q < 0 || H < 1 || n_win < 0)
    return V4A_ERR_INVALID;
  if (!valid_kv(comp) || !valid_kv(win)) return V4A_ERR_INVALID;
  if (comp->fmt != win->fmt || comp->d_nope != win->d_nope || comp->d_rope != win->d_rope)
    return V4A_ERR_INVALID;
  if (q_dtype != V4A_F32 && q_dtype != V4A_BF16) return V4A_ERR_INVALID;
  if (out_dtype != V4A_F32 && out_dtype != V4A_BF16) return V4A_ERR_INVALID;
  if (win->cap < n_win) return V4A_ERR_INVALID;
  if (H > 128) return V4A_ERR_UNSUPPORTED;
  const int D = comp->d_nope + comp->d_rope;
  if (comp->fmt == V4A_KV_FP8_BF16ROPE) {
    if (comp->d_nope != 448 || comp->d_rope != 64 || q_dtype != V4A_BF16 || H % 16 != 0)
      return V4A_ERR_UNSUPPORTED;
  } else if (D > 512 || D % 8 != 0) {
    return V4A_ERR_UNSUPPORTED;
  }
  return V4A_OK;
}

void fill_attend(AttendArgs& a, const void* q, int32_t q_dtype, const v4a_kv* comp,
                 const v4a_kv* win, int32_t n_win, const int64_t* pos, const float* sink,
                 float sm_scale, int32_t B, int32_t Q, int32_t H, void* out, int32_t out_dtype) {
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.q_bf16 = q_dtype == V4A_BF16;
  a.c_nope = (const uint8_t*)comp->nope;
  a.c_rope = (const uint16_t*)comp->rope;
  a.c_scale = comp->scale;
  a.c_cap = comp->cap;
  a.w_nope = (const uint8_t*)win->nope;
  a.w_rope = (const uint16_t*)win->rope;
  a.w_scale = win->scale;
  a.w_cap = win->cap;
  a.n_win = n_win;
  a.pos = pos;
  a.sink = sink;
  a.sm_scale = sm_scale;
  a.B = B;
  a.Q = Q;
  a.H = H;
  a.d_nope = comp->d_nope;
  a.d_rope = comp->d_rope;
  a.out = out;
  a.out_bf16 = out_dtype == V4A_BF16;
  a.fp8 = comp->fmt == V4A_KV_FP8_BF16ROPE;
}

v4a_status run_attend(AttendArgs& a, int64_t n_entries_max, void* ws, size_t ws_bytes,
                      void* stream, const v4a_norm_rope* nr = nullptr) {
  attend_plan(a, n_entries_max);
  const size_t need = attend_workspace_bytes(a);
  if (need > 0) {
    if (!ws || ws_bytes < need) return V4A_ERR_WORKSPACE;
    attend_carve(a, ws);
  }
  if (nr) {
    a.nr_gamma = nr->gamma;
    a.nr_eps = nr->eps;
    a.nr_inv = a.d_rope > 0 ? nr->inv_freq : nullptr;
  }
  log_attend(a.csa ? "csa_attend" : "hca_attend", a);
  KernelEvents ev;
  return hip_status(launch_attend(a, (hipStream_t)stream, take_events(&ev)));
}

// Extra checks of the _nr attend calls.
v4a_status check_nr(const v4a_kv* comp, const v4a_norm_rope* nr) {
  if (!nr) return V4A_OK;
  if (!(nr->eps >= 0.0f)) return V4A_ERR_INVALID;
  if (comp->fmt != V4A_KV_FP8_BF16ROPE) return V4A_ERR_UNSUPPORTED;
  return V4A_OK;
}

// Validates a page table for a cache of `pool_rows` rows and rate m; fills
// the kernel's view and the sequence's logical capacity.
v4a_status check_pages(const v4a_pages* pg, int m, int64_t pool_rows, int64_t min_per_page,
                       Pages* out, int64_t* lcap) {
  if (!pg || !pg->table || pg->max_pages < 1 || m < 1) return V4A_ERR_INVALID;
  const int64_t pt = pg->page_tokens;
  if (pt < 128 || pt > ((int64_t)1 << 30) || (pt & (pt - 1)) != 0 || m > pt)
    return V4A_ERR_UNSUPPORTED;
  const int64_t P = pt / m;
  if (P < min_per_page) return V4A_ERR_UNSUPPORTED;
  if (pool_rows < P || pool_rows % P != 0) return V4A_ERR_INVALID;
  if (pool_rows >= ((int64_t)1 << 31) || (int64_t)pg->max_pages * P >= ((int64_t)1 << 31))
    return V4A_ERR_UNSUPPORTED;
  int sh = 0;
  while (((int64_t)1 << sh) < P) sh++;
  out->tab = pg->table;
  out->tab_ld = pg->max_pages;
  out->psh = sh;
  out->n_pages = pool_rows / P;
  *lcap = (int64_t)pg->max_pages * P;
  return V4A_OK;
}

}  // namespace

extern "C" {

static v4a_status compress_impl(const void* kv_cur, const void* gate_cur, const void* kv_prev,
                                const void* gate_prev, const float* pos_bias, int32_t in_dtype,
                                int32_t B, int32_t T, int32_t d, int32_t m, int64_t t0,
                                int32_t out_kind, const void* out, const v4a_norm_rope* nr,
                                void* stream, const v4a_pages* pages = nullptr,
                                const int64_t* apos = nullptr, float* state = nullptr,
                                CompressArgs* built = nullptr) {
  // built: validate and fill the kernel arguments only (no launch)
  if (built) {
    memset(built, 0, sizeof(*built));
    built->B = 0;
  }
  if (B < 0 || T < 0 || d < 1 || t0 < 0) return V4A_ERR_INVALID;
  if (B == 0 || (!apos && T == 0)) return V4A_OK;   // nothing to read or write
  if (!kv_cur) return V4A_ERR_INVALID;
  if (!out && !apos) return V4A_ERR_INVALID;
  if (nr && !(nr->eps >= 0.0f)) return V4A_ERR_INVALID;
  if (nr && out_kind != V4A_OUT_KV) return V4A_ERR_UNSUPPORTED;
  if (in_dtype != V4A_F32 && in_dtype != V4A_BF16) return V4A_ERR_INVALID;
  if (!is_pow2_le(m, 128)) return V4A_ERR_UNSUPPORTED;
  if (T % m != 0 || t0 % m != 0) return V4A_ERR_INVALID;
  if (gate_prev && !kv_prev) return V4A_ERR_INVALID;
  if (d > 1024) return V4A_ERR_UNSUPPORTED;
  CompressArgs a;
  memset(&a, 0, sizeof(a));
  a.kv_cur = kv_cur;
  a.gate_cur = gate_cur;
  a.kv_prev = kv_prev;
  a.gate_prev = gate_prev;
  a.bias = pos_bias;
  a.in_bf16 = in_dtype == V4A_BF16;
  a.B = B;
  a.T = T;
  a.d = d;
  a.m = m;
  a.t0 = t0;
  a.out_kind = out_kind;
  if (!out) {
    // a state-only append: nothing is stored
    a.no_store = 1;
    a.d_nope = d;
  } else if (out_kind == V4A_OUT_KV) {
    const v4a_kv* kv = (const v4a_kv*)out;
    if (!valid_kv(kv) || kv->d_nope + kv->d_rope != d) return V4A_ERR_INVALID;
    if (kv->fmt == V4A_KV_FP8_BF16ROPE && kv->d_nope % 32 != 0) return V4A_ERR_UNSUPPORTED;
    a.out_fmt = kv->fmt;
    a.d_nope = kv->d_nope;
    a.cap = kv->cap;
    a.o_a = kv->nope;
    a.o_b = kv->rope;
    a.o_scale = kv->scale;
    if (nr) {
      if (kv->d_nope % 2 != 0 || kv->d_rope % 2 != 0) return V4A_ERR_UNSUPPORTED;
      a.nr_gamma = nr->gamma;
      a.nr_inv = kv->d_rope > 0 ? nr->inv_freq : nullptr;
      a.nr_eps = nr->eps;
    }
  } else if (out_kind == V4A_OUT_IDX) {
    const v4a_idx* ix = (const v4a_idx*)out;
    if (!ix->codes || ix->cap < 1 || ix->d != d) return V4A_ERR_INVALID;
    if (ix->fmt == V4A_IDX_MXFP4) {
      if (!ix->scales) return V4A_ERR_INVALID;
      if (d % 32 != 0) return V4A_ERR_UNSUPPORTED;
    } else if (ix->fmt != V4A_F32) {
      return V4A_ERR_INVALID;
    }
    a.out_fmt = ix->fmt;
    a.cap = ix->cap;
    a.o_a = ix->codes;
    a.o_b = ix->scales;
  } else {
    return V4A_ERR_INVALID;
  }
  if (pages && out) {
    int64_t lcap = 0;
    v4a_status s = check_pages(pages, m, a.cap, 1, &a.pg, &lcap);
    if (s != V4A_OK) return s;
    if (!apos && t0 / m + T / m > lcap) return V4A_ERR_INVALID;
    a.cap = lcap;
  }
  if (apos) {
    // decode-time append: one token per sequence folded into the state
    if (!state && (m > 1 || kv_prev)) return V4A_ERR_INVALID;
    a.apos = apos;
    a.state = state;
    if (built) {
      *built = a;
      return V4A_OK;
    }
    log_compress("append", a);
    return hip_status(launch_compress(a, (hipStream_t)stream));
  }
  if (B == 0 || T == 0) return V4A_OK;
  log_compress("compress", a);
  return hip_status(launch_compress(a, (hipStream_t)stream));
}

v4a_status v4attn_compress_paged(const void* kv_cur, const void* gate_cur, const void* kv_prev,
                                 const void* gate_prev, const float* pos_bias, int32_t in_dtype,
                                 int32_t B, int32_t T, int32_t d, int32_t m, int64_t t0,
                                 int32_t out_kind, const void* out, const v4a_pages* pages,
                                 const v4a_norm_rope* nr, void* stream) {
  if (!pages && B > 0 && T > 0) return V4A_ERR_INVALID;
  return compress_impl(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, in_dtype, B, T, d, m, t0,
                       out_kind, out, nr, stream, pages);
}

v4a_status v4attn_append(const void* kv_cur, const void* gate_cur, const void* kv_prev,
                         const void* gate_prev, float* state, const int64_t* pos,
                         const float* pos_bias, int32_t in_dtype, int32_t B, int32_t d, int32_t m,
                         int32_t out_kind, const void* out, const v4a_pages* pages,
                         const v4a_norm_rope* nr, void* stream) {
  if (!pos && B > 0) return V4A_ERR_INVALID;
  // T = m, t0 = 0 pass the shape checks of the chunked call; the append
  // kernel takes its blocks from pos
  return compress_impl(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, in_dtype, B, m, d, m, 0,
                       out_kind, out, nr, stream, pages, pos, state);
}

v4a_status v4attn_compress(const void* kv_cur, const void* gate_cur, const void* kv_prev,
                           const void* gate_prev, const float* pos_bias, int32_t in_dtype,
                           int32_t B, int32_t T, int32_t d, int32_t m, int64_t t0,
                           int32_t out_kind, const void* out, void* stream) {
  return compress_impl(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, in_dtype, B, T, d, m, t0,
                       out_kind, out, nullptr, stream);
}

v4a_status v4attn_compress_nr(const void* kv_cur, const void* gate_cur, const void* kv_prev,
                              const void* gate_prev, const float* pos_bias, int32_t in_dtype,
                              int32_t B, int32_t T, int32_t d, int32_t m, int64_t t0,
                              int32_t out_kind, const void* out, const v4a_norm_rope* nr,
                              void* stream) {
  return compress_impl(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, in_dtype, B, T, d, m, t0,
                       out_kind, out, nr, stream);
}

// Validates an index call (B, Q >= 1) and fills its kernel arguments; the
// workspace is carved by the caller.
static v4a_status index_prepare(IndexArgs& a, const void* q_idx, int32_t q_dtype, const float* w,
                                const v4a_idx* keys, const int64_t* pos, int32_t B, int32_t Q,
                                int32_t H_I, int32_t m, int32_t k, int32_t* topk, int score_bf16,
                                const v4a_pages* pages) {
  if (!q_idx || !w || !keys || !pos || !topk || H_I < 1 || k < 1 || m < 1)
    return V4A_ERR_INVALID;
  if (q_dtype != V4A_F32 && q_dtype != V4A_BF16) return V4A_ERR_INVALID;
  if (!keys->codes || keys->cap < 1 || keys->d < 1) return V4A_ERR_INVALID;
  if (k > 4096 || H_I > 64) return V4A_ERR_UNSUPPORTED;
  if (keys->cap >= ((int64_t)1 << 31)) return V4A_ERR_UNSUPPORTED;
  memset(&a, 0, sizeof(a));
  if (keys->fmt == V4A_IDX_MXFP4) {
    if (!keys->scales) return V4A_ERR_INVALID;
    if (keys->d != 128 || H_I % 16 != 0) return V4A_ERR_UNSUPPORTED;
    a.key_mx = 1;
  } else if (keys->fmt == V4A_F32) {
    if (keys->d > 256 || (int64_t)keys->d * H_I > 8192) return V4A_ERR_UNSUPPORTED;
  } else {
    return V4A_ERR_INVALID;
  }
  a.q = q_idx;
  a.q_bf16 = q_dtype == V4A_BF16;
  a.w = w;
  a.codes = keys->codes;
  a.kscales = keys->scales;
  a.cap = keys->cap;
  a.d = keys->d;
  a.pos = pos;
  a.B = B;
  a.Q = Q;
  a.H = H_I;
  a.m = m;
  a.k = k;
  a.topk = topk;
  a.score_bf16 = score_bf16;
  if (pages) {
    if (!a.key_mx) return V4A_ERR_UNSUPPORTED;
    v4a_status s = check_pages(pages, m, keys->cap, 128, &a.pg, &a.cap);
    if (s != V4A_OK) return s;
  }
  return V4A_OK;
}

static v4a_status index_topk(const void* q_idx, int32_t q_dtype, const float* w,
                             const v4a_idx* keys, const int64_t* pos, int32_t B, int32_t Q,
                             int32_t H_I, int32_t m, int32_t k, int32_t* topk, void* ws,
                             size_t ws_bytes, void* stream, int score_bf16,
                             const v4a_pages* pages = nullptr, bool fixed_scratch = false) {
  if (B < 0 || Q < 0) return V4A_ERR_INVALID;
  if (B == 0 || Q == 0) return V4A_OK;     // nothing to read or write
  IndexArgs a;
  v4a_status s = index_prepare(a, q_idx, q_dtype, w, keys, pos, B, Q, H_I, m, k, topk, score_bf16,
                               pages);
  if (s != V4A_OK) return s;
  size_t need = index_workspace_bytes(B, Q, H_I, keys->d, a.cap, a.key_mx);
  if (fixed_scratch) {
    // the library's own device array (no allocation): the call's scratch
    // must fit it
    if (need > kIndexScratchBytes) return V4A_ERR_SCRATCH;
    hipError_t e = index_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  } else if (!ws || ws_bytes < need) {
    return V4A_ERR_WORKSPACE;
  }
  index_carve(a, ws);
  if (B == 0 || Q == 0) return V4A_OK;
  log_index(score_bf16 ? "index_topk_bf16" : "index_topk", a);
  KernelEvents ev;
  return hip_status(launch_index_topk(a, (hipStream_t)stream, take_events(&ev)));
}

v4a_status v4attn_index_topk(const void* q_idx, int32_t q_dtype, const float* w,
                             const v4a_idx* keys, const int64_t* pos, int32_t B, int32_t Q,
                             int32_t H_I, int32_t m, int32_t k, int32_t* topk, void* ws,
                             size_t ws_bytes, void* stream) {
  return index_topk(q_idx, q_dtype, w, keys, pos, B, Q, H_I, m, k, topk, ws, ws_bytes, stream, 0);
}

v4a_status v4attn_index_topk_noalloc(const void* q_idx, int32_t q_dtype, const float* w,
                                     const v4a_idx* keys, const int64_t* pos, int32_t B,
                                     int32_t Q, int32_t H_I, int32_t m, int32_t k, int32_t* topk,
                                     void* stream) {
  return index_topk(q_idx, q_dtype, w, keys, pos, B, Q, H_I, m, k, topk, nullptr, 0, stream, 0,
                    nullptr, true);
}

v4a_status v4attn_index_topk_bf16(const void* q_idx, int32_t q_dtype, const float* w,
                                  const v4a_idx* keys, const int64_t* pos, int32_t B, int32_t Q,
                                  int32_t H_I, int32_t m, int32_t k, int32_t* topk, void* ws,
                                  size_t ws_bytes, void* stream) {
  return index_topk(q_idx, q_dtype, w, keys, pos, B, Q, H_I, m, k, topk, ws, ws_bytes, stream, 1);
}

v4a_status v4attn_append_batch(int32_t n, const v4a_append* calls, void* stream) {
  if (n < 0 || (n > 0 && !calls)) return V4A_ERR_INVALID;
  if (n > V4A_MAX_APPEND) return V4A_ERR_UNSUPPORTED;
  AppendBatch ab;
  memset(&ab, 0, sizeof(ab));
  ab.n = n;
  for (int j = 0; j < n; j++) {
    const v4a_append& c = calls[j];
    if (!c.pos && c.B > 0) return V4A_ERR_INVALID;
    const v4a_status s = compress_impl(c.kv_cur, c.gate_cur, c.kv_prev, c.gate_prev, c.pos_bias,
                                       c.in_dtype, c.B, c.m, c.d, c.m, 0, c.out_kind, c.out, c.nr,
                                       stream, c.pages, c.pos, c.state, &ab.c[j]);
    if (s != V4A_OK) return s;
  }
  for (int j = 0; j < n; j++) log_compress("append_batch", ab.c[j]);
  return hip_status(launch_append_batch(ab, (hipStream_t)stream));
}

v4a_status v4attn_index_topk_paged(const void* q_idx, int32_t q_dtype, const float* w,
                                   const v4a_idx* keys, const v4a_pages* pages,
                                   const int64_t* pos, int32_t B, int32_t Q, int32_t H_I,
                                   int32_t m, int32_t k, int32_t score_bf16, int32_t* topk,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!pages && B > 0 && Q > 0) return V4A_ERR_INVALID;
  return index_topk(q_idx, q_dtype, w, keys, pos, B, Q, H_I, m, k, topk, ws, ws_bytes, stream,
                    score_bf16 ? 1 : 0, pages);
}

v4a_status v4attn_csa_attend_paged(const void* q, int32_t q_dtype, const v4a_kv* comp,
                                   const v4a_pages* pages, int32_t m, const int32_t* topk,
                                   int32_t k, const v4a_kv* win, int32_t n_win,
                                   const int64_t* pos, const float* sink, float sm_scale,
                                   int32_t B, int32_t Q, int32_t H, void* out, int32_t out_dtype,
                                   const v4a_norm_rope* nr, void* ws, size_t ws_bytes,
                                   void* stream) {
  bool empty;
  v4a_status s = check_attend(q, q_dtype, comp, win, n_win, pos, B, Q, H, out, out_dtype, &empty);
  if (s != V4A_OK || empty) return s;
  if ((s = check_nr(comp, nr)) != V4A_OK) return s;
  if (k < 0 || (k > 0 && !topk)) return V4A_ERR_INVALID;
  if (comp->fmt != V4A_KV_FP8_BF16ROPE) return V4A_ERR_UNSUPPORTED;
  AttendArgs a;
  fill_attend(a, q, q_dtype, comp, win, n_win, pos, sink, sm_scale, B, Q, H, out, out_dtype);
  if ((s = check_pages(pages, m, comp->cap, 1, &a.c_pg, &a.c_cap)) != V4A_OK) return s;
  a.csa = 1;
  a.topk = topk;
  a.k = k;
  a.m = 1;
  if (B == 0 || Q == 0) return V4A_OK;
  return run_attend(a, (int64_t)k + n_win, ws, ws_bytes, stream, nr);
}

v4a_status v4attn_hca_attend_paged(const void* q, int32_t q_dtype, const v4a_kv* comp,
                                   const v4a_pages* pages, int32_t m, const v4a_kv* win,
                                   int32_t n_win, const int64_t* pos, const float* sink,
                                   float sm_scale, int32_t B, int32_t Q, int32_t H, void* out,
                                   int32_t out_dtype, const v4a_norm_rope* nr, void* ws,
                                   size_t ws_bytes, void* stream) {
  bool empty;
  v4a_status s = check_attend(q, q_dtype, comp, win, n_win, pos, B, Q, H, out, out_dtype, &empty);
  if (s != V4A_OK || empty) return s;
  if ((s = check_nr(comp, nr)) != V4A_OK) return s;
  if (m < 1) return V4A_ERR_INVALID;
  if (comp->fmt != V4A_KV_FP8_BF16ROPE) return V4A_ERR_UNSUPPORTED;
  AttendArgs a;
  fill_attend(a, q, q_dtype, comp, win, n_win, pos, sink, sm_scale, B, Q, H, out, out_dtype);
  if ((s = check_pages(pages, m, comp->cap, 1, &a.c_pg, &a.c_cap)) != V4A_OK) return s;
  a.csa = 0;
  a.topk = nullptr;
  a.m = m;
  if (B == 0 || Q == 0) return V4A_OK;
  return run_attend(a, a.c_cap + n_win, ws, ws_bytes, stream, nr);
}

v4a_status v4attn_csa_attend_nr(const void* q, int32_t q_dtype, const v4a_kv* comp,
                                const int32_t* topk, int32_t k, const v4a_kv* win, int32_t n_win,
                                const int64_t* pos, const float* sink, float sm_scale, int32_t B,
                                int32_t Q, int32_t H, void* out, int32_t out_dtype,
                                const v4a_norm_rope* nr, void* ws, size_t ws_bytes, void* stream) {
  bool empty;
  v4a_status s = check_attend(q, q_dtype, comp, win, n_win, pos, B, Q, H, out, out_dtype, &empty);
  if (s != V4A_OK || empty) return s;
  if ((s = check_nr(comp, nr)) != V4A_OK) return s;
  if (k < 0 || (k > 0 && !topk)) return V4A_ERR_INVALID;
  AttendArgs a;
  fill_attend(a, q, q_dtype, comp, win, n_win, pos, sink, sm_scale, B, Q, H, out, out_dtype);
  a.csa = 1;
  a.topk = topk;
  a.k = k;
  a.m = 1;
  if (B == 0 || Q == 0) return V4A_OK;
  return run_attend(a, (int64_t)k + n_win, ws, ws_bytes, stream, nr);
}

v4a_status v4attn_csa_attend(const void* q, int32_t q_dtype, const v4a_kv* comp,
                             const int32_t* topk, int32_t k, const v4a_kv* win, int32_t n_win,
                             const int64_t* pos, const float* sink, float sm_scale, int32_t B,
                             int32_t Q, int32_t H, void* out, int32_t out_dtype, void* ws,
                             size_t ws_bytes, void* stream) {
  return v4attn_csa_attend_nr(q, q_dtype, comp, topk, k, win, n_win, pos, sink, sm_scale, B, Q, H,
                              out, out_dtype, nullptr, ws, ws_bytes, stream);
}

v4a_status v4attn_csa_index_attend(const void* q_idx, int32_t q_idx_dtype, const float* w,
                                   const v4a_idx* keys, int32_t H_I, int32_t m, int32_t k,
                                   int32_t* topk, const void* q, int32_t q_dtype,
                                   const v4a_kv* comp, const v4a_kv* win, int32_t n_win,
                                   const int64_t* pos, const float* sink, float sm_scale,
                                   int32_t B, int32_t Q, int32_t H, void* out, int32_t out_dtype,
                                   void* ws_index, size_t ws_index_bytes, void* ws_attend,
                                   size_t ws_attend_bytes, void* stream) {
  bool empty;
  v4a_status s = check_attend(q, q_dtype, comp, win, n_win, pos, B, Q, H, out, out_dtype, &empty);
  if (s != V4A_OK || empty) return s;
  IndexArgs ia;
  s = index_prepare(ia, q_idx, q_idx_dtype, w, keys, pos, B, Q, H_I, m, k, topk, 0, nullptr);
  if (s != V4A_OK) return s;
  AttendArgs aa;
  fill_attend(aa, q, q_dtype, comp, win, n_win, pos, sink, sm_scale, B, Q, H, out, out_dtype);
  aa.csa = 1;
  aa.topk = topk;
  aa.k = k;
  aa.m = 1;
  attend_plan(aa, (int64_t)k + n_win);
  // the emit step moves into the attention when the rows take the
  // three-filter selection and the attention is the FP8 kernel with splits
  // of at most 256 entries; otherwise the two calls run as they are
  const int fused = aa.fp8 && index_filter_path(ia) &&
                    aa.split_size <= 256;
  const size_t need_i = index_workspace_bytes(B, Q, H_I, keys->d, ia.cap, ia.key_mx, fused);
  if (!ws_index || ws_index_bytes < need_i) return V4A_ERR_WORKSPACE;
  const size_t need_a = attend_workspace_bytes(aa);
  if (need_a > 0) {
    if (!ws_attend || ws_attend_bytes < need_a) return V4A_ERR_WORKSPACE;
    attend_carve(aa, ws_attend);
  }
  index_carve(ia, ws_index, fused);
  log_index("csa_index_attend: index", ia);
  hipError_t e = launch_index_topk(ia, (hipStream_t)stream, nullptr);
  if (e != hipSuccess) return hip_status(e);
  if (fused) {
    aa.sel_ctr = ia.ctr;
    aa.sel_cand = ia.cand;
    aa.sel_elist = ia.elist;
    aa.sel_elen = ia.elen;
    aa.sel_scores = ia.scores;
    aa.sel_sc_ld = ia.sc_ld;
    aa.sel_cap = ia.cap;
    aa.sel_m = m;
    aa.sel_topk = topk;
  }
  log_attend("csa_index_attend: attend", aa);
  return hip_status(launch_attend(aa, (hipStream_t)stream, nullptr));
}

v4a_status v4attn_hca_attend_nr(const void* q, int32_t q_dtype, const v4a_kv* comp, int32_t m,
                                const v4a_kv* win, int32_t n_win, const int64_t* pos,
                                const float* sink, float sm_scale, int32_t B, int32_t Q, int32_t H,
                                void* out, int32_t out_dtype, const v4a_norm_rope* nr, void* ws,
                                size_t ws_bytes, void* stream) {
  bool empty;
  v4a_status s = check_attend(q, q_dtype, comp, win, n_win, pos, B, Q, H, out, out_dtype, &empty);
  if (s != V4A_OK || empty) return s;
  if ((s = check_nr(comp, nr)) != V4A_OK) return s;
  if (m < 1) return V4A_ERR_INVALID;
  AttendArgs a;
  fill_attend(a, q, q_dtype, comp, win, n_win, pos, sink, sm_scale, B, Q, H, out, out_dtype);
  a.csa = 0;
  a.topk = nullptr;
  a.m = m;
  if (B == 0 || Q == 0) return V4A_OK;
  return run_attend(a, comp->cap + n_win, ws, ws_bytes, stream, nr);
}

v4a_status v4attn_hca_attend(const void* q, int32_t q_dtype, const v4a_kv* comp, int32_t m,
                             const v4a_kv* win, int32_t n_win, const int64_t* pos,
                             const float* sink, float sm_scale, int32_t B, int32_t Q, int32_t H,
                             void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                             void* stream) {
  return v4attn_hca_attend_nr(q, q_dtype, comp, m, win, n_win, pos, sink, sm_scale, B, Q, H, out,
                              out_dtype, nullptr, ws, ws_bytes, stream);
}

size_t v4attn_workspace_bytes(int32_t op, int32_t B, int32_t Q, int32_t H, int32_t d, int64_t cap,
                              int32_t k, int32_t n_win) {
  if (B < 0 || Q < 0 || H < 1 || d < 1) return (size_t)-1;
  if (op == V4A_OP_INDEX_TOPK || op == V4A_OP_CSA_INDEX) {
    if (cap < 1) return (size_t)-1;
    return index_workspace_bytes(B, Q, H, d, cap, d == 128 && H % 16 == 0 ? 1 : 0,
                                 op == V4A_OP_CSA_INDEX);
  }
  if (op == V4A_OP_CSA_ATTEND_NR) op = V4A_OP_CSA_ATTEND;
  if (op == V4A_OP_HCA_ATTEND_NR) op = V4A_OP_HCA_ATTEND;
  if (op != V4A_OP_CSA_ATTEND && op != V4A_OP_HCA_ATTEND) return (size_t)-1;
  if (n_win < 0 || k < 0) return (size_t)-1;
  AttendArgs a;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.Q = Q;
  a.H = H;
  a.d_nope = d;
  a.d_rope = 0;
  a.fp8 = 0;                      // fp32 partials: the larger of the two formats
  int64_t n = op == V4A_OP_CSA_ATTEND ? (int64_t)k + n_win : cap + n_win;
  attend_plan(a, n);
  // the plan of the fp32 partials bounds the FP8 one (the _nr calls need no
  // more: their queries are normalised inside the attention kernel)
  return attend_workspace_bytes(a);
}

const char* v4attn_status_str(v4a_status s) {
  switch (s) {
    case V4A_OK: return "ok";
    case V4A_ERR_INVALID: return "invalid argument";
    case V4A_ERR_UNSUPPORTED: return "unsupported shape or format";
    case V4A_ERR_WORKSPACE: return "workspace missing or too small";
    case V4A_ERR_HIP: return "HIP runtime error";
    case V4A_ERR_SCRATCH:
      return "the call needs more scratch than the allocation-free entry point's fixed 32 MiB";
    default: return "unknown status";
  }
}

int32_t v4attn_last_hip_error(void) { return g_last_hip; }

void v4attn_time_next_kernel(void* start, void* stop) {
  g_time_next = {(hipEvent_t)start, (hipEvent_t)stop};
}

int32_t v4attn_version(void) { return 100; }

}  // extern "C"
