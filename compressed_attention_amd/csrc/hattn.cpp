// C ABI of libhattn: argument validation, workspace sizing, dispatch, timer.
// Every check happens before anything is enqueued; see include/hattn.h.
#include "hattn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

hattn_status_t fail(hattn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

hattn_status_t ok() {
  g_err[0] = 0;
  return HATTN_OK;
}

hattn_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int dt) { return dt == HATTN_F32 || dt == HATTN_BF16; }
int elem_bytes(int dt) { return dt == HATTN_F32 ? 4 : 2; }

// Workspace protocol shared by every entry point that takes one.  Returns
// true when the call must end here: a size query (HATTN_OK) or a missing /
// too small workspace.  ws_bytes == NULL means "no workspace given", which
// is fine exactly when the call needs none.
bool ws_query(void* ws, size_t* ws_bytes, size_t need, hattn_status_t* st) {
  if (!ws_bytes) {
    if (need == 0) {
      *st = HATTN_OK;
      return false;
    }
    *st = fail(HATTN_ERR_WORKSPACE, "a workspace of %zu bytes is required", need);
    return true;
  }
  if (!ws) {
    *ws_bytes = need;
    *st = ok();
    return true;
  }
  if (*ws_bytes < need) {
    *st = fail(HATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", *ws_bytes, need);
    return true;
  }
  *st = HATTN_OK;
  return false;
}

// ---- kernel timer ----------------------------------------------------------
struct Pending {
  std::string name;
  hipEvent_t e0, e1;
};
bool g_timer_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
std::map<std::string, std::pair<double, int64_t>> g_totals;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace hattn {

thread_local LaunchScope* t_scope = nullptr;

LaunchScope::LaunchScope(const char* name, hipStream_t s)
    : name_(name), stream_(s), ev0_(nullptr), ev1_(nullptr), used_(false), outer_(t_scope) {
  t_scope = this;
  if (!g_timer_on) return;
  ev0_ = take_event();
  ev1_ = take_event();
}

LaunchScope::~LaunchScope() {
  t_scope = outer_;
  if (used_ && ev0_ && ev1_) {
    g_pending.push_back({name_, ev0_, ev1_});
  } else {
    if (ev0_) g_free.push_back(ev0_);
    if (ev1_) g_free.push_back(ev1_);
  }
}

bool timer_events(hipEvent_t* e0, hipEvent_t* e1) {
  LaunchScope* sc = t_scope;
  if (!sc || sc->used_ || !sc->ev0_ || !sc->ev1_) return false;
  sc->used_ = true;
  *e0 = sc->ev0_;
  *e1 = sc->ev1_;
  return true;
}

}  // namespace hattn

extern "C" {

const char* hattn_status_string(int status) {
  switch (status) {
    case HATTN_OK: return "HATTN_OK";
    case HATTN_ERR_ARG: return "HATTN_ERR_ARG: invalid argument";
    case HATTN_ERR_UNSUPPORTED: return "HATTN_ERR_UNSUPPORTED: no kernel for this configuration";
    case HATTN_ERR_WORKSPACE: return "HATTN_ERR_WORKSPACE: workspace too small";
    case HATTN_ERR_HIP: return "HATTN_ERR_HIP: HIP runtime error";
    default: return "unknown hattn status";
  }
}

const char* hattn_last_error(void) { return g_err; }

int hattn_abi_version(void) { return 3; }

// Arrays that kernels access with 16-byte vector loads or stores; NULL passes.
static bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15u) return false;
  return true;
}
#define HATTN_REQUIRE_ALIGNED(fn, ...) \
  if (!aligned16({__VA_ARGS__})) return fail(HATTN_ERR_ARG, "%s: arrays must be 16-byte aligned", fn)

hattn_status_t hattn_compress(int dtype, const void* x, int64_t bt, int64_t L, int32_t C, const float* logits,
                              const float* pos_bias, int32_t w, int32_t stride, int64_t e_begin, int64_t e_end,
                              void* y, void* stream) {
  if (!dtype_ok(dtype)) return fail(HATTN_ERR_ARG, "compress: bad dtype %d", dtype);
  if (bt < 0 || L < 0) return fail(HATTN_ERR_ARG, "compress: negative size");
  if (w < 1 || w > 4096 || stride < 1) return fail(HATTN_ERR_ARG, "compress: need 1 <= w <= 4096 and stride >= 1");
  const int vec = 16 / elem_bytes(dtype);
  if (C <= 0 || C % vec) return fail(HATTN_ERR_ARG, "compress: C=%d must be a positive multiple of %d", C, vec);
  if (L < w) return fail(HATTN_ERR_ARG, "compress: L=%lld shorter than the window %d", (long long)L, w);
  const int64_t N = (L - w) / stride + 1;
  if (e_begin < 0 || e_end < e_begin || e_end > N)
    return fail(HATTN_ERR_ARG, "compress: entry range [%lld, %lld) outside [0, %lld]", (long long)e_begin,
                (long long)e_end, (long long)N);
  if (bt == 0 || e_end == e_begin) return ok();
  if (!x || !y) return fail(HATTN_ERR_ARG, "compress: NULL x or y");
  HATTN_REQUIRE_ALIGNED("compress", x, y);
  return hip_status(hattn::launch_compress(dtype, x, bt, L, C, logits, pos_bias, w, stride, N, e_begin, e_end, y,
                                           (hipStream_t)stream),
                    "compress");
}

hattn_status_t hattn_compress_with_index(int dtype, const void* x, const void* x_i, int64_t bt, int64_t L, int32_t C,
                                        int32_t C_i, const float* logits, const float* pos_bias, int32_t w,
                                        int32_t stride, int64_t e_begin, int64_t e_end, void* y, void* y_i,
                                        void* stream) {
  if (!dtype_ok(dtype)) return fail(HATTN_ERR_ARG, "compress_with_index: bad dtype %d", dtype);
  if (bt < 0 || L < 0) return fail(HATTN_ERR_ARG, "compress_with_index: negative size");
  if (w < 1 || w > 4096 || stride < 1)
    return fail(HATTN_ERR_ARG, "compress_with_index: need 1 <= w <= 4096 and stride >= 1");
  const int vec = 16 / elem_bytes(dtype);
  if (C <= 0 || C % vec || C_i <= 0 || C_i % vec)
    return fail(HATTN_ERR_ARG, "compress_with_index: C=%d and C_i=%d must be positive multiples of %d", C, C_i, vec);
  if (L < w) return fail(HATTN_ERR_ARG, "compress_with_index: L=%lld shorter than the window %d", (long long)L, w);
  const int64_t N = (L - w) / stride + 1;
  if (e_begin < 0 || e_end < e_begin || e_end > N)
    return fail(HATTN_ERR_ARG, "compress_with_index: entry range [%lld, %lld) outside [0, %lld]", (long long)e_begin,
                (long long)e_end, (long long)N);
  if (bt == 0 || e_end == e_begin) return ok();
  if (!x || !y || !x_i || !y_i) return fail(HATTN_ERR_ARG, "compress_with_index: NULL x, x_i, y or y_i");
  HATTN_REQUIRE_ALIGNED("compress_with_index", x, y, x_i, y_i);
  return hip_status(hattn::launch_compress(dtype, x, bt, L, C, logits, pos_bias, w, stride, N, e_begin, e_end, y,
                                           (hipStream_t)stream, x_i, y_i, C_i),
                    "compress_with_index");
}

hattn_status_t hattn_compress_channel_logits(int dtype, const void* x, int64_t bt, int64_t L, int32_t C,
                                            const float* logits, const float* pos_bias, int32_t w, int32_t stride,
                                            int64_t e_begin, int64_t e_end, void* y, void* stream) {
  if (!dtype_ok(dtype)) return fail(HATTN_ERR_ARG, "compress_channel_logits: bad dtype %d", dtype);
  if (bt < 0 || L < 0) return fail(HATTN_ERR_ARG, "compress_channel_logits: negative size");
  if (w < 1 || w > 4096 || stride < 1)
    return fail(HATTN_ERR_ARG, "compress_channel_logits: need 1 <= w <= 4096 and stride >= 1");
  const int vec = 16 / elem_bytes(dtype);
  if (C <= 0 || C % vec)
    return fail(HATTN_ERR_ARG, "compress_channel_logits: C=%d must be a positive multiple of %d", C, vec);
  if (L < w) return fail(HATTN_ERR_ARG, "compress_channel_logits: L=%lld shorter than the window %d", (long long)L, w);
  const int64_t N = (L - w) / stride + 1;
  if (e_begin < 0 || e_end < e_begin || e_end > N)
    return fail(HATTN_ERR_ARG, "compress_channel_logits: entry range outside [0, %lld]", (long long)N);
  if (bt == 0 || e_end == e_begin) return ok();
  if (!x || !y || !logits) return fail(HATTN_ERR_ARG, "compress_channel_logits: NULL x, logits or y");
  HATTN_REQUIRE_ALIGNED("compress_channel_logits", x, y, logits);
  return hip_status(hattn::launch_compress_channel(dtype, x, bt, L, C, logits, pos_bias, w, stride, N, e_begin,
                                                   e_end, y, (hipStream_t)stream),
                    "compress_channel_logits");
}

hattn_status_t hattn_visible_count(const int32_t* pos, int64_t count, int32_t w, int32_t stride, int64_t n_entries,
                                   int32_t* n_vis, void* stream) {
  if (count < 0 || w < 1 || stride < 1 || n_entries < 0 || n_entries > INT32_MAX)
    return fail(HATTN_ERR_ARG, "visible_count: bad sizes");
  if (count == 0) return ok();
  if (!pos || !n_vis) return fail(HATTN_ERR_ARG, "visible_count: NULL pointer");
  return hip_status(hattn::launch_visible_count(pos, count, w, stride, n_entries, n_vis, (hipStream_t)stream),
                    "visible_count");
}

static hattn_status_t check_index_args(const char* fn, int dtype, const void* q_i, const void* k_i, const float* w_i,
                                       const int32_t* n_vis, int64_t bt, int64_t nq, int32_t h_i, int32_t d_i,
                                       int64_t n, int32_t k, const int32_t* idx) {
  if (!dtype_ok(dtype)) return fail(HATTN_ERR_ARG, "%s: bad dtype %d", fn, dtype);
  if (bt < 0 || nq < 0 || n < 0 || n > INT32_MAX) return fail(HATTN_ERR_ARG, "%s: bad sizes", fn);
  if (k < 1 || k > 8192) return fail(HATTN_ERR_ARG, "%s: need 1 <= k <= 8192 (k=%d)", fn, k);
  if (h_i < 1 || h_i > 64) return fail(HATTN_ERR_ARG, "%s: need 1 <= h_i <= 64", fn);
  if (d_i < 1 || d_i > 256) return fail(HATTN_ERR_ARG, "%s: need 1 <= d_i <= 256", fn);
  if (h_i * d_i > 8192) return fail(HATTN_ERR_UNSUPPORTED, "%s: h_i*d_i > 8192", fn);
  if (bt * nq > 0 && (!q_i || !w_i || !n_vis || !idx || (n > 0 && !k_i)))
    return fail(HATTN_ERR_ARG, "%s: NULL required pointer", fn);
  HATTN_REQUIRE_ALIGNED(fn, q_i, k_i, w_i);
  return HATTN_OK;
}

hattn_status_t hattn_index_topk(int dtype, const void* q_i, const void* k_i, const float* w_i, const int32_t* n_vis,
                                int64_t bt, int64_t nq, int32_t h_i, int32_t d_i, int64_t n, int32_t k, int32_t* idx,
                                float* score, void* ws, size_t* ws_bytes, void* stream) {
  hattn_status_t st = check_index_args("index_topk", dtype, q_i, k_i, w_i, n_vis, bt, nq, h_i, d_i, n, k, idx);
  if (st != HATTN_OK) return st;
  hattn::IndexArgs a{dtype, q_i, k_i, w_i, n_vis, bt, nq, h_i, d_i, n};
  const size_t need = bt * nq > 0 ? hattn::flat_topk_ws_bytes(a, k) : 0;
  HATTN_REQUIRE_ALIGNED("index_topk", ws);
  if (ws_query(ws, ws_bytes, need, &st)) return st;
  if (bt * nq == 0) return ok();
  return hip_status(hattn::launch_flat_topk(a, k, idx, score, ws, (hipStream_t)stream), "index_topk");
}

hattn_status_t hattn_hisa_pool(int dtype, const void* k_i, int64_t bt, int64_t n, int32_t d_i, int32_t B,
                               int64_t j_begin, int64_t j_end, float* reps, void* stream) {
  if (!dtype_ok(dtype)) return fail(HATTN_ERR_ARG, "hisa_pool: bad dtype %d", dtype);
  if (bt < 0 || n < 0 || B < 1 || d_i < 1 || d_i > 1024) return fail(HATTN_ERR_ARG, "hisa_pool: bad sizes");
  const int vec = 16 / elem_bytes(dtype);
  if (d_i % vec) return fail(HATTN_ERR_ARG, "hisa_pool: d_i=%d must be a multiple of %d", d_i, vec);
  const int64_t nb = (n + B - 1) / B;
  if (j_begin < 0 || j_end < j_begin || j_end > nb) return fail(HATTN_ERR_ARG, "hisa_pool: block range outside [0, %lld]", (long long)nb);
  if (bt == 0 || j_end == j_begin) return ok();
  if (!k_i || !reps) return fail(HATTN_ERR_ARG, "hisa_pool: NULL pointer");
  HATTN_REQUIRE_ALIGNED("hisa_pool", k_i, reps);
  return hip_status(hattn::launch_pool(dtype, k_i, bt, n, d_i, B, j_begin, j_end, reps, (hipStream_t)stream),
                    "hisa_pool");
}

static hattn_status_t hisa_check(int dtype, const void* q_i, const void* k_i, const float* w_i,
                                 const int32_t* n_vis, int64_t bt, int64_t nq, int32_t h_i, int32_t d_i, int64_t n,
                                 const float* reps, int32_t B, int32_t m, int32_t k, const int32_t* idx, void* ws) {
  hattn_status_t st = check_index_args("hisa_topk", dtype, q_i, k_i, w_i, n_vis, bt, nq, h_i, d_i, n, k, idx);
  if (st != HATTN_OK) return st;
  if (B < 1 || B > 1024 || m < 1 || int64_t(m) * B > 16384)
    return fail(HATTN_ERR_ARG, "hisa_topk: need 1 <= B <= 1024, m >= 1, m*B <= 16384");
  if ((n + B - 1) / B > 16384) return fail(HATTN_ERR_UNSUPPORTED, "hisa_topk: more than 16384 blocks");
  if (bt * nq > 0 && n > 0 && !reps) return fail(HATTN_ERR_ARG, "hisa_topk: NULL reps");
  HATTN_REQUIRE_ALIGNED("hisa_topk", reps, ws);
  return HATTN_OK;
}

hattn_status_t hattn_hisa_topk(int dtype, const void* q_i, const void* k_i, const float* w_i, const int32_t* n_vis,
                               int64_t bt, int64_t nq, int32_t h_i, int32_t d_i, int64_t n, const float* reps,
                               int32_t B, int32_t m, int32_t k, int32_t* idx, int32_t* blk, void* ws,
                               size_t* ws_bytes, void* stream) {
  hattn_status_t st = hisa_check(dtype, q_i, k_i, w_i, n_vis, bt, nq, h_i, d_i, n, reps, B, m, k, idx, ws);
  if (st != HATTN_OK) return st;
  hattn::IndexArgs a{dtype, q_i, k_i, w_i, n_vis, bt, nq, h_i, d_i, n};
  const size_t need = bt * nq > 0 ? hattn::hisa_topk_ws_bytes(a, B, m, k) : 0;
  if (ws_query(ws, ws_bytes, need, &st)) return st;
  if (bt * nq == 0) return ok();
  return hip_status(hattn::launch_hisa_topk(a, reps, B, m, k, idx, blk, ws, (hipStream_t)stream), "hisa_topk");
}

hattn_status_t hattn_block_sparse_topk(int dtype, const void* q_i, const void* k_i, const float* w_i,
                                      const int32_t* n_vis, int64_t bt, int64_t nq, int32_t h_i, int32_t d_i,
                                      int64_t n, const float* reps, int32_t B, int32_t m, int32_t* idx, int32_t* blk,
                                      void* ws, size_t* ws_bytes, void* stream) {
  if (m < 1 || B < 1 || int64_t(m) * B > 16384)
    return fail(HATTN_ERR_ARG, "block_sparse_topk: need B >= 1, m >= 1, m*B <= 16384");
  // the selection length m*B plays the part of k in the shared checks
  hattn_status_t st = hisa_check(dtype, q_i, k_i, w_i, n_vis, bt, nq, h_i, d_i, n, reps, B, m, std::min(m * B, 8192),
                                 idx, ws);
  if (st != HATTN_OK) return st;
  hattn::IndexArgs a{dtype, q_i, k_i, w_i, n_vis, bt, nq, h_i, d_i, n};
  const size_t need = bt * nq > 0 ? hattn::block_sparse_ws_bytes(a, B, m) : 0;
  if (ws_query(ws, ws_bytes, need, &st)) return st;
  if (bt * nq == 0) return ok();
  return hip_status(hattn::launch_block_sparse(a, reps, B, m, idx, blk, ws, (hipStream_t)stream), "block_sparse_topk");
}

static hattn_status_t attn_check(const char* fn, const hattn::AttnArgs& a, void* ws) {
  if (!dtype_ok(a.dtype)) return fail(HATTN_ERR_ARG, "%s: bad dtype %d", fn, a.dtype);
  if (a.bt < 0 || a.nq < 0 || a.n < 0 || a.L < 1 || a.window < 1)
    return fail(HATTN_ERR_ARG, "%s: bad sizes (need L >= 1, window >= 1)", fn);
  if (a.raw_rows < 0 || (a.raw_rows > 0 && (a.raw_rows < a.window || a.raw_rows > a.L)))
    return fail(HATTN_ERR_ARG, "%s: a ring of raw_rows=%d must hold window=%d to L=%lld rows", fn, a.raw_rows,
                a.window, (long long)a.L);
  if (a.h < 1 || a.d < 1 || a.d % 8) return fail(HATTN_ERR_ARG, "%s: bad head shape h=%d d=%d", fn, a.h, a.d);
  if (!(a.scale > 0.f) || a.scale != a.scale) return fail(HATTN_ERR_ARG, "%s: scale must be > 0", fn);
  if (!hattn::attn_supported(a)) return fail(HATTN_ERR_UNSUPPORTED, "%s: h=%d d=%d has no kernel", fn, a.h, a.d);
  const int64_t rows = a.bt * a.nq;
  if (rows > 0 && (!a.q || !a.raw_kv || !a.q_pos || !a.out || (a.n > 0 && !a.ckv)))
    return fail(HATTN_ERR_ARG, "%s: NULL required pointer", fn);
  HATTN_REQUIRE_ALIGNED(fn, a.q, a.ckv, a.raw_kv, a.out, ws);
  return HATTN_OK;
}

static hattn_status_t attn_common(const char* fn, hattn::AttnArgs& a, void* ws, size_t* ws_bytes, void* stream) {
  hattn_status_t st = attn_check(fn, a, ws);
  if (st != HATTN_OK) return st;
  const int64_t rows = a.bt * a.nq;
  const size_t need = rows > 0 ? hattn::attn_ws_bytes(a) : 0;
  if (ws_query(ws, ws_bytes, need, &st)) return st;
  if (rows == 0) return ok();
  return hip_status(hattn::launch_attn(a, ws, (hipStream_t)stream), fn);
}

// A ring length that does not fit in int32 is passed on as -1 so that
// attn_check rejects it.
static int32_t ring_arg(int64_t raw_rows) { return raw_rows > INT32_MAX ? -1 : int32_t(raw_rows); }

hattn_status_t hattn_sparse_attn(int dtype, const void* q, const void* ckv, int64_t n, const int32_t* idx, int32_t k,
                                 const void* raw_kv, int64_t L, int64_t raw_rows, const int32_t* q_pos,
                                 int32_t window, float scale, int64_t bt, int64_t nq, int32_t h, int32_t d, float* out,
                                 float* lse, void* ws, size_t* ws_bytes, void* stream) {
  if (k < 0) return fail(HATTN_ERR_ARG, "sparse_attn: k < 0");
  if (bt * nq > 0 && k > 0 && !idx) return fail(HATTN_ERR_ARG, "sparse_attn: NULL idx");
  // With k == 0 no index is ever used; the kernels still read a clamped
  // slot, so hand them a valid device int32 array (q_pos has >= 1 entry).
  hattn::AttnArgs a{dtype, q, ckv, n, k > 0 ? idx : q_pos, k, nullptr, raw_kv, L, q_pos, window, scale,
                    bt, nq, h, d, out, lse, ring_arg(raw_rows)};
  return attn_common("sparse_attn", a, ws, ws_bytes, stream);
}

hattn_status_t hattn_sparse_attn_noalloc(int dtype, const void* q, const void* ckv, int64_t n, const int32_t* idx,
                                         int32_t k, const void* raw_kv, int64_t L, int64_t raw_rows,
                                         const int32_t* q_pos, int32_t window, float scale, int64_t bt, int64_t nq,
                                         int32_t h, int32_t d, float* out, float* lse, void* stream) {
  if (k < 0) return fail(HATTN_ERR_ARG, "sparse_attn_noalloc: k < 0");
  if (bt * nq > 0 && k > 0 && !idx) return fail(HATTN_ERR_ARG, "sparse_attn_noalloc: NULL idx");
  hattn::AttnArgs a{dtype, q, ckv, n, k > 0 ? idx : q_pos, k, nullptr, raw_kv, L, q_pos, window, scale,
                    bt, nq, h, d, out, lse, ring_arg(raw_rows)};
  hattn_status_t st = attn_check("sparse_attn_noalloc", a, nullptr);
  if (st != HATTN_OK) return st;
  const int64_t rows = bt * nq;
  if (rows == 0) return ok();
  const size_t need = hattn::attn_ws_bytes(a);
  if (need > hattn::kStaticScratchBytes)
    return fail(HATTN_ERR_WORKSPACE, "sparse_attn_noalloc: needs %zu bytes of scratch, the static limit is %zu",
                need, hattn::kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = hattn::static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "sparse_attn_noalloc (scratch address)");
  }
  return hip_status(hattn::launch_attn(a, ws, (hipStream_t)stream), "sparse_attn_noalloc");
}

hattn_status_t hattn_dense_compressed_attn(int dtype, const void* q, const void* ckv, int64_t n, const int32_t* n_vis,
                                           const void* raw_kv, int64_t L, int64_t raw_rows, const int32_t* q_pos,
                                           int32_t window, float scale, int64_t bt, int64_t nq, int32_t h, int32_t d,
                                           float* out, float* lse, void* ws, size_t* ws_bytes, void* stream) {
  if (bt * nq > 0 && !n_vis) return fail(HATTN_ERR_ARG, "dense_compressed_attn: NULL n_vis");
  hattn::AttnArgs a{dtype, q, ckv, n, nullptr, 0, n_vis, raw_kv, L, q_pos, window, scale, bt, nq, h, d, out, lse,
                    ring_arg(raw_rows)};
  return attn_common("dense_compressed_attn", a, ws, ws_bytes, stream);
}

static hattn_status_t append_check(int dtype, const void* raw_kv, int64_t bt, int64_t L, int32_t C, int32_t w,
                                   int32_t stride, const int32_t* q_pos, const void* ckv, const int32_t* n_vis,
                                   const void* k_i, int32_t d_i, int32_t B, const float* reps, int64_t* N,
                                   int64_t raw_rows = 0) {
  if (!dtype_ok(dtype)) return fail(HATTN_ERR_ARG, "decode_append: bad dtype %d", dtype);
  if (bt < 0 || L < 0) return fail(HATTN_ERR_ARG, "decode_append: negative size");
  if (w < 1 || w > 4096 || stride < 1) return fail(HATTN_ERR_ARG, "decode_append: need 1 <= w <= 4096, stride >= 1");
  if (L < w) return fail(HATTN_ERR_ARG, "decode_append: L=%lld shorter than the window %d", (long long)L, w);
  if (raw_rows < 0 || raw_rows > INT32_MAX || (raw_rows > 0 && (raw_rows < w || raw_rows > L)))
    return fail(HATTN_ERR_ARG, "decode_append: a ring of raw_rows=%lld must hold w=%d to L=%lld rows",
                (long long)raw_rows, w, (long long)L);
  const int vec = 16 / elem_bytes(dtype);
  if (C <= 0 || C % vec || C / vec > 256)
    return fail(HATTN_ERR_ARG, "decode_append: C=%d must be a positive multiple of %d, at most %d", C, vec, 256 * vec);
  if ((k_i == nullptr) != (reps == nullptr)) return fail(HATTN_ERR_ARG, "decode_append: give both k_i and reps, or neither");
  if (reps && (B < 1 || d_i <= 0 || d_i % vec || d_i / vec > 256))
    return fail(HATTN_ERR_ARG, "decode_append: bad B=%d or d_i=%d", B, d_i);
  *N = (L - w) / stride + 1;
  if (*N > INT32_MAX) return fail(HATTN_ERR_ARG, "decode_append: too many entries");
  if (bt == 0) return HATTN_OK;
  if (!raw_kv || !q_pos || !ckv || !n_vis) return fail(HATTN_ERR_ARG, "decode_append: NULL pointer");
  HATTN_REQUIRE_ALIGNED("decode_append", raw_kv, ckv, k_i);
  return HATTN_OK;
}

hattn_status_t hattn_decode_append(int dtype, const void* raw_kv, int64_t bt, int64_t L, int64_t raw_rows, int32_t C,
                                   const float* logits, const float* pos_bias, int32_t w, int32_t stride,
                                   const int32_t* q_pos, void* ckv, int32_t* n_vis, const void* k_i, int32_t d_i,
                                   int32_t B, float* reps, void* stream) {
  int64_t N = 0;
  const hattn_status_t st =
      append_check(dtype, raw_kv, bt, L, C, w, stride, q_pos, ckv, n_vis, k_i, d_i, B, reps, &N, raw_rows);
  if (st != HATTN_OK) return st;
  if (bt == 0) return ok();
  return hip_status(hattn::launch_append(dtype, raw_kv, bt, L, C, logits, pos_bias, w, stride, q_pos, ckv, N, n_vis,
                                         k_i, d_i, B, reps, (hipStream_t)stream, int(raw_rows)),
                    "decode_append");
}

hattn_status_t hattn_timer_enable(int on) {
  if (on) {
    g_totals.clear();
    for (auto& p : g_pending) {
      g_free.push_back(p.e0);
      g_free.push_back(p.e1);
    }
    g_pending.clear();
  }
  g_timer_on = on != 0;
  return ok();
}

hattn_status_t hattn_timer_collect(void) {
  hipError_t err = hipSuccess;
  for (auto& p : g_pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(p.e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.e0, p.e1);
    if (e == hipSuccess) {
      auto& t = g_totals[p.name];
      t.first += ms;
      t.second += 1;
    } else {
      err = e;
    }
    g_free.push_back(p.e0);
    g_free.push_back(p.e1);
  }
  g_pending.clear();
  return hip_status(err, "timer_collect");
}

hattn_status_t hattn_timer_query(const char* name, double* total_ms, int64_t* count) {
  if (!name || !total_ms || !count) return fail(HATTN_ERR_ARG, "timer_query: NULL pointer");
  auto it = g_totals.find(name);
  if (it == g_totals.end()) return fail(HATTN_ERR_ARG, "timer_query: no kernel named %s was recorded", name);
  *total_ms = it->second.first;
  *count = it->second.second;
  return ok();
}

hattn_status_t hattn_timer_names(char* buf, int64_t len) {
  if (!buf || len < 1) return fail(HATTN_ERR_ARG, "timer_names: bad buffer");
  std::string s;
  for (auto& kv : g_totals) {
    if (!s.empty()) s += '\n';
    s += kv.first;
  }
  const size_t n = std::min<size_t>(s.size(), size_t(len - 1));
  std::memcpy(buf, s.data(), n);
  buf[n] = 0;
  return ok();
}


// ---- decode plan -----------------------------------------------------------
}  // extern "C"

struct hattn_decode_plan {
  ~hattn_decode_plan() {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
  }
  int device = -1;
  // the step captured once by hattn_decode_plan_run_graph
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool front = false;  // stage 1 and cache maintenance in one launch
  int dtype = 0;
  int64_t bt = 0, L = 0;
  int C = 0;
  int raw_rows = 0;  // 0: full raw arrays; R > 0: rings of the newest R rows
  const int32_t* q_pos = nullptr;
  // CSA branch
  const void* csa_raw_kv = nullptr;
  const float *csa_logits = nullptr, *csa_pos_bias = nullptr;
  int csa_w = 0, csa_stride = 0;
  int64_t csa_N = 0;
  void* csa_ckv = nullptr;
  const void* k_i = nullptr;
  float* reps = nullptr;
  int d_i = 0, B = 0, m = 0, k = 0;
  int32_t* nv_csa = nullptr;
  int32_t* idx = nullptr;
  hattn::IndexArgs ia{};
  void* hisa_ws = nullptr;
  hattn::AttnArgs sa{};
  void* sa_ws = nullptr;
  // HCA branch
  const void* hca_raw_kv = nullptr;
  const float *hca_logits = nullptr, *hca_pos_bias = nullptr;
  int hca_w = 0, hca_stride = 0;
  int64_t hca_N = 0;
  void* hca_ckv = nullptr;
  int32_t* nv_hca = nullptr;
  hattn::AttnArgs da{};
  void* da_ws = nullptr;
};

namespace {

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Validates the descriptor and lays the workspace out (offsets from ws);
// fills `p` when it is given.
hattn_status_t decode_layout(const hattn_decode_desc* d, size_t* total, hattn_decode_plan* p) {
  if (!d) return fail(HATTN_ERR_ARG, "decode_plan: NULL descriptor");
  if (d->bt < 1) return fail(HATTN_ERR_ARG, "decode_plan: need bt >= 1");
  const int C = 2 * d->d;
  int64_t Nc = 0, Nh = 0;
  hattn_status_t st = append_check(d->dtype, d->csa_raw_kv, d->bt, d->L, C, d->csa_w, d->csa_stride, d->q_pos,
                                   d->csa_ckv, d->q_pos, d->k_i, d->d_i, d->B, d->reps, &Nc, d->raw_rows);
  if (st != HATTN_OK) return st;
  if (!d->k_i) return fail(HATTN_ERR_ARG, "decode_plan: the CSA branch needs k_i and reps");
  st = append_check(d->dtype, d->hca_raw_kv, d->bt, d->L, C, d->hca_w, d->hca_stride, d->q_pos, d->hca_ckv,
                    d->q_pos, nullptr, 0, 0, nullptr, &Nh, d->raw_rows);
  if (st != HATTN_OK) return st;
  if (d->raw_rows > 0 && d->raw_rows < d->window)
    return fail(HATTN_ERR_ARG, "decode_plan: a ring of %lld raw rows cannot hold the %d-row window",
                (long long)d->raw_rows, d->window);
  // Workspace: counts, selected indices, then each call's own workspace.
  const size_t o_nvc = 0;
  const size_t o_nvh = o_nvc + al256(size_t(d->bt) * 4);
  const size_t o_idx = o_nvh + al256(size_t(d->bt) * 4);
  const size_t o_hisa = o_idx + al256(size_t(d->bt) * std::max(d->k, 1) * 4);
  char* base = reinterpret_cast<char*>(d->ws);
  auto at = [&](size_t off) -> void* { return base ? base + off : reinterpret_cast<void*>(uintptr_t(256)); };
  // the selected indices: the caller's array when given, else the workspace's
  int32_t* idx = d->csa_idx ? d->csa_idx : reinterpret_cast<int32_t*>(at(o_idx));
  hattn::IndexArgs ia{d->dtype, d->q_i, d->k_i, d->w_i, (const int32_t*)at(o_nvc), d->bt, 1, d->h_i, d->d_i, Nc};
  st = hisa_check(d->dtype, d->q_i, d->k_i, d->w_i, ia.n_vis, d->bt, 1, d->h_i, d->d_i, Nc, d->reps, d->B, d->m,
                  d->k, idx, d->ws);
  if (st != HATTN_OK) return st;
  const size_t o_sa = o_hisa + al256(hattn::hisa_topk_ws_bytes(ia, d->B, d->m, d->k));
  hattn::AttnArgs sa{d->dtype, d->csa_q, d->csa_ckv, Nc, idx, d->k, nullptr, d->csa_raw_kv,
                     d->L, d->q_pos, d->window, d->scale, d->bt, 1, d->h, d->d, d->csa_out, d->csa_lse,
                     int(d->raw_rows)};
  st = attn_check("decode_plan (CSA attention)", sa, d->ws);
  if (st != HATTN_OK) return st;
  const size_t o_da = o_sa + al256(hattn::attn_ws_bytes(sa));
  hattn::AttnArgs da{d->dtype, d->hca_q, d->hca_ckv, Nh, nullptr, 0, (const int32_t*)at(o_nvh), d->hca_raw_kv,
                     d->L, d->q_pos, d->window, d->scale, d->bt, 1, d->h, d->d, d->hca_out, d->hca_lse,
                     int(d->raw_rows)};
  st = attn_check("decode_plan (HCA attention)", da, d->ws);
  if (st != HATTN_OK) return st;
  *total = o_da + al256(hattn::attn_ws_bytes(da));
  if (!p) return HATTN_OK;
  p->dtype = d->dtype;
  p->bt = d->bt;
  p->L = d->L;
  p->C = C;
  p->raw_rows = int(d->raw_rows);
  p->q_pos = d->q_pos;
  p->csa_raw_kv = d->csa_raw_kv;
  p->csa_logits = d->csa_logits;
  p->csa_pos_bias = d->csa_pos_bias;
  p->csa_w = d->csa_w;
  p->csa_stride = d->csa_stride;
  p->csa_N = Nc;
  p->csa_ckv = d->csa_ckv;
  p->k_i = d->k_i;
  p->reps = d->reps;
  p->d_i = d->d_i;
  p->B = d->B;
  p->m = d->m;
  p->k = d->k;
  p->nv_csa = reinterpret_cast<int32_t*>(at(o_nvc));
  p->idx = idx;
  p->ia = ia;
  p->hisa_ws = at(o_hisa);
  p->sa = sa;
  p->sa_ws = at(o_sa);
  p->hca_raw_kv = d->hca_raw_kv;
  p->hca_logits = d->hca_logits;
  p->hca_pos_bias = d->hca_pos_bias;
  p->hca_w = d->hca_w;
  p->hca_stride = d->hca_stride;
  p->hca_N = Nh;
  p->hca_ckv = d->hca_ckv;
  p->nv_hca = reinterpret_cast<int32_t*>(at(o_nvh));
  p->da = da;
  p->da_ws = at(o_da);
  p->front = hattn::decode_front_ok(ia, d->B, d->m, std::max(d->csa_w, d->hca_w));
  return HATTN_OK;
}

}  // namespace

extern "C" {

int64_t hattn_decode_desc_size(void) { return int64_t(sizeof(hattn_decode_desc)); }

hattn_status_t hattn_decode_plan_ws_bytes(const hattn_decode_desc* desc, size_t* ws_bytes) {
  if (!ws_bytes) return fail(HATTN_ERR_ARG, "decode_plan_ws_bytes: NULL ws_bytes");
  size_t total = 0;
  hattn_status_t st = decode_layout(desc, &total, nullptr);
  if (st != HATTN_OK) return st;
  *ws_bytes = total;
  return ok();
}

hattn_status_t hattn_decode_plan_create(const hattn_decode_desc* desc, hattn_decode_plan_t* plan) {
  if (!plan) return fail(HATTN_ERR_ARG, "decode_plan_create: NULL plan");
  *plan = nullptr;
  size_t total = 0;
  hattn_status_t st = decode_layout(desc, &total, nullptr);
  if (st != HATTN_OK) return st;
  if (!desc->ws || desc->ws_bytes < total)
    return fail(HATTN_ERR_WORKSPACE, "decode_plan_create: workspace of %zu bytes is smaller than the %zu required",
                desc->ws ? desc->ws_bytes : size_t(0), total);
  hattn_decode_plan* p = new hattn_decode_plan();
  decode_layout(desc, &total, p);
  const hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_status(e, "decode_plan_create");
  }
  *plan = p;
  return ok();
}

}  // extern "C"

namespace {

// The step's launches, in order, on st.
hipError_t plan_enqueue(hattn_decode_plan* p, hipStream_t st) {
  hipError_t e;
  // Both branches on one stream: the HCA work rides in the CSA launches
  // (one cache-maintenance launch, one attention launch, one merge launch).
  if (p->front) {
    // cache maintenance of both layers + HISA stage 1 in one launch
    e = hattn::launch_decode_front(p->ia, p->reps, p->B, p->m, p->hisa_ws, p->q_pos, p->csa_raw_kv, p->csa_logits,
                                   p->csa_pos_bias, p->csa_w, p->csa_stride, p->csa_ckv, p->nv_csa, p->hca_raw_kv,
                                   p->hca_logits, p->hca_pos_bias, p->hca_w, p->hca_stride, p->hca_ckv, p->hca_N,
                                   p->nv_hca, p->L, p->C, st, p->raw_rows);
    if (e == hipSuccess)
      e = hattn::launch_hisa_topk(p->ia, p->reps, p->B, p->m, p->k, p->idx, nullptr, p->hisa_ws, st, true);
  } else {
    e = hattn::launch_append_pair(p->dtype, p->bt, p->q_pos, p->csa_raw_kv, p->csa_logits, p->csa_pos_bias,
                                  p->csa_w, p->csa_stride, p->csa_ckv, p->csa_N, p->nv_csa, p->k_i, p->d_i, p->B,
                                  p->reps, p->hca_raw_kv, p->hca_logits, p->hca_pos_bias, p->hca_w, p->hca_stride,
                                  p->hca_ckv, p->hca_N, p->nv_hca, p->L, p->C, st, p->raw_rows);
    if (e == hipSuccess)
      e = hattn::launch_hisa_topk(p->ia, p->reps, p->B, p->m, p->k, p->idx, nullptr, p->hisa_ws, st);
  }
  if (e == hipSuccess) e = hattn::launch_attn_pair(p->sa, p->sa_ws, p->da, p->da_ws, st);
  return e;
}

hattn_status_t plan_device_check(hattn_decode_plan* p, const char* fn) {
  if (!p) return fail(HATTN_ERR_ARG, "%s: NULL plan", fn);
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev != p->device) return fail(HATTN_ERR_ARG, "%s: plan made on device %d, current %d", fn, p->device, dev);
  return HATTN_OK;
}

// Captures the step into p->graph / p->exec on a private stream.
hipError_t plan_capture(hattn_decode_plan* p) {
  hipStream_t cap = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
  if (e != hipSuccess) return e;
  e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    const hipError_t el = plan_enqueue(p, cap);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(cap, &g);
    if (el != hipSuccess) e = el;
    if (e == hipSuccess) {
      hipGraphExec_t x = nullptr;
      e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
      if (e == hipSuccess) {
        p->graph = g;
        p->exec = x;
      }
    }
    if (e != hipSuccess && g) (void)hipGraphDestroy(g);
  }
  (void)hipStreamDestroy(cap);
  return e;
}

}  // namespace

extern "C" {

hattn_status_t hattn_decode_plan_run(hattn_decode_plan_t p, void* stream) {
  hattn_status_t s = plan_device_check(p, "decode_plan_run");
  if (s != HATTN_OK) return s;
  return hip_status(plan_enqueue(p, (hipStream_t)stream), "decode_plan_run");
}

hattn_status_t hattn_decode_plan_run_graph(hattn_decode_plan_t p, void* stream) {
  hattn_status_t s = plan_device_check(p, "decode_plan_run_graph");
  if (s != HATTN_OK) return s;
  if (!p->exec) {
    if (g_timer_on)
      return fail(HATTN_ERR_ARG, "decode_plan_run_graph: the first call captures the step; turn the timer off");
    const hipError_t e = plan_capture(p);
    if (e != hipSuccess) return hip_status(e, "decode_plan_run_graph (capture)");
  }
  return hip_status(hipGraphLaunch(p->exec, (hipStream_t)stream), "decode_plan_run_graph");
}

hattn_status_t hattn_decode_plan_destroy(hattn_decode_plan_t p) {
  delete p;
  return ok();
}

}  // extern "C"
