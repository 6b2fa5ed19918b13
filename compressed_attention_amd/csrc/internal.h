// Internal host-side interface between the C ABI (hattn.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hattn {

// Names the kernel launched inside its lifetime.  When the kernel timer is
// on, the scope owns a start/stop event pair that HATTN_LAUNCH hands to
// hipExtLaunchKernelGGL, so the events carry the dispatch's own start and end
// times (no marker packets around the kernel); the destructor queues the pair
// for hattn_timer_collect().  One timed launch per scope.
struct LaunchScope {
  LaunchScope(const char* name, hipStream_t s);
  ~LaunchScope();
  const char* name_;
  hipStream_t stream_;
  hipEvent_t ev0_, ev1_;
  bool used_;
  LaunchScope* outer_;
};

// Events of the innermost live scope if the timer is on and the scope has
// not timed a launch yet (then the scope counts as used); false otherwise.
bool timer_events(hipEvent_t* e0, hipEvent_t* e1);

#define HATTN_LAUNCH(kernel, grid, block, shm, st, ...)                                             \
  do {                                                                                               \
    hipEvent_t hattn_e0_, hattn_e1_;                                                                 \
    if (::hattn::timer_events(&hattn_e0_, &hattn_e1_))                                               \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, st, hattn_e0_, hattn_e1_, 0u, __VA_ARGS__);    \
    else                                                                                             \
      hipLaunchKernelGGL(kernel, grid, block, shm, st, __VA_ARGS__);                                 \
  } while (0)

// ---- compression / geometry / pooling -------------------------------------
// With x2 (indexer keys [bt][L][C2]) the same weights also compress x2 into
// y2 [bt][N][C2].
hipError_t launch_compress(int dtype, const void* x, int64_t bt, int64_t L, int C, const float* z,
                           const float* bias, int w, int s, int64_t N, int64_t e0, int64_t e1, void* y,
                           hipStream_t st, const void* x2 = nullptr, void* y2 = nullptr, int C2 = 0);
// Per-channel logits Z [bt][L][C] fp32.
hipError_t launch_compress_channel(int dtype, const void* x, int64_t bt, int64_t L, int C, const float* Z,
                                   const float* bias, int w, int s, int64_t N, int64_t e0, int64_t e1, void* y,
                                   hipStream_t st);
hipError_t launch_visible_count(const int32_t* pos, int64_t count, int w, int s, int64_t n_entries,
                                int32_t* n_vis, hipStream_t st);
hipError_t launch_pool(int dtype, const void* k_i, int64_t bt, int64_t n, int d_i, int B, int64_t j0,
                       int64_t j1, float* reps, hipStream_t st);
size_t append_lds_bytes(int dtype, int C, int w, int d_i, bool with_reps);
// Two layers of the same sequences in one launch: layer 1 (with block means
// when k_i / reps are given) and layer 2 (entries only).
// raw_rows: 0 when x and z hold all L rows; R > 0 when they are rings of the
// newest R rows (row r at slot r % R; R >= w).
hipError_t launch_append_pair(int dtype, int64_t bt, const int32_t* q_pos, const void* x1, const float* z1,
                              const float* bias1, int w1, int s1, void* y1, int64_t N1, int32_t* n_vis1,
                              const void* k_i, int d_i, int B, float* reps, const void* x2, const float* z2,
                              const float* bias2, int w2, int s2, void* y2, int64_t N2, int32_t* n_vis2, int64_t L,
                              int C, hipStream_t st, int raw_rows = 0);
hipError_t launch_append(int dtype, const void* x, int64_t bt, int64_t L, int C, const float* z, const float* bias,
                         int w, int s, const int32_t* q_pos, void* y, int64_t N, int32_t* n_vis, const void* k_i,
                         int d_i, int B, float* reps, hipStream_t st, int raw_rows = 0);

// ---- indexer ---------------------------------------------------------------
struct IndexArgs {
  int dtype;
  const void* q_i;
  const void* k_i;
  const float* w_i;
  const int32_t* n_vis;
  int64_t bt, nq;
  int h_i, d_i;
  int64_t n;
};

size_t flat_topk_ws_bytes(const IndexArgs& a, int k);
hipError_t launch_flat_topk(const IndexArgs& a, int k, int32_t* idx, float* score, void* ws, hipStream_t st);

size_t hisa_topk_ws_bytes(const IndexArgs& a, int B, int m, int k);
// Block-sparse baseline: HISA's first stage (top-m blocks) and every visible
// entry of the chosen blocks as the selection, idx [rows][m*B].
size_t block_sparse_ws_bytes(const IndexArgs& a, int B, int m);
hipError_t launch_block_sparse(const IndexArgs& a, const float* reps, int B, int m, int32_t* idx, int32_t* blk,
                               void* ws, hipStream_t st);
hipError_t launch_hisa_topk(const IndexArgs& a, const float* reps, int B, int m, int k, int32_t* idx,
                            int32_t* blk, void* ws, hipStream_t st, bool stage1_done = false);
// Decode front: HISA stage 1 for one query per sequence (into ws's S1, as
// launch_hisa_topk lays it out) fused with the cache maintenance of the
// layer behind the indexer (layer 1: its entry, visible count and the block
// mean holding the new entry) and optionally a second layer (layer 2: entry
// and visible count).  Then launch_hisa_topk(..., stage1_done = true).
// max_w: the longest compression window of the layers whose entries the
// launch maintains (the roles reuse the kernel's LDS tile as scratch).
bool decode_front_ok(const IndexArgs& a, int B, int m, int max_w);
hipError_t launch_decode_front(const IndexArgs& a, float* reps, int B, int m, void* ws, const int32_t* q_pos,
                               const void* x1, const float* z1, const float* bias1, int w1, int s1, void* y1,
                               int32_t* n_vis1, const void* x2, const float* z2, const float* bias2, int w2, int s2,
                               void* y2, int64_t N2, int32_t* n_vis2, int64_t L, int C, hipStream_t st,
                               int raw_rows = 0);

// ---- attention -------------------------------------------------------------
struct AttnArgs {
  int dtype;
  const void* q;
  const void* ckv;
  int64_t n;
  const int32_t* idx;    // sparse: [bt][nq][k]
  int k;                 // sparse list length
  const int32_t* n_vis;  // dense: [bt][nq]
  const void* raw_kv;
  int64_t L;
  const int32_t* q_pos;
  int window;
  float scale;
  int64_t bt, nq;
  int h, d;
  float* out;
  float* lse;
  int raw_rows = 0;  // 0: raw_kv holds all L rows; R > 0: a ring of the newest R (row r at slot r % R)
};

size_t attn_ws_bytes(const AttnArgs& a);
// The library's static device scratch (used in place of a workspace by the
// no-allocation entry point): its size, and its address on the current
// device (resolved on the first call per device).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr);
hipError_t launch_attn(const AttnArgs& a, void* ws, hipStream_t st);
// A sparse and a dense set (each with its own attn_ws_bytes workspace) in
// shared launches; the same results as launch_attn on each.
hipError_t launch_attn_pair(const AttnArgs& s, void* ws_s, const AttnArgs& d, void* ws_d, hipStream_t st);
bool attn_supported(const AttnArgs& a);

}  // namespace hattn
