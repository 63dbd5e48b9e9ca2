// Host-side launchers of the libvjp kernels (internal; the public C ABI is
// include/libvjp.h).  Each returns the hipError_t of its launch(es); shapes
// and pointers have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vjp {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

inline int dtype_size(int dt) { return dt == kF32 ? 4 : 2; }

// Stage 2: out[j] = (accumulate ? out[j] : 0) + fixed-order sum_t P[t * d + j].
hipError_t launch_reduce_partials(const float* P, int64_t T, int64_t d, float* out,
                                  int accumulate, hipStream_t s);
// As above with columns j >= split written to out2[j - split].
hipError_t launch_reduce_partials_split(const float* P, int64_t T, int64_t d, float* out,
                                        float* out2, int64_t split, int accumulate,
                                        hipStream_t s);

// Streaming device copy of `bytes` bytes (the measurement reference), with
// its launch shape (vectors in flight per lane: 1, 2, 4 or 8; grid bound).
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
hipError_t launch_copy_shaped(const void* src, void* dst, int64_t bytes, int vectors_per_lane,
                              int64_t max_groups, hipStream_t s);

// Weighted sum.
hipError_t launch_weighted_sum_fwd(const void* x, int64_t ld_x, const void* w, void* y,
                                   int64_t n, int64_t d, int act, int wdt, bool vec,
                                   hipStream_t s);
hipError_t launch_weighted_sum_bwd_stage1(const void* dy, const void* x, int64_t ld_x,
                                          const void* w, void* dx, int64_t ld_dx, float* P,
                                          int64_t n, int64_t d, int block_rows, int64_t tiles,
                                          int act, int wdt, bool vec, hipStream_t s);

// Scaled SiLU.
hipError_t launch_scaled_silu_fwd(const void* x, const float* w, void* y, int64_t n, int act,
                                  bool vec, hipStream_t s);
hipError_t launch_scaled_silu_bwd_stage1(const void* dy, const void* x, const float* w,
                                         void* dx, float* P, int64_t n, int64_t elems_per_tile,
                                         int act, bool vec, hipStream_t s);

// Softmax.  row_lse may be null (forward: not written; backward: src is the
// saved y).  With row_lse given, the backward's src is x.  A null y in the
// forward writes the statistics only.
hipError_t launch_softmax_fwd(const void* x, int64_t ld_x, void* y, int64_t ld_y,
                              float* row_lse, int64_t rows, int64_t cols, int act, bool vec,
                              hipStream_t s);
hipError_t launch_softmax_bwd(const void* dy, int64_t ld_dy, const void* src, int64_t ld_src,
                              const float* row_lse, void* dx, int64_t ld_dx, int64_t rows,
                              int64_t cols, int act, bool vec, hipStream_t s);

// Softmax cross-entropy.
hipError_t launch_softmax_xent(const void* z, int64_t ld, const int32_t* targets, int64_t rows,
                               int64_t classes, int act, float grad_scale, float* row_max,
                               float* row_lse, float* row_loss, void* dz, int64_t ld_dz,
                               bool vec, hipStream_t s);
// Statistics only (row_max may be null): the forward of the split form.
hipError_t launch_softmax_xent_stats(const void* z, int64_t ld, const int32_t* targets,
                                     int64_t rows, int64_t classes, int act, float* row_max,
                                     float* row_lse, float* row_loss, bool vec, hipStream_t s);
// dz = (*dloss / total_rows) * (exp(z - row_lse) - onehot(t)) for `rows` rows.
hipError_t launch_softmax_xent_bwd(const void* z, int64_t ld, const int32_t* targets,
                                   const float* row_lse, const float* dloss, int64_t total_rows,
                                   int64_t rows, int64_t classes, int act, void* dz,
                                   int64_t ld_dz, bool vec, hipStream_t s);
hipError_t launch_xent_finalize(const float* row_loss, const int32_t* targets, int64_t rows,
                                int64_t classes, float* loss, int32_t* n_invalid,
                                hipStream_t s);

// LayerNorm (rms = false) / RMSNorm (rms = true).  Rows wider than
// norm_max_cols(act, vec) are not supported (hipErrorInvalidValue).
int64_t norm_max_cols(int act, bool vec);
hipError_t launch_norm_fwd(bool rms, const void* x, int64_t ld_x, const void* w, const void* b,
                           int wdt, void* y, int64_t ld_y, float* row_mean, float* row_rstd,
                           int64_t rows, int64_t cols, float eps, int act, bool vec,
                           hipStream_t s);
// Stage 1 of the backward: dx and the per-tile partials P[tiles][cols] (dw)
// followed, for LayerNorm, by P[tiles][cols .. 2 cols) (db) in each row.
// row_rstd (and row_mean) null: the statistics are recomputed from x.
hipError_t launch_norm_bwd_stage1(bool rms, const void* dy, int64_t ld_dy, const void* x,
                                  int64_t ld_x, const void* w, int wdt, const float* row_mean,
                                  const float* row_rstd, void* dx, int64_t ld_dx, float* P,
                                  int64_t rows, int64_t cols, int64_t tiles, float eps, int act,
                                  bool vec, hipStream_t s);

// Row gather and its scatter-add backward.  The backward's workspace holds
// gather_workspace_ints(M, V, D) 4-byte values, sorted keys [M] first and the
// sorted positions [M] next (layout in gather.hip).
int gather_sort_passes(int64_t V);
int64_t gather_workspace_ints(int64_t M, int64_t V, int64_t D);
hipError_t launch_gather_rows_fwd(const void* x, int64_t ld_x, const int32_t* idx, int64_t M,
                                  int64_t V, int64_t D, void* y, int64_t ld_y, int act, bool vec,
                                  hipStream_t s);
hipError_t launch_gather_rows_bwd(const void* dy, int64_t ld_dy, const int32_t* idx, int64_t M,
                                  int64_t V, int64_t D, float* dt, int64_t ld_dt, int accumulate,
                                  int32_t* n_invalid, int32_t* ws, int act, bool vec, bool pvec,
                                  hipStream_t s);

}  // namespace vjp
