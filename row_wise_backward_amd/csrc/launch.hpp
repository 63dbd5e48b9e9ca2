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

}  // namespace vjp
