// Row softmax forward (saves y) and backward (needs only y).
//
// Source: "Backprop for kernel writers".  Section 01 "The only idea": the
// backward is a vector-Jacobian product and the cols x cols softmax Jacobian
// is never formed.  The softmax section after 04 "The duality": the VJP
// collapses to one row scalar s = sum_j dy_j y_j accumulated in one pass and
// applied elementwise, dx_j = y_j (dy_j - s), in a second; the backward is a
// function of y alone; the forward's max shift is free (shift invariance).
// "Backward in Triton -- autograd.Function and the backward grid", section
// "Save vs recompute": the row max is a one-scalar-per-row statistic the
// forward recomputes on chip.
//
// Save-statistics variant ("Backprop for kernel writers", the softmax section
// after 04: save y, or recompute it from the saved max and logsumexp; section
// 07 "Fusion": store only L = m + log l per row and rebuild any probability
// as exp(x - L)): the forward can also write row_lse (and may skip y), and
// the backward can take x and row_lse instead of y, recomputing
// y = exp(x - L) on chip in fp32 in both of its passes.
//
// Resident path (rows up to 8 waves * 64 * K * VEC columns): the row is read
// once into VGPRs (layout in rowops.hpp), the statistics are reduced with
// wave butterflies and, for multi-wave rows, LDS in wave order, and the
// output pass works from the registers.  Streaming path (wider rows): 256
// threads per row, an online max / sum pass and an output pass, so x (or
// dy and y) is read twice.
#include "launch.hpp"
#include "rowops.hpp"

namespace vjp {

namespace {

// Forward, resident.  KEEP = true holds exp(x - m) in fp32 VGPRs between
// the sum and the output pass; KEEP = false recomputes it from the stored row
// (more VALU work, far fewer VGPRs, so more rows in flight per CU).  Both
// produce bitwise identical results.
template <typename T, int VEC, int WAVES, int K, bool KEEP>
__global__ __launch_bounds__(row_block_threads<WAVES>()) void softmax_fwd_resident(
    const T* __restrict__ x, int64_t ld_x, T* __restrict__ y, int64_t ld_y,
    float* __restrict__ row_lse, int64_t rows, int64_t cols) {
  __shared__ float buf[2][WAVES];   // one slot per reduction of the row
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t row = WAVES == 1 ? int64_t(blockIdx.x) * rows_per_block<1>() + wave
                                 : int64_t(blockIdx.x);
  const int wv = WAVES == 1 ? 0 : wave;
  if (WAVES == 1 && row >= rows) return;
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  const int64_t lane_col = (int64_t(wv) * kWave + lane) * VEC;

  Vec<T, VEC> raw[K];
  float mx, mn;
  load_row_minmax<T, VEC, WAVES, K>(x + row * ld_x, cols, lane_col, raw, mx, mn);
  const float m = row_reduce_max<WAVES>(mx, buf[0]);
  const bool safe = needs_denorm_exp(mn, m);
  fence_row<T, VEC, K>(raw);

  float keep[KEEP ? K : 1][VEC];
  float l = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k * kStep < cols) {
      float e[VEC];
      exp_vec<T, VEC>(raw[k], m, safe, e);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        l += e[i];
        if constexpr (KEEP) keep[k][i] = e[i];
      }
    }
  }
  l = row_reduce_sum<WAVES>(l, buf[1]);
  const float inv = 1.0f / l;
  if constexpr (!KEEP) fence_row<T, VEC, K>(raw);
  if (row_lse != nullptr && wv == 0 && lane == 0) row_lse[row] = row_lse_of(m, l);
  if (y == nullptr) return;   // statistics only (uniform across the workgroup)

  T* yr = y + row * ld_y;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k * kStep < cols) {
      const int64_t col = k * kStep + lane_col;
      if (col < cols) {
        float o[VEC];
        if constexpr (KEEP) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[i] = keep[k][i];
        } else {
          exp_vec<T, VEC>(raw[k], m, safe, o);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] *= inv;
        store_row_vec<T, VEC>(yr, col, cols, o);
      }
    }
  }
}

// Backward, resident.  FROM_LSE = false: `src` is the saved y.  FROM_LSE =
// true: `src` is x and y = exp(x - row_lse) is rebuilt in fp32 in the s pass
// and again in the output pass, so only the stored rows stay in VGPRs.
template <typename T, int VEC, int WAVES, int K, bool FROM_LSE>
__global__ __launch_bounds__(row_block_threads<WAVES>()) void softmax_bwd_resident(
    const T* __restrict__ dy, int64_t ld_dy, const T* __restrict__ src, int64_t ld_src,
    const float* __restrict__ row_lse, T* __restrict__ dx, int64_t ld_dx, int64_t rows,
    int64_t cols) {
  __shared__ float buf[2][WAVES];   // one slot per reduction of the row
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t row = WAVES == 1 ? int64_t(blockIdx.x) * rows_per_block<1>() + wave
                                 : int64_t(blockIdx.x);
  const int wv = WAVES == 1 ? 0 : wave;
  if (WAVES == 1 && row >= rows) return;
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  const int64_t lane_col = (int64_t(wv) * kWave + lane) * VEC;
  const T* gr = dy + row * ld_dy;
  const T* sr = src + row * ld_src;

  Vec<T, VEC> rg[K], ry[K];
  float L = 0.0f;
  bool safe = false;
  // x padding = -inf (y = 0 there), y padding = 0
  load_row_resident<T, VEC, WAVES, K>(sr, cols, lane_col, FROM_LSE ? neg_inf_of<T>() : zero_of<T>(), ry);
  load_row_resident<T, VEC, WAVES, K>(gr, cols, lane_col, zero_of<T>(), rg);
  if constexpr (FROM_LSE) {
    float mx, mn;
    lane_minmax<T, VEC, WAVES, K>(ry, cols, lane_col, mx, mn);
    L = row_lse[row];
    safe = needs_denorm_exp(mn, L);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k * kStep < cols) {
      float yv[VEC];
      if constexpr (FROM_LSE) {
        exp_vec<T, VEC>(ry[k], L, safe, yv);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) yv[i] = to_f32(ry[k].v[i]);
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) s = fmaf(to_f32(rg[k].v[i]), yv[i], s);
    }
  }
  s = row_reduce_sum<WAVES>(s, buf[0]);
  fence_row<T, VEC, K>(rg);
  fence_row<T, VEC, K>(ry);

  T* dr = dx + row * ld_dx;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k * kStep < cols) {
      const int64_t col = k * kStep + lane_col;
      if (col < cols) {
        float yv[VEC];
        if constexpr (FROM_LSE) {
          exp_vec<T, VEC>(ry[k], L, safe, yv);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) yv[i] = to_f32(ry[k].v[i]);
        }
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = yv[i] * (to_f32(rg[k].v[i]) - s);
        store_row_vec<T, VEC>(dr, col, cols, o);
      }
    }
  }
}

template <typename T, int VEC>
__global__ __launch_bounds__(kStreamThreads) void softmax_fwd_stream(
    const T* __restrict__ x, int64_t ld_x, T* __restrict__ y, int64_t ld_y,
    float* __restrict__ row_lse, int64_t cols) {
  __shared__ float bm[kStreamThreads / kWave], bl[kStreamThreads / kWave];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * ld_x;
  float m = -__builtin_inff(), l = 0.0f;
  for (int64_t col = int64_t(threadIdx.x) * VEC; col < cols; col += int64_t(kStreamThreads) * VEC) {
    Vec<T, VEC> r;
    load_row_vec<T, VEC>(xr, col, cols, neg_inf_of<T>(), r);
#pragma unroll
    for (int i = 0; i < VEC; ++i) online_step(to_f32(r.v[i]), m, l);
  }
  block_merge_ml(m, l, bm, bl);
  const float inv = 1.0f / l;
  if (row_lse != nullptr && threadIdx.x == 0) row_lse[row] = row_lse_of(m, l);
  if (y == nullptr) return;
  T* yr = y + row * ld_y;
  for (int64_t col = int64_t(threadIdx.x) * VEC; col < cols; col += int64_t(kStreamThreads) * VEC) {
    Vec<T, VEC> r;
    load_row_vec<T, VEC>(xr, col, cols, neg_inf_of<T>(), r);
    float o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = exp2_denorm_safe((to_f32(r.v[i]) - m) * kLog2e) * inv;
    store_row_vec<T, VEC>(yr, col, cols, o);
  }
}

template <typename T, int VEC, bool FROM_LSE>
__global__ __launch_bounds__(kStreamThreads) void softmax_bwd_stream(
    const T* __restrict__ dy, int64_t ld_dy, const T* __restrict__ src, int64_t ld_src,
    const float* __restrict__ row_lse, T* __restrict__ dx, int64_t ld_dx, int64_t cols) {
  __shared__ float buf[kStreamThreads / kWave];
  const int64_t row = blockIdx.x;
  const T* gr = dy + row * ld_dy;
  const T* sr = src + row * ld_src;
  T* dr = dx + row * ld_dx;
  const float L = FROM_LSE ? row_lse[row] : 0.0f;
  auto y_of = [&](const Vec<T, VEC>& b, float (&yv)[VEC]) {
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      yv[i] = FROM_LSE ? exp2_denorm_safe((to_f32(b.v[i]) - L) * kLog2e) : to_f32(b.v[i]);
  };
  const T fill = FROM_LSE ? neg_inf_of<T>() : zero_of<T>();
  float s = 0.0f;
  for (int64_t col = int64_t(threadIdx.x) * VEC; col < cols; col += int64_t(kStreamThreads) * VEC) {
    Vec<T, VEC> a, b;
    load_row_vec<T, VEC>(gr, col, cols, zero_of<T>(), a);
    load_row_vec<T, VEC>(sr, col, cols, fill, b);
    float yv[VEC];
    y_of(b, yv);
#pragma unroll
    for (int i = 0; i < VEC; ++i) s = fmaf(to_f32(a.v[i]), yv[i], s);
  }
  s = block_sum_stream<kStreamThreads / kWave>(s, buf);
  for (int64_t col = int64_t(threadIdx.x) * VEC; col < cols; col += int64_t(kStreamThreads) * VEC) {
    Vec<T, VEC> a, b;
    load_row_vec<T, VEC>(gr, col, cols, zero_of<T>(), a);
    load_row_vec<T, VEC>(sr, col, cols, fill, b);
    float yv[VEC];
    y_of(b, yv);
    float o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = yv[i] * (to_f32(a.v[i]) - s);
    store_row_vec<T, VEC>(dr, col, cols, o);
  }
}

// Launch tiers, smallest first: (waves per row, vectors per lane, keep the
// exponentials in VGPRs).  The first tier whose capacity WAVES * 64 * K * VEC
// holds the row is used; wider rows take the streaming path.  Measured on
// MI355X: rows of 4096 16-bit values run best as 4 waves x 2 vectors with
// the exponentials kept (forward) and 8 waves x 1 vector (backward); K >= 4
// recomputes the exponentials so that the row fits in fewer VGPRs.
template <typename T, int VEC, int WAVES, int K, bool KEEP>
bool fwd_try(const T* xp, int64_t ld_x, T* yp, int64_t ld_y, float* lse, int64_t rows,
             int64_t cols, hipStream_t s) {
  if (int64_t(WAVES) * kWave * K * VEC < cols) return false;
  const unsigned grid = unsigned((rows + rows_per_block<WAVES>() - 1) / rows_per_block<WAVES>());
  softmax_fwd_resident<T, VEC, WAVES, K, KEEP>
      <<<grid, row_block_threads<WAVES>(), 0, s>>>(xp, ld_x, yp, ld_y, lse, rows, cols);
  return true;
}

template <typename T, int VEC, int WAVES, int K, bool FROM_LSE>
bool bwd_try(const T* gp, int64_t ld_dy, const T* sp, int64_t ld_src, const float* lse, T* dp,
             int64_t ld_dx, int64_t rows, int64_t cols, hipStream_t s) {
  if (int64_t(WAVES) * kWave * K * VEC < cols) return false;
  const unsigned grid = unsigned((rows + rows_per_block<WAVES>() - 1) / rows_per_block<WAVES>());
  softmax_bwd_resident<T, VEC, WAVES, K, FROM_LSE><<<grid, row_block_threads<WAVES>(), 0, s>>>(
      gp, ld_dy, sp, ld_src, lse, dp, ld_dx, rows, cols);
  return true;
}

template <typename T, int VEC>
hipError_t fwd_vec(const void* x, int64_t ld_x, void* y, int64_t ld_y, float* lse, int64_t rows,
                   int64_t cols, hipStream_t s) {
  const T* xp = static_cast<const T*>(x);
  T* yp = static_cast<T*>(y);
  if (!(fwd_try<T, VEC, 1, 2, true>(xp, ld_x, yp, ld_y, lse, rows, cols, s) ||
        fwd_try<T, VEC, 2, 2, true>(xp, ld_x, yp, ld_y, lse, rows, cols, s) ||
        fwd_try<T, VEC, 4, 2, true>(xp, ld_x, yp, ld_y, lse, rows, cols, s) ||
        fwd_try<T, VEC, 8, 2, true>(xp, ld_x, yp, ld_y, lse, rows, cols, s) ||
        fwd_try<T, VEC, 8, 4, false>(xp, ld_x, yp, ld_y, lse, rows, cols, s) ||
        fwd_try<T, VEC, 8, 8, false>(xp, ld_x, yp, ld_y, lse, rows, cols, s)))
    softmax_fwd_stream<T, VEC><<<unsigned(rows), kStreamThreads, 0, s>>>(xp, ld_x, yp, ld_y, lse,
                                                                        cols);
  return hipGetLastError();
}

// Tiers of the backward.  Saved y: 8 waves x 1 vector for rows of 4096 16-bit
// values measured fastest (127 us for 32768 x 4096 bf16).  Rebuilt y (two
// exponentials per element): 4 waves x 2 vectors (129 us, against 169 us for
// 8 waves x 1 vector), the forward's tiers.
template <typename T, int VEC, bool FROM_LSE>
hipError_t bwd_vec(const void* dy, int64_t ld_dy, const void* src, int64_t ld_src,
                   const float* lse, void* dx, int64_t ld_dx, int64_t rows, int64_t cols,
                   hipStream_t s) {
  const T* gp = static_cast<const T*>(dy);
  const T* sp = static_cast<const T*>(src);
  T* dp = static_cast<T*>(dx);
#define VJP_SMB_TRY(W, K) \
  bwd_try<T, VEC, W, K, FROM_LSE>(gp, ld_dy, sp, ld_src, lse, dp, ld_dx, rows, cols, s)
  const bool done =
      FROM_LSE ? (VJP_SMB_TRY(1, 2) || VJP_SMB_TRY(2, 2) || VJP_SMB_TRY(4, 2) ||
                  VJP_SMB_TRY(8, 2) || VJP_SMB_TRY(8, 4) || VJP_SMB_TRY(8, 8))
               : (VJP_SMB_TRY(1, 1) || VJP_SMB_TRY(2, 1) || VJP_SMB_TRY(4, 1) ||
                  VJP_SMB_TRY(8, 1) || VJP_SMB_TRY(8, 2) || VJP_SMB_TRY(8, 4) ||
                  VJP_SMB_TRY(8, 8));
  if (!done)
    softmax_bwd_stream<T, VEC, FROM_LSE><<<unsigned(rows), kStreamThreads, 0, s>>>(
        gp, ld_dy, sp, ld_src, lse, dp, ld_dx, cols);
#undef VJP_SMB_TRY
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_typed(const void* x, int64_t ld_x, void* y, int64_t ld_y, float* lse,
                     int64_t rows, int64_t cols, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  return vec ? fwd_vec<T, V>(x, ld_x, y, ld_y, lse, rows, cols, s)
             : fwd_vec<T, 1>(x, ld_x, y, ld_y, lse, rows, cols, s);
}

template <typename T>
hipError_t bwd_typed(const void* dy, int64_t ld_dy, const void* src, int64_t ld_src,
                     const float* lse, void* dx, int64_t ld_dx, int64_t rows, int64_t cols,
                     bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  if (lse != nullptr)
    return vec ? bwd_vec<T, V, true>(dy, ld_dy, src, ld_src, lse, dx, ld_dx, rows, cols, s)
               : bwd_vec<T, 1, true>(dy, ld_dy, src, ld_src, lse, dx, ld_dx, rows, cols, s);
  return vec ? bwd_vec<T, V, false>(dy, ld_dy, src, ld_src, lse, dx, ld_dx, rows, cols, s)
             : bwd_vec<T, 1, false>(dy, ld_dy, src, ld_src, lse, dx, ld_dx, rows, cols, s);
}

}  // namespace

hipError_t launch_softmax_fwd(const void* x, int64_t ld_x, void* y, int64_t ld_y,
                              float* row_lse, int64_t rows, int64_t cols, int act, bool vec,
                              hipStream_t s) {
  switch (act) {
    case kF32: return fwd_typed<float>(x, ld_x, y, ld_y, row_lse, rows, cols, vec, s);
    case kF16: return fwd_typed<_Float16>(x, ld_x, y, ld_y, row_lse, rows, cols, vec, s);
    default: return fwd_typed<bf16>(x, ld_x, y, ld_y, row_lse, rows, cols, vec, s);
  }
}

hipError_t launch_softmax_bwd(const void* dy, int64_t ld_dy, const void* src, int64_t ld_src,
                              const float* row_lse, void* dx, int64_t ld_dx, int64_t rows,
                              int64_t cols, int act, bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return bwd_typed<float>(dy, ld_dy, src, ld_src, row_lse, dx, ld_dx, rows, cols, vec, s);
    case kF16: return bwd_typed<_Float16>(dy, ld_dy, src, ld_src, row_lse, dx, ld_dx, rows, cols, vec, s);
    default: return bwd_typed<bf16>(dy, ld_dy, src, ld_src, row_lse, dx, ld_dx, rows, cols, vec, s);
  }
}

}  // namespace vjp
