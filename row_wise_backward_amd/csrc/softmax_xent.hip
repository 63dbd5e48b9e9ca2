// Fused softmax-cross-entropy: forward statistics and logit gradient in one
// pass over the logits.
//
// Source: "Backprop for kernel writers", section 02 "See it move" (for
// softmax followed by cross-entropy the two derivatives cancel: the logit
// gradient is the softmax minus the one-hot of the target class, which is
// why the two are fused) and section 07 "Fusion" (keep only the per-row
// m and l, i.e. L = m + log l, and rebuild any probability as
// exp(z - L); recompute what is cheap from data already on chip).
//
// Per row r with target t_r and C classes:
//   m_r = max_j z_rj                 -> row_max[r]
//   l_r = sum_j exp(z_rj - m_r)
//   lse_r = m_r + log l_r            -> row_lse[r]
//   loss_r = lse_r - z_{r, t_r}      -> row_loss[r] (workspace; NaN if t_r is
//                                       outside [0, C))
//   dz_rj = scale * (p_rj - [j == t_r]),  p_rj = exp(z_rj - m_r) / l_r
// The probabilities are rebuilt from the exponentials held in VGPRs (resident
// path) or recomputed from m and l (streaming path); they never reach HBM.
// The mean loss is formed by the fixed-order xent_finalize_kernel.
//
// Split form (section 07: save only the row statistics, rebuild p in the
// backward): GRAD = false runs the statistics pass alone (the logits are read
// once, nothing of their size is written); xent_bwd_kernel is then a map over
// the logits with dz = scale * (exp(z - lse) - [j == t]), where the upstream
// gradient of the mean loss is read from device memory, scale = dloss / rows.
//
// Every kernel here takes its row from xcd_block_x(): the workgroups of one
// XCD work through one contiguous band of rows.  Which workgroup takes a row
// does not change its results.
#include "launch.hpp"
#include "rowops.hpp"

namespace vjp {

namespace {

__device__ __forceinline__ void write_row_stats(int64_t row, float m, float lse, float zt,
                                                bool valid, float* __restrict__ row_max,
                                                float* __restrict__ row_lse,
                                                float* __restrict__ row_loss) {
  if (row_max != nullptr) row_max[row] = m;
  row_lse[row] = lse;
  row_loss[row] = valid ? lse - zt : __builtin_nanf("");
}

// Backward of the split form: one workgroup per (row, chunk of NT * VEC * U
// columns); U vectors per lane are loaded before any is used.  In place
// (dz == z with the same leading dimension) is safe: every element is read
// and then written by the same lane.
template <typename T, int VEC, int U, int NT = kStreamThreads>
__global__ __launch_bounds__(NT) void xent_bwd_kernel(
    const T* z, int64_t ld, const int32_t* __restrict__ targets,
    const float* __restrict__ row_lse, const float* __restrict__ dloss, int64_t total_rows,
    int64_t C, T* dz, int64_t ld_dz) {
  const int64_t row = xcd_block_x();
  const float L = row_lse[row];
  const int64_t t = targets[row];
  const float scale = *dloss / float(total_rows);
  const T* zr = z + row * ld;
  T* dr = dz + row * ld_dz;
  constexpr int64_t kChunk = int64_t(NT) * VEC;
  const int64_t c0 = int64_t(blockIdx.y) * kChunk * U + int64_t(threadIdx.x) * VEC;
  words_t<T, VEC> w[U];
#pragma unroll
  for (int u = 0; u < U; ++u) issue_vec<T, VEC>(zr + c0 + u * kChunk, C - (c0 + u * kChunk), w[u]);
#pragma unroll
  for (int u = 0; u < U; ++u)
    fix_vec<T, VEC>(zr + c0 + u * kChunk, C - (c0 + u * kChunk), neg_inf_of<T>(), w[u]);
  Vec<T, VEC> r[U];
#pragma unroll
  for (int u = 0; u < U; ++u) r[u] = as_vec<T, VEC>(w[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t col = c0 + u * kChunk;
    if (col < C) {
      float a[VEC], e[VEC];
      float amin = __builtin_inff();
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        a[i] = (to_f32(r[u].v[i]) - L) * kLog2e;
        amin = fminf(amin, a[i]);
      }
      if (amin < -126.0f) {   // some result may be subnormal
#pragma unroll
        for (int i = 0; i < VEC; ++i) e[i] = exp2_denorm_safe(a[i]);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) e[i] = exp2_fast(a[i]);
      }
      float o[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = e[i] * scale;
      if (uint64_t(t - col) < uint64_t(VEC)) {   // this vector holds the target column
#pragma unroll
        for (int i = 0; i < VEC; ++i)
          if (col + i == t) o[i] = (e[i] - 1.0f) * scale;
      }
      store_row_vec<T, VEC>(dr, col, C, o);
    }
  }
}

// Resident kernel: the row is loaded once; KEEP = true holds exp(z - m) in
// fp32 VGPRs for the gradient pass, KEEP = false recomputes it from the
// stored row (bitwise the same values, fewer VGPRs, more rows per CU).
template <typename T, int VEC, int WAVES, int K, bool KEEP, bool GRAD>
__global__ __launch_bounds__(row_block_threads<WAVES>()) void xent_resident(
    const T* __restrict__ z, int64_t ld, const int32_t* __restrict__ targets, int64_t rows,
    int64_t C, float scale, float* __restrict__ row_max, float* __restrict__ row_lse,
    float* __restrict__ row_loss, T* __restrict__ dz, int64_t ld_dz) {
  __shared__ float buf[2][WAVES];   // one slot per reduction of the row
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t row = WAVES == 1 ? xcd_block_x() * rows_per_block<1>() + wave : xcd_block_x();
  const int wv = WAVES == 1 ? 0 : wave;
  if (WAVES == 1 && row >= rows) return;
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  const int64_t lane_col = (int64_t(wv) * kWave + lane) * VEC;
  const T* zr = z + row * ld;
  const int64_t t = targets[row];
  const bool valid = t >= 0 && t < C;

  Vec<T, VEC> raw[K];
  float mx, mn;
  load_row_minmax<T, VEC, WAVES, K>(zr, C, lane_col, raw, mx, mn);
  const float m = row_reduce_max<WAVES>(mx, buf[0]);
  const bool safe = needs_denorm_exp(mn, m);
  fence_row<T, VEC, K>(raw);

  float keep[KEEP ? K : 1][VEC];
  float l = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k * kStep < C) {
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
  const float ps = scale * inv;

  const float lse = row_lse_of(m, l);
  if constexpr (!GRAD) {
    if (wv == 0 && lane == 0) {
      if (row_max != nullptr) row_max[row] = m;
      row_lse[row] = lse;
      row_loss[row] = valid ? lse - to_f32(zr[t]) : __builtin_nanf("");
    }
    return;
  }
  if (wv == 0 && lane == 0) {
    row_max[row] = m;
    row_lse[row] = lse;
    if (!valid) row_loss[row] = __builtin_nanf("");
  }

  T* dr = dz + row * ld_dz;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k * kStep < C) {
      const int64_t col = k * kStep + lane_col;
      if (col < C) {
        // The lane holding z_t writes the row loss (an invalid target past the
        // last column can fall in the last vector's padding: the NaN written
        // above stands).
        if (valid && uint64_t(t - col) < uint64_t(VEC)) {
#pragma unroll
          for (int i = 0; i < VEC; ++i)
            if (col + i == t) row_loss[row] = lse - to_f32(raw[k].v[i]);
        }
        float e[VEC];
        if constexpr (KEEP) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) e[i] = keep[k][i];
        } else {
          exp_vec<T, VEC>(raw[k], m, safe, e);
        }
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = e[i] * ps;
        if (uint64_t(t - col) < uint64_t(VEC)) {  // this vector holds the target column
#pragma unroll
          for (int i = 0; i < VEC; ++i)
            if (col + i == t) o[i] = (e[i] * inv - 1.0f) * scale;
        }
        store_row_vec<T, VEC>(dr, col, C, o);
      }
    }
  }
}

template <typename T, int VEC, bool GRAD>
__global__ __launch_bounds__(kStreamThreads) void xent_stream(
    const T* __restrict__ z, int64_t ld, const int32_t* __restrict__ targets, int64_t C,
    float scale, float* __restrict__ row_max, float* __restrict__ row_lse,
    float* __restrict__ row_loss, T* __restrict__ dz, int64_t ld_dz) {
  __shared__ float bm[kStreamThreads / kWave], bl[kStreamThreads / kWave];
  const int64_t row = xcd_block_x();
  const T* zr = z + row * ld;
  T* dr = dz + row * ld_dz;
  const int64_t t = targets[row];
  const bool valid = t >= 0 && t < C;
  float m = -__builtin_inff(), l = 0.0f;
  for (int64_t col = int64_t(threadIdx.x) * VEC; col < C; col += int64_t(kStreamThreads) * VEC) {
    Vec<T, VEC> r;
    load_row_vec<T, VEC>(zr, col, C, neg_inf_of<T>(), r);
#pragma unroll
    for (int i = 0; i < VEC; ++i) online_step(to_f32(r.v[i]), m, l);
  }
  block_merge_ml(m, l, bm, bl);
  const float inv = 1.0f / l;
  const float ps = scale * inv;
  if (threadIdx.x == 0) {
    write_row_stats(row, m, row_lse_of(m, l), valid ? to_f32(zr[t]) : 0.0f, valid, row_max,
                    row_lse, row_loss);
  }
  if constexpr (!GRAD) return;
  for (int64_t col = int64_t(threadIdx.x) * VEC; col < C; col += int64_t(kStreamThreads) * VEC) {
    Vec<T, VEC> r;
    load_row_vec<T, VEC>(zr, col, C, neg_inf_of<T>(), r);
    float o[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float e = exp2_denorm_safe((to_f32(r.v[i]) - m) * kLog2e);
      o[i] = (col + i == t) ? (e * inv - 1.0f) * scale : e * ps;
    }
    store_row_vec<T, VEC>(dr, col, C, o);
  }
}

// Launch tiers, smallest first, as for the softmax forward: (waves per row,
// vectors per lane, keep the exponentials).  Measured on MI355X: rows of
// 32000 16-bit logits run best recomputing the exponentials; keeping them in
// fp32 VGPRs cuts the waves per SIMD from 5 to 3 (484-498 us against 364 us),
// and keeping them rounded to bf16 in place of the stored row did not help
// either (the exponentials are not what limits this kernel), nor did one
// workgroup exchange per row instead of two (each wave's max and sum merged
// online: 360-373 us against 359-361 us), nor a persistent kernel staging its
// next row in LDS by direct loads while computing the current one (446-490
// us); a plain copy of the same bytes takes 344-351 us.  The
// statistics-only form never keeps the exponentials (an online max / sum
// folding each vector as it arrives measured slower: 217 us against 189 us
// for the read of 16384 x 32000 bf16).
template <typename T, int VEC, int WAVES, int K, bool KEEP, bool GRAD>
bool resident_try(const T* zp, int64_t ld, const int32_t* tg, int64_t rows, int64_t C,
                  float scale, float* rmax, float* rlse, float* rloss, T* dp, int64_t ld_dz,
                  hipStream_t s) {
  if (int64_t(WAVES) * kWave * K * VEC < C) return false;
  const unsigned grid = unsigned((rows + rows_per_block<WAVES>() - 1) / rows_per_block<WAVES>());
  xent_resident<T, VEC, WAVES, K, KEEP && GRAD, GRAD><<<grid, row_block_threads<WAVES>(), 0, s>>>(
      zp, ld, tg, rows, C, scale, rmax, rlse, rloss, dp, ld_dz);
  return true;
}

template <typename T, int VEC, bool GRAD>
hipError_t run_vec(const void* z, int64_t ld, const int32_t* tg, int64_t rows, int64_t C,
                   float scale, float* rmax, float* rlse, float* rloss, void* dz, int64_t ld_dz,
                   hipStream_t s) {
  const T* zp = static_cast<const T*>(z);
  T* dp = static_cast<T*>(dz);

#define VJP_XENT_TRY(W, K, KEEP) \
  resident_try<T, VEC, W, K, KEEP, GRAD>(zp, ld, tg, rows, C, scale, rmax, rlse, rloss, dp, ld_dz, s)
  // Rows up to 8 waves x 8 vectors: with the gradient as 16 waves x 4 vectors
  // (measured on MI355X for 16384 x 32000 bf16: 358-361 us against 364-365
  // us), statistics only as 8 waves x 8 vectors (159 us against 184 us).
  // (Each try launches when its capacity holds the row, so the widest tier
  // is tried only after the narrower ones.)
  bool done = VJP_XENT_TRY(1, 2, true) || VJP_XENT_TRY(2, 2, true) || VJP_XENT_TRY(4, 2, true) ||
              VJP_XENT_TRY(8, 2, true) || VJP_XENT_TRY(8, 4, false);
  if (!done) done = GRAD ? VJP_XENT_TRY(16, 4, false) : VJP_XENT_TRY(8, 8, false);
  if (!done)
    xent_stream<T, VEC, GRAD><<<unsigned(rows), kStreamThreads, 0, s>>>(
        zp, ld, tg, C, scale, rmax, rlse, rloss, dp, ld_dz);
#undef VJP_XENT_TRY
  return hipGetLastError();
}

template <typename T, bool GRAD>
hipError_t run_typed(const void* z, int64_t ld, const int32_t* tg, int64_t rows, int64_t C,
                     float scale, float* rmax, float* rlse, float* rloss, void* dz,
                     int64_t ld_dz, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  return vec ? run_vec<T, V, GRAD>(z, ld, tg, rows, C, scale, rmax, rlse, rloss, dz, ld_dz, s)
             : run_vec<T, 1, GRAD>(z, ld, tg, rows, C, scale, rmax, rlse, rloss, dz, ld_dz, s);
}

// Split backward launch: 1024 threads x 4 vectors per workgroup, so a row of
// up to 32768 16-bit logits is one workgroup with every load in flight
// (measured on MI355X for 16384 x 32000 bf16: 347 us against 399 us for 256
// threads x 4 vectors).
constexpr int kBwdUnroll = 4;
constexpr int kBwdThreads = 1024;

template <typename T>
hipError_t bwd_typed(const void* z, int64_t ld, const int32_t* tg, const float* rlse,
                     const float* dloss, int64_t total_rows, int64_t rows, int64_t C, void* dz,
                     int64_t ld_dz, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  const int v = vec ? V : 1;
  const int64_t per_block = int64_t(kBwdThreads) * v * kBwdUnroll;
  const dim3 grid(unsigned(rows), unsigned((C + per_block - 1) / per_block));
  if (vec)
    xent_bwd_kernel<T, V, kBwdUnroll, kBwdThreads><<<grid, kBwdThreads, 0, s>>>(
        static_cast<const T*>(z), ld, tg, rlse, dloss, total_rows, C, static_cast<T*>(dz), ld_dz);
  else
    xent_bwd_kernel<T, 1, kBwdUnroll, kBwdThreads><<<grid, kBwdThreads, 0, s>>>(
        static_cast<const T*>(z), ld, tg, rlse, dloss, total_rows, C, static_cast<T*>(dz), ld_dz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_xent(const void* z, int64_t ld, const int32_t* targets, int64_t rows,
                               int64_t classes, int act, float grad_scale, float* row_max,
                               float* row_lse, float* row_loss, void* dz, int64_t ld_dz,
                               bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return run_typed<float, true>(z, ld, targets, rows, classes, grad_scale, row_max, row_lse, row_loss, dz, ld_dz, vec, s);
    case kF16: return run_typed<_Float16, true>(z, ld, targets, rows, classes, grad_scale, row_max, row_lse, row_loss, dz, ld_dz, vec, s);
    default: return run_typed<bf16, true>(z, ld, targets, rows, classes, grad_scale, row_max, row_lse, row_loss, dz, ld_dz, vec, s);
  }
}

hipError_t launch_softmax_xent_stats(const void* z, int64_t ld, const int32_t* targets,
                                     int64_t rows, int64_t classes, int act, float* row_max,
                                     float* row_lse, float* row_loss, bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return run_typed<float, false>(z, ld, targets, rows, classes, 0.0f, row_max, row_lse, row_loss, nullptr, 0, vec, s);
    case kF16: return run_typed<_Float16, false>(z, ld, targets, rows, classes, 0.0f, row_max, row_lse, row_loss, nullptr, 0, vec, s);
    default: return run_typed<bf16, false>(z, ld, targets, rows, classes, 0.0f, row_max, row_lse, row_loss, nullptr, 0, vec, s);
  }
}

hipError_t launch_softmax_xent_bwd(const void* z, int64_t ld, const int32_t* targets,
                                   const float* row_lse, const float* dloss, int64_t total_rows,
                                   int64_t rows, int64_t classes, int act, void* dz,
                                   int64_t ld_dz, bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return bwd_typed<float>(z, ld, targets, row_lse, dloss, total_rows, rows, classes, dz, ld_dz, vec, s);
    case kF16: return bwd_typed<_Float16>(z, ld, targets, row_lse, dloss, total_rows, rows, classes, dz, ld_dz, vec, s);
    default: return bwd_typed<bf16>(z, ld, targets, row_lse, dloss, total_rows, rows, classes, dz, ld_dz, vec, s);
  }
}

}  // namespace vjp
