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
#include "launch.hpp"
#include "rowops.hpp"

namespace vjp {

namespace {

template <int WAVES> constexpr int block_threads() { return WAVES == 1 ? 256 : WAVES * kWave; }

__device__ __forceinline__ void write_row_stats(int64_t row, float m, float lse, float zt,
                                                bool valid, float* __restrict__ row_max,
                                                float* __restrict__ row_lse,
                                                float* __restrict__ row_loss) {
  row_max[row] = m;
  row_lse[row] = lse;
  row_loss[row] = valid ? lse - zt : __builtin_nanf("");
}

template <typename T, int VEC, int WAVES>
__global__ __launch_bounds__(block_threads<WAVES>()) void xent_resident(
    const T* __restrict__ z, int64_t ld, const int32_t* __restrict__ targets, int64_t rows,
    int64_t C, float scale, float* __restrict__ row_max, float* __restrict__ row_lse,
    float* __restrict__ row_loss, T* __restrict__ dz, int64_t ld_dz) {
  __shared__ float buf[WAVES];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t row = WAVES == 1 ? int64_t(blockIdx.x) * 4 + wave : int64_t(blockIdx.x);
  const int wv = WAVES == 1 ? 0 : wave;
  if (WAVES == 1 && row >= rows) return;
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  const int64_t lane_col = (int64_t(wv) * kWave + lane) * VEC;
  const T* zr = z + row * ld;
  const int64_t t = targets[row];
  const bool valid = t >= 0 && t < C;

  Vec<T, VEC> raw[kChunks];
  float mx = -__builtin_inff(), mn = __builtin_inff();
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    if (k * kStep < C) {
      const int64_t col = k * kStep + lane_col;
      if (load_row_vec<T, VEC>(zr, col, C, neg_inf_of<T>(), raw[k])) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float f = to_f32(raw[k].v[i]);
          mx = fmaxf(mx, f);
          mn = fminf(mn, f);
        }
      } else {  // ragged end of the row: padding counts for neither max nor min
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float f = to_f32(raw[k].v[i]);
          mx = fmaxf(mx, f);
          mn = fminf(mn, col + i < C ? f : __builtin_inff());
        }
      }
    }
  }
  const float m = row_reduce_max<WAVES>(mx, buf);

  float e[kChunks][VEC];
  float l = 0.0f;
  if (!((mn - m) * kLog2e < -126.0f)) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      if (k * kStep < C) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          e[k][i] = exp2_fast((to_f32(raw[k].v[i]) - m) * kLog2e);
          l += e[k][i];
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      if (k * kStep < C) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          e[k][i] = exp2_denorm_safe((to_f32(raw[k].v[i]) - m) * kLog2e);
          l += e[k][i];
        }
      }
    }
  }
  l = row_reduce_sum<WAVES>(l, buf);
  const float inv = 1.0f / l;
  const float ps = scale * inv;

  if (wv == 0 && lane == 0) {
    const float lse = m + log2_fast(l) * kLn2;
    write_row_stats(row, m, lse, valid ? to_f32(zr[t]) : 0.0f, valid, row_max, row_lse,
                    row_loss);
  }

  T* dr = dz + row * ld_dz;
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    if (k * kStep < C) {
      const int64_t col = k * kStep + lane_col;
      if (col < C) {
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = e[k][i] * ps;
        if (uint64_t(t - col) < uint64_t(VEC)) {  // this vector holds the target column
#pragma unroll
          for (int i = 0; i < VEC; ++i)
            if (col + i == t) o[i] = (e[k][i] * inv - 1.0f) * scale;
        }
        store_row_vec<T, VEC>(dr, col, C, o);
      }
    }
  }
}

template <typename T, int VEC>
__global__ __launch_bounds__(kStreamThreads) void xent_stream(
    const T* __restrict__ z, int64_t ld, const int32_t* __restrict__ targets, int64_t C,
    float scale, float* __restrict__ row_max, float* __restrict__ row_lse,
    float* __restrict__ row_loss, T* __restrict__ dz, int64_t ld_dz) {
  __shared__ float bm[kStreamThreads / kWave], bl[kStreamThreads / kWave];
  const int64_t row = blockIdx.x;
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
    const float lse = m + log2_fast(l) * kLn2;
    write_row_stats(row, m, lse, valid ? to_f32(zr[t]) : 0.0f, valid, row_max, row_lse,
                    row_loss);
  }
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

int resident_waves(int64_t cols, int vec) {
  for (int w = 1; w <= 8; w <<= 1)
    if (int64_t(w) * kWave * kChunks * vec >= cols) return w;
  return 0;
}

template <typename T, int VEC>
hipError_t run_vec(const void* z, int64_t ld, const int32_t* tg, int64_t rows, int64_t C,
                   float scale, float* rmax, float* rlse, float* rloss, void* dz, int64_t ld_dz,
                   hipStream_t s) {
  const T* zp = static_cast<const T*>(z);
  T* dp = static_cast<T*>(dz);
  const unsigned rb = unsigned(rows);
  switch (resident_waves(C, VEC)) {
    case 1: xent_resident<T, VEC, 1><<<unsigned((rows + 3) / 4), 256, 0, s>>>(zp, ld, tg, rows, C, scale, rmax, rlse, rloss, dp, ld_dz); break;
    case 2: xent_resident<T, VEC, 2><<<rb, 128, 0, s>>>(zp, ld, tg, rows, C, scale, rmax, rlse, rloss, dp, ld_dz); break;
    case 4: xent_resident<T, VEC, 4><<<rb, 256, 0, s>>>(zp, ld, tg, rows, C, scale, rmax, rlse, rloss, dp, ld_dz); break;
    case 8: xent_resident<T, VEC, 8><<<rb, 512, 0, s>>>(zp, ld, tg, rows, C, scale, rmax, rlse, rloss, dp, ld_dz); break;
    default: xent_stream<T, VEC><<<rb, kStreamThreads, 0, s>>>(zp, ld, tg, C, scale, rmax, rlse, rloss, dp, ld_dz); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t run_typed(const void* z, int64_t ld, const int32_t* tg, int64_t rows, int64_t C,
                     float scale, float* rmax, float* rlse, float* rloss, void* dz,
                     int64_t ld_dz, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  return vec ? run_vec<T, V>(z, ld, tg, rows, C, scale, rmax, rlse, rloss, dz, ld_dz, s)
             : run_vec<T, 1>(z, ld, tg, rows, C, scale, rmax, rlse, rloss, dz, ld_dz, s);
}

}  // namespace

hipError_t launch_softmax_xent(const void* z, int64_t ld, const int32_t* targets, int64_t rows,
                               int64_t classes, int act, float grad_scale, float* row_max,
                               float* row_lse, float* row_loss, void* dz, int64_t ld_dz,
                               bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return run_typed<float>(z, ld, targets, rows, classes, grad_scale, row_max, row_lse, row_loss, dz, ld_dz, vec, s);
    case kF16: return run_typed<_Float16>(z, ld, targets, rows, classes, grad_scale, row_max, row_lse, row_loss, dz, ld_dz, vec, s);
    default: return run_typed<bf16>(z, ld, targets, rows, classes, grad_scale, row_max, row_lse, row_loss, dz, ld_dz, vec, s);
  }
}

}  // namespace vjp
