// LayerNorm and RMSNorm over the last dimension: forward and backward.
//
// Source: "Backprop for kernel writers", the LayerNorm passage after 04 "The
// duality" (every element of a row is coupled through its mean and variance,
// yet the backward collapses to two row scalars; the parameter gradients
// reduce over the batch axis and need cross-block accumulation) and section
// 07 (save normalisation constants: one float per row).  "Backward in Triton
// -- autograd.Function and the backward grid", sections "Save vs recompute"
// (the rstd is a one-scalar-per-row statistic) and "The backward grid is not
// the forward grid" (RMSNorm's dw: a length-d partial from every row, summed
// by a second, deterministic pass).
//
//   LayerNorm: mu = mean(x), rstd = 1 / sqrt(mean((x - mu)^2) + eps),
//              xhat = (x - mu) rstd, y = xhat w + b
//   RMSNorm:   mu = 0,       rstd = 1 / sqrt(mean(x^2) + eps), y = xhat w
//   backward:  g = dy w, a = mean(g) (LayerNorm only), c = mean(g xhat),
//              dx = rstd (g - a - xhat c); dw = sum_rows dy xhat, db = sum_rows dy
//
// Forward: one row per workgroup in the resident row layout of rowops.hpp,
// the row read once; the variance is the two-pass mean of squared deviations
// of the values held in registers.  Backward: workgroup t owns the rows t, t + tiles, t + 2 tiles,
// ... (a round-robin deal, so all workgroups stream neighbouring rows at the
// same moment); for each row it loads x and dy into registers, forms the two
// row scalars with one exchange, writes dx, and adds dy xhat (and dy) into
// fp32 column partials that stay in its lanes' registers: every lane owns
// fixed columns, so no cross-lane reduction is needed.  The tile's partial
// rows go to P[t][0 .. cols) (dw) and P[t][cols .. 2 cols) (db), summed by
// the fixed-order stage-2 kernel.
#include <type_traits>

#include "launch.hpp"
#include "rowops.hpp"

namespace vjp {

namespace {

// Loads the lane's K vectors of row `row` (padding reads 0), all in flight
// together.
template <typename T, int VEC, int WAVES, int K>
__device__ __forceinline__ void load_lane_row(const T* __restrict__ r, int64_t cols,
                                              int64_t lane_col, Vec<T, VEC> (&v)[K]) {
  load_row_resident<T, VEC, WAVES, K>(r, cols, lane_col, zero_of<T>(), v);
}

// VEC consecutive parameter values starting at column col, in two phases
// like issue_vec / fix_vec: issue_params starts the load (one aligned vector
// of VEC elements, PB bytes each: 4 for fp32, 2 for fp16 / bf16) when the
// parameter vectors are 16-byte aligned (pvec) and the VEC columns lie inside
// the row; params_f32 widens the loaded values to fp32, or loads a ragged or
// unaligned vector element by element (zero past cols).  The loaded values
// stay packed in their own width until they are used.  fp16 against bf16 is
// a launch-wide value, so its branch is uniform.
template <int VEC, int PB>
using param_words_t =
    typename std::conditional<PB == 4, words_t<float, VEC>, words_t<uint16_t, VEC>>::type;

template <int VEC, int PB>
__device__ __forceinline__ void issue_params(const void* __restrict__ p, int64_t col, int64_t cols,
                                             bool pvec, param_words_t<VEC, PB>& r) {
  if (pvec && col + VEC <= cols)
    r = *reinterpret_cast<const param_words_t<VEC, PB>*>(static_cast<const char*>(p) + col * PB);
}

template <int VEC, int PB>
__device__ __forceinline__ void params_f32(const void* __restrict__ p, int64_t col, int64_t cols,
                                           int wdt, bool pvec, const param_words_t<VEC, PB>& r,
                                           float (&o)[VEC]) {
  if (pvec && col + VEC <= cols) {
    if constexpr (PB == 4) {
      const Vec<float, VEC> f = __builtin_bit_cast(Vec<float, VEC>, r);
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = f.v[i];
    } else {
      const Vec<uint16_t, VEC> h = __builtin_bit_cast(Vec<uint16_t, VEC>, r);
      if (wdt == kF16) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = to_f32(__builtin_bit_cast(_Float16, h.v[i]));
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) o[i] = to_f32(bf16{h.v[i]});
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) o[i] = (col + i < cols) ? load_param_f32(p, col + i, wdt) : 0.0f;
}

// A lane's K vectors of parameter values (the columns k * step + lane_col,
// k < K, VEC each), every load issued before any is widened to fp32.
template <int VEC, int PB, int K>
__device__ __forceinline__ void lane_params_f32(const void* __restrict__ p, int64_t lane_col,
                                                int64_t step, int64_t cols, int wdt, bool pvec,
                                                float (&o)[K][VEC]) {
  param_words_t<VEC, PB> r[K];
#pragma unroll
  for (int k = 0; k < K; ++k) issue_params<VEC, PB>(p, k * step + lane_col, cols, pvec, r[k]);
#pragma unroll
  for (int k = 0; k < K; ++k) params_f32<VEC, PB>(p, k * step + lane_col, cols, wdt, pvec, r[k], o[k]);
}

// Forward: RB consecutive rows per workgroup of WAVES waves (WAVES = 1: one
// wave per row, four rows per 256-thread workgroup, RB = 1), the resident
// layout of rowops.hpp, every row read once and all RB rows loaded before any
// is reduced; w and b read once per workgroup with vector loads (they stay in
// L2: every workgroup reads the same values), the RB means and then the RB
// variances exchanged together.
template <typename T, int VEC, int WAVES, int K, bool RMS, int RB, int PB>
__global__ __launch_bounds__(row_block_threads<WAVES>()) void norm_fwd_resident(
    const T* __restrict__ x, int64_t ld_x, const void* __restrict__ w,
    const void* __restrict__ b, int wdt, bool pvec, T* __restrict__ y, int64_t ld_y,
    float* __restrict__ row_mean, float* __restrict__ row_rstd, int64_t rows, int64_t cols,
    float eps) {
  static_assert(WAVES > 1 || RB == 1, "one-wave rows take one row per wave");
  __shared__ float buf[2][RB][WAVES];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t row0 = WAVES == 1 ? int64_t(blockIdx.x) * rows_per_block<1>() + wave
                                  : int64_t(blockIdx.x) * RB;
  const int wv = WAVES == 1 ? 0 : wave;
  if (WAVES == 1 && row0 >= rows) return;
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  const int64_t lane_col = (int64_t(wv) * kWave + lane) * VEC;
  const float inv_cols = 1.0f / float(cols);

  // Every load of the parameters and rows is issued before the first wait
  // (the parameters first: they are L2 hits and arrive before the rows).
  param_words_t<VEC, PB> rw[K], rb[RMS ? 1 : K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    issue_params<VEC, PB>(w, k * kStep + lane_col, cols, pvec, rw[k]);
    if constexpr (!RMS) issue_params<VEC, PB>(b, k * kStep + lane_col, cols, pvec, rb[k]);
  }
  Vec<T, VEC> raw[RB][K];
#pragma unroll
  for (int q = 0; q < RB; ++q)
    if (row0 + q < rows) load_lane_row<T, VEC, WAVES, K>(x + (row0 + q) * ld_x, cols, lane_col, raw[q]);

  float mean[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q) mean[q] = 0.0f;
  if constexpr (!RMS) {
#pragma unroll
    for (int q = 0; q < RB; ++q) {
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (k * kStep < cols)
#pragma unroll
          for (int i = 0; i < VEC; ++i) mean[q] += to_f32(raw[q][k].v[i]);   // padding reads 0
    }
    row_reduce_sum_n<WAVES, RB>(mean, buf[0]);
#pragma unroll
    for (int q = 0; q < RB; ++q) mean[q] *= inv_cols;
#pragma unroll
    for (int q = 0; q < RB; ++q) fence_row<T, VEC, K>(raw[q]);   // convert again below
  }
  float rstd[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q) {
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k * kStep < cols) {
        const int64_t col = k * kStep + lane_col;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float d = to_f32(raw[q][k].v[i]) - mean[q];
          if (col + i < cols) ss = fmaf(d, d, ss);
        }
      }
    }
    rstd[q] = ss;
  }
  row_reduce_sum_n<WAVES, RB>(rstd, buf[1]);
#pragma unroll
  for (int q = 0; q < RB; ++q) rstd[q] = 1.0f / __builtin_sqrtf(rstd[q] * inv_cols + eps);
#pragma unroll
  for (int q = 0; q < RB; ++q) fence_row<T, VEC, K>(raw[q]);

#pragma unroll
  for (int q = 0; q < RB; ++q) {
    const int64_t row = row0 + q;
    if (row >= rows) break;
    if (wv == 0 && lane == 0) {
      if (row_mean != nullptr) row_mean[row] = mean[q];
      if (row_rstd != nullptr) row_rstd[row] = rstd[q];
    }
    T* yr = y + row * ld_y;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k * kStep < cols) {
        const int64_t col = k * kStep + lane_col;
        if (col < cols) {
          float pw[VEC], pb[VEC];   // widened here: packed until now
          params_f32<VEC, PB>(w, col, cols, wdt, pvec, rw[k], pw);
          if constexpr (!RMS) params_f32<VEC, PB>(b, col, cols, wdt, pvec, rb[k], pb);
          float o[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i)
            o[i] = fmaf((to_f32(raw[q][k].v[i]) - mean[q]) * rstd[q], pw[i], RMS ? 0.0f : pb[i]);
          store_row_vec<T, VEC>(yr, col, cols, o);
        }
      }
    }
  }
}

template <typename T, int VEC, int WAVES, int K, bool RMS>
__global__ __launch_bounds__(WAVES * kWave) void norm_bwd_tile(
    const T* __restrict__ dy, int64_t ld_dy, const T* __restrict__ x, int64_t ld_x,
    const void* __restrict__ w, int wdt, const float* __restrict__ row_mean,
    const float* __restrict__ row_rstd, T* __restrict__ dx, int64_t ld_dx,
    float* __restrict__ P, int64_t rows, int64_t cols, int64_t tiles, float eps) {
  // Reduction slots, double-buffered by row parity: a wave may start the next
  // row's exchange while a slower wave still reads this row's values.
  __shared__ float buf[2][4][WAVES];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  const int64_t lane_col = (int64_t(wave) * kWave + lane) * VEC;
  const float inv_cols = 1.0f / float(cols);
  const int64_t tile = blockIdx.x;

  // w is loaded once per workgroup, all of a lane's vectors issued before
  // any is widened to fp32.  (Element by element, each load waited for
  // before the next, a workgroup's start took 8 round trips to L2: 134.9
  // against 133.1 us for LayerNorm and 126.4 against 125.6 us for RMSNorm,
  // medians of 80 interleaved runs at 32768 x 4096 bf16, the same bits.)
  float wv[K][VEC], pdw[K][VEC], pdb[RMS ? 1 : K][VEC];
  {
    const bool pvec = reinterpret_cast<uintptr_t>(w) % 16 == 0;
    if (wdt == kF32) lane_params_f32<VEC, 4, K>(w, lane_col, kStep, cols, wdt, pvec, wv);
    else lane_params_f32<VEC, 2, K>(w, lane_col, kStep, cols, wdt, pvec, wv);
  }
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      pdw[k][i] = 0.0f;
      if constexpr (!RMS) pdb[k][i] = 0.0f;
    }

  // RMSNorm requests the next row of the tile before it processes the
  // current one (while a lane holds at most 8 values of a row; wider rows
  // load in turn); LayerNorm loads each row when it comes to it.  The
  // compiler's wait before a row's first use also covers the next row's
  // loads (on some paths none are issued, so it waits for all), so with the
  // early request a wave has two rows in flight and then processes one.
  // Measured on MI355X at 32768 x 4096 bf16, medians of 80 interleaved runs,
  // the same bits: without the early request LayerNorm took 134.2 against
  // 137.4 us and 133.8 against 137.0 us (two runs), RMSNorm 129.2 against
  // 127.1 us.  A true overlap, the next row kept pending as raw words
  // through the current row's work and viewed as elements after a copy at
  // the top of the next iteration (no wait left before the work), was
  // slower for both: 137.1 against 132.7 us and 136.6 against 125.5 us; so
  // were two rows per wave at once (rows r and r + tiles loaded together,
  // their four row scalars in one exchange, the partials added in the same
  // order): 135.3 against 133.6 us and 134.6 against 125.8 us.
  constexpr bool kPrefetch = RMS && K * VEC <= 8;
  constexpr int KN = kPrefetch ? K : 1;
  Vec<T, VEC> rx[K], rg[K], nx[KN], ng[KN];
  if (kPrefetch && tile < rows) {
    load_lane_row<T, VEC, WAVES, K>(x + tile * ld_x, cols, lane_col, rx);
    load_lane_row<T, VEC, WAVES, K>(dy + tile * ld_dy, cols, lane_col, rg);
  }
  int par = 0;
  for (int64_t row = tile; row < rows; row += tiles, par ^= 1) {
    const int64_t next = row + tiles;
    if constexpr (kPrefetch) {
      if (next < rows) {
        load_lane_row<T, VEC, WAVES, KN>(x + next * ld_x, cols, lane_col, nx);
        load_lane_row<T, VEC, WAVES, KN>(dy + next * ld_dy, cols, lane_col, ng);
      }
    } else {
      load_lane_row<T, VEC, WAVES, K>(x + row * ld_x, cols, lane_col, rx);
      load_lane_row<T, VEC, WAVES, K>(dy + row * ld_dy, cols, lane_col, rg);
    }
    float mean = 0.0f, rstd;
    if (row_rstd != nullptr) {          // saved statistics (uniform branch)
      rstd = row_rstd[row];
      if constexpr (!RMS) mean = row_mean[row];
    } else {                            // recomputed from the row in registers
      if constexpr (!RMS) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k)
          if (k * kStep < cols)
#pragma unroll
            for (int i = 0; i < VEC; ++i) s += to_f32(rx[k].v[i]);
        mean = row_reduce_sum<WAVES>(s, buf[par][2]) * inv_cols;
      }
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (k * kStep < cols) {
          const int64_t col = k * kStep + lane_col;
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            const float d = to_f32(rx[k].v[i]) - mean;
            if (col + i < cols) ss = fmaf(d, d, ss);
          }
        }
      }
      rstd = 1.0f / __builtin_sqrtf(row_reduce_sum<WAVES>(ss, buf[par][3]) * inv_cols + eps);
    }
    // Row scalars.  Padding has dy = 0 and w = 0, so g = 0 there.
    float a = 0.0f, c = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k * kStep < cols) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float xh = (to_f32(rx[k].v[i]) - mean) * rstd;
          const float g = to_f32(rg[k].v[i]) * wv[k][i];
          if constexpr (!RMS) a += g;
          c = fmaf(g, xh, c);
        }
      }
    }
    row_reduce_sum2<WAVES>(a, c, buf[par][0], buf[par][1]);
    a *= inv_cols;
    c *= inv_cols;
    if constexpr (RMS) a = 0.0f;

    T* dr = dx + row * ld_dx;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k * kStep < cols) {
        const int64_t col = k * kStep + lane_col;
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float xh = (to_f32(rx[k].v[i]) - mean) * rstd;
          const float gy = to_f32(rg[k].v[i]);
          o[i] = rstd * (gy * wv[k][i] - a - xh * c);
          pdw[k][i] = fmaf(gy, xh, pdw[k][i]);
          if constexpr (!RMS) pdb[k][i] += gy;
        }
        if (col < cols) store_row_vec<T, VEC>(dr, col, cols, o);
      }
    }
    if constexpr (kPrefetch) {
#pragma unroll
      for (int k = 0; k < KN; ++k) {
        rx[k] = nx[k];
        rg[k] = ng[k];
      }
    }
  }

  // The tile's partial rows, in 16-byte stores where the workspace and the
  // row width allow.  (Every tile writes them at its end, so they form the
  // kernel's tail: LayerNorm's backward at 32768 x 4096 bf16 took 132.3 us
  // with 16-byte stores against 137.0-143.3 us with one fp32 store per
  // element, in one process, bitwise the same results.)
  const int64_t pw = RMS ? cols : 2 * cols;   // partial row width
  const bool pvec = cols % 4 == 0 && reinterpret_cast<uintptr_t>(P) % 16 == 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t col = k * kStep + lane_col;
    if constexpr (VEC % 4 == 0) {
      if (pvec && col + VEC <= cols) {
#pragma unroll
        for (int i = 0; i < VEC; i += 4) {
          *reinterpret_cast<Vec<float, 4>*>(P + tile * pw + col + i) =
              Vec<float, 4>{{pdw[k][i], pdw[k][i + 1], pdw[k][i + 2], pdw[k][i + 3]}};
          if constexpr (!RMS)
            *reinterpret_cast<Vec<float, 4>*>(P + tile * pw + cols + col + i) =
                Vec<float, 4>{{pdb[k][i], pdb[k][i + 1], pdb[k][i + 2], pdb[k][i + 3]}};
        }
        continue;
      }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      if (col + i < cols) {
        P[tile * pw + col + i] = pdw[k][i];
        if constexpr (!RMS) P[tile * pw + cols + col + i] = pdb[k][i];
      }
    }
  }
}

// Launch tiers, smallest first: (waves per row, vectors per lane).  The first
// tier whose capacity WAVES * 64 * K * VEC holds the row is used.  A lane
// holds at most 16 elements of a row (the backward keeps w and the dw / db
// partials of its columns in fp32 registers besides x and dy), so rows of
// up to 16 waves * 64 lanes * 16 = 16384 columns are supported.
constexpr int kLaneElems = 16;
// Rows per workgroup of the forward with 16-bit parameters (rows of 2 to 16
// waves with at most two vectors per lane; wider rows would hold too many
// registers).  Measured on MI355X for 32768 x 4096 bf16 with bf16
// parameters: LayerNorm 101 us with one row per workgroup, 97 us with two
// (w and b read once per two rows), 111 us with four; RMSNorm 90 us with
// one, 91 us with two.  Workgroups that loop over rows with the parameters
// held in registers measured 127 us.  (The bias loads cost LayerNorm 11 us:
// 89-90 us without them; with the register fences below, 95.6 against
// 90.7 us in one process, RMSNorm 88.1.  Two row pairs per workgroup with w
// and b loaded once take 251 VGPRs, or spill 780 bytes per lane at 64.)  Those figures predate the register fences between
// the phases of the forward: with them LayerNorm's two-row form holds 64
// VGPRs instead of 80 (eight waves per SIMD instead of six) and took 96 us;
// RMSNorm with two rows (47 VGPRs) took 92 us against 90 us with one, and
// LayerNorm with four rows (88 VGPRs, w and b read by half as many
// workgroups) 95.0 against 93.0 us with two, medians of 80 interleaved
// runs, the same bits.  The same fences in the backward
// raised its VGPRs and were left out.  LayerNorm statistics from one
// exchange (each wave's sum and its sum of squares about its own mean,
// merged across the waves with the pairwise variance update) instead of two
// (the mean, then the squares about it) measured 95.5 us for two rows per
// workgroup and 100.5 us for one, against 94.1 us, in one process.
template <bool RMS> constexpr int kFwdRowsPerBlock = RMS ? 1 : 2;

template <typename T, int VEC, int WAVES, int K, bool RMS>
bool fwd_try(const T* xp, int64_t ld_x, const void* w, const void* b, int wdt, bool pvec, T* yp,
             int64_t ld_y, float* mean, float* rstd, int64_t rows, int64_t cols, float eps,
             hipStream_t s) {
  if constexpr (K * VEC > kLaneElems) {
    return false;
  } else {
    if (int64_t(WAVES) * kWave * K * VEC < cols) return false;
    // fp32 parameters stay at one row per workgroup (two rows would take
    // 96-107 VGPRs).
    constexpr int RB2 = (WAVES == 1 || K > 2) ? 1 : kFwdRowsPerBlock<RMS>;
    auto grid = [&](int rb) {
      const int64_t per = WAVES == 1 ? rows_per_block<1>() : rb;
      return unsigned((rows + per - 1) / per);
    };
    if (wdt == kF32)
      norm_fwd_resident<T, VEC, WAVES, K, RMS, 1, 4><<<grid(1), row_block_threads<WAVES>(), 0, s>>>(
          xp, ld_x, w, b, wdt, pvec, yp, ld_y, mean, rstd, rows, cols, eps);
    else
      norm_fwd_resident<T, VEC, WAVES, K, RMS, RB2, 2><<<grid(RB2), row_block_threads<WAVES>(), 0, s>>>(
          xp, ld_x, w, b, wdt, pvec, yp, ld_y, mean, rstd, rows, cols, eps);
    return true;
  }
}

template <typename T, int VEC, int WAVES, int K, bool RMS>
bool bwd_try(const T* gp, int64_t ld_dy, const T* xp, int64_t ld_x, const void* w, int wdt,
             const float* mean, const float* rstd, T* dp, int64_t ld_dx, float* P, int64_t rows,
             int64_t cols, int64_t tiles, float eps, hipStream_t s) {
  if constexpr (K * VEC > kLaneElems) {
    return false;
  } else {
    if (int64_t(WAVES) * kWave * K * VEC < cols) return false;
    norm_bwd_tile<T, VEC, WAVES, K, RMS><<<unsigned(tiles), WAVES * kWave, 0, s>>>(
        gp, ld_dy, xp, ld_x, w, wdt, mean, rstd, dp, ld_dx, P, rows, cols, tiles, eps);
    return true;
  }
}

template <typename T, int VEC, bool RMS>
hipError_t fwd_vec(const void* x, int64_t ld_x, const void* w, const void* b, int wdt, bool pvec,
                   void* y, int64_t ld_y, float* mean, float* rstd, int64_t rows, int64_t cols,
                   float eps, hipStream_t s) {
  const T* xp = static_cast<const T*>(x);
  T* yp = static_cast<T*>(y);
#define VJP_NF_TRY(W, K) \
  fwd_try<T, VEC, W, K, RMS>(xp, ld_x, w, b, wdt, pvec, yp, ld_y, mean, rstd, rows, cols, eps, s)
  const bool done = VJP_NF_TRY(1, 2) || VJP_NF_TRY(2, 2) || VJP_NF_TRY(4, 2) ||
                    VJP_NF_TRY(8, 2) || VJP_NF_TRY(16, 2) || VJP_NF_TRY(16, 4) ||
                    VJP_NF_TRY(16, 8) || VJP_NF_TRY(16, 16);
#undef VJP_NF_TRY
  return done ? hipGetLastError() : hipErrorInvalidValue;
}

template <typename T, int VEC, bool RMS>
hipError_t bwd_vec(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x, const void* w,
                   int wdt, const float* mean, const float* rstd, void* dx, int64_t ld_dx,
                   float* P, int64_t rows, int64_t cols, int64_t tiles, float eps,
                   hipStream_t s) {
  const T* gp = static_cast<const T*>(dy);
  const T* xp = static_cast<const T*>(x);
  T* dp = static_cast<T*>(dx);
#define VJP_NB_TRY(W, K)                                                                  \
  bwd_try<T, VEC, W, K, RMS>(gp, ld_dy, xp, ld_x, w, wdt, mean, rstd, dp, ld_dx, P, rows, \
                             cols, tiles, eps, s)
  const bool done = VJP_NB_TRY(1, 1) || VJP_NB_TRY(2, 1) || VJP_NB_TRY(4, 1) ||
                    VJP_NB_TRY(8, 1) || VJP_NB_TRY(16, 1) || VJP_NB_TRY(16, 2) ||
                    VJP_NB_TRY(16, 4) || VJP_NB_TRY(16, 8) || VJP_NB_TRY(16, 16);
#undef VJP_NB_TRY
  return done ? hipGetLastError() : hipErrorInvalidValue;
}

template <typename T, bool RMS>
hipError_t fwd_typed(const void* x, int64_t ld_x, const void* w, const void* b, int wdt, void* y,
                     int64_t ld_y, float* mean, float* rstd, int64_t rows, int64_t cols,
                     float eps, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  const bool pvec = reinterpret_cast<uintptr_t>(w) % 16 == 0 &&
                    (RMS || reinterpret_cast<uintptr_t>(b) % 16 == 0);
  return vec ? fwd_vec<T, V, RMS>(x, ld_x, w, b, wdt, pvec, y, ld_y, mean, rstd, rows, cols, eps, s)
             : fwd_vec<T, 1, RMS>(x, ld_x, w, b, wdt, pvec, y, ld_y, mean, rstd, rows, cols, eps, s);
}

template <typename T, bool RMS>
hipError_t bwd_typed(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x, const void* w,
                     int wdt, const float* mean, const float* rstd, void* dx, int64_t ld_dx,
                     float* P, int64_t rows, int64_t cols, int64_t tiles, float eps, bool vec,
                     hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  return vec ? bwd_vec<T, V, RMS>(dy, ld_dy, x, ld_x, w, wdt, mean, rstd, dx, ld_dx, P, rows,
                                  cols, tiles, eps, s)
             : bwd_vec<T, 1, RMS>(dy, ld_dy, x, ld_x, w, wdt, mean, rstd, dx, ld_dx, P, rows,
                                  cols, tiles, eps, s);
}

}  // namespace

int64_t norm_max_cols(int, bool) { return int64_t(16) * kWave * kLaneElems; }

hipError_t launch_norm_fwd(bool rms, const void* x, int64_t ld_x, const void* w, const void* b,
                           int wdt, void* y, int64_t ld_y, float* row_mean, float* row_rstd,
                           int64_t rows, int64_t cols, float eps, int act, bool vec,
                           hipStream_t s) {
#define VJP_NF(T, R) \
  fwd_typed<T, R>(x, ld_x, w, b, wdt, y, ld_y, row_mean, row_rstd, rows, cols, eps, vec, s)
  if (rms) {
    switch (act) {
      case kF32: return VJP_NF(float, true);
      case kF16: return VJP_NF(_Float16, true);
      default: return VJP_NF(bf16, true);
    }
  }
  switch (act) {
    case kF32: return VJP_NF(float, false);
    case kF16: return VJP_NF(_Float16, false);
    default: return VJP_NF(bf16, false);
  }
#undef VJP_NF
}

hipError_t launch_norm_bwd_stage1(bool rms, const void* dy, int64_t ld_dy, const void* x,
                                  int64_t ld_x, const void* w, int wdt, const float* row_mean,
                                  const float* row_rstd, void* dx, int64_t ld_dx, float* P,
                                  int64_t rows, int64_t cols, int64_t tiles, float eps, int act,
                                  bool vec, hipStream_t s) {
#define VJP_NB(T, R)                                                                          \
  bwd_typed<T, R>(dy, ld_dy, x, ld_x, w, wdt, row_mean, row_rstd, dx, ld_dx, P, rows, cols, \
                  tiles, eps, vec, s)
  if (rms) {
    switch (act) {
      case kF32: return VJP_NB(float, true);
      case kF16: return VJP_NB(_Float16, true);
      default: return VJP_NB(bf16, true);
    }
  }
  switch (act) {
    case kF32: return VJP_NB(float, false);
    case kF16: return VJP_NB(_Float16, false);
    default: return VJP_NB(bf16, false);
  }
#undef VJP_NB
}

}  // namespace vjp
