// Row-wise building blocks for the softmax and softmax-cross-entropy
// kernels: the register-resident row layout and workgroup reductions.
//
// Resident layout.  A row is owned by WAVES waves (WAVES = 1: one wave per
// row, four rows per 256-thread workgroup).  Lane `lane` of wave `wv` holds
// K vectors of VEC elements; vector k starts at column
//   (k * WAVES * 64 + wv * 64 + lane) * VEC,
// so each step k reads WAVES * 64 * VEC contiguous elements (1 KB per wave
// for 16-byte vectors).  Capacity: WAVES * 64 * K * VEC columns.  The whole
// row stays in VGPRs (as loaded, in its storage type) between the statistics
// pass and the output pass, so it is read from HBM exactly once.
#pragma once

#include "common.hpp"

namespace vjp {

template <int WAVES> constexpr int row_block_threads() { return WAVES == 1 ? 256 : WAVES * kWave; }

// Launch geometry of a resident row kernel: rows per workgroup and grid size.
template <int WAVES> constexpr int rows_per_block() { return WAVES == 1 ? 256 / kWave : 1; }

template <typename T> __device__ __forceinline__ T neg_inf_of();
template <> __device__ __forceinline__ float neg_inf_of<float>() { return -__builtin_inff(); }
template <> __device__ __forceinline__ _Float16 neg_inf_of<_Float16>() {
  return __builtin_bit_cast(_Float16, uint16_t(0xfc00));
}
template <> __device__ __forceinline__ bf16 neg_inf_of<bf16>() { return bf16{0xff80}; }

template <typename T> __device__ __forceinline__ T zero_of() { return T{}; }

// Load vector `col` of a row; elements at or beyond `cols` read as `fill`.
// Returns true when the whole vector lies inside the row.
template <typename T, int VEC>
__device__ __forceinline__ bool load_row_vec(const T* __restrict__ row, int64_t col, int64_t cols,
                                             T fill, Vec<T, VEC>& r) {
  words_t<T, VEC> w;
  issue_vec<T, VEC>(row + col, cols - col, w);
  fix_vec<T, VEC>(row + col, cols - col, fill, w);
  r = as_vec<T, VEC>(w);
  return col + VEC <= cols;
}

// Loads the lane's K vectors of a row in the resident layout, all K loads
// issued before any is completed or used; elements at or beyond `cols`
// (including vectors wholly past the end) read as `fill`.
template <typename T, int VEC, int WAVES, int K>
__device__ __forceinline__ void load_row_resident(const T* __restrict__ row, int64_t cols,
                                                  int64_t lane_col, T fill, Vec<T, VEC> (&r)[K]) {
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  words_t<T, VEC> w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t col = k * kStep + lane_col;
    issue_vec<T, VEC>(row + col, cols - col, w[k]);
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t col = k * kStep + lane_col;
    fix_vec<T, VEC>(row + col, cols - col, fill, w[k]);
  }
#pragma unroll
  for (int k = 0; k < K; ++k) r[k] = as_vec<T, VEC>(w[k]);
}

// Store vector `col` of a row, dropping elements at or beyond `cols`.
template <typename T, int VEC>
__device__ __forceinline__ void store_row_vec(T* __restrict__ row, int64_t col, int64_t cols,
                                              const float (&v)[VEC]) {
  store_f32_tail<T, VEC>(row + col, cols - col, v);
}

// Workgroup-wide reductions for rows owned by WAVES > 1 waves.  Every thread
// receives the same value; waves are combined in wave order.  `buf` holds
// WAVES floats and must not be reused until every wave has read it (the
// kernels give each reduction of a row its own slot).
template <int WAVES>
__device__ __forceinline__ float row_reduce_max(float v, float* buf) {
  v = wave_max(v);
  if constexpr (WAVES > 1) {
    if ((threadIdx.x % kWave) == 0) buf[threadIdx.x / kWave] = v;
    lds_barrier();
    v = buf[0];
#pragma unroll
    for (int k = 1; k < WAVES; ++k) v = fmaxf(v, buf[k]);
  }
  return v;
}

template <int WAVES>
__device__ __forceinline__ float row_reduce_sum(float v, float* buf) {
  v = wave_sum(v);
  if constexpr (WAVES > 1) {
    if ((threadIdx.x % kWave) == 0) buf[threadIdx.x / kWave] = v;
    lds_barrier();
    v = buf[0];
#pragma unroll
    for (int k = 1; k < WAVES; ++k) v += buf[k];
  }
  return v;
}

// Two sums of a row in one exchange (one barrier): waves combined in order.
template <int WAVES>
__device__ __forceinline__ void row_reduce_sum2(float& a, float& b, float* bufa, float* bufb) {
  a = wave_sum(a);
  b = wave_sum(b);
  if constexpr (WAVES > 1) {
    if ((threadIdx.x % kWave) == 0) {
      bufa[threadIdx.x / kWave] = a;
      bufb[threadIdx.x / kWave] = b;
    }
    lds_barrier();
    a = bufa[0];
    b = bufb[0];
#pragma unroll
    for (int k = 1; k < WAVES; ++k) {
      a += bufa[k];
      b += bufb[k];
    }
  }
}

// N sums of a row (or of N rows owned by the same waves) in one exchange.
template <int WAVES, int N>
__device__ __forceinline__ void row_reduce_sum_n(float (&v)[N], float (*buf)[WAVES]) {
#pragma unroll
  for (int n = 0; n < N; ++n) v[n] = wave_sum(v[n]);
  if constexpr (WAVES > 1) {
    if ((threadIdx.x % kWave) == 0) {
#pragma unroll
      for (int n = 0; n < N; ++n) buf[n][threadIdx.x / kWave] = v[n];
    }
    lds_barrier();
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float t = buf[n][0];
#pragma unroll
      for (int k = 1; k < WAVES; ++k) t += buf[n][k];
      v[n] = t;
    }
  }
}

// 2^t without flushing subnormal results: v_exp_f32 is only trusted for
// results >= 2^-126, below that the argument is shifted up by 64 and the
// result scaled back (an exact power-of-two scaling, one rounding).
__device__ __forceinline__ float exp2_denorm_safe(float t) {
  return t < -126.0f ? exp2_fast(t + 64.0f) * 5.421010862427522e-20f /* 2^-64 */
                     : exp2_fast(t);
}

// e[i] = exp(x_i - m) = 2^((x_i - m) log2 e) for one vector of a row, x_i
// as stored.  x_i - m is exact for 16-bit inputs, so the row max maps to
// exactly 1.  Lanes whose row range can produce results below 2^-126
// (flagged by `safe`) take the subnormal-preserving form; the two forms
// agree wherever both are exact.
template <typename T, int VEC>
__device__ __forceinline__ void exp_vec(const Vec<T, VEC>& r, float m, bool safe,
                                        float (&e)[VEC]) {
  if (!safe) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) e[i] = exp2_fast((to_f32(r.v[i]) - m) * kLog2e);
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) e[i] = exp2_denorm_safe((to_f32(r.v[i]) - m) * kLog2e);
  }
}

// Row logsumexp from the row max m and the row sum l of exp(x - m).
__device__ __forceinline__ float row_lse_of(float m, float l) { return m + log2_fast(l) * kLn2; }

// The lane's max over its K vectors (padding read as -inf) and min over its
// valid elements.
template <typename T, int VEC, int WAVES, int K>
__device__ __forceinline__ void lane_minmax(const Vec<T, VEC> (&raw)[K], int64_t cols,
                                            int64_t lane_col, float& mx, float& mn) {
  constexpr int64_t kStep = int64_t(WAVES) * kWave * VEC;
  mx = -__builtin_inff();
  mn = __builtin_inff();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k * kStep < cols) {
      const int64_t rem = cols - (k * kStep + lane_col);
      const int nv = rem >= VEC ? VEC : (rem > 0 ? int(rem) : 0);   // valid elements
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float f = to_f32(raw[k].v[i]);
        mx = fmaxf(mx, f);   // padding is -inf
        mn = fminf(mn, i < nv ? f : __builtin_inff());
      }
    }
  }
}

// Loads the lane's K vectors of a row (padding reads as -inf) and returns the
// lane's max over its elements and min over its valid elements.
template <typename T, int VEC, int WAVES, int K>
__device__ __forceinline__ void load_row_minmax(const T* __restrict__ row, int64_t cols,
                                                int64_t lane_col, Vec<T, VEC> (&raw)[K],
                                                float& mx, float& mn) {
  load_row_resident<T, VEC, WAVES, K>(row, cols, lane_col, neg_inf_of<T>(), raw);
  lane_minmax<T, VEC, WAVES, K>(raw, cols, lane_col, mx, mn);
}

// Register barrier on a loaded vector: the compiler must treat its contents
// as new, so values converted from it in an earlier phase are not kept alive
// for reuse.  This keeps only the packed storage-type row in VGPRs between
// phases (the conversion is redone, one VALU op per element) and raises the
// number of rows in flight per CU.  Emits no instruction.
template <typename T, int N>
__device__ __forceinline__ void fence_vec(Vec<T, N>& r) {
  constexpr int kBytes = sizeof(T) * N;
  if constexpr (kBytes == 16) {
    u32x4_t u = __builtin_bit_cast(u32x4_t, r);
    asm volatile("" : "+v"(u));
    r = __builtin_bit_cast(Vec<T, N>, u);
  } else if constexpr (kBytes == 8) {
    u32x2_t u = __builtin_bit_cast(u32x2_t, r);
    asm volatile("" : "+v"(u));
    r = __builtin_bit_cast(Vec<T, N>, u);
  } else if constexpr (kBytes == 4) {
    unsigned u = __builtin_bit_cast(unsigned, r);
    asm volatile("" : "+v"(u));
    r = __builtin_bit_cast(Vec<T, N>, u);
  }
}

template <typename T, int VEC, int K>
__device__ __forceinline__ void fence_row(Vec<T, VEC> (&raw)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k) fence_vec<T, VEC>(raw[k]);
}

// Whether a lane needs the subnormal-preserving exponential: its smallest
// element lies more than 126 binades below the row max.
__device__ __forceinline__ bool needs_denorm_exp(float lane_min, float m) {
  return (lane_min - m) * kLog2e < -126.0f;
}

// Smallest WAVES in {1, 2, 4, 8} whose resident capacity with K vectors per
// lane holds `cols`; 0 means the row needs the streaming path.
inline int resident_waves(int64_t cols, int vec, int k) {
  for (int w = 1; w <= 8; w <<= 1)
    if (int64_t(w) * kWave * k * vec >= cols) return w;
  return 0;
}

// Streaming-path workgroup: 256 threads per row.
constexpr int kStreamThreads = 256;

// Combine per-thread online-softmax states (m, l) with l relative to m:
// M = max m_i, L = sum_i l_i * 2^((m_i - M) log2 e), threads in index order
// (wave butterflies, then the W waves in order).  Every thread receives (M, L).
template <int W>
__device__ __forceinline__ void block_merge_ml_w(float& m, float& l, float* bm, float* bl) {
  float M = wave_max(m);
  float contrib = (m == -__builtin_inff()) ? 0.0f : l * exp2_denorm_safe((m - M) * kLog2e);
  float Lw = wave_sum(contrib);
  lds_barrier();
  if ((threadIdx.x % kWave) == 0) {
    bm[threadIdx.x / kWave] = M;
    bl[threadIdx.x / kWave] = Lw;
  }
  lds_barrier();
  float Mg = bm[0];
#pragma unroll
  for (int k = 1; k < W; ++k) Mg = fmaxf(Mg, bm[k]);
  float Lg = 0.0f;
#pragma unroll
  for (int k = 0; k < W; ++k)
    Lg += (bm[k] == -__builtin_inff()) ? 0.0f : bl[k] * exp2_denorm_safe((bm[k] - Mg) * kLog2e);
  m = Mg;
  l = Lg;
}

__device__ __forceinline__ void block_merge_ml(float& m, float& l, float* bm, float* bl) {
  block_merge_ml_w<kStreamThreads / kWave>(m, l, bm, bl);
}

// One element of an online softmax: fold x into the running (m, l).  An
// element equal to -inf adds nothing; a NaN element turns l into NaN.
__device__ __forceinline__ void online_step(float x, float& m, float& l) {
  if (x > m) {
    l = (m == -__builtin_inff()) ? 1.0f : fmaf(l, exp2_denorm_safe((m - x) * kLog2e), 1.0f);
    m = x;
  } else if (x != -__builtin_inff()) {
    l += exp2_denorm_safe((x - m) * kLog2e);
  }
}

template <int W>
__device__ __forceinline__ float block_sum_stream(float v, float* buf) {
  v = wave_sum(v);
  lds_barrier();
  if ((threadIdx.x % kWave) == 0) buf[threadIdx.x / kWave] = v;
  lds_barrier();
  float s = buf[0];
#pragma unroll
  for (int k = 1; k < W; ++k) s += buf[k];
  return s;
}

}  // namespace vjp
