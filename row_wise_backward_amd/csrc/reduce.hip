// Stage 2 of the two-stage parameter-gradient reduction, and the
// cross-entropy mean.
//
// "Writing Triton Kernels with Autograd: A Minimal End-to-End Example",
// section 3: each program of the backward writes one partial row per tile of
// rows; a second reduction over the tiles gives grad_w.  "Backward in Triton
// -- autograd.Function and the backward grid", section "The backward grid is
// not the forward grid": a partials buffer reduced in a second pass is the
// deterministic choice.  Here the second pass is a HIP kernel with a fixed
// summation order, so the result does not depend on scheduling:
//
//   d >= 2: CL = min(16, next_pow2(d)) column lanes, RL = 1024 / CL row
//   lanes; thread (r, c) of block b owns column j = b * CL + c and sums
//   P[r][j], P[r + RL][j], P[r + 2 RL][j], ... in increasing t, starting
//   from 0; the RL per-thread sums are then combined by the pairwise tree
//   v[r] += v[r + s] for s = RL / 2, RL / 4, ..., 1.
//
//   d = 1 (and the cross-entropy mean): one workgroup of 1024 threads;
//   thread r sums P[r], P[r + 1024], ... in increasing t, starting from 0;
//   each wave's 64 sums are combined by the DPP tree of wave_sum (neighbour
//   swap, pair swap, half-row mirror, row mirror, then rows (0 + 1) + (2 + 3));
//   the sixteen wave sums are added in wave order, ((w0 + w1) + w2) + ... .
#include "common.hpp"
#include "launch.hpp"

namespace vjp {

constexpr int kReduceThreads = 1024;

template <int CL>
__global__ __launch_bounds__(kReduceThreads) void reduce_partials_kernel(
    const float* __restrict__ P, int64_t T, int64_t d, float* __restrict__ out, int accumulate) {
  constexpr int RL = kReduceThreads / CL;
  __shared__ float red[kReduceThreads];
  const int c = threadIdx.x % CL;
  const int r = threadIdx.x / CL;
  const int64_t j = int64_t(blockIdx.x) * CL + c;
  float v = 0.0f;
  if (j < d) {
#pragma unroll 8
    for (int64_t t = r; t < T; t += RL) v += P[t * d + j];
  }
  red[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int s = RL / 2; s > 0; s >>= 1) {
    if (r < s) red[r * CL + c] += red[(r + s) * CL + c];
    __syncthreads();
  }
  if (r == 0 && j < d) out[j] = accumulate ? out[j] + red[c] : red[c];
}

constexpr int kScalarThreads = 1024;
constexpr int kScalarWaves = kScalarThreads / kWave;

__global__ __launch_bounds__(kScalarThreads) void reduce_scalar_kernel(
    const float* __restrict__ P, int64_t T, float* __restrict__ out, int accumulate) {
  __shared__ float red[kScalarWaves];
  float v = 0.0f;
#pragma unroll 8
  for (int64_t t = threadIdx.x; t < T; t += kScalarThreads) v += P[t];
  v = wave_sum(v);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = red[0];
#pragma unroll
    for (int k = 1; k < kScalarWaves; ++k) s += red[k];
    *out = accumulate ? *out + s : s;
  }
}

hipError_t launch_reduce_partials(const float* P, int64_t T, int64_t d, float* out,
                                  int accumulate, hipStream_t s) {
  if (d == 1) {
    reduce_scalar_kernel<<<1, kScalarThreads, 0, s>>>(P, T, out, accumulate);
    return hipGetLastError();
  }
  int cl = 1;
  while (cl < d && cl < 16) cl <<= 1;
  const dim3 grid(unsigned((d + cl - 1) / cl)), block(kReduceThreads);
  switch (cl) {
    case 1: reduce_partials_kernel<1><<<grid, block, 0, s>>>(P, T, d, out, accumulate); break;
    case 2: reduce_partials_kernel<2><<<grid, block, 0, s>>>(P, T, d, out, accumulate); break;
    case 4: reduce_partials_kernel<4><<<grid, block, 0, s>>>(P, T, d, out, accumulate); break;
    case 8: reduce_partials_kernel<8><<<grid, block, 0, s>>>(P, T, d, out, accumulate); break;
    default: reduce_partials_kernel<16><<<grid, block, 0, s>>>(P, T, d, out, accumulate); break;
  }
  return hipGetLastError();
}

// Mean cross-entropy over rows: the row losses are summed in the same fixed
// order as the d = 1 reduction above (1024 threads, DPP wave tree, waves
// in order) and the sum is divided by rows.  Targets outside [0, classes) are
// counted exactly in integers.
__global__ __launch_bounds__(kScalarThreads) void xent_finalize_kernel(
    const float* __restrict__ row_loss, const int32_t* __restrict__ targets, int64_t rows,
    int64_t classes, float* __restrict__ loss, int32_t* __restrict__ n_invalid) {
  __shared__ float red[kScalarWaves];
  __shared__ int cnt[kScalarWaves];
  float v = 0.0f;
  int bad = 0;
#pragma unroll 4
  for (int64_t t = threadIdx.x; t < rows; t += kScalarThreads) {
    v += row_loss[t];
    const int32_t tg = targets[t];
    bad += (tg < 0 || int64_t(tg) >= classes) ? 1 : 0;
  }
  v = wave_sum(v);
  bad = wave_sum_i32(bad);
  if (threadIdx.x % kWave == 0) {
    red[threadIdx.x / kWave] = v;
    cnt[threadIdx.x / kWave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = red[0];
    int c = cnt[0];
#pragma unroll
    for (int k = 1; k < kScalarWaves; ++k) {
      s += red[k];
      c += cnt[k];
    }
    *loss = rows > 0 ? s / float(rows) : __builtin_nanf("");
    if (n_invalid) *n_invalid = c;
  }
}

hipError_t launch_xent_finalize(const float* row_loss, const int32_t* targets, int64_t rows,
                                int64_t classes, float* loss, int32_t* n_invalid,
                                hipStream_t s) {
  xent_finalize_kernel<<<1, kScalarThreads, 0, s>>>(row_loss, targets, rows, classes, loss,
                                                    n_invalid);
  return hipGetLastError();
}

}  // namespace vjp
