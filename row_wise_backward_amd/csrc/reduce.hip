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
//   d >= 2: workgroup b owns the 32 columns 32 b .. 32 b + 31 (one 128-byte
//   line of every partial row, so no line is read by two workgroups); its
//   1024 threads are 128 row lanes r times 8 column lanes c, and lane (r, c)
//   owns the four columns j = 32 b + 4 c + k, k = 0..3.  Each lane sums
//   P[r][j], P[r + 128][j], P[r + 256][j], ... in increasing t, starting from
//   0; the 128 row sums of a column are then combined by the pairwise tree
//   v[r] += v[r + s] for s = 64, 32, ..., 1.  The 16-byte and the element
//   load paths add the same values in the same order.
//
//   d = 1 (and the cross-entropy mean): one workgroup of 1024 threads;
//   thread r sums P[r], P[r + 1024], ... in increasing t, starting from 0;
//   each wave's 64 sums are combined by the DPP tree of wave_sum (neighbour
//   swap, pair swap, half-row mirror, row mirror, then rows (0 + 1) + (2 + 3));
//   the sixteen wave sums are added in wave order, ((w0 + w1) + w2) + ... .
//
// Stage 2 stays a kernel of its own.  Run by the last workgroup of stage 1
// instead (a device-scope counter finds it), it gives the same bits, but
// each stage-1 workgroup then needs a device-scope release before it counts,
// and on gfx950 that is an L2 write-back: the scaled-SiLU backward at 2^24
// fp16 elements (4096 workgroups) took 197 us with one wave per workgroup
// releasing and 618 us with every thread fencing, against 22.5 us for the
// stage-1 kernel plus this one.
#include "common.hpp"
#include "launch.hpp"

namespace vjp {

constexpr int kReduceThreads = 1024;
constexpr int kRowLanes = 128;
constexpr int kColLanes = kReduceThreads / kRowLanes;   // 8
constexpr int kColsPerBlock = 4 * kColLanes;            // 32

// VEC4: d % 4 == 0 and P 16-byte aligned, so a lane's four columns are one
// aligned 16-byte load (all four in range or none).
// Column j of the sum goes to out[j] for j < split and to out2[j - split]
// otherwise (two parameter gradients from one partials buffer).
template <bool VEC4>
__global__ __launch_bounds__(kReduceThreads) void reduce_partials_kernel(
    const float* __restrict__ P, int64_t T, int64_t d, float* __restrict__ out,
    float* __restrict__ out2, int64_t split, int accumulate) {
  __shared__ float4 red[kRowLanes][kColLanes];
  const int c = threadIdx.x % kColLanes;
  const int r = threadIdx.x / kColLanes;
  const int64_t j = int64_t(blockIdx.x) * kColsPerBlock + 4 * c;
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (VEC4) {
    if (j < d) {
#pragma unroll 8
      for (int64_t t = r; t < T; t += kRowLanes) {
        const float4 p = *reinterpret_cast<const float4*>(P + t * d + j);
        v.x += p.x;
        v.y += p.y;
        v.z += p.z;
        v.w += p.w;
      }
    }
  } else {
#pragma unroll 4
    for (int64_t t = r; t < T; t += kRowLanes) {
      const float* p = P + t * d + j;
      if (j < d) v.x += p[0];
      if (j + 1 < d) v.y += p[1];
      if (j + 2 < d) v.z += p[2];
      if (j + 3 < d) v.w += p[3];
    }
  }
  red[r][c] = v;
  __syncthreads();
#pragma unroll
  for (int s = kRowLanes / 2; s > 0; s >>= 1) {
    if (r < s) {
      float4 a = red[r][c];
      const float4 b = red[r + s][c];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
      red[r][c] = a;
    }
    __syncthreads();
  }
  if (r == 0) {
    const float4 s = red[0][c];
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (j + k < d) {
        float* o = j + k < split ? out + (j + k) : out2 + (j + k - split);
        *o = accumulate ? *o + sv[k] : sv[k];
      }
    }
  }
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
  return launch_reduce_partials_split(P, T, d, out, nullptr, d, accumulate, s);
}

hipError_t launch_reduce_partials_split(const float* P, int64_t T, int64_t d, float* out,
                                        float* out2, int64_t split, int accumulate,
                                        hipStream_t s) {
  if (d == 1 && split >= 1) {
    reduce_scalar_kernel<<<1, kScalarThreads, 0, s>>>(P, T, out, accumulate);
    return hipGetLastError();
  }
  const dim3 grid(unsigned((d + kColsPerBlock - 1) / kColsPerBlock)), block(kReduceThreads);
  const bool vec4 = d % 4 == 0 && reinterpret_cast<uintptr_t>(P) % 16 == 0;
  if (vec4)
    reduce_partials_kernel<true><<<grid, block, 0, s>>>(P, T, d, out, out2, split, accumulate);
  else
    reduce_partials_kernel<false><<<grid, block, 0, s>>>(P, T, d, out, out2, split, accumulate);
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
