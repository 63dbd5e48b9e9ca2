// Fused scaled-SiLU y = w * x * sigmoid(x): forward and stage-1 backward.
//
// Source: "Backward in Triton -- autograd.Function and the backward grid",
// section "A complete minimal example -- fused scaled-SiLU, end to end"
// (fp32 compute; dx = dy * w * (s + silu (1 - s)); dw = sum dy * silu, a
// scalar reduced over every element) and section "Save vs recompute -- the
// decision at the Triton level" (the backward reads x and recomputes
// s = sigmoid(x) instead of reading a saved s).  The page combines per-block
// dw partials with one float atomic per block; here each tile writes its
// fp32 partial to P[t] and the fixed-order stage-2 kernel sums them.
//
// gfx950 mapping: flat elementwise stream, 16-byte accesses (8 x fp16/bf16,
// 4 x fp32) per lane, 256-thread workgroups, kUnroll vectors per lane
// issued before any is used.  sigmoid(x) from e = 2^(-|x| log2 e) on v_exp_f32
// and v_rcp_f32 (both accurate to about 1 ulp in fp32): 1 / (1 + e) for
// x >= 0, e / (1 + e) for x < 0, so nothing overflows, with a 2^64 scale
// carried through where sigmoid(x) is an fp32 subnormal (fp16 storage, whose
// results there are +-0, takes 1 / (1 + 2^(-x log2 e))).  The scalar w is read
// from device memory by every workgroup (no host synchronisation).
#include "common.hpp"
#include "launch.hpp"

namespace vjp {

namespace {

constexpr int kThreads = 256;

template <typename T, int VEC, int kUnroll>
__global__ __launch_bounds__(kThreads) void silu_fwd_kernel(const T* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            T* __restrict__ y, int64_t n,
                                                            int64_t elems_per_block) {
  const float wv = *w;
  const int64_t beg = int64_t(blockIdx.x) * elems_per_block;
  const int64_t end = min(beg + elems_per_block, n);
  const int64_t stride = int64_t(kThreads) * VEC;
  for (int64_t base = beg + int64_t(threadIdx.x) * VEC; base < end; base += kUnroll * stride) {
    // All kUnroll loads in flight before the first is used.
    words_t<T, VEC> xw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) issue_vec<T, VEC>(x + base + u * stride, end - base - u * stride, xw[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      fix_vec<T, VEC>(x + base + u * stride, end - base - u * stride, T{}, xw[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i0 = base + u * stride;
      if (i0 < end) {
        const Vec<T, VEC> xv = as_vec<T, VEC>(xw[u]);
        float yv[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float xf = to_f32(xv.v[i]);
          const ScaledSigmoid sg = sigmoid_for<T>(xf);
          yv[i] = (wv * xf * sg.s) * sg.k;
        }
        store_f32_tail<T, VEC>(y + i0, end - i0, yv);
      }
    }
  }
}

template <typename T, int VEC, int kUnroll>
__global__ __launch_bounds__(kThreads) void silu_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ x, const float* __restrict__ w,
    T* __restrict__ dx, float* __restrict__ P, int64_t n, int64_t elems_per_tile) {
  __shared__ float red[kThreads / kWave];
  const float wv = *w;
  const int64_t tile = blockIdx.x;
  const int64_t beg = tile * elems_per_tile;
  const int64_t end = min(beg + elems_per_tile, n);
  const int64_t stride = int64_t(kThreads) * VEC;
  float acc = 0.0f;
  for (int64_t base = beg + int64_t(threadIdx.x) * VEC; base < end; base += kUnroll * stride) {
    // All loads of the step in flight before the first is used; elements past
    // the end read as zeros (they add nothing to the partial).
    words_t<T, VEC> xw[kUnroll], gw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t left = end - base - u * stride;
      issue_vec<T, VEC>(x + base + u * stride, left, xw[u]);
      issue_vec<T, VEC>(dy + base + u * stride, left, gw[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t left = end - base - u * stride;
      fix_vec<T, VEC>(x + base + u * stride, left, T{}, xw[u]);
      fix_vec<T, VEC>(dy + base + u * stride, left, T{}, gw[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i0 = base + u * stride;
      const Vec<T, VEC> xv = as_vec<T, VEC>(xw[u]), gv = as_vec<T, VEC>(gw[u]);
      float dxv[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float xf = to_f32(xv.v[i]), gf = to_f32(gv.v[i]);
        // s = sg.s * sg.k; silu = x s.  Where k < 1, s < 2^-126 so 1 - s
        // rounds to 1 and dx is formed from the scaled s and scaled back once.
        const ScaledSigmoid sg = sigmoid_for<T>(xf);
        const float silu = xf * sg.s;
        dxv[i] = (gf * wv * fmaf(silu, 1.0f - sg.s * sg.k, sg.s)) * sg.k;
        acc = fmaf(gf, silu * sg.k, acc);
      }
      if (i0 < end) store_f32_tail<T, VEC>(dx + i0, end - i0, dxv);
    }
  }
  acc = wave_sum(acc);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = acc;
  lds_barrier();
  if (threadIdx.x == 0) {
    float s = red[0];
#pragma unroll
    for (int k = 1; k < kThreads / kWave; ++k) s += red[k];
    P[tile] = s;
  }
}

// Vectors per thread and step, every load of a step in flight together
// (measured on MI355X for n = 2^24 fp16, HIP events: forward 8 vectors
// 14.1-14.3 us, 4 vectors 15.4-15.9 us; backward over tiles of 4096
// elements, 2 vectors 20.5-20.8 us, 1 vector 21.3-21.7 us).  Under a
// cache-flushed median the backward kept the same order: tiles of 4096
// elements with 2 vectors 18.2 us, 1 vector 19.5 us; tiles of 8192 or 16384
// elements with 2 to 8 vectors 18.7-20.2 us; tiles of 2048 with 1 vector 18.2.
// Workgroup sizes (one process, flushed medians): the forward 12.8 us with
// 256 threads against 12.9 / 13.5 / 14.7 us with 128 / 512 / 1024 (each over
// 16384 elements); the backward 18.2 us against 18.4 / 19.0 / 20.7 us with
// 512 / 128 / 64 threads over the same 4096-element tiles, 19.6 us with 1024
// threads over tiles of 8192.
constexpr int kFwdUnroll = 8;
constexpr int kBwdUnroll = 2;

// Elements per forward launch (a multiple of every elements-per-workgroup
// value, so chunks keep the 16-byte alignment of vectorised pointers).
constexpr int64_t kFwdLaunchElems = int64_t(1) << 30;

template <typename T>
hipError_t fwd_typed(const void* x, const float* w, void* y, int64_t n, bool vec,
                     hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  const int64_t epb = int64_t(kThreads) * (vec ? V : 1) * kFwdUnroll;
  for (int64_t off = 0; off < n; off += kFwdLaunchElems) {
    const int64_t m = n - off < kFwdLaunchElems ? n - off : kFwdLaunchElems;
    const dim3 grid(unsigned((m + epb - 1) / epb));
    const T* xp = static_cast<const T*>(x) + off;
    T* yp = static_cast<T*>(y) + off;
    if (vec)
      silu_fwd_kernel<T, V, kFwdUnroll><<<grid, kThreads, 0, s>>>(xp, w, yp, m, epb);
    else
      silu_fwd_kernel<T, 1, kFwdUnroll><<<grid, kThreads, 0, s>>>(xp, w, yp, m, epb);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_typed(const void* dy, const void* x, const float* w, void* dx, float* P,
                     int64_t n, int64_t ept, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  const dim3 grid(unsigned((n + ept - 1) / ept));
  if (vec)
    silu_bwd_kernel<T, V, kBwdUnroll><<<grid, kThreads, 0, s>>>(static_cast<const T*>(dy),
                                                    static_cast<const T*>(x), w,
                                                    static_cast<T*>(dx), P, n, ept);
  else
    silu_bwd_kernel<T, 1, kBwdUnroll><<<grid, kThreads, 0, s>>>(static_cast<const T*>(dy),
                                                    static_cast<const T*>(x), w,
                                                    static_cast<T*>(dx), P, n, ept);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scaled_silu_fwd(const void* x, const float* w, void* y, int64_t n, int act,
                                  bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return fwd_typed<float>(x, w, y, n, vec, s);
    case kF16: return fwd_typed<_Float16>(x, w, y, n, vec, s);
    default: return fwd_typed<bf16>(x, w, y, n, vec, s);
  }
}

hipError_t launch_scaled_silu_bwd_stage1(const void* dy, const void* x, const float* w,
                                         void* dx, float* P, int64_t n, int64_t elems_per_tile,
                                         int act, bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return bwd_typed<float>(dy, x, w, dx, P, n, elems_per_tile, vec, s);
    case kF16: return bwd_typed<_Float16>(dy, x, w, dx, P, n, elems_per_tile, vec, s);
    default: return bwd_typed<bf16>(dy, x, w, dx, P, n, elems_per_tile, vec, s);
  }
}

}  // namespace vjp
