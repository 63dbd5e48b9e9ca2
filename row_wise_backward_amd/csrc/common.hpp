// Device-side building blocks shared by the libvjp kernels (gfx950, wave64).
//
// Storage types: float (fp32), _Float16 (fp16), bf16 (raw 16-bit pattern).
// Everything is computed in fp32; conversions to 16-bit storage round to
// nearest even (v_cvt_pk_bf16_f32 for bf16, v_cvt_f16_f32 for fp16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vjp {

constexpr int kWave = 64;

struct bf16 {
  uint16_t bits;
};

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float(uint32_t(v.bits) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) {
  return static_cast<_Float16>(v);
}
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return bf16{__builtin_bit_cast(uint16_t, static_cast<__bf16>(v))};
}

// ------------------------------------------------------------------ vector memory
// N consecutive elements moved as one access (16 bytes -> one 128-bit load).
template <typename T, int N> struct alignas(sizeof(T) * N) Vec {
  T v[N];
};

template <typename T, int N>
__device__ __forceinline__ void load_f32(const T* __restrict__ p, float (&out)[N]) {
  Vec<T, N> r = *reinterpret_cast<const Vec<T, N>*>(p);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = to_f32(r.v[i]);
}

template <typename T, int N>
__device__ __forceinline__ void store_f32(T* __restrict__ p, const float (&in)[N]) {
  Vec<T, N> r;
#pragma unroll
  for (int i = 0; i < N; ++i) r.v[i] = from_f32<T>(in[i]);
  *reinterpret_cast<Vec<T, N>*>(p) = r;
}

// Guarded variants for the ragged end of a row or array: a full vector when
// all N elements lie below `limit` elements from p, else element by element.
template <typename T, int N>
__device__ __forceinline__ void load_f32_tail(const T* __restrict__ p, int64_t avail,
                                              float fill, float (&out)[N]) {
  if (avail >= N) {
    load_f32<T, N>(p, out);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = (i < avail) ? to_f32(p[i]) : fill;
  }
}

template <typename T, int N>
__device__ __forceinline__ void store_f32_tail(T* __restrict__ p, int64_t avail,
                                               const float (&in)[N]) {
  if (avail >= N) {
    store_f32<T, N>(p, in);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i < avail) p[i] = from_f32<T>(in[i]);
  }
}

// ------------------------------------------------------------------ wave reductions
// Butterfly over lanes that differ in bits [lo, 64): every lane ends with the
// same bitwise result (each step adds the same two operands on both sides).
template <int LO = 1>
__device__ __forceinline__ float wave_sum_from(float v) {
#pragma unroll
  for (int o = LO; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return wave_sum_from<1>(v); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum within aligned groups of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ------------------------------------------------------------------ math
// exp(x) as 2^(x * log2 e) on the hardware exp2; sigmoid as 1 / (1 + e^-x).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float sigmoid(float x) {
  return rcp_fast(1.0f + exp2_fast(-x * kLog2e));
}

}  // namespace vjp
