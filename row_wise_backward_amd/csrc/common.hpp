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

template <typename T> inline constexpr bool is_bf16 = false;
template <> inline constexpr bool is_bf16<bf16> = true;

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

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x8_t __attribute__((ext_vector_type(8)));

// The vector of 32-bit words (or the one narrower word) with the bytes of a
// Vec<T, N>.
template <int kBytes> struct WordVec;
template <> struct WordVec<32> { using type = u32x8_t; };
template <> struct WordVec<16> { using type = u32x4_t; };
template <> struct WordVec<8> { using type = u32x2_t; };
template <> struct WordVec<4> { using type = unsigned; };
template <> struct WordVec<2> { using type = unsigned short; };
template <typename T, int N> using words_t = typename WordVec<sizeof(T) * N>::type;

// Streaming accesses: data read or written exactly once by the kernel are
// moved with the nontemporal hint, which on gfx950 lets a 128-bit load stream
// reach close to the HBM peak instead of being held in the caches.
template <typename T, int N>
__device__ __forceinline__ Vec<T, N> load_stream(const T* __restrict__ p) {
  constexpr int kBytes = sizeof(T) * N;
  if constexpr (kBytes == 16) {
    return __builtin_bit_cast(Vec<T, N>, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  } else if constexpr (kBytes == 8) {
    return __builtin_bit_cast(Vec<T, N>, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)));
  } else if constexpr (kBytes == 4) {
    return __builtin_bit_cast(Vec<T, N>, __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p)));
  } else {
    static_assert(kBytes == 2, "unsupported vector width");
    return __builtin_bit_cast(Vec<T, N>, __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p)));
  }
}

template <typename T, int N>
__device__ __forceinline__ void store_stream(T* __restrict__ p, const Vec<T, N>& v) {
  constexpr int kBytes = sizeof(T) * N;
  if constexpr (kBytes == 16) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
  } else if constexpr (kBytes == 8) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2_t, v), reinterpret_cast<u32x2_t*>(p));
  } else if constexpr (kBytes == 4) {
    __builtin_nontemporal_store(__builtin_bit_cast(unsigned, v), reinterpret_cast<unsigned*>(p));
  } else {
    static_assert(kBytes == 2, "unsupported vector width");
    __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, v), reinterpret_cast<unsigned short*>(p));
  }
}

template <typename T, int N>
__device__ __forceinline__ void load_f32(const T* __restrict__ p, float (&out)[N]) {
  const Vec<T, N> r = load_stream<T, N>(p);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = to_f32(r.v[i]);
}

template <typename T, int N>
__device__ __forceinline__ void store_f32(T* __restrict__ p, const float (&in)[N]) {
  Vec<T, N> r;
#pragma unroll
  for (int i = 0; i < N; ++i) r.v[i] = from_f32<T>(in[i]);
  store_stream<T, N>(p, r);
}

// Loads split in two so that several vectors of a lane are in flight at
// once.  issue_vec starts one streaming vector load of the N elements at p
// when all of them lie below `avail` elements from p, and otherwise leaves w
// as it is; fix_vec completes such a vector element by element (elements at
// or past avail read as `fill`; avail may be zero or negative).  A caller
// issues all of its vectors, fixes them, and only then views them as
// elements (as_vec).  Both steps work on whole 32-bit words for the sake of
// the code the compiler emits: where a value loaded in one arm of a branch
// merges with another, any work the merge needs on the loaded data (a copy,
// or the split of a word into 16-bit elements) waits for the load right
// where it is issued, and the loads of a lane then run one at a time.
template <typename T, int N>
__device__ __forceinline__ void issue_vec(const T* __restrict__ p, int64_t avail,
                                          words_t<T, N>& w) {
  if (avail >= N) w = __builtin_nontemporal_load(reinterpret_cast<const words_t<T, N>*>(p));
}

template <typename T, int N>
__device__ __forceinline__ void fix_vec(const T* __restrict__ p, int64_t avail, T fill,
                                        words_t<T, N>& w) {
  if (avail < N) {
    Vec<T, N> t;
#pragma unroll
    for (int i = 0; i < N; ++i) t.v[i] = (i < avail) ? p[i] : fill;
    w = __builtin_bit_cast(words_t<T, N>, t);
  }
}

template <typename T, int N>
__device__ __forceinline__ Vec<T, N> as_vec(const words_t<T, N>& w) {
  return __builtin_bit_cast(Vec<T, N>, w);
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

// Raw (storage-type) load of up to N elements: a streaming vector when all N
// lie below `avail`, else element by element with zeros past the end.
template <typename T, int N>
__device__ __forceinline__ Vec<T, N> load_raw_tail(const T* __restrict__ p, int64_t avail) {
  if (avail >= N) return load_stream<T, N>(p);
  Vec<T, N> r;
#pragma unroll
  for (int i = 0; i < N; ++i) r.v[i] = (i < avail) ? p[i] : T{};
  return r;
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
// Full-wave reductions on DPP.  Within each row of 16 lanes: swap neighbours
// (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), mirror the half-row,
// mirror the row -- after these four steps every lane of a row holds the row
// total, and because each step adds the same two operands on both sides the
// lanes of a row agree bitwise.  The four row totals are then read from lanes
// 0, 16, 32 and 48 and combined as (r0 + r1) + (r2 + r3), so every lane of the
// wave receives the same value in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppSwap1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppSwap1>(v);
  v += dpp_f32<kDppSwap2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppSwap1>(v));
  v = fmaxf(v, dpp_f32<kDppSwap2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppSwap1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppSwap2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// Sum within aligned groups of L consecutive lanes (L a power of two, 1..64,
// wave-uniform), on DPP: every lane of a group receives the group total, the
// same bitwise value across the group.  Groups of 32 and 64 combine the
// 16-lane row totals read from lanes 0 / 16 (and 32 / 48) in that order.
__device__ __forceinline__ float group_sum_dpp(float v, int L) {
  if (L >= 2) v += dpp_f32<kDppSwap1>(v);
  if (L >= 4) v += dpp_f32<kDppSwap2>(v);
  if (L >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if (L >= 16) v += dpp_f32<kDppMirror>(v);
  if (L >= 32) {
    const float a = readlane_f32(v, 0) + readlane_f32(v, 16);
    const float b = readlane_f32(v, 32) + readlane_f32(v, 48);
    v = L == 64 ? a + b : ((threadIdx.x & 32) ? b : a);
  }
  return v;
}

// Butterfly over lanes that differ in bits [LO, 64) (lanes sharing the low
// bits are combined): every lane ends with the same bitwise result.
template <int LO = 1>
__device__ __forceinline__ float wave_sum_from(float v) {
#pragma unroll
  for (int o = LO; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
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
// exp(x) as 2^(x * log2 e) on the hardware exp2.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid(x) as s * k, evaluated without overflow and without flushing
// results below 2^-126 (x < -87.3, where sigmoid(x) is an fp32 subnormal
// that bf16 and fp32 outputs such as w x sigmoid(x) can still hold).  With
// e = 2^(-|x| log2 e) = exp(-|x|) <= 1: sigmoid(x) = 1 / (1 + e) for x >= 0
// and e / (1 + e) for x < 0, so neither form can overflow.  Where e itself
// would be subnormal (x < 0 only), it is formed as 2^(t + 64) and k = 2^-64
// carries the scale: products formed from s stay normal and round once when
// finally multiplied by k.  k = 1 elsewhere (a multiply by k is then exact).
struct ScaledSigmoid {
  float s;
  float k;
};

__device__ __forceinline__ ScaledSigmoid sigmoid_scaled(float x) {
  const float t = -__builtin_fabsf(x) * kLog2e;
  const bool tiny = x < 0.0f && t < -126.0f;
  const float e = exp2_fast(tiny ? t + 64.0f : t);
  const float r = rcp_fast(1.0f + (tiny ? 0.0f : e));
  return {x >= 0.0f ? r : e * r, tiny ? 5.421010862427522e-20f /* 2^-64 */ : 1.0f};
}

// The sigmoid a kernel with storage type T needs.  fp16 values and results
// are zero below 2^-24 in magnitude: where 1 / (1 + 2^(-x log2 e)) underflows
// or overflows (x < -87), every fp16 result formed from it (w x s, dy w s
// (1 + x (1 - s))) is +-0 either way, so the two-operation form serves, with
// k = 1.  bf16 and fp32 results reach down to 2^-133 and 2^-149 and take the
// scaled form.
template <typename T>
__device__ __forceinline__ ScaledSigmoid sigmoid_for(float x) {
  if constexpr (sizeof(T) == 2 && !is_bf16<T>) {
    return {rcp_fast(1.0f + exp2_fast(-x * kLog2e)), 1.0f};
  } else {
    return sigmoid_scaled(x);
  }
}

// Workgroups of a launch are dispatched to the 8 XCDs (accelerator dies,
// each with its own L2) round-robin: workgroup b runs on XCD b % 8.
// xcd_group(b, count) renumbers [0, count) so that consecutive numbers run on
// one XCD (XCD k takes the k-th eighth of them): work items that share cache
// lines then share one L2 instead of fetching the lines once per XCD.  The
// last count % 8 numbers map to themselves.
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t xcd_group(int64_t b, int64_t count) {
  const int64_t full = count / kXcds * kXcds;
  if (b >= full) return b;
  return (b % kXcds) * (full / kXcds) + b / kXcds;
}

// blockIdx.x renumbered by xcd_group over the grid's x extent: the row a
// workgroup takes in the cross-entropy kernels, so that each XCD works
// through one contiguous band of rows (16384 x 32000 bf16, fused forward +
// backward, bitwise the same results: 339 us against 357-362 us in one
// process, median of 20 flushed runs).  Not used elsewhere: the same
// renumbering made the forward kernels slower (scaled SiLU 11.4 -> 14.0 us,
// LayerNorm 90.5 -> 104.6 us, row gather 45.3 -> 52.9 us, weighted sum and
// softmax +4-5%) and left the other backward kernels within 1%.
__device__ __forceinline__ int64_t xcd_block_x() { return xcd_group(blockIdx.x, gridDim.x); }

// Workgroup barrier that orders LDS accesses only.  The kernels exchange only
// LDS data across their barriers, so global loads (a prefetched next row) and
// stores (the previous row's output) issued before it stay in flight instead
// of being drained as a full __syncthreads() would.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One element of a parameter vector stored as fp32, fp16 or bf16 (dt is the
// library's dtype code: 0 fp32, 1 fp16, 2 bf16), widened to fp32.
__device__ __forceinline__ float load_param_f32(const void* __restrict__ w, int64_t j, int dt) {
  if (dt == 0) return static_cast<const float*>(w)[j];
  if (dt == 1) return to_f32(static_cast<const _Float16*>(w)[j]);
  return to_f32(static_cast<const bf16*>(w)[j]);
}

}  // namespace vjp
