// A plain streaming device copy: the measurement reference for the row
// kernels.  Every op here reads and writes each byte once at most, so a copy
// of as many bytes as an op moves, timed in the same process, is the rate
// its kernel can approach on the chip it runs on (the published 8 TB/s is
// not reached by any access pattern).
//
// 16-byte nontemporal loads and stores, U vectors in flight per lane, a grid
// of at most G workgroups that loops over the data; the full groups of U
// vectors are copied without per-access bounds checks so that a lane's loads
// are all in flight together.  Unaligned pointers and the tail below 16
// bytes take a byte loop.  vjp_copy uses U = 4 and G = 32768: the fastest
// shape measured on MI355X for copies of 0.5 to 1 GB (rocprofv3 kernel
// trace, median of 20 flushed runs: 6.2-6.3 TB/s against 5.95-6.0 TB/s for
// G = 8192); vjp_copy_shaped takes both as arguments, for sweeps.
#include "common.hpp"
#include "launch.hpp"

namespace vjp {

namespace {

constexpr int kCopyThreads = 256;

template <int U>
__global__ __launch_bounds__(kCopyThreads) void copy_vec16(const u32x4_t* __restrict__ src,
                                                           u32x4_t* __restrict__ dst,
                                                           int64_t n16) {
  constexpr int64_t kGroup = int64_t(kCopyThreads) * U;
  const int64_t stride = int64_t(gridDim.x) * kGroup;
  int64_t base = int64_t(blockIdx.x) * kGroup;
  for (; base + kGroup <= n16; base += stride) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_nontemporal_load(src + base + u * kCopyThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u)
      __builtin_nontemporal_store(v[u], dst + base + u * kCopyThreads + threadIdx.x);
  }
  if (base < n16) {   // the last, partial group (one workgroup)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = base + u * kCopyThreads + threadIdx.x;
      if (j < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + j), dst + j);
    }
  }
}

__global__ __launch_bounds__(kCopyThreads) void copy_bytes(const uint8_t* __restrict__ src,
                                                           uint8_t* __restrict__ dst, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * kCopyThreads + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * kCopyThreads)
    dst[i] = src[i];
}

unsigned grid_for(int64_t units, int64_t per_group, int64_t max_groups) {
  const int64_t g = (units + per_group - 1) / per_group;
  return unsigned(g < 1 ? 1 : (g < max_groups ? g : max_groups));
}

template <int U>
void launch_vec16(const uint8_t* a, uint8_t* b, int64_t n16, int64_t max_groups, hipStream_t s) {
  copy_vec16<U><<<grid_for(n16, int64_t(kCopyThreads) * U, max_groups), kCopyThreads, 0, s>>>(
      reinterpret_cast<const u32x4_t*>(a), reinterpret_cast<u32x4_t*>(b), n16);
}

}  // namespace

hipError_t launch_copy_shaped(const void* src, void* dst, int64_t bytes, int vectors_per_lane,
                              int64_t max_groups, hipStream_t s) {
  const uint8_t* a = static_cast<const uint8_t*>(src);
  uint8_t* b = static_cast<uint8_t*>(dst);
  int64_t done = 0;
  if (reinterpret_cast<uintptr_t>(a) % 16 == 0 && reinterpret_cast<uintptr_t>(b) % 16 == 0) {
    const int64_t n16 = bytes / 16;
    if (n16 > 0) {
      switch (vectors_per_lane) {
        case 1: launch_vec16<1>(a, b, n16, max_groups, s); break;
        case 2: launch_vec16<2>(a, b, n16, max_groups, s); break;
        case 8: launch_vec16<8>(a, b, n16, max_groups, s); break;
        default: launch_vec16<4>(a, b, n16, max_groups, s); break;
      }
    }
    done = n16 * 16;
  }
  if (bytes > done)
    copy_bytes<<<grid_for(bytes - done, kCopyThreads, 8192), kCopyThreads, 0, s>>>(
        a + done, b + done, bytes - done);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  return launch_copy_shaped(src, dst, bytes, 4, 32768, s);
}

}  // namespace vjp
