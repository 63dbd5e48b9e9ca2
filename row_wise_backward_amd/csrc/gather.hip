// Row gather (embedding lookup) and its backward, a deterministic scatter-add.
//
// Source: "Backprop for kernel writers", section 06 "Top-k & routing": a
// selection y_m = x[i_m] sends gradient only to the selected rows, so the
// backward is the scatter-add  xbar_j = sum over m with i_m = j of ybar_m;
// with repeated indices every duplicate must be summed, and atomic adds make
// the result depend on scheduling.  Section 04 "The duality": a value read by
// many outputs sums their gradients.
//
// Deterministic scatter-add without float atomics:
//   1. a stable LSD radix sort of the indices (8-bit digits, as many passes
//      as the index range needs), carrying the position m; an index outside
//      [0, V) gets the key V and sorts after every valid one;
//   2. the bounds [begin, end) of each table row's run in the sorted order;
//   3. runs longer than kRun positions are cut into consecutive chunks of
//      kRun positions; one workgroup per (chunk, column block) sums its dy
//      rows in sorted order into an fp32 partial row (so a row selected
//      thousands of times is summed by many workgroups at once);
//   4. one workgroup per (table row, column block) writes (or adds into) the
//      fp32 gradient row: a run of at most kRun positions is summed directly
//      from dy in sorted order, a longer one as the in-order sum of its chunk
//      partials; rows never selected get zeros (or stay unchanged).
// The sorted order is unique (equal keys keep increasing m), so every
// summation order, hence every result bit, is fixed by the input.
//
// Radix pass (blocks of 1024 keys, 256 threads): the upsweep counts each
// block's digits (integer LDS atomics: exact); one workgroup scans the
// digit-major table hist[digit][block]; the downsweep places the keys of a
// block in four rounds of 256 (thread order within a round, rounds in
// order), ranking equal digits within a wave with eight ballots and across
// waves and rounds with counts in LDS.
#include "launch.hpp"
#include "common.hpp"

namespace vjp {

namespace {

constexpr int kSortThreads = 256;
constexpr int kSortRounds = 4;
constexpr int kSortBlock = kSortThreads * kSortRounds;   // keys per block
constexpr int kDigits = 256;
constexpr int kSortWaves = kSortThreads / kWave;

__device__ __forceinline__ int32_t key_of(const int32_t* __restrict__ idx, int64_t m, int64_t V) {
  const int32_t v = idx[m];
  return (v >= 0 && int64_t(v) < V) ? v : int32_t(V);
}

// Pass input: the raw indices (first pass, position = m) or the previous
// pass's keys / positions.
__global__ __launch_bounds__(kSortThreads) void radix_upsweep(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ keys_in, int64_t M, int64_t V,
    int shift, int32_t* __restrict__ hist, int64_t nblocks) {
  __shared__ int cnt[kDigits];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    const int64_t j = b * kSortBlock + r * kSortThreads + threadIdx.x;
    if (j < M) {
      const int32_t k = keys_in ? keys_in[j] : key_of(idx, j, V);
      atomicAdd(&cnt[(uint32_t(k) >> shift) & (kDigits - 1)], 1);
    }
  }
  __syncthreads();
  hist[int64_t(threadIdx.x) * nblocks + b] = cnt[threadIdx.x];
}

// Exclusive scan of n integers in place, one workgroup of 1024 threads:
// thread t owns the contiguous chunk [t c, (t + 1) c).
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_exclusive(int32_t* __restrict__ a,
                                                               int64_t n) {
  __shared__ int32_t part[kScanThreads];
  const int64_t c = (n + kScanThreads - 1) / kScanThreads;
  const int64_t lo = int64_t(threadIdx.x) * c;
  const int64_t hi = lo + c < n ? lo + c : n;
  int32_t s = 0;
#pragma unroll 8
  for (int64_t i = lo; i < hi; ++i) s += a[i];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan of the chunk sums.
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int32_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0;
#pragma unroll 8
  for (int64_t i = lo; i < hi; ++i) {
    const int32_t v = a[i];
    a[i] = run;
    run += v;
  }
}

__global__ __launch_bounds__(kSortThreads) void radix_downsweep(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ keys_in,
    const int32_t* __restrict__ vals_in, int64_t M, int64_t V, int shift,
    const int32_t* __restrict__ offs, int64_t nblocks, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ vals_out) {
  __shared__ int32_t base[kDigits];
  __shared__ int32_t wave_cnt[kSortWaves][kDigits];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.x;
  base[threadIdx.x] = offs[int64_t(threadIdx.x) * nblocks + b];   // running start of each digit
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int r = 0; r < kSortRounds; ++r) {
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) wave_cnt[w][threadIdx.x] = 0;
    __syncthreads();
    const int64_t j = b * kSortBlock + r * kSortThreads + threadIdx.x;
    const bool in = j < M;
    int32_t k = 0, v = 0;
    if (in) {
      k = keys_in ? keys_in[j] : key_of(idx, j, V);
      v = vals_in ? vals_in[j] : int32_t(j);
    }
    // Lanes past the end carry digit 256 (bit 8), which matches no real digit.
    const int d = in ? int((uint32_t(k) >> shift) & (kDigits - 1)) : kDigits;
    uint64_t same = ~uint64_t(0);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      const bool on = (d >> bit) & 1;
      const uint64_t m = __ballot(on);
      same &= on ? m : ~m;
    }
    const int rank = __popcll(same & below);
    if (in && rank == 0) wave_cnt[wave][d] = __popcll(same);
    __syncthreads();
    if (in) {
      int32_t pre = base[d];
      for (int w = 0; w < wave; ++w) pre += wave_cnt[w][d];
      const int32_t pos = pre + rank;
      keys_out[pos] = k;
      vals_out[pos] = v;
    }
    __syncthreads();
    int32_t add = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) add += wave_cnt[w][threadIdx.x];
    base[threadIdx.x] += add;
    __syncthreads();
  }
}

// seg_begin / seg_end (V + 1 entries each) and *n_invalid were zero-filled;
// position j opens a run where the key changes and closes one before a
// change.  The run of key V (invalid indices) runs to the end: its start
// gives the invalid count.
__global__ __launch_bounds__(256) void segment_bounds(const int32_t* __restrict__ keys,
                                                      int64_t M, int64_t V,
                                                      int32_t* __restrict__ seg_begin,
                                                      int32_t* __restrict__ seg_end,
                                                      int32_t* __restrict__ n_invalid) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= M) return;
  const int32_t k = keys[j];
  const bool first = j == 0 || keys[j - 1] != k;
  if (first) seg_begin[k] = int32_t(j);
  if (j == M - 1 || keys[j + 1] != k) seg_end[k] = int32_t(j + 1);
  if (first && int64_t(k) == V && n_invalid != nullptr) *n_invalid = int32_t(M - j);
}

// Runs of at most kRun sorted positions are summed directly; longer runs in
// chunks of kRun positions.  Every long run has more than kRun positions, so
// it has fewer than len / 16 chunks, and all chunks together fewer than M / 16.
// (Measured on MI355X for 16384 Zipf ids into 32000 x 4096: 32-position runs
// 218 us for the whole backward; 64-position runs with the chunk counts
// folded into a strided scan, 330 us.)
constexpr int kRun = 32;

// acc[i] += dy[pos[j], col + i] for j = j0 .. j1 - 1 in order, U rows in flight.
template <typename T, int VEC, int U>
__device__ __forceinline__ void sum_dy_rows(const T* __restrict__ dy, int64_t ld_dy,
                                            const int32_t* __restrict__ pos, int32_t j0,
                                            int32_t j1, int64_t col, int64_t left,
                                            float (&acc)[VEC]) {
  for (int32_t j = j0; j < j1; j += U) {
    float r[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < j1 && left > 0) {
        load_f32_tail<T, VEC>(dy + int64_t(pos[j + u]) * ld_dy + col, left, 0.0f, r[u]);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) r[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += r[u][i];
  }
}

// n_chunks[v] = number of kRun-position chunks of a long run (0 for a short
// one); scanned afterwards into chunk offsets.
__global__ __launch_bounds__(256) void count_chunks(const int32_t* __restrict__ seg_begin,
                                                    const int32_t* __restrict__ seg_end,
                                                    int64_t V, int32_t* __restrict__ n_chunks) {
  const int64_t v = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v > V) return;
  const int32_t len = v < V ? seg_end[v] - seg_begin[v] : 0;
  n_chunks[v] = len > kRun ? (len + kRun - 1) / kRun : 0;
}

// owner[q] = the table row whose run chunk q belongs to.
__global__ __launch_bounds__(256) void chunk_owners(const int32_t* __restrict__ chunk_off,
                                                    int64_t V, int32_t* __restrict__ owner) {
  const int64_t v = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= V) return;
  for (int32_t q = chunk_off[v]; q < chunk_off[v + 1]; ++q) owner[q] = int32_t(v);
}

// Stage A: workgroup (q, c) sums chunk q of a long run into Q[q][chunk c].
template <typename T, int VEC, int U>
__global__ __launch_bounds__(kSortThreads) void chunk_sums(
    const T* __restrict__ dy, int64_t ld_dy, const int32_t* __restrict__ sorted_pos,
    const int32_t* __restrict__ seg_begin, const int32_t* __restrict__ seg_end,
    const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ owner, int64_t V,
    int64_t D, float* __restrict__ Q, int64_t ldq) {
  const int64_t q = blockIdx.x;
  if (q >= chunk_off[V]) return;   // the grid is an upper bound on the chunk count
  const int32_t v = owner[q];
  const int32_t j0 = seg_begin[v] + int32_t(q - chunk_off[v]) * kRun;
  const int32_t j1 = min(j0 + kRun, seg_end[v]);
  const int64_t col = int64_t(blockIdx.y) * kSortThreads * VEC + int64_t(threadIdx.x) * VEC;
  const int64_t left = D - col;
  if (left <= 0) return;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
  sum_dy_rows<T, VEC, U>(dy, ld_dy, sorted_pos, j0, j1, col, left, acc);
  float* out = Q + q * ldq + col;   // rows of ldq (a multiple of 4) floats, 16-byte aligned
  if (left >= VEC && VEC % 4 == 0) {
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
      Vec<float, 4> o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o.v[k] = acc[i + k];
      *reinterpret_cast<Vec<float, 4>*>(out + i) = o;
    }
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      if (i < left) out[i] = acc[i];
  }
}

// Stage B: workgroup (v, c) forms the gradient of table row v for chunk c of
// the columns and writes (or adds into) it.  PVEC: the gradient rows are
// 16-byte aligned, so each lane's VEC fp32 values go out as 16-byte stores.
template <typename T, int VEC, int U, bool PVEC>
__global__ __launch_bounds__(kSortThreads) void scatter_add_rows(
    const T* __restrict__ dy, int64_t ld_dy, const int32_t* __restrict__ sorted_pos,
    const int32_t* __restrict__ seg_begin, const int32_t* __restrict__ seg_end,
    const int32_t* __restrict__ chunk_off, const float* __restrict__ Q, int64_t ldq, int64_t D,
    float* __restrict__ dt, int64_t ld_dt, int accumulate) {
  const int64_t v = blockIdx.x;
  const int64_t col = int64_t(blockIdx.y) * kSortThreads * VEC + int64_t(threadIdx.x) * VEC;
  const int64_t left = D - col;
  if (left <= 0) return;
  const int32_t beg = seg_begin[v], end = seg_end[v];
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
  if (end - beg <= kRun) {
    sum_dy_rows<T, VEC, U>(dy, ld_dy, sorted_pos, beg, end, col, left, acc);
  } else {
    // The chunk partials of the run, U rows in flight, added in chunk order.
    const int32_t q0 = chunk_off[v], q1 = chunk_off[v + 1];
    for (int32_t q = q0; q < q1; q += U) {
      float r[U][VEC];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* part = Q + int64_t(q + u) * ldq + col;
        if (q + u < q1 && left >= VEC && VEC % 4 == 0) {
#pragma unroll
          for (int i = 0; i < VEC; i += 4) {
            const Vec<float, 4> p4 = *reinterpret_cast<const Vec<float, 4>*>(part + i);
#pragma unroll
            for (int k = 0; k < 4; ++k) r[u][i + k] = p4.v[k];
          }
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) r[u][i] = (q + u < q1 && i < left) ? part[i] : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += r[u][i];
    }
  }
  float* out = dt + v * ld_dt + col;
  if (PVEC && left >= VEC && VEC % 4 == 0) {
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
      Vec<float, 4> o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o.v[q] = acc[i + q];
      if (accumulate) {
        const Vec<float, 4> old = *reinterpret_cast<const Vec<float, 4>*>(out + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) o.v[q] += old.v[q];
      }
      store_stream<float, 4>(out + i, o);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      if (i < left) out[i] = accumulate ? out[i] + acc[i] : acc[i];
  }
}

// Forward: workgroup (m, c) copies the columns of chunk c of x[idx[m]] to
// y[m] (zeros for an index outside [0, V)).
template <typename T, int VEC>
__global__ __launch_bounds__(kSortThreads) void gather_rows_fwd(
    const T* __restrict__ x, int64_t ld_x, const int32_t* __restrict__ idx, int64_t V,
    int64_t D, T* __restrict__ y, int64_t ld_y) {
  const int64_t m = blockIdx.x;
  const int64_t col = int64_t(blockIdx.y) * kSortThreads * VEC + int64_t(threadIdx.x) * VEC;
  if (col >= D) return;
  const int32_t v = idx[m];
  float o[VEC];
  if (v >= 0 && int64_t(v) < V) {
    load_f32_tail<T, VEC>(x + int64_t(v) * ld_x + col, D - col, 0.0f, o);
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = 0.0f;
  }
  store_f32_tail<T, VEC>(y + m * ld_y + col, D - col, o);
}

__global__ void fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

template <typename T>
hipError_t fwd_typed(const void* x, int64_t ld_x, const int32_t* idx, int64_t M, int64_t V,
                     int64_t D, void* y, int64_t ld_y, bool vec, hipStream_t s) {
  constexpr int V8 = 16 / sizeof(T);
  const int v = vec ? V8 : 1;
  const int64_t chunk = int64_t(kSortThreads) * v;
  const dim3 grid(unsigned(M), unsigned((D + chunk - 1) / chunk));
  if (vec)
    gather_rows_fwd<T, V8><<<grid, kSortThreads, 0, s>>>(static_cast<const T*>(x), ld_x, idx, V,
                                                        D, static_cast<T*>(y), ld_y);
  else
    gather_rows_fwd<T, 1><<<grid, kSortThreads, 0, s>>>(static_cast<const T*>(x), ld_x, idx, V,
                                                       D, static_cast<T*>(y), ld_y);
  return hipGetLastError();
}

// Rows summed per step of the backward (loads in flight per lane).
constexpr int kScatterUnroll = 8;

template <typename T>
hipError_t scatter_typed(const void* dy, int64_t ld_dy, const int32_t* pos, const int32_t* beg,
                         const int32_t* end, const int32_t* chunk_off, const int32_t* owner,
                         float* Q, int64_t ldq, int64_t nq_max, int64_t V, int64_t D, float* dt,
                         int64_t ld_dt, int accumulate, bool vec, bool pvec, hipStream_t s) {
  // Four columns per lane: each lane's fp32 results are one 16-byte store,
  // so a wave's stores cover 1 KB contiguously (eight 16-bit columns per lane
  // would leave every store instruction writing half of each 32-byte span).
  constexpr int V4 = 4;
  const int v = vec ? V4 : 1;
  const int64_t chunk = int64_t(kSortThreads) * v;
  const unsigned cb = unsigned((D + chunk - 1) / chunk);
  const T* g = static_cast<const T*>(dy);
  constexpr int U = kScatterUnroll;
  if (nq_max > 0) {
    const dim3 ga(unsigned(nq_max), cb);
    if (vec)
      chunk_sums<T, V4, U><<<ga, kSortThreads, 0, s>>>(g, ld_dy, pos, beg, end, chunk_off, owner,
                                                       V, D, Q, ldq);
    else
      chunk_sums<T, 1, U><<<ga, kSortThreads, 0, s>>>(g, ld_dy, pos, beg, end, chunk_off, owner,
                                                      V, D, Q, ldq);
  }
  const dim3 gb(unsigned(V), cb);
  if (vec && pvec)
    scatter_add_rows<T, V4, U, true><<<gb, kSortThreads, 0, s>>>(
        g, ld_dy, pos, beg, end, chunk_off, Q, ldq, D, dt, ld_dt, accumulate);
  else if (vec)
    scatter_add_rows<T, V4, U, false><<<gb, kSortThreads, 0, s>>>(
        g, ld_dy, pos, beg, end, chunk_off, Q, ldq, D, dt, ld_dt, accumulate);
  else
    scatter_add_rows<T, 1, U, false><<<gb, kSortThreads, 0, s>>>(
        g, ld_dy, pos, beg, end, chunk_off, Q, ldq, D, dt, ld_dt, accumulate);
  return hipGetLastError();
}

}  // namespace

int gather_sort_passes(int64_t V) {
  int bits = 1;
  while (bits < 32 && (int64_t(1) << bits) <= V) ++bits;   // keys 0 .. V
  return (bits + 7) / 8;
}

// Workspace, in 4-byte units: sorted keys [M], sorted positions [M], two
// ping-pong key / position buffers [4 M], the digit table [256 nb], run
// starts and ends [2 (V + 1)], chunk offsets [V + 1], chunk owners [nq], then
// (16-byte aligned) the chunk partials Q [nq][ldq] fp32, with
// nq = M / 16 + 1 (an upper bound on the chunk count) and ldq = D rounded up
// to a multiple of 4.
int64_t gather_max_chunks(int64_t M) { return M / 16 + 1; }

int64_t gather_ws_q_offset(int64_t M, int64_t V) {
  const int64_t nb = (M + kSortBlock - 1) / kSortBlock;
  const int64_t ints = 6 * M + int64_t(kDigits) * nb + 3 * (V + 1) + gather_max_chunks(M);
  return (ints + 3) / 4 * 4;
}

int64_t gather_workspace_ints(int64_t M, int64_t V, int64_t D) {
  return gather_ws_q_offset(M, V) + gather_max_chunks(M) * ((D + 3) / 4 * 4);
}

hipError_t launch_gather_rows_fwd(const void* x, int64_t ld_x, const int32_t* idx, int64_t M,
                                  int64_t V, int64_t D, void* y, int64_t ld_y, int act, bool vec,
                                  hipStream_t s) {
  switch (act) {
    case kF32: return fwd_typed<float>(x, ld_x, idx, M, V, D, y, ld_y, vec, s);
    case kF16: return fwd_typed<_Float16>(x, ld_x, idx, M, V, D, y, ld_y, vec, s);
    default: return fwd_typed<bf16>(x, ld_x, idx, M, V, D, y, ld_y, vec, s);
  }
}

hipError_t launch_gather_rows_bwd(const void* dy, int64_t ld_dy, const int32_t* idx, int64_t M,
                                  int64_t V, int64_t D, float* dt, int64_t ld_dt, int accumulate,
                                  int32_t* n_invalid, int32_t* ws, int act, bool vec, bool pvec,
                                  hipStream_t s) {
  const int64_t nb = (M + kSortBlock - 1) / kSortBlock;
  int32_t* sk = ws;                 // sorted keys
  int32_t* sv = ws + M;             // sorted positions
  int32_t* ak = ws + 2 * M;
  int32_t* av = ws + 3 * M;
  int32_t* bk = ws + 4 * M;
  int32_t* bv = ws + 5 * M;
  int32_t* hist = ws + 6 * M;
  int32_t* seg_begin = hist + int64_t(kDigits) * nb;
  int32_t* seg_end = seg_begin + (V + 1);
  int32_t* chunk_off = seg_end + (V + 1);
  int32_t* owner = chunk_off + (V + 1);
  const int64_t ldq = (D + 3) / 4 * 4;
  float* Q = reinterpret_cast<float*>(ws + gather_ws_q_offset(M, V));
  hipError_t e;
  if (M > 0) {
    const int passes = gather_sort_passes(V);
    const int32_t* ik = nullptr;
    const int32_t* iv = nullptr;
    for (int p = 0; p < passes; ++p) {
      int32_t* ok = p == passes - 1 ? sk : (p % 2 == 0 ? ak : bk);
      int32_t* ov = p == passes - 1 ? sv : (p % 2 == 0 ? av : bv);
      radix_upsweep<<<unsigned(nb), kSortThreads, 0, s>>>(idx, ik, M, V, 8 * p, hist, nb);
      scan_exclusive<<<1, kScanThreads, 0, s>>>(hist, int64_t(kDigits) * nb);
      radix_downsweep<<<unsigned(nb), kSortThreads, 0, s>>>(idx, ik, iv, M, V, 8 * p, hist, nb,
                                                            ok, ov);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      ik = ok;
      iv = ov;
    }
  }
  fill_i32<<<64, 256, 0, s>>>(seg_begin, 2 * (V + 1), 0);
  if (n_invalid != nullptr) fill_i32<<<1, 64, 0, s>>>(n_invalid, 1, 0);
  if (M > 0)
    segment_bounds<<<unsigned((M + 255) / 256), 256, 0, s>>>(sk, M, V, seg_begin, seg_end,
                                                             n_invalid);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (V == 0 || D == 0) return hipSuccess;
  // Long runs: chunk counts, their offsets (the total lands in chunk_off[V]),
  // and the owner of each chunk.
  const unsigned gv = unsigned((V + 1 + 255) / 256);
  count_chunks<<<gv, 256, 0, s>>>(seg_begin, seg_end, V, chunk_off);
  scan_exclusive<<<1, kScanThreads, 0, s>>>(chunk_off, V + 1);
  chunk_owners<<<gv, 256, 0, s>>>(chunk_off, V, owner);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nq_max = M > kRun ? gather_max_chunks(M) : 0;
#define VJP_SC(T)                                                                          \
  scatter_typed<T>(dy, ld_dy, sv, seg_begin, seg_end, chunk_off, owner, Q, ldq, nq_max, V, D, \
                   dt, ld_dt, accumulate, vec, pvec, s)
  switch (act) {
    case kF32: return VJP_SC(float);
    case kF16: return VJP_SC(_Float16);
    default: return VJP_SC(bf16);
  }
#undef VJP_SC
}

}  // namespace vjp
