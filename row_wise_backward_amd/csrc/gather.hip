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
//
// For M <= 16384 the plan takes one launch when the keys fit 15 bits
// (V + 1 <= 32768: a stable counting sort, plan_count) and three otherwise
// (one kernel per radix pass, each block counting the digits of all M keys
// itself instead of reading a scanned table, then one workgroup for the run
// bounds, the chunks and a list of the selected rows), instead of a dozen;
// step 4 then runs from the list of selected rows.  The rows never selected
// are zero-filled by extra workgroups of the plan's own launches, which
// otherwise leave most of the chip idle.  The sorted keys and positions, the
// run bounds of the keys that occur (an absent key's empty run may sit at a
// different place), the chunk offsets of long runs and every result bit are
// the same on all paths.
#include "launch.hpp"
#include "common.hpp"

#include <atomic>

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
    const int32_t v = int(threadIdx.x) >= o ? part[threadIdx.x - o] : 0;
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
// chunks of kRun positions (a run of len positions has ceil(len / kRun)).  Every long run has more than kRun positions, so
// it has fewer than len / 16 chunks, and all chunks together fewer than M / 16.
// (Measured on MI355X for 16384 Zipf ids into 32000 x 4096: 32-position runs
// 218 us for the whole backward; 64-position runs with the chunk counts
// folded into a strided scan, 330 us.)
constexpr int kRun = 32;

// Sorted-index range [j0, j1) of one chunk of a long run.
struct ChunkSpan {
  int32_t j0, j1;
};
__device__ __forceinline__ ChunkSpan chunk_span(int32_t run_begin, int32_t run_end, int32_t c) {
  const int32_t j0 = run_begin + c * kRun;
  return ChunkSpan{j0, min(j0 + kRun, run_end)};
}

// Plans for 0 < M <= kPlanMaxM take three launches: one kernel per radix
// pass, in which every block counts the digits of all M keys itself (the
// keys are L2 resident), so that it knows both where each digit starts and
// how many keys of each digit the blocks before it hold, and then places its
// own 1024 keys exactly as radix_downsweep does; and one workgroup that
// writes the run bounds, chunk offsets and chunk owners.  The arrays are the
// same, bit for bit, as those of the separate kernels above.
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanRounds = 16;
constexpr int64_t kPlanMaxM = int64_t(kPlanThreads) * kPlanRounds;

// Exclusive prefix of v over a workgroup of W waves in thread order; `total`
// gets the sum.  wsum: W ints of LDS (LDS barriers only).
template <int W>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* wsum,
                                                        int32_t& total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  lds_barrier();
  int32_t pre = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int32_t t = wsum[w];
    if (w < wave) pre += t;
    total += t;
  }
  lds_barrier();   // wsum is free again
  return pre + x - v;
}

// Keys read per thread per step of the digit count (loads in flight).
constexpr int kCountUnroll = 16;

// Zero rows beside the plan.  The plan kernels run on a few CUs; extra
// workgroups of the same launches write the zeros of the table rows no index
// selects (when the gradient is written, not added into).  Each such
// workgroup takes `rows` consecutive table rows of the launch's share
// [r0, r1), finds which of them are selected by reading all M indices itself
// (so it needs nothing from the plan), and writes zeros to the others.  The
// rows it writes are disjoint from those the listed-rows kernel writes
// later, so the two never touch the same bytes.
struct FillShare {
  int64_t r0, r1;               // table rows of this launch
  int64_t rows;                 // rows per fill workgroup (<= kFillMaxRows)
  int64_t groups;               // fill workgroups of this launch (0: none)
  const int32_t* idx;           // the M indices
  int64_t M, D;
  float* dt;                    // the gradient table
  int64_t ld_dt;
  bool pvec;                    // gradient rows 16-byte aligned
};
constexpr int64_t kFillMaxRows = 1024;
constexpr int64_t kFillBytes = int64_t(128) << 10;       // zeros per fill workgroup (target)
// Zeros beside the plan launches, at most: about what each launch writes in
// the time of its own work.  (Measured on MI355X for 16384 Zipf ids into
// 32000 x 4096: 162 us for the backward, against 172 us with every zero row
// written by the listed-rows kernel, 172 us with 192 / 128 MB beside the
// second pass / plan_tail, and 182 us with 96 MB more beside the chunk sums
// of long runs, whose own work streams dy.)
constexpr int64_t kFillFirstPassBytes = int64_t(64) << 20;
constexpr int64_t kFillPassBytes = int64_t(128) << 20;
constexpr int64_t kFillTailBytes = int64_t(96) << 20;
// Zeros beside the single-launch plan (plan_count), whose 16 sort
// workgroups take about 25 us on their own.  (Measured for the same
// workload: plan_count 28.7 / 33.4 / 40.6 / 44.1 us with 96 / 128 / 160 /
// 192 MB beside it, the listed-rows kernel 88.1 / 84.2 / 80.6 / 77.0 us: the
// zeros it sheds cost it less than they cost the plan.  Fill workgroups that
// zero every row of their share, skipping the scan of the indices and
// leaving the selected rows to be overwritten later, gave the same whole
// backward, 132.0 against 132.2 us.  The whole backward by the share, later
// and in one process: 48 / 64 / 80 / 96 / 112 MB 136.5 / 135.2 / 132.5 /
// 131.9-132.7 / 133.6 us.)
constexpr int64_t kFillCountBytes = int64_t(96) << 20;
constexpr int kFillUnroll = 16;

// Zeros to one fp32 row of D values, by the whole workgroup.
template <int THREADS>
__device__ __forceinline__ void zero_row(float* __restrict__ out, int64_t D, bool pvec) {
  for (int64_t col = int64_t(threadIdx.x) * 4; col < D; col += int64_t(THREADS) * 4) {
    if (pvec && col + 4 <= D) {
      store_stream<float, 4>(out + col, Vec<float, 4>{});
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (col + i < D) out[col + i] = 0.0f;
    }
  }
}

// sel: kFillMaxRows / 32 words of LDS.
template <int THREADS>
__device__ void zero_unselected_rows(const FillShare& fs, int64_t f, uint32_t* sel) {
  const int32_t* __restrict__ idx = fs.idx;
  const int64_t M = fs.M, D = fs.D, ld_dt = fs.ld_dt;
  float* __restrict__ dt = fs.dt;
  const bool pvec = fs.pvec;
  const int64_t a = fs.r0 + f * fs.rows;
  const int64_t e = a + fs.rows < fs.r1 ? a + fs.rows : fs.r1;
  if (a >= e) return;   // uniform
  const int n = int(e - a);
  for (int i = threadIdx.x; i < (n + 31) / 32; i += THREADS) sel[i] = 0;
  lds_barrier();
  // Mark the selected rows (integer LDS atomics), kFillUnroll loads in
  // flight per thread (positions past the end read index M - 1 again, and
  // mark nothing: marking those repeats put tens of thousands of atomics on
  // one LDS word in the workgroup whose rows hold index M - 1, which then
  // finished last); groups of four indices when the array is 16-byte
  // aligned, else single.
  auto mark = [&](int32_t k) {
    const int64_t d = int64_t(k) - a;
    if (d >= 0 && d < n) atomicOr(&sel[d >> 5], 1u << (d & 31));
  };
  if (reinterpret_cast<uintptr_t>(idx) % 16 == 0) {
    const int64_t M4 = M / 4;
    const Vec<int32_t, 4>* idx4 = reinterpret_cast<const Vec<int32_t, 4>*>(idx);
    for (int64_t j0 = threadIdx.x; j0 < M4; j0 += int64_t(kFillUnroll) * THREADS) {
      Vec<int32_t, 4> k[kFillUnroll];
#pragma unroll
      for (int u = 0; u < kFillUnroll; ++u) {
        const int64_t j = j0 + int64_t(u) * THREADS;
        k[u] = idx4[j < M4 ? j : M4 - 1];
      }
#pragma unroll
      for (int u = 0; u < kFillUnroll; ++u)
        if (j0 + int64_t(u) * THREADS < M4)   // clamped repeats mark nothing
#pragma unroll
          for (int i = 0; i < 4; ++i) mark(k[u].v[i]);
    }
    for (int64_t j = 4 * M4 + threadIdx.x; j < M; j += THREADS) mark(idx[j]);
  } else {
    for (int64_t j0 = threadIdx.x; j0 < M; j0 += int64_t(kFillUnroll) * THREADS) {
      int32_t k[kFillUnroll];
#pragma unroll
      for (int u = 0; u < kFillUnroll; ++u) {
        const int64_t j = j0 + int64_t(u) * THREADS;
        k[u] = idx[j < M ? j : M - 1];
      }
#pragma unroll
      for (int u = 0; u < kFillUnroll; ++u)
        if (j0 + int64_t(u) * THREADS < M) mark(k[u]);   // clamped repeats mark nothing
    }
  }
  lds_barrier();
  for (int r = 0; r < n; ++r)
    if (!((sel[r >> 5] >> (r & 31)) & 1u)) zero_row<THREADS>(dt + (a + r) * ld_dt, D, pvec);
}

// zero / nzero: the first pass also zero-fills the run bounds (2 (V + 1)
// entries) and the invalid count for the plan_tail kernel that follows.  The
// workgroup exchanges data only through LDS (its sorted keys are read by the
// next kernel), so its barriers leave the global stores in flight.
// FIRST: the pass reads the raw indices (position = m), otherwise the
// previous pass's keys and positions.  Loads are unconditional (indices past
// the end are clamped to M - 1 and their values discarded), so that a
// thread's loads are all in flight together.
template <bool FIRST>
__global__ __launch_bounds__(kSortThreads) void radix_pass_fused(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ keys_in,
    const int32_t* __restrict__ vals_in, int64_t M, int64_t V, int shift,
    int32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out, int32_t* __restrict__ zero,
    int64_t nzero, int32_t* __restrict__ n_invalid, FillShare fs) {
  // Digit counts in four copies (by lane mod 4): keys concentrated on a few
  // digits then collide on one LDS address four times less often.
  __shared__ int32_t all[4][kDigits], before[4][kDigits], base[kDigits];
  __shared__ int32_t wave_cnt[kSortWaves][kDigits];
  __shared__ int32_t wsum[kSortWaves];
  static_assert(4 * kDigits >= kFillMaxRows / 32, "fill bitmap fits in all[][]");
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.x;
  const int64_t nb = (M + kSortBlock - 1) / kSortBlock;   // the sort's own workgroups
  if (b >= nb) {
    zero_unselected_rows<kSortThreads>(fs, b - nb, reinterpret_cast<uint32_t*>(&all[0][0]));
    return;
  }
  const int64_t lo = b * kSortBlock;
  if (zero != nullptr) {
    for (int64_t i = b * kSortThreads + threadIdx.x; i < nzero; i += nb * kSortThreads)
      zero[i] = 0;
    if (b == 0 && threadIdx.x == 0 && n_invalid != nullptr) *n_invalid = 0;
  }
  // This block's keys, all four rounds in flight.
  const int32_t* __restrict__ src = FIRST ? idx : keys_in;
  int32_t key[kSortRounds], val[kSortRounds];
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
    const int64_t j = lo + r * kSortThreads + threadIdx.x;
    const int64_t jj = j < M ? j : M - 1;
    key[r] = src[jj];
    val[r] = FIRST ? int32_t(jj) : vals_in[jj];
  }
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r)
    if (FIRST) key[r] = (key[r] >= 0 && int64_t(key[r]) < V) ? key[r] : int32_t(V);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    all[c][threadIdx.x] = 0;
    before[c][threadIdx.x] = 0;
  }
  lds_barrier();
  // Digit counts of all keys and of the keys before this block (integer
  // atomics: exact), kCountUnroll loads in flight per thread.
  for (int64_t j0 = threadIdx.x; j0 < M; j0 += int64_t(kCountUnroll) * kSortThreads) {
    int32_t k[kCountUnroll];
#pragma unroll
    for (int u = 0; u < kCountUnroll; ++u) {
      const int64_t j = j0 + int64_t(u) * kSortThreads;
      k[u] = src[j < M ? j : M - 1];
    }
#pragma unroll
    for (int u = 0; u < kCountUnroll; ++u) {
      const int64_t j = j0 + int64_t(u) * kSortThreads;
      if (j >= M) break;
      const int32_t kv = FIRST ? ((k[u] >= 0 && int64_t(k[u]) < V) ? k[u] : int32_t(V)) : k[u];
      const int d = int((uint32_t(kv) >> shift) & (kDigits - 1));
      atomicAdd(&all[lane & 3][d], 1);
      if (j < lo) atomicAdd(&before[lane & 3][d], 1);
    }
  }
  lds_barrier();
  int32_t tot;
  const int32_t n_all = all[0][threadIdx.x] + all[1][threadIdx.x] + all[2][threadIdx.x] +
                        all[3][threadIdx.x];
  const int32_t n_before = before[0][threadIdx.x] + before[1][threadIdx.x] +
                           before[2][threadIdx.x] + before[3][threadIdx.x];
  base[threadIdx.x] = block_exclusive_scan<kSortWaves>(n_all, wsum, tot) + n_before;
  const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
  for (int r = 0; r < kSortRounds; ++r) {
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) wave_cnt[w][threadIdx.x] = 0;
    lds_barrier();
    const int64_t j = lo + r * kSortThreads + threadIdx.x;
    const bool in = j < M;
    const int32_t k = key[r], v = val[r];
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
    lds_barrier();
    if (in) {
      int32_t pre = base[d];
      for (int w = 0; w < wave; ++w) pre += wave_cnt[w][d];
      keys_out[pre + rank] = k;
      vals_out[pre + rank] = v;
    }
    lds_barrier();
    int32_t add = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) add += wave_cnt[w][threadIdx.x];
    base[threadIdx.x] += add;
    lds_barrier();
  }
}

// Run bounds, invalid count, chunk offsets, chunk owners and the list of
// selected rows (in key order, with its length in *n_rows) from the sorted
// keys, in one workgroup (M <= kPlanMaxM; the bounds and the invalid count
// arrive zero-filled).  Thread t takes the sorted positions [16 t, 16 t +
// 16); a run that starts there ends at the next run start, found in the
// thread's own positions or, past them, as the smallest first run start of
// the threads after it (a suffix minimum over the workgroup).  The workgroup
// exchanges data only through LDS; its global writes are never read back.
__global__ __launch_bounds__(kPlanThreads) void plan_tail(
    const int32_t* __restrict__ sk, int64_t M, int64_t V, int32_t* __restrict__ seg_begin,
    int32_t* __restrict__ seg_end, int32_t* __restrict__ chunk_off, ChunkSpan* __restrict__ ctab,
    int32_t* __restrict__ rows, int32_t* __restrict__ rbeg, int32_t* __restrict__ n_rows,
    int32_t* __restrict__ n_invalid, FillShare fs) {
  __shared__ int32_t wmin[kPlanWaves];
  __shared__ int32_t wsum[kPlanWaves];
  __shared__ uint32_t sel[kFillMaxRows / 32];
  if (blockIdx.x > 0) {   // the plan is workgroup 0; the others write zero rows
    zero_unselected_rows<kPlanThreads>(fs, int64_t(blockIdx.x) - 1, sel);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int32_t M32 = int32_t(M);
  // Loads are unconditional (indices clamped into [0, M)), values past the
  // end replaced afterwards, so a thread's loads are in flight together.
  const int64_t j0 = int64_t(tid) * kPlanRounds;
  auto clampj = [M](int64_t j) { return j < 0 ? int64_t(0) : (j < M ? j : M - 1); };
  int32_t prev = sk[clampj(j0 - 1)];
  int32_t kk[kPlanRounds];
#pragma unroll
  for (int i = 0; i < kPlanRounds; ++i) kk[i] = sk[clampj(j0 + i)];
  // Run starts among my positions, and the first of them (M if none).
  bool st[kPlanRounds];
  int32_t first = M32;
#pragma unroll
  for (int i = 0; i < kPlanRounds; ++i) {
    const int64_t j = j0 + i;
    st[i] = j < M && (j == 0 || (i == 0 ? prev : kk[i - 1]) != kk[i]);
    if (st[i] && first == M32) first = int32_t(j);
  }
  // Smallest first run start over the threads after me.
  int32_t x = first;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_down(x, o, kWave);
    if (lane + o < kWave) x = min(x, y);
  }
  if (lane == 0) wmin[wave] = x;   // minimum over the wave
  lds_barrier();
  int32_t next = __shfl_down(x, 1, kWave);
  if (lane == kWave - 1) next = M32;
  for (int w = wave + 1; w < kPlanWaves; ++w) next = min(next, wmin[w]);
  // Each run starting here: its bounds, its chunks, and whether it is a row.
  int32_t end[kPlanRounds], nch[kPlanRounds];
#pragma unroll
  for (int i = kPlanRounds - 1; i >= 0; --i) {
    end[i] = next;
    if (st[i]) next = int32_t(j0 + i);
  }
  int32_t my_chunks = 0, my_rows = 0;
#pragma unroll
  for (int i = 0; i < kPlanRounds; ++i) {
    nch[i] = 0;
    if (!st[i]) continue;
    const int32_t j = int32_t(j0 + i);
    seg_begin[kk[i]] = j;
    seg_end[kk[i]] = end[i];
    if (int64_t(kk[i]) == V) {
      if (n_invalid != nullptr) *n_invalid = M32 - j;
      continue;
    }
    const int32_t len = end[i] - j;
    nch[i] = len > kRun ? (len + kRun - 1) / kRun : 0;
    my_chunks += nch[i];
    my_rows += 1;
  }
  int32_t total_chunks, total_rows;
  int32_t q = block_exclusive_scan<kPlanWaves>(my_chunks, wsum, total_chunks);
  int32_t r = block_exclusive_scan<kPlanWaves>(my_rows, wsum, total_rows);
#pragma unroll
  for (int i = 0; i < kPlanRounds; ++i) {
    if (!st[i]) continue;
    const int32_t j = int32_t(j0 + i);
    if (int64_t(kk[i]) == V) {   // the run after the last listed row's
      rbeg[total_rows] = j;
      continue;
    }
    rbeg[r] = j;
    rows[r++] = kk[i];
    if (nch[i] > 0) {
      chunk_off[kk[i]] = q;
      for (int32_t c = 0; c < nch[i]; ++c) ctab[q + c] = chunk_span(j, end[i], c);
      q += nch[i];
    }
  }
  if (tid == 0) {
    chunk_off[V] = total_chunks;
    *n_rows = total_rows;
    if (sk[M - 1] != int32_t(V)) rbeg[total_rows] = M32;   // no invalid index
  }
}

// Single-launch plan (M <= kPlanMaxM indices, keys 0 .. V with V + 1 <=
// kCountKeys): a stable counting sort.  Every sort workgroup counts the keys
// of all M indices, and those of the indices before its own kCountBlock, in
// LDS; the prefix sum of the counts is where each key's run starts, so the
// workgroup places each of its keys at: run start + equal keys in earlier
// workgroups + rank among equal keys in its own block, the rank coming from a
// bitonic sort of its (key, local position) pairs (the composite is unique,
// so equal keys keep increasing position: the stable order, which is unique,
// hence the same sorted keys and positions as the radix passes).  The same
// prefix sums give the run bounds of every key, the chunk offsets and owners
// of runs longer than kRun, the list of selected rows and the invalid count
// (the run of key V): the sparse ones (row list, chunk offsets and owners)
// from the scan, by sort workgroup t mod (sort workgroups) for thread t's
// keys, the run bounds afterwards in coalesced stores, each sort workgroup
// a contiguous share of the keys.  Workgroups past the sort's write zero
// rows, as beside the radix passes.  One launch instead of three.
//
// One LDS word per key holds both counts (all indices in the low half, those
// before this block in the high half: one atomic increment per index).  A
// duplicate-matching step (ballots over the 15 key bits, one add per
// distinct key) cost more than the serialised adds it saves, even on
// Zipf-skewed ids.  Thread t owns the 32 keys [32 t, 32 t + 32): it loads
// their words into registers, sums them, takes its offset from one
// workgroup scan, and walks them in order, leaving in each word the key's
// run start (low half) beside its count before this block (high half); key
// k's word sits at k + k / 32, so the lanes of a wave reading their strips
// in step hit distinct banks.
constexpr int kCountThreads = 1024;
constexpr int kCountWaves = kCountThreads / kWave;
constexpr int64_t kCountKeys = 32768;             // keys 0 .. V, V + 1 <= kCountKeys
constexpr int kCountBlock = 1024;                 // keys placed per workgroup
constexpr int kCountLoads = 16;                   // index loads in flight per lane (counting)
constexpr int kStrip = int(kCountKeys / kCountThreads);      // keys per thread in the scan
constexpr int kCountWords = int(kCountKeys + kCountKeys / kStrip);
static_assert(kCountBlock == kCountThreads, "one key per thread in the placement");
static_assert(kPlanMaxM <= 32767, "16-bit counts");
static_assert(kStrip == 32, "one padding word per strip");

__device__ __forceinline__ int64_t cnt_slot(int64_t k) { return k + (k >> 5); }

// Inclusive prefix sum over the 64 lanes of a wave (integers, exact): a
// doubling scan within each row of 16 lanes on DPP row shifts (lanes shifted
// in from before the row read 0), then the totals of rows 0, 1 and 2, read
// from lanes 15, 31 and 47, added to the rows after them.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xF, 0xF, false));   // row_shr:1
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xF, 0xF, false));   // row_shr:2
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xF, 0xF, false));   // row_shr:4
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xF, 0xF, false));   // row_shr:8
  const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(x), 15));
  const uint32_t r1 = uint32_t(__builtin_amdgcn_readlane(int(x), 31));
  const uint32_t r2 = uint32_t(__builtin_amdgcn_readlane(int(x), 47));
  const int row = int(threadIdx.x % kWave) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Per key: its count plus 2^16 if it is a selected table row (so one sum
// carries both the run starts and the row-list offsets; neither total
// exceeds M < 2^16), and its number of chunks.  Key V (invalid indices) has
// a run but is no table row; keys past V count nothing.
__device__ __forceinline__ uint32_t key_ar(uint32_t n, int64_t k, int64_t V) {
  return n + ((k < V && n > 0) ? 0x10000u : 0u);
}
__device__ __forceinline__ uint32_t key_chunks(uint32_t n, int64_t k, int64_t V) {
  return (k < V && n > uint32_t(kRun)) ? (n + kRun - 1) / kRun : 0u;
}

// The sparse plan entries of key k < V selected n > 0 times: its place
// ar >> 16 in the row list with its run start, and for a long run its chunk
// offset q and the spans of its nch chunks.
__device__ __forceinline__ void emit_row(int64_t k, uint32_t n, uint32_t ar, uint32_t q,
                                         uint32_t nch, int32_t* __restrict__ chunk_off,
                                         ChunkSpan* __restrict__ ctab, int32_t* __restrict__ rows,
                                         int32_t* __restrict__ rbeg) {
  const int32_t run = int32_t(ar & 0xFFFFu);
  rows[ar >> 16] = int32_t(k);
  rbeg[ar >> 16] = run;
  if (nch > 0) {
    chunk_off[k] = int32_t(q);
    for (uint32_t c = 0; c < nch; ++c) ctab[q + c] = chunk_span(run, run + int32_t(n), int32_t(c));
  }
}

__global__ __launch_bounds__(kCountThreads) void plan_count(
    const int32_t* __restrict__ idx, int64_t M, int64_t V, int32_t* __restrict__ sk,
    int32_t* __restrict__ sv, int32_t* __restrict__ seg_begin, int32_t* __restrict__ seg_end,
    int32_t* __restrict__ chunk_off, ChunkSpan* __restrict__ ctab, int32_t* __restrict__ rows,
    int32_t* __restrict__ rbeg, int32_t* __restrict__ n_rows, int32_t* __restrict__ n_invalid,
    FillShare fs) {
  __shared__ uint32_t cnt[kCountWords];   // per key: counts, then run start + earlier equals
  __shared__ uint32_t srt[kCountBlock];   // this block's (key, position) pairs
  __shared__ uint32_t srt2[kCountBlock];  // the bitonic network's second buffer
  __shared__ uint32_t wsum[2][kCountWaves];
  static_assert(kCountBlock >= kFillMaxRows / 32, "fill bitmap fits in srt");
  const int64_t nb = (M + kCountBlock - 1) / kCountBlock;
  const int64_t b = blockIdx.x;
  if (b >= nb) {
    zero_unselected_rows<kCountThreads>(fs, b - nb, srt);
    return;
  }
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t lo = b * kCountBlock;
  const int64_t mine_j = lo + tid;
  const int32_t mine_key = key_of(idx, mine_j < M ? mine_j : M - 1, V);   // loaded early
  for (int i = tid; i < kCountWords; i += kCountThreads) cnt[i] = 0;
  lds_barrier();
  constexpr int64_t kStride = int64_t(kCountThreads);
  for (int64_t j0 = tid; j0 < M; j0 += kStride * kCountLoads) {
    int32_t key[kCountLoads];
#pragma unroll
    for (int u = 0; u < kCountLoads; ++u) {
      const int64_t j = j0 + u * kStride;
      key[u] = key_of(idx, j < M ? j : M - 1, V);
    }
#pragma unroll
    for (int u = 0; u < kCountLoads; ++u) {
      const int64_t j = j0 + u * kStride;
      if (j < M) atomicAdd(&cnt[cnt_slot(key[u])], j < lo ? 0x10001u : 1u);
    }
  }
  lds_barrier();
  // This thread's strip: its sums (its words read kBatch at a time, all in
  // flight together), its offsets from the scan.
  constexpr int kBatch = 8;
  const int64_t k0 = int64_t(tid) * kStrip;
  uint32_t* const strip = cnt + cnt_slot(k0);
  uint32_t ar = 0, ch = 0;
#pragma unroll
  for (int g = 0; g < kStrip; g += kBatch) {
    uint32_t w[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) w[i] = strip[g + i];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      ar += key_ar(w[i] & 0xFFFFu, k0 + g + i, V);
      ch += key_chunks(w[i] & 0xFFFFu, k0 + g + i, V);
    }
  }
  const uint32_t ar_i = wave_scan_incl(ar), ch_i = wave_scan_incl(ch);
  if (lane == kWave - 1) {
    wsum[0][wave] = ar_i;
    wsum[1][wave] = ch_i;
  }
  lds_barrier();
  uint32_t run_ar = ar_i - ar, q = ch_i - ch, tot_ar = 0, tot_ch = 0;
#pragma unroll
  for (int v = 0; v < kCountWaves; ++v) {
    const uint32_t x = wsum[0][v], y = wsum[1][v];
    if (v < wave) {
      run_ar += x;
      q += y;
    }
    tot_ar += x;
    tot_ch += y;
  }
  if (b == 0 && tid == 0) {
    chunk_off[V] = int32_t(tot_ch);
    *n_rows = int32_t(tot_ar >> 16);
  }
  // Walk the strip: each key's word becomes its run start beside the equal
  // keys in earlier workgroups (only this thread reads or writes these words).
  const bool writes = int64_t(tid) % nb == b;
#pragma unroll 1
  for (int g = 0; g < kStrip; g += kBatch) {
    uint32_t w[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) w[i] = strip[g + i];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t k = k0 + g + i;
      const uint32_t n = w[i] & 0xFFFFu;
      const uint32_t x = key_ar(n, k, V), y = key_chunks(n, k, V);
      strip[g + i] = (run_ar & 0xFFFFu) | (w[i] & 0xFFFF0000u);
      if (writes && k < V && n > 0) emit_row(k, n, run_ar, q, y, chunk_off, ctab, rows, rbeg);
      run_ar += x;
      q += y;
    }
  }
  // Placement: sort this block's (key, local position) pairs, ascending, on
  // a bitonic network.  Its stages whose partners lie in the same wave run on
  // register shuffles; the ten others exchange through LDS, alternating
  // between srt and srt2.
  uint32_t e = mine_j < M ? (uint32_t(mine_key) << 10) | uint32_t(tid) : 0xFFFFFFFFu;
  int stage = 0;
#pragma unroll
  for (int kk = 2; kk <= kCountBlock; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      uint32_t y;
      if (jj >= kWave) {
        uint32_t* buf = (stage++ & 1) ? srt2 : srt;
        buf[tid] = e;
        lds_barrier();
        y = buf[tid ^ jj];
      } else {
        y = uint32_t(__shfl_xor(int(e), jj, kWave));
      }
      // ascending runs (tid & kk clear) keep the smaller key at the lower index
      e = (((tid & kk) == 0) == ((tid & jj) == 0)) ? min(e, y) : max(e, y);
    }
  }
  srt[tid] = e;
  lds_barrier();
  // Run bounds of this workgroup's share of the keys 0 .. V (run V + 1
  // starts at M), the invalid count, and the end of the listed rows' runs.
  const int64_t share = (V + 1 + nb - 1) / nb;
  const int64_t s1 = (b + 1) * share < V + 1 ? (b + 1) * share : V + 1;
  for (int64_t k = b * share + tid; k < s1; k += kCountThreads) {
    const int32_t r0 = int32_t(cnt[cnt_slot(k)] & 0xFFFFu);
    const int32_t r1 = k == V ? int32_t(M) : int32_t(cnt[cnt_slot(k + 1)] & 0xFFFFu);
    seg_begin[k] = r0;
    seg_end[k] = r1;
    if (k == V) {
      if (n_invalid != nullptr) *n_invalid = r1 - r0;
      rbeg[tot_ar >> 16] = r0;
    }
  }
  if (e != 0xFFFFFFFFu) {
    const uint32_t k = e >> 10;
    // first sorted index holding key k (binary search in [0, tid])
    int f0 = 0, f1 = tid;
    while (f0 < f1) {
      const int mid = (f0 + f1) >> 1;
      if ((srt[mid] >> 10) < k) f0 = mid + 1; else f1 = mid;
    }
    const uint32_t w = cnt[cnt_slot(k)];
    const int32_t pos = int32_t((w & 0xFFFFu) + (w >> 16)) + (tid - f0);
    sk[pos] = int32_t(k);
    sv[pos] = int32_t(lo + (e & 1023u));
  }
}

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

// The same sums for lanes whose VEC columns lie inside the row (left >=
// VEC): the U loads of a step are unconditional (positions past j1 - 1 read
// the row at pos[j1 - 1] again and add zeros, as sum_dy_rows adds zeros), so
// they are all in flight together.  Bitwise the same results.
template <typename T, int VEC, int U>
__device__ __forceinline__ void sum_dy_rows_full(const T* __restrict__ dy, int64_t ld_dy,
                                                 const int32_t* __restrict__ pos, int32_t j0,
                                                 int32_t j1, int64_t col, float (&acc)[VEC]) {
  for (int32_t j = j0; j < j1; j += U) {
    words_t<T, VEC> w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t p = pos[j + u < j1 ? j + u : j1 - 1];
      w[u] = __builtin_nontemporal_load(
          reinterpret_cast<const words_t<T, VEC>*>(dy + int64_t(p) * ld_dy + col));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const Vec<T, VEC> r = as_vec<T, VEC>(w[u]);
      const bool in = j + u < j1;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += in ? to_f32(r.v[i]) : 0.0f;
    }
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

// ctab[q] = the sorted-index span of chunk q (of its table row's run).
__global__ __launch_bounds__(256) void chunk_spans(const int32_t* __restrict__ chunk_off,
                                                    const int32_t* __restrict__ seg_begin,
                                                    const int32_t* __restrict__ seg_end, int64_t V,
                                                    ChunkSpan* __restrict__ ctab) {
  const int64_t v = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= V) return;
  const int32_t q0 = chunk_off[v], q1 = chunk_off[v + 1], b = seg_begin[v], e = seg_end[v];
  for (int32_t q = q0; q < q1; ++q) ctab[q] = chunk_span(b, e, q - q0);
}

// The partial sum of chunk q (sorted indices [j0, j1)) for the VEC columns
// of this lane at col (left = D - col > 0), stored to Q[q].
template <typename T, int VEC, int U>
__device__ __forceinline__ void chunk_partial(const T* __restrict__ dy, int64_t ld_dy,
                                              const int32_t* __restrict__ sorted_pos, int32_t j0,
                                              int32_t j1, int64_t q, int64_t col, int64_t left,
                                              float* __restrict__ Q, int64_t ldq) {
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
  if (left >= VEC)
    sum_dy_rows_full<T, VEC, U>(dy, ld_dy, sorted_pos, j0, j1, col, acc);
  else
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

// Stage A: workgroup (q, c) sums chunk q of a long run into Q[q][chunk c].
// (Zero rows beside it, as beside the plan, made the backward slower: 137 to
// 144 us against 135 with 32 to 96 MB of them for 16384 Zipf ids into
// 32000 x 4096 on MI355X; on the odd workgroups only, the chunk sums on the
// even ones, 145 to 150 us against 137 with 64 to 192 MB, whether the zero
// workgroups read all M indices or the plan's run bounds: the zero stream
// slows the latency-bound chunk reads even from the other XCDs, 28 -> 39 us
// for the chunk sums on four XCDs beside 96 MB.)
template <typename T, int VEC, int U>
__global__ __launch_bounds__(kSortThreads) void chunk_sums(
    const T* __restrict__ dy, int64_t ld_dy, const int32_t* __restrict__ sorted_pos,
    const int32_t* __restrict__ chunk_off, const ChunkSpan* __restrict__ ctab, int64_t V,
    int64_t D, float* __restrict__ Q, int64_t ldq) {
  const int64_t q = blockIdx.x;
  if (q >= chunk_off[V]) return;   // the grid is an upper bound on the chunk count
  const int64_t col = int64_t(blockIdx.y) * kSortThreads * VEC + int64_t(threadIdx.x) * VEC;
  if (col >= D) return;
  const ChunkSpan c = ctab[q];
  chunk_partial<T, VEC, U>(dy, ld_dy, sorted_pos, c.j0, c.j1, q, col, D - col, Q, ldq);
}

// Stage B for table row v (its run: sorted indices [beg, end)) and the VEC
// columns of this lane at col (left = D - col > 0): the gradient row,
// written (or added into dt).  PVEC: the gradient rows are 16-byte aligned,
// so each lane's VEC fp32 values go out as 16-byte stores.
template <typename T, int VEC, int U, bool PVEC>
__device__ __forceinline__ void row_gradient(
    int64_t v, int32_t beg, int32_t end, int64_t col, const T* __restrict__ dy, int64_t ld_dy,
    const int32_t* __restrict__ sorted_pos, const int32_t* __restrict__ chunk_off,
    const float* __restrict__ Q, int64_t ldq, int64_t D, float* __restrict__ dt, int64_t ld_dt,
    int accumulate) {
  const int64_t left = D - col;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
  if (end - beg <= kRun) {
    if (left >= VEC)
      sum_dy_rows_full<T, VEC, U>(dy, ld_dy, sorted_pos, beg, end, col, acc);
    else
      sum_dy_rows<T, VEC, U>(dy, ld_dy, sorted_pos, beg, end, col, left, acc);
  } else {
    // The chunk partials of the run, U rows in flight, added in chunk order.
    const int32_t q0 = chunk_off[v], q1 = q0 + (end - beg + kRun - 1) / kRun;
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

// Stage B over every table row: workgroup (v, c) writes (or adds into) the
// gradient of row v for chunk c of the columns; rows never selected get
// zeros (or stay unchanged).
template <typename T, int VEC, int U, bool PVEC>
__global__ __launch_bounds__(kSortThreads) void scatter_add_rows(
    const T* __restrict__ dy, int64_t ld_dy, const int32_t* __restrict__ sorted_pos,
    const int32_t* __restrict__ seg_begin, const int32_t* __restrict__ seg_end,
    const int32_t* __restrict__ chunk_off, const float* __restrict__ Q, int64_t ldq, int64_t D,
    float* __restrict__ dt, int64_t ld_dt, int accumulate) {
  const int64_t col = int64_t(blockIdx.y) * kSortThreads * VEC + int64_t(threadIdx.x) * VEC;
  if (col >= D) return;
  row_gradient<T, VEC, U, PVEC>(blockIdx.x, seg_begin[blockIdx.x], seg_end[blockIdx.x], col, dy,
                                ld_dy, sorted_pos, chunk_off, Q, ldq, D, dt, ld_dt, accumulate);
}

// Stage B from the list of selected rows (plans of M <= kPlanMaxM).  When
// the share fs holds rows to zero-fill (writing, not accumulating), the even
// workgroups loop over the (listed row, column chunk) pairs and the odd ones
// write zeros to the share's rows never selected (an empty run), so that the
// latency-bound sums and the bandwidth-bound zero rows run side by side; the
// rows before the share were zero-filled beside the plan.  Otherwise every
// workgroup takes listed pairs.  Needs gridDim.x >= 2.
// Consecutive workgroups go to the 8 XCDs in turn, so the sums run on XCDs
// 0, 2, 4, 6 and the zero rows on 1, 3, 5, 7.  (Measured on MI355X for
// 16384 Zipf ids into 32000 x 4096: 88 us; the sums alone 43 us, the zero
// rows alone 77 us (67 us from all XCDs).  Other splits were slower: both
// roles on every XCD, 105 us (the sums' reads queue behind the zero
// stream); sums on XCDs 0-3 and zeros on 4-7, 95 us; sums on 3 or 2 XCDs,
// 105 or 123 us; the chunk sums and the listed sums in one launch and the
// zero rows in the next, 113 us for both (against 88 + 21 here); the even
// workgroups left without a pair writing zero rows too, 93 us; two or four
// column groups per lane (all their loads in flight), 90-94 us; all zero
// rows here with the pairs first in every workgroup, 132 us; one workgroup
// per table row and column chunk, 128 us; every zero row written by a
// kernel of its own on a second stream, beside the plan, the chunk sums and
// the listed sums on the first, 143-175 us for the whole backward against
// 134: its workgroups hold the CUs the latency-bound sums wait for, and the
// chunk sums alone stretched from 20 to 43-104 us; the chunk sums moved into
// this launch beside the short rows' sums, and the long rows' chunk sums
// added up in a third launch, 164-171 us against 132 (this launch 128 us,
// the third 13-20 us: a long row's chain of up to 92 partials is exposed).)
template <typename T, int VEC, int U, bool PVEC>
__global__ __launch_bounds__(kSortThreads) void scatter_listed_rows(
    const T* __restrict__ dy, int64_t ld_dy, const int32_t* __restrict__ sorted_pos,
    const int32_t* __restrict__ seg_begin, const int32_t* __restrict__ seg_end,
    const int32_t* __restrict__ chunk_off, const float* __restrict__ Q, int64_t ldq, int64_t D,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ rbeg,
    const int32_t* __restrict__ n_rows, int64_t cb, float* __restrict__ dt, int64_t ld_dt,
    int accumulate, FillShare fs) {
  const int64_t b = blockIdx.x;
  const bool split = fs.r1 > fs.r0;
  if (!split || b % 2 == 0) {
    const int64_t me = split ? b / 2 : b;
    const int64_t stride = split ? int64_t(gridDim.x + 1) / 2 : int64_t(gridDim.x);
    const int64_t items = int64_t(*n_rows) * cb;
    for (int64_t it = me; it < items; it += stride) {
      const int64_t col = (it % cb) * kSortThreads * VEC + int64_t(threadIdx.x) * VEC;
      const int64_t r = it / cb;   // the run of listed row r ends where row r + 1's begins
      if (col < D)
        row_gradient<T, VEC, U, PVEC>(rows[r], rbeg[r], rbeg[r + 1], col, dy, ld_dy, sorted_pos,
                                      chunk_off, Q, ldq, D, dt, ld_dt, accumulate);
    }
    return;
  }
  const int64_t stride = int64_t(gridDim.x) / 2;
  for (int64_t v = fs.r0 + b / 2; v < fs.r1; v += stride)
    if (seg_end[v] == seg_begin[v]) zero_row<kSortThreads>(dt + v * ld_dt, D, PVEC);   // uniform
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

// Vector lanes per row of the forward: each lane carries kGatherK 16-byte
// vectors of its row, all loads issued before the first store, so one
// workgroup of 256 lanes covers a 4096-element bf16 row.  (Measured on
// MI355X, 16384 Zipf ids into 32000 x 4096 bf16, median of 20 flushed runs:
// 36.9 us against 44.5 us for one vector per lane and two workgroups per
// row; with uniform ids 47.2 against 46.3 us.  Cached loads of the table
// took 34.1 us for the Zipf ids but 66.8 us for uniform ones: the loads stay
// nontemporal.)
constexpr int kGatherK = 2;

// Forward, 16-byte vectors (rows 16-byte aligned): workgroup (m, c) copies
// the bits of column chunk c (kGatherK vectors per lane) of x[idx[m]] to
// y[m]; zeros for an index outside [0, V).
template <typename T, int VEC>
__global__ __launch_bounds__(kSortThreads) void gather_rows_fwd_vec(
    const T* __restrict__ x, int64_t ld_x, const int32_t* __restrict__ idx, int64_t V,
    int64_t D, T* __restrict__ y, int64_t ld_y) {
  constexpr int64_t kStep = int64_t(kSortThreads) * VEC;
  const int64_t m = blockIdx.x;
  const int64_t c0 = int64_t(blockIdx.y) * kStep * kGatherK + int64_t(threadIdx.x) * VEC;
  if (c0 >= D) return;
  const int32_t v = idx[m];
  words_t<T, VEC> w[kGatherK];
#pragma unroll
  for (int k = 0; k < kGatherK; ++k) w[k] = words_t<T, VEC>{};
  if (v >= 0 && int64_t(v) < V) {
    const T* src = x + int64_t(v) * ld_x;
#pragma unroll
    for (int k = 0; k < kGatherK; ++k) issue_vec<T, VEC>(src + c0 + k * kStep, D - (c0 + k * kStep), w[k]);
#pragma unroll
    for (int k = 0; k < kGatherK; ++k)
      fix_vec<T, VEC>(src + c0 + k * kStep, D - (c0 + k * kStep), from_f32<T>(0.0f), w[k]);
  }
  T* dst = y + m * ld_y;
#pragma unroll
  for (int k = 0; k < kGatherK; ++k) {
    const int64_t col = c0 + k * kStep, avail = D - col;
    if (avail >= VEC) {
      __builtin_nontemporal_store(w[k], reinterpret_cast<words_t<T, VEC>*>(dst + col));
    } else if (avail > 0) {
      const Vec<T, VEC> e = as_vec<T, VEC>(w[k]);
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        if (i < avail) dst[col + i] = e.v[i];
    }
  }
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
  if (vec) {
    const int64_t chunk = int64_t(kSortThreads) * V8 * kGatherK;
    const dim3 grid(unsigned(M), unsigned((D + chunk - 1) / chunk));
    gather_rows_fwd_vec<T, V8><<<grid, kSortThreads, 0, s>>>(static_cast<const T*>(x), ld_x, idx,
                                                            V, D, static_cast<T*>(y), ld_y);
  } else {
    const int64_t chunk = kSortThreads;
    const dim3 grid(unsigned(M), unsigned((D + chunk - 1) / chunk));
    gather_rows_fwd<T, 1><<<grid, kSortThreads, 0, s>>>(static_cast<const T*>(x), ld_x, idx, V,
                                                       D, static_cast<T*>(y), ld_y);
  }
  return hipGetLastError();
}

// Rows summed per step of the backward (loads in flight per lane).
constexpr int kScatterUnroll = 8;

// Workgroups of the listed-rows stage B (each loops over its items).
constexpr int64_t kListedGrid = 32768;

// rows / n_rows: the list of selected rows (then stage B runs from the list),
// or null (stage B over every table row).
template <typename T>
hipError_t scatter_typed(const void* dy, int64_t ld_dy, const int32_t* pos, const int32_t* beg,
                         const int32_t* end, const int32_t* chunk_off, const ChunkSpan* ctab,
                         float* Q, int64_t ldq, int64_t nq_max, int64_t V, int64_t D,
                         const int32_t* rows, const int32_t* rbeg, const int32_t* n_rows,
                         float* dt, int64_t ld_dt,
                         int accumulate, bool vec, bool pvec, const FillShare& fill_listed,
                         hipStream_t s) {
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
    // A chunk's kRun rows all in flight at once: its positions and then its
    // dy rows are one round trip each (with U rows per round the dependent
    // position and row loads took kRun / U rounds of both).
    const dim3 ga(unsigned(nq_max), cb);
    if (vec)
      chunk_sums<T, V4, kRun><<<ga, kSortThreads, 0, s>>>(g, ld_dy, pos, chunk_off, ctab, V, D, Q,
                                                          ldq);
    else
      chunk_sums<T, 1, kRun><<<ga, kSortThreads, 0, s>>>(g, ld_dy, pos, chunk_off, ctab, V, D, Q,
                                                         ldq);
  }
  if (rows != nullptr) {
    const int64_t want = 2 * V * int64_t(cb);
    const unsigned gl = unsigned(want < 2 ? 2 : (want < kListedGrid ? want : kListedGrid));
#define VJP_LISTED(VV, PV)                                                                      \
  scatter_listed_rows<T, VV, U, PV><<<gl, kSortThreads, 0, s>>>(                              \
      g, ld_dy, pos, beg, end, chunk_off, Q, ldq, D, rows, rbeg, n_rows, cb, dt, ld_dt,         \
      accumulate,                                                                             \
      fill_listed)
    if (vec && pvec)
      VJP_LISTED(V4, true);
    else if (vec)
      VJP_LISTED(V4, false);
    else
      VJP_LISTED(1, false);
#undef VJP_LISTED
    return hipGetLastError();
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
// starts and ends [2 (V + 1)], chunk offsets [V + 1], chunk spans [2 nq], then
// (16-byte aligned) the chunk partials Q [nq][ldq] fp32, with
// nq = M / 16 + 1 (an upper bound on the chunk count) and ldq = D rounded up
// to a multiple of 4.
int64_t gather_max_chunks(int64_t M) { return M / 16 + 1; }

int64_t gather_ws_q_offset(int64_t M, int64_t V) {
  const int64_t nb = (M + kSortBlock - 1) / kSortBlock;
  const int64_t ints = 6 * M + int64_t(kDigits) * nb + 3 * (V + 1) + 2 * gather_max_chunks(M);
  return (ints + 3) / 4 * 4;
}

int64_t gather_workspace_ints(int64_t M, int64_t V, int64_t D) {
  return gather_ws_q_offset(M, V) + gather_max_chunks(M) * ((D + 3) / 4 * 4);
}

// The plan for any M: radix passes of three kernels each, then the run
// bounds, chunk counts, their scan and the chunk spans as separate kernels.
static hipError_t plan_multi(const int32_t* idx, int64_t M, int64_t V, int64_t D, int32_t* sk,
                             int32_t* sv, int32_t* ak, int32_t* av, int32_t* bk, int32_t* bv,
                             int32_t* hist, int64_t nb, int32_t* seg_begin, int32_t* seg_end,
                             int32_t* chunk_off, ChunkSpan* ctab, int32_t* n_invalid,
                             hipStream_t s) {
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
  chunk_spans<<<gv, 256, 0, s>>>(chunk_off, seg_begin, seg_end, V, ctab);
  return hipGetLastError();
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

namespace {
// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}
}  // namespace

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
  ChunkSpan* ctab = reinterpret_cast<ChunkSpan*>(chunk_off + (V + 1));
  const int64_t ldq = (D + 3) / 4 * 4;
  float* Q = reinterpret_cast<float*>(ws + gather_ws_q_offset(M, V));
  // Plans of M <= kPlanMaxM also list the selected rows: the list reuses the
  // sort's spare key buffer, its length the digit table's first entry.
  int32_t* rows = bk;
  int32_t* rbeg = ak;   // run start of each listed row, then the end of the last
  int32_t* n_rows = hist;
  hipError_t e;
  const int64_t nq_max = M > kRun ? gather_max_chunks(M) : 0;
  const bool listed = M > 0 && M <= kPlanMaxM;
  // Zero rows beside the plan: when writing, each radix pass and plan_tail
  // take up to a fixed number of bytes of the zero rows, in order of rows,
  // and the listed-rows kernel the rest.  A FillShare with r0 = r1 fills
  // nothing.
  const int passes = listed ? gather_sort_passes(V) : 0;
  const bool fill_rows = listed && !accumulate && V > 0 && D > 0;
  int64_t per = (kFillBytes / 4 + D - 1) / (D > 0 ? D : 1);
  per = per < 1 ? 1 : (per > kFillMaxRows ? kFillMaxRows : per);
  int64_t cursor = 0;   // next unassigned row
  // bytes: the most zeros this launch takes (-1: all the rest); wide: its
  // workgroups have kPlanThreads threads, and take four times the rows;
  // max_groups > 0: at most that many fill workgroups, each taking more rows
  // (up to kFillMaxRows; the share shrinks if even that is not enough).
  auto share = [&](int64_t bytes, bool wide, int64_t max_groups) {
    int64_t rows = wide ? (4 * per < kFillMaxRows ? 4 * per : kFillMaxRows) : per;
    FillShare f{cursor, cursor, rows, 0, idx, M, D, dt, ld_dt, pvec};
    if (fill_rows) {
      const int64_t budget = bytes < 0 ? V : (bytes / 4 + D - 1) / D;
      f.r1 = V - cursor < budget ? V : cursor + budget;
      if (max_groups > 0) {
        const int64_t need = (f.r1 - f.r0 + max_groups - 1) / max_groups;
        rows = need > rows ? (need < kFillMaxRows ? need : kFillMaxRows) : rows;
        f.rows = rows;
        if (f.r1 - f.r0 > max_groups * rows) f.r1 = f.r0 + max_groups * rows;
      }
      f.groups = (f.r1 - f.r0 + rows - 1) / rows;
      cursor = f.r1;
    }
    return f;
  };
  if (listed && V + 1 <= kCountKeys) {
    // Every workgroup of this launch holds the sort's LDS, so one fits per
    // CU: the fill workgroups take the CUs the sort leaves, in one round.
    const int64_t nbc = (M + kCountBlock - 1) / kCountBlock;
    const int cus = device_cus();
    const FillShare f = share(kFillCountBytes, true, cus > nbc + 1 ? cus - nbc : 1);
    plan_count<<<unsigned(nbc + f.groups), kCountThreads, 0, s>>>(
        idx, M, V, sk, sv, seg_begin, seg_end, chunk_off, ctab, rows, rbeg, n_rows, n_invalid, f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (V == 0 || D == 0) return hipSuccess;
  } else if (listed) {
    const int32_t* ik = nullptr;
    const int32_t* iv = nullptr;
    for (int p = 0; p < passes; ++p) {
      int32_t* ok = p == passes - 1 ? sk : (p % 2 == 0 ? ak : bk);
      int32_t* ov = p == passes - 1 ? sv : (p % 2 == 0 ? av : bv);
      const FillShare f = share(p == 0 ? kFillFirstPassBytes : kFillPassBytes, false, 0);
      const unsigned grid = unsigned(nb + f.groups);
      if (p == 0)
        radix_pass_fused<true><<<grid, kSortThreads, 0, s>>>(
            idx, ik, iv, M, V, 8 * p, ok, ov, seg_begin, 2 * (V + 1), n_invalid, f);
      else
        radix_pass_fused<false><<<grid, kSortThreads, 0, s>>>(
            idx, ik, iv, M, V, 8 * p, ok, ov, nullptr, 0, nullptr, f);
      ik = ok;
      iv = ov;
    }
    const FillShare f = share(kFillTailBytes, true, 0);
    plan_tail<<<unsigned(1 + f.groups), kPlanThreads, 0, s>>>(sk, M, V, seg_begin, seg_end,
                                                             chunk_off, ctab, rows, rbeg, n_rows,
                                                             n_invalid, f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (V == 0 || D == 0) return hipSuccess;
  } else {
    if ((e = plan_multi(idx, M, V, D, sk, sv, ak, av, bk, bv, hist, nb, seg_begin, seg_end,
                        chunk_off, ctab, n_invalid, s)) != hipSuccess ||
        V == 0 || D == 0)
      return e;
  }
  const FillShare fl = share(-1, false, 0);   // the listed-rows kernel: the rest
#define VJP_SC(T)                                                                            \
  scatter_typed<T>(dy, ld_dy, sv, seg_begin, seg_end, chunk_off, ctab, Q, ldq, nq_max, V, D,    \
                   listed ? rows : nullptr, rbeg, listed ? n_rows : nullptr, dt, ld_dt,       \
                   accumulate,                                                                \
                   vec, pvec, fl, s)
  switch (act) {
    case kF32: return VJP_SC(float);
    case kF16: return VJP_SC(_Float16);
    default: return VJP_SC(bf16);
  }
#undef VJP_SC
}

}  // namespace vjp
