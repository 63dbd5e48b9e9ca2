// Row-wise weighted sum y = x . w: forward and the stage-1 backward.
//
// Source: "Writing Triton Kernels with Autograd: A Minimal End-to-End
// Example" -- section 1 (y[i] = sum_j x[i, j] w[j]), section 2 (tile over
// rows, loop over D, accumulate locally), section 3 (grad_x = dy outer w is
// a map over x; grad_w reduces over the batch, so each tile of rows writes
// one partial row and a second pass sums them), section 4 (the backward
// kernel writes grad_x and the partial row of its tile).
//
// gfx950 mapping.  A row is spread over L consecutive lanes of a wave64
// (L = smallest power of two with L * VEC >= d, at most 64), each lane
// moving VEC elements per access (16 bytes: 8 x bf16/fp16 or 4 x fp32) so a
// wave reads 64 * 16 B contiguous bytes per instruction.  A wave therefore
// covers G = 64 / L rows at once and a 256-thread workgroup 4 G rows; U such
// row groups are loaded before any is used.  Rows wider than 64 * VEC loop
// over column chunks.
//
// Forward: per-lane fp32 dot over its columns, then a DPP reduction over the
// L lanes of the row.  Backward stage 1: workgroup (t, cb) owns row tile t and
// column block cb (64 * VEC columns at most); each lane keeps VEC fp32
// partial sums for its columns over the rows it visits, lanes holding the
// same columns are combined by a butterfly, the 4 waves through LDS in wave
// order, and the tile's partial row is written to P[t][.] -- no atomics.
#include "common.hpp"
#include "launch.hpp"

namespace vjp {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

__device__ __forceinline__ float load_param(const void* __restrict__ w, int64_t j, int dt) {
  if (dt == kF32) return static_cast<const float*>(w)[j];
  if (dt == kF16) return to_f32(static_cast<const _Float16*>(w)[j]);
  return to_f32(static_cast<const bf16*>(w)[j]);
}

template <int VEC>
__device__ __forceinline__ void load_params(const void* __restrict__ w, int64_t col, int64_t d,
                                            int dt, float (&out)[VEC]) {
  // 16-byte loads when this lane's VEC values lie inside the row and start
  // on a 16-byte boundary (VEC fp32 values, or VEC 16-bit ones with VEC a
  // multiple of 8), else one load per element; the same values either way.
  // (The grad_x writers, 32768 short workgroups at 1048576 x 256 bf16, load
  // w first: 175.3 against 177.9 us for the backward with one load per
  // element, interleaved medians of 77 flushed launches.)
  const bool inside = col + VEC <= d;
  if constexpr (VEC % 4 == 0) {
    if (dt == kF32 && inside && (reinterpret_cast<uintptr_t>(static_cast<const float*>(w) + col) % 16) == 0) {
#pragma unroll
      for (int i = 0; i < VEC; i += 4) {
        const Vec<float, 4> f = *reinterpret_cast<const Vec<float, 4>*>(static_cast<const float*>(w) + col + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) out[i + k] = f.v[k];
      }
      return;
    }
  }
  if constexpr (VEC % 8 == 0) {
    const uint16_t* h16 = static_cast<const uint16_t*>(w) + col;
    if (dt != kF32 && inside && (reinterpret_cast<uintptr_t>(h16) % 16) == 0) {
#pragma unroll
      for (int i = 0; i < VEC; i += 8) {
        const Vec<uint16_t, 8> h = *reinterpret_cast<const Vec<uint16_t, 8>*>(h16 + i);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          out[i + k] = dt == kF16 ? to_f32(__builtin_bit_cast(_Float16, h.v[k])) : to_f32(bf16{h.v[k]});
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) out[i] = (col + i < d) ? load_param(w, col + i, dt) : 0.0f;
}

// Forward.  The rows are cut into chunks of U workgroup steps (U * 4 G
// rows); workgroup g takes chunks g, g + gridDim.x, ..., so at any moment the
// workgroups stream neighbouring chunks.  The row loop is uniform across the
// wave (lanes past the last row carry zeros), so the per-row DPP reductions
// always see every lane.  WIDE: rows wider than 64 * VEC elements, whose
// further column chunks are looped over (a separate instantiation, so that
// the common case holds fewer registers).
template <typename T, int VEC, int U, bool WIDE>
__global__ __launch_bounds__(kThreads) void ws_fwd_kernel(const T* __restrict__ x, int64_t ld,
                                                          const void* __restrict__ w, int wdt,
                                                          T* __restrict__ y, int64_t n, int64_t d,
                                                          int L) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int G = kWave / L;
  const int sub = lane / L;
  const int c = lane % L;
  const int64_t cw = int64_t(L) * VEC;                 // columns per chunk
  const int64_t step = int64_t(kWavesPerBlock) * G;    // rows per workgroup step
  const int64_t row_end = n;

  float w0[VEC];
  load_params<VEC>(w, int64_t(c) * VEC, d, wdt, w0);

  for (int64_t q = blockIdx.x; q * U * step < n; q += gridDim.x) {
    const int64_t wbase = q * U * step + int64_t(wave) * G;
    // All U loads in flight before the first is used (rows past the end of
    // the block have nothing available and read as zeros).
    const int64_t col = int64_t(c) * VEC;
    words_t<T, VEC> xw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = wbase + sub + u * step;
      issue_vec<T, VEC>(x + row * ld + col, row < row_end ? d - col : 0, xw[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = wbase + sub + u * step;
      fix_vec<T, VEC>(x + row * ld + col, row < row_end ? d - col : 0, T{}, xw[u]);
    }
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const Vec<T, VEC> xv = as_vec<T, VEC>(xw[u]);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) a = fmaf(to_f32(xv.v[i]), w0[i], a);
      acc[u] = a;
    }
    // Remaining column chunks (rows wider than 64 * VEC elements).
    for (int64_t col0 = cw; WIDE && col0 < d; col0 += cw) {
      const int64_t colk = col0 + int64_t(c) * VEC;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t row = wbase + sub + u * step;
        issue_vec<T, VEC>(x + row * ld + colk, row < row_end ? d - colk : 0, xw[u]);
      }
      float wk[VEC];
      load_params<VEC>(w, colk, d, wdt, wk);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t row = wbase + sub + u * step;
        fix_vec<T, VEC>(x + row * ld + colk, row < row_end ? d - colk : 0, T{}, xw[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const Vec<T, VEC> xk = as_vec<T, VEC>(xw[u]);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[u] = fmaf(to_f32(xk.v[i]), wk[i], acc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float a = group_sum_dpp(acc[u], L);
      const int64_t row = wbase + sub + u * step;
      if (c == 0 && row < row_end) y[row] = from_f32<T>(a);
    }
  }
}

// Row groups per step of a grad_x writer workgroup (their dy values loaded
// together: 182-185 us against 184-192 us one group at a time, 1048576 x 256
// bf16 with 32768 writers, one process).
constexpr int kWriterUnroll = 4;

// Backward stage 1.  grad_x = dy (x) w needs no x, so it is written by its
// own workgroups while others read x for grad_w: workgroups g < readers
// form the partials, the rest write grad_x, side by side, so a pure read
// stream and a pure write stream share HBM (measured on MI355X for
// 1048576 x 256 bf16, old and new in one process: 185-188 us with 512
// readers and 32768 writers on two boxes, against 205 us on one and 186 us
// on the other with every workgroup reading x and writing its grad_x rows).
//
// Readers.  Rows are cut into blocks of block_rows rows; tile t holds blocks
// t, t + tiles, t + 2 tiles, ... (with tiles = number of blocks this is one
// contiguous block per tile).  Reader (g, cb) takes tiles r, r + readers,
// ... with r = xcd_group(g, readers), and column block cb, so that readers
// of neighbouring tiles (whose dy values share cache lines) run on one XCD.
// Each lane accumulates VEC fp32 partials over its rows in increasing row
// order; the lanes holding the same columns are combined by a butterfly and
// the four waves through LDS in wave order, and the tile's partial row is
// written to P[t][.].  Which reader forms a tile does not change its partial.
//
// Writers.  Writer (h, cb) writes grad_x for column block cb and the spans of
// kWriterUnroll row groups (4 G consecutive rows each) numbered
// m, m + writers, ... with m = xcd_group(h, writers): each span's dy values
// are one contiguous run, and neighbouring spans run on one XCD.
// grad_x[i, j] = dy[i] w[j], one fp32 product rounded once.
template <typename T, int VEC, int U>
__global__ __launch_bounds__(kThreads) void ws_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ x, int64_t ld_x, const void* __restrict__ w,
    int wdt, T* __restrict__ dx, int64_t ld_dx, float* __restrict__ P, int64_t n, int64_t d,
    int L, int block_rows, int64_t tiles, int64_t readers) {
  __shared__ float red[kWavesPerBlock][kWave * VEC];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform per wave
  const int G = kWave / L;
  const int sub = lane / L;
  const int c = lane % L;
  const int64_t col0 = int64_t(blockIdx.y) * L * VEC;
  const int64_t col = col0 + int64_t(c) * VEC;
  const int64_t cols_left = d - col;
  if (int64_t(blockIdx.x) >= readers) {
    float wr[VEC];
    load_params<VEC>(w, col, d, wdt, wr);
    const int64_t writers = int64_t(gridDim.x) - readers;
    const int64_t me = xcd_group(int64_t(blockIdx.x) - readers, writers);
    // One span of kWriterUnroll row groups per step: their dy values are
    // loaded together (rows past the end read dy[n - 1] and store nothing).
    const int64_t group = int64_t(kWavesPerBlock) * G;
    const int64_t span = int64_t(kWriterUnroll) * group;
    for (int64_t r0 = me * span; r0 < n; r0 += writers * span) {
      T gv[kWriterUnroll];
#pragma unroll
      for (int u = 0; u < kWriterUnroll; ++u) {
        const int64_t row = r0 + u * group + int64_t(wave) * G + sub;
        gv[u] = dy[row < n ? row : n - 1];
      }
#pragma unroll
      for (int u = 0; u < kWriterUnroll; ++u) {
        const int64_t row = r0 + u * group + int64_t(wave) * G + sub;
        if (row < n && cols_left > 0) {
          const float g = to_f32(gv[u]);
          float gx[VEC];
#pragma unroll
          for (int i = 0; i < VEC; ++i) gx[i] = g * wr[i];
          store_f32_tail<T, VEC>(dx + row * ld_dx + col, cols_left, gx);
        }
      }
    }
    return;
  }
  // The four waves interleave: one workgroup step covers 4 G consecutive rows
  // (wave w takes rows w G .. w G + G - 1 of it, one per L-lane group), so a
  // workgroup streams one contiguous window of a block.  Row indices are
  // relative to the block; loop bounds are uniform across the wave.
  const int wg_rows = kWavesPerBlock * G;
  const int my_row = wave * G + sub;
  const int64_t xstep = int64_t(wg_rows) * ld_x;

  for (int64_t tile = xcd_group(blockIdx.x, readers); tile < tiles; tile += readers) {
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
    for (int64_t r0 = tile * block_rows; r0 < n; r0 += tiles * block_rows) {
      const int nrows = int(min(int64_t(block_rows), n - r0));
      const T* __restrict__ gw = dy + r0;
      const T* __restrict__ xp = x + (r0 + my_row) * ld_x + col;
      for (int base = 0; base < nrows; base += U * wg_rows) {
        // Rows stay in storage type until used; all U row loads (and the dy
        // values, read at a clamped row and zeroed past the end) are in
        // flight before the first is used.
        words_t<T, VEC> xw[U];
        T gr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = base + u * wg_rows + my_row;
          gr[u] = gw[r < nrows ? r : nrows - 1];
          issue_vec<T, VEC>(xp + u * xstep, r < nrows ? cols_left : 0, xw[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = base + u * wg_rows + my_row;
          fix_vec<T, VEC>(xp + u * xstep, r < nrows ? cols_left : 0, T{}, xw[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = base + u * wg_rows + my_row;
          const float g = r < nrows ? to_f32(gr[u]) : 0.0f;
          const Vec<T, VEC> xr = as_vec<T, VEC>(xw[u]);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] = fmaf(to_f32(xr.v[i]), g, acc[i]);
        }
        xp += U * xstep;
      }
    }

    // Lanes c, c + L, c + 2L, ... hold the same columns: butterfly over them.
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      for (int o = L; o < kWave; o <<= 1) acc[i] += __shfl_xor(acc[i], o, kWave);
    if (sub == 0) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) red[wave][c * VEC + i] = acc[i];
    }
    lds_barrier();
    if (wave == 0 && sub == 0) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        float s = red[0][c * VEC + i];
#pragma unroll
        for (int k = 1; k < kWavesPerBlock; ++k) s += red[k][c * VEC + i];
        if (col + i < d) P[tile * d + col + i] = s;
      }
    }
    lds_barrier();   // red is reused by the next tile of this workgroup
  }
}

int lanes_per_row(int64_t d, int vec) {
  int L = 1;
  while (L < kWave && int64_t(L) * vec < d) L <<= 1;
  return L;
}

// Launch shapes (measured on MI355X for 1048576 x 256 bf16): the forward
// keeps four row groups per lane in flight, in chunks dealt to at most 8192
// workgroups (86 us; contiguous blocks of 512 rows per workgroup with one
// row group per step, 89.5 us); the backward keeps four row groups per lane
// in flight in up to 512 reader workgroups (which loop over the tiles beyond
// that; one row group: 235 us, two: 188 us, four: 185 us) beside up to
// 32768 writer workgroups (four row groups each at this size).  More tiles
// and readers (1024 to 4096 of each) or 16384 writers took 185-206 us.
// A later sweep of the forward under cache-flushed medians of 20 (one
// process): 83.6-85.2 us here; 2, 8 or 16 row groups per lane with 2048 to
// 32768 workgroups 83.9-125.9 us, none better by more than the run-to-run
// spread.  The one 16-bit y store per row (a lane per row) costs at most
// 1.5 us: 80.5 against 82.0 us with the stores taken out (interleaved
// medians of 77), less than an LDS exchange to widen them would add.
constexpr int kFwdUnroll = 4;
constexpr int64_t kFwdMaxGrid = 8192;
constexpr int kBwdUnroll = 4;
constexpr int64_t kBwdReaders = 512;
constexpr int64_t kBwdWriters = 32768;

template <typename T>
hipError_t fwd_typed(const void* x, int64_t ld_x, const void* w, int wdt, void* y, int64_t n,
                     int64_t d, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  const int v = vec ? V : 1;
  const int L = lanes_per_row(d, v);
  const int64_t rows_per_chunk = int64_t(kWavesPerBlock) * (kWave / L) * kFwdUnroll;
  const int64_t chunks = (n + rows_per_chunk - 1) / rows_per_chunk;
  const dim3 grid(unsigned(chunks < kFwdMaxGrid ? chunks : kFwdMaxGrid));
  const bool wide = d > int64_t(kWave) * v;
  const T* xp = static_cast<const T*>(x);
  T* yp = static_cast<T*>(y);
  if (vec && wide)
    ws_fwd_kernel<T, V, kFwdUnroll, true><<<grid, kThreads, 0, s>>>(xp, ld_x, w, wdt, yp, n, d, L);
  else if (vec)
    ws_fwd_kernel<T, V, kFwdUnroll, false><<<grid, kThreads, 0, s>>>(xp, ld_x, w, wdt, yp, n, d, L);
  else if (wide)
    ws_fwd_kernel<T, 1, kFwdUnroll, true><<<grid, kThreads, 0, s>>>(xp, ld_x, w, wdt, yp, n, d, L);
  else
    ws_fwd_kernel<T, 1, kFwdUnroll, false><<<grid, kThreads, 0, s>>>(xp, ld_x, w, wdt, yp, n, d, L);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_typed(const void* dy, const void* x, int64_t ld_x, const void* w, int wdt,
                     void* dx, int64_t ld_dx, float* P, int64_t n, int64_t d, int block_rows,
                     int64_t tiles, bool vec, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  const int v = vec ? V : 1;
  const int L = lanes_per_row(d, v);
  const int64_t cw = int64_t(L) * v;
  const int64_t readers = tiles < kBwdReaders ? tiles : kBwdReaders;
  const int64_t span = int64_t(kWavesPerBlock) * (kWave / L) * kWriterUnroll;
  const int64_t spans = (n + span - 1) / span;
  const int64_t writers = spans < kBwdWriters ? spans : kBwdWriters;
  const dim3 grid(unsigned(readers + writers), unsigned((d + cw - 1) / cw));
  if (vec)
    ws_bwd_kernel<T, V, kBwdUnroll><<<grid, kThreads, 0, s>>>(
        static_cast<const T*>(dy), static_cast<const T*>(x), ld_x, w, wdt, static_cast<T*>(dx),
        ld_dx, P, n, d, L, block_rows, tiles, readers);
  else
    ws_bwd_kernel<T, 1, kBwdUnroll><<<grid, kThreads, 0, s>>>(
        static_cast<const T*>(dy), static_cast<const T*>(x), ld_x, w, wdt, static_cast<T*>(dx),
        ld_dx, P, n, d, L, block_rows, tiles, readers);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_weighted_sum_fwd(const void* x, int64_t ld_x, const void* w, void* y,
                                   int64_t n, int64_t d, int act, int wdt, bool vec,
                                   hipStream_t s) {
  switch (act) {
    case kF32: return fwd_typed<float>(x, ld_x, w, wdt, y, n, d, vec, s);
    case kF16: return fwd_typed<_Float16>(x, ld_x, w, wdt, y, n, d, vec, s);
    default: return fwd_typed<bf16>(x, ld_x, w, wdt, y, n, d, vec, s);
  }
}

hipError_t launch_weighted_sum_bwd_stage1(const void* dy, const void* x, int64_t ld_x,
                                          const void* w, void* dx, int64_t ld_dx, float* P,
                                          int64_t n, int64_t d, int block_rows, int64_t tiles,
                                          int act, int wdt, bool vec, hipStream_t s) {
  switch (act) {
    case kF32: return bwd_typed<float>(dy, x, ld_x, w, wdt, dx, ld_dx, P, n, d, block_rows, tiles, vec, s);
    case kF16: return bwd_typed<_Float16>(dy, x, ld_x, w, wdt, dx, ld_dx, P, n, d, block_rows, tiles, vec, s);
    default: return bwd_typed<bf16>(dy, x, ld_x, w, wdt, dx, ld_dx, P, n, d, block_rows, tiles, vec, s);
  }
}

}  // namespace vjp
