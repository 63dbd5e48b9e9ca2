// The libvjp C ABI (declared in include/libvjp.h): argument validation,
// workspace sizing, choice of the 128-bit or element-wise kernel variant,
// and the launch sequence of each entry point.  Nothing here allocates device
// memory or synchronises the host.
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>
#include <mutex>

#include "launch.hpp"
#include "libvjp.h"

#define VJP_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace vjp;

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return VJP_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(VJP_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Sizes beyond this are rejected so that no element offset can overflow int64.
constexpr int64_t kMaxElems = int64_t(1) << 46;
// Widest rows of the ops whose launches put column blocks in the second grid
// dimension (at most 65535 blocks): the weighted-sum backward (blocks of 64
// columns in its narrowest form) and the row gather / scatter-add (blocks of
// 256 columns).
constexpr int64_t kWsMaxCols = int64_t(65535) * 64;
constexpr int64_t kGatherMaxCols = int64_t(65535) * 256;
// Widest rows of the split cross-entropy backward, which also puts column
// blocks in the second grid dimension: 4096 columns a block when its rows are
// not 16-byte aligned (1024 threads x 4 elements).
constexpr int64_t kXentBwdMaxClasses = int64_t(65535) * 4096;
// Rows per launch of the row kernels (keeps every grid far below 2^31 threads).
constexpr int64_t kRowsPerLaunch = int64_t(1) << 20;

bool dtype_ok(int dt) { return dt == kF32 || dt == kF16 || dt == kBF16; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo = 0, hi = 0;
  const char* name = "";
};

Range span(const void* p, int64_t bytes, const char* name) {
  Range r;
  r.name = name;
  if (p && bytes > 0) {
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + uint64_t(bytes);
  }
  return r;
}

// Bytes touched by a row-major [rows, cols] matrix with leading dimension ld.
int64_t mat_bytes(int64_t rows, int64_t cols, int64_t ld, int esize) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((rows - 1) * ld + cols) * esize;
}

bool overlaps(const Range& a, const Range& b) {
  return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}

int check_alias(std::initializer_list<Range> outs, std::initializer_list<Range> ins) {
  for (const Range* o = outs.begin(); o != outs.end(); ++o) {
    for (const Range& i : ins)
      if (overlaps(*o, i)) return fail(VJP_EALIAS, "output %s overlaps input %s", o->name, i.name);
    for (const Range* p = o + 1; p != outs.end(); ++p)
      if (overlaps(*o, *p)) return fail(VJP_EALIAS, "outputs %s and %s overlap", o->name, p->name);
  }
  return VJP_OK;
}

int check_matrix(const char* name, const void* p, int64_t rows, int64_t cols, int64_t ld,
                 int esize) {
  if (ld < cols) return fail(VJP_EINVAL, "%s: ld (%lld) < columns (%lld)", name, (long long)ld, (long long)cols);
  if (rows > 0 && cols > 0) {
    if (!p) return fail(VJP_EINVAL, "%s is NULL", name);
    if (!aligned(p, esize)) return fail(VJP_EALIGN, "%s is not aligned to its element size", name);
    if (ld > kMaxElems || rows > kMaxElems || (rows - 1) > kMaxElems / (ld > 0 ? ld : 1))
      return fail(VJP_EINVAL, "%s: size too large", name);
  }
  return VJP_OK;
}

int check_vector(const char* name, const void* p, int64_t n, int esize) {
  if (n > 0) {
    if (!p) return fail(VJP_EINVAL, "%s is NULL", name);
    if (!aligned(p, esize)) return fail(VJP_EALIGN, "%s is not aligned to its element size", name);
  }
  return VJP_OK;
}

// 128-bit accesses need 16-byte aligned rows.
bool rows_vec_ok(const void* p, int64_t ld, int esize) {
  return aligned(p, 16) && ((ld * esize) % 16) == 0;
}

#define VJP_TRY(expr)          \
  do {                         \
    const int _st = (expr);    \
    if (_st != VJP_OK) return _st; \
  } while (0)

// Row tiling of the weighted-sum backward.  An explicit rows_per_tile gives
// contiguous tiles of that many rows.  The automatic tiling cuts the rows into
// blocks of kAutoBlockRows and deals them round-robin to at most kAutoTiles
// tiles, so that the workgroups, one per tile, stream neighbouring blocks at
// the same time (measured on MI355X: about 15 % more bandwidth than
// contiguous tiles of 512 rows for 1048576 x 256 bf16; 1024 tiles, four
// workgroups per CU, beat 512, 768, 1280, 1536, 2048 and 4096).
constexpr int64_t kAutoBlockRows = 32;
constexpr int64_t kMaxRowsPerTile = int64_t(1) << 30;
constexpr int64_t kAutoTiles = 1024;

struct WsTiling {
  int64_t block_rows, tiles;
};

WsTiling resolve_ws_tiling(int64_t n_rows, int64_t rpt) {
  if (rpt > 0) return {rpt, (n_rows + rpt - 1) / rpt};
  const int64_t blocks = (n_rows + kAutoBlockRows - 1) / kAutoBlockRows;
  return {kAutoBlockRows, blocks < kAutoTiles ? blocks : kAutoTiles};
}

int64_t resolve_elems_per_tile(int64_t n) {
  const int64_t per = (n + 4095) / 4096;
  const int64_t e = ((per + 2047) / 2048) * 2048;
  return e < 2048 ? 2048 : e;
}

}  // namespace

VJP_API int vjp_version(void) { return VJP_VERSION; }

VJP_API const char* vjp_status_string(int status) {
  switch (status) {
    case VJP_OK: return "ok";
    case VJP_EINVAL: return "invalid argument";
    case VJP_EDTYPE: return "unknown dtype";
    case VJP_EALIGN: return "misaligned pointer";
    case VJP_EWORKSPACE: return "workspace missing or too small";
    case VJP_EALIAS: return "output overlaps another buffer";
    case VJP_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

VJP_API const char* vjp_last_error(void) { return g_err; }

VJP_API int vjp_copy(const void* src, void* dst, int64_t bytes, vjp_stream_t stream) {
  if (bytes < 0) return fail(VJP_EINVAL, "negative size");
  if (bytes == 0) return ok();
  if (!src || !dst) return fail(VJP_EINVAL, "NULL pointer");
  VJP_TRY(check_alias({span(dst, bytes, "dst")}, {span(src, bytes, "src")}));
  return hip_status(launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream)), "copy");
}

VJP_API int vjp_copy_shaped(const void* src, void* dst, int64_t bytes, int vectors_per_lane,
                            int64_t max_workgroups, vjp_stream_t stream) {
  if (bytes < 0) return fail(VJP_EINVAL, "negative size");
  if (vectors_per_lane != 1 && vectors_per_lane != 2 && vectors_per_lane != 4 &&
      vectors_per_lane != 8)
    return fail(VJP_EINVAL, "vectors_per_lane must be 1, 2, 4 or 8");
  if (max_workgroups < 1 || max_workgroups > (int64_t(1) << 31) - 1)
    return fail(VJP_EINVAL, "max_workgroups must be in [1, 2^31 - 1]");
  if (bytes == 0) return ok();
  if (!src || !dst) return fail(VJP_EINVAL, "NULL pointer");
  VJP_TRY(check_alias({span(dst, bytes, "dst")}, {span(src, bytes, "src")}));
  return hip_status(launch_copy_shaped(src, dst, bytes, vectors_per_lane, max_workgroups,
                                       static_cast<hipStream_t>(stream)),
                    "copy");
}

// ------------------------------------------------------------------ weighted sum

VJP_API int vjp_weighted_sum_fwd(const void* x, int64_t ld_x, const void* w, void* y,
                                 int64_t n_rows, int64_t d, vjp_dtype_t act, vjp_dtype_t w_dtype,
                                 vjp_stream_t stream) {
  if (!dtype_ok(act) || !dtype_ok(w_dtype)) return fail(VJP_EDTYPE, "unknown dtype");
  if (n_rows < 0 || d < 0) return fail(VJP_EINVAL, "negative size");
  if (n_rows > kMaxElems || d > kMaxElems) return fail(VJP_EINVAL, "size too large");
  const int es = dtype_size(act), ws = dtype_size(w_dtype);
  VJP_TRY(check_matrix("x", x, n_rows, d, ld_x, es));
  VJP_TRY(check_vector("w", w, d, ws));
  VJP_TRY(check_vector("y", y, n_rows, es));
  VJP_TRY(check_alias({span(y, n_rows * es, "y")},
                      {span(x, mat_bytes(n_rows, d, ld_x, es), "x"), span(w, d * ws, "w")}));
  if (n_rows == 0) return ok();
  const bool vec = rows_vec_ok(x, ld_x, es);
  return hip_status(launch_weighted_sum_fwd(x, ld_x, w, y, n_rows, d, act, w_dtype, vec,
                                            static_cast<hipStream_t>(stream)),
                    "weighted_sum_fwd");
}

VJP_API int vjp_weighted_sum_tiling(int64_t n_rows, int64_t rows_per_tile, int64_t* block_rows,
                                    int64_t* tiles) {
  if (n_rows < 0 || rows_per_tile < 0) return fail(VJP_EINVAL, "negative size");
  if (rows_per_tile > kMaxRowsPerTile) return fail(VJP_EINVAL, "rows_per_tile above 2^30");
  if (!block_rows || !tiles) return fail(VJP_EINVAL, "null output pointer");
  const WsTiling t = resolve_ws_tiling(n_rows, rows_per_tile);
  *block_rows = t.block_rows;
  *tiles = t.tiles;
  return ok();
}

VJP_API size_t vjp_weighted_sum_bwd_workspace_size(int64_t n_rows, int64_t d,
                                                   int64_t rows_per_tile) {
  if (n_rows < 0 || d < 0 || rows_per_tile < 0 || rows_per_tile > kMaxRowsPerTile) return 0;
  return size_t(resolve_ws_tiling(n_rows, rows_per_tile).tiles) * size_t(d) * sizeof(float);
}

VJP_API int vjp_weighted_sum_bwd(const void* dy, const void* x, int64_t ld_x, const void* w,
                                 void* dx, int64_t ld_dx, float* dw, int accumulate,
                                 int64_t n_rows, int64_t d, int64_t rows_per_tile, vjp_dtype_t act,
                                 vjp_dtype_t w_dtype, void* workspace, size_t workspace_bytes,
                                 vjp_stream_t stream) {
  if (!dtype_ok(act) || !dtype_ok(w_dtype)) return fail(VJP_EDTYPE, "unknown dtype");
  if (n_rows < 0 || d < 0 || rows_per_tile < 0) return fail(VJP_EINVAL, "negative size");
  if (n_rows > kMaxElems || d > kMaxElems) return fail(VJP_EINVAL, "size too large");
  if (d > kWsMaxCols) return fail(VJP_EINVAL, "d above %lld", (long long)kWsMaxCols);
  if (rows_per_tile > kMaxRowsPerTile) return fail(VJP_EINVAL, "rows_per_tile above 2^30");
  if (accumulate != 0 && accumulate != 1) return fail(VJP_EINVAL, "accumulate must be 0 or 1");
  const int es = dtype_size(act), ws = dtype_size(w_dtype);
  VJP_TRY(check_vector("dy", dy, n_rows, es));
  VJP_TRY(check_matrix("x", x, n_rows, d, ld_x, es));
  VJP_TRY(check_vector("w", w, d, ws));
  VJP_TRY(check_matrix("dx", dx, n_rows, d, ld_dx, es));
  VJP_TRY(check_vector("dw", dw, d, 4));
  const size_t need = vjp_weighted_sum_bwd_workspace_size(n_rows, d, rows_per_tile);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(VJP_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 4)) return fail(VJP_EALIGN, "workspace is not 4-byte aligned");
  }
  VJP_TRY(check_alias({span(dx, mat_bytes(n_rows, d, ld_dx, es), "dx"), span(dw, d * 4, "dw"),
                       span(workspace, int64_t(need), "workspace")},
                      {span(dy, n_rows * es, "dy"), span(x, mat_bytes(n_rows, d, ld_x, es), "x"),
                       span(w, d * ws, "w")}));
  if (d == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const WsTiling tl = resolve_ws_tiling(n_rows, rows_per_tile);
  const int64_t T = tl.tiles;
  float* P = static_cast<float*>(workspace);
  if (T > 0) {
    const bool vec = rows_vec_ok(x, ld_x, es) && rows_vec_ok(dx, ld_dx, es);
    const hipError_t e = launch_weighted_sum_bwd_stage1(dy, x, ld_x, w, dx, ld_dx, P, n_rows, d,
                                                        int(tl.block_rows), T, act, w_dtype, vec,
                                                        s);
    if (e != hipSuccess) return hip_status(e, "weighted_sum_bwd stage 1");
  }
  return hip_status(launch_reduce_partials(P, T, d, dw, accumulate, s), "weighted_sum_bwd stage 2");
}

// ------------------------------------------------------------------ scaled SiLU

VJP_API int vjp_scaled_silu_fwd(const void* x, const float* w, void* y, int64_t n, vjp_dtype_t act,
                                vjp_stream_t stream) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (n < 0) return fail(VJP_EINVAL, "negative size");
  if (n > kMaxElems) return fail(VJP_EINVAL, "size too large");
  const int es = dtype_size(act);
  VJP_TRY(check_vector("x", x, n, es));
  VJP_TRY(check_vector("w", w, n > 0 ? 1 : 0, 4));
  VJP_TRY(check_vector("y", y, n, es));
  VJP_TRY(check_alias({span(y, n * es, "y")}, {span(x, n * es, "x"), span(w, 4, "w")}));
  if (n == 0) return ok();
  const bool vec = aligned(x, 16) && aligned(y, 16);
  return hip_status(launch_scaled_silu_fwd(x, w, y, n, act, vec, static_cast<hipStream_t>(stream)),
                    "scaled_silu_fwd");
}

VJP_API int64_t vjp_scaled_silu_elems_per_tile(int64_t n) {
  if (n < 0) return -1;
  return resolve_elems_per_tile(n);
}

VJP_API size_t vjp_scaled_silu_bwd_workspace_size(int64_t n) {
  if (n < 0) return 0;
  const int64_t e = resolve_elems_per_tile(n);
  return size_t((n + e - 1) / e) * sizeof(float);
}

namespace {

// Shared body of the two scaled-SiLU backwards: validation of everything but
// the partials buffer P (T = tiles(n) floats, checked by the caller), then
// stage 1 and the fixed-order stage 2.
int scaled_silu_bwd_impl(const void* dy, const void* x, const float* w, void* dx, float* dw,
                         int accumulate, int64_t n, int act, Range scratch, float* P,
                         vjp_stream_t stream) {
  const int es = dtype_size(act);
  VJP_TRY(check_alias({span(dx, n * es, "dx"), span(dw, 4, "dw"), scratch},
                      {span(dy, n * es, "dy"), span(x, n * es, "x"), span(w, n > 0 ? 4 : 0, "w")}));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ept = resolve_elems_per_tile(n);
  const int64_t T = (n + ept - 1) / ept;
  if (T > 0) {
    const bool vec = aligned(dy, 16) && aligned(x, 16) && aligned(dx, 16);
    const hipError_t e = launch_scaled_silu_bwd_stage1(dy, x, w, dx, P, n, ept, act, vec, s);
    if (e != hipSuccess) return hip_status(e, "scaled_silu_bwd stage 1");
  }
  return hip_status(launch_reduce_partials(P, T, 1, dw, accumulate, s), "scaled_silu_bwd stage 2");
}

int scaled_silu_bwd_args(const void* dy, const void* x, const float* w, void* dx, float* dw,
                         int accumulate, int64_t n, int act) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (n < 0) return fail(VJP_EINVAL, "negative size");
  if (n > kMaxElems) return fail(VJP_EINVAL, "size too large");
  if (accumulate != 0 && accumulate != 1) return fail(VJP_EINVAL, "accumulate must be 0 or 1");
  const int es = dtype_size(act);
  VJP_TRY(check_vector("dy", dy, n, es));
  VJP_TRY(check_vector("x", x, n, es));
  VJP_TRY(check_vector("w", w, n > 0 ? 1 : 0, 4));
  VJP_TRY(check_vector("dx", dx, n, es));
  VJP_TRY(check_vector("dw", dw, 1, 4));
  return VJP_OK;
}

}  // namespace

VJP_API int vjp_scaled_silu_bwd(const void* dy, const void* x, const float* w, void* dx,
                                float* dw, int accumulate, int64_t n, vjp_dtype_t act, void* workspace,
                                size_t workspace_bytes, vjp_stream_t stream) {
  VJP_TRY(scaled_silu_bwd_args(dy, x, w, dx, dw, accumulate, n, act));
  const size_t need = vjp_scaled_silu_bwd_workspace_size(n);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(VJP_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 4)) return fail(VJP_EALIGN, "workspace is not 4-byte aligned");
  }
  return scaled_silu_bwd_impl(dy, x, w, dx, dw, accumulate, n, act,
                              span(workspace, int64_t(need), "workspace"),
                              static_cast<float*>(workspace), stream);
}

// ------------------------------------------------------------------ no-allocation variant
//
// Scratch of vjp_scaled_silu_bwd_noalloc: the stage-1 partials, one float per
// tile.  The tiling never forms more than 4096 tiles (resolve_elems_per_tile),
// so 16 KB serve every n.  A __device__ array: each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and only that address reaches kernels.
constexpr int64_t kNoallocScratchFloats = 4096;
static __device__ __align__(256) float scratch[kNoallocScratchFloats];

namespace {

constexpr int kMaxDevices = 256;
std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the calling thread's current device.
hipError_t scratch_address(float** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<float*>(p) : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

VJP_API int vjp_scaled_silu_bwd_noalloc(const void* dy, const void* x, const float* w, void* dx,
                                        float* dw, int accumulate, int64_t n, vjp_dtype_t act,
                                        vjp_stream_t stream) {
  VJP_TRY(scaled_silu_bwd_args(dy, x, w, dx, dw, accumulate, n, act));
  const int64_t ept = resolve_elems_per_tile(n);
  const int64_t T = (n + ept - 1) / ept;
  if (T > kNoallocScratchFloats)
    return fail(VJP_EINVAL, "n = %lld needs %lld partials, above the %lld of the scratch",
                static_cast<long long>(n), static_cast<long long>(T),
                static_cast<long long>(kNoallocScratchFloats));
  float* P = nullptr;
  if (T > 0) {
    const hipError_t e = scratch_address(&P);
    if (e != hipSuccess) return hip_status(e, "scaled_silu_bwd_noalloc scratch address");
  }
  return scaled_silu_bwd_impl(dy, x, w, dx, dw, accumulate, n, act,
                              span(P, T * int64_t(sizeof(float)), "scratch"), P, stream);
}

// ------------------------------------------------------------------ softmax

namespace {

// Shared body of the two softmax forwards (row_lse null: y required).
int softmax_fwd_impl(const void* x, int64_t ld_x, void* y, int64_t ld_y, float* row_lse,
                     int64_t rows, int64_t cols, int act, vjp_stream_t stream) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (rows < 0 || cols < 0) return fail(VJP_EINVAL, "negative size");
  if (rows > 0 && cols == 0) return fail(VJP_EINVAL, "softmax over zero columns");
  const int es = dtype_size(act);
  VJP_TRY(check_matrix("x", x, rows, cols, ld_x, es));
  if (y != nullptr || row_lse == nullptr) VJP_TRY(check_matrix("y", y, rows, cols, ld_y, es));
  if (row_lse != nullptr) VJP_TRY(check_vector("row_lse", row_lse, rows, 4));
  VJP_TRY(check_alias({span(y, y ? mat_bytes(rows, cols, ld_y, es) : 0, "y"),
                       span(row_lse, row_lse ? rows * 4 : 0, "row_lse")},
                      {span(x, mat_bytes(rows, cols, ld_x, es), "x")}));
  const bool vec = rows_vec_ok(x, ld_x, es) && (y == nullptr || rows_vec_ok(y, ld_y, es));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
    const hipError_t e = launch_softmax_fwd(
        static_cast<const char*>(x) + r0 * ld_x * es, ld_x,
        y ? static_cast<char*>(y) + r0 * ld_y * es : nullptr, ld_y,
        row_lse ? row_lse + r0 : nullptr, nr, cols, act, vec, s);
    if (e != hipSuccess) return hip_status(e, "softmax_fwd");
  }
  return ok();
}

// Shared body of the two softmax backwards (row_lse null: src is y, else x).
int softmax_bwd_impl(const void* dy, int64_t ld_dy, const void* src, int64_t ld_src,
                     const float* row_lse, void* dx, int64_t ld_dx, int64_t rows, int64_t cols,
                     int act, vjp_stream_t stream) {
  const char* src_name = row_lse ? "x" : "y";
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (rows < 0 || cols < 0) return fail(VJP_EINVAL, "negative size");
  if (rows > 0 && cols == 0) return fail(VJP_EINVAL, "softmax over zero columns");
  const int es = dtype_size(act);
  VJP_TRY(check_matrix("dy", dy, rows, cols, ld_dy, es));
  VJP_TRY(check_matrix(src_name, src, rows, cols, ld_src, es));
  VJP_TRY(check_matrix("dx", dx, rows, cols, ld_dx, es));
  VJP_TRY(check_alias({span(dx, mat_bytes(rows, cols, ld_dx, es), "dx")},
                      {span(dy, mat_bytes(rows, cols, ld_dy, es), "dy"),
                       span(src, mat_bytes(rows, cols, ld_src, es), src_name),
                       span(row_lse, row_lse ? rows * 4 : 0, "row_lse")}));
  const bool vec = rows_vec_ok(dy, ld_dy, es) && rows_vec_ok(src, ld_src, es) &&
                   rows_vec_ok(dx, ld_dx, es);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
    const hipError_t e = launch_softmax_bwd(
        static_cast<const char*>(dy) + r0 * ld_dy * es, ld_dy,
        static_cast<const char*>(src) + r0 * ld_src * es, ld_src,
        row_lse ? row_lse + r0 : nullptr, static_cast<char*>(dx) + r0 * ld_dx * es, ld_dx, nr,
        cols, act, vec, s);
    if (e != hipSuccess) return hip_status(e, "softmax_bwd");
  }
  return ok();
}

}  // namespace

VJP_API int vjp_softmax_fwd(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows,
                            int64_t cols, vjp_dtype_t act, vjp_stream_t stream) {
  return softmax_fwd_impl(x, ld_x, y, ld_y, nullptr, rows, cols, act, stream);
}

VJP_API int vjp_softmax_bwd(const void* dy, int64_t ld_dy, const void* y, int64_t ld_y,
                            void* dx, int64_t ld_dx, int64_t rows, int64_t cols, vjp_dtype_t act,
                            vjp_stream_t stream) {
  return softmax_bwd_impl(dy, ld_dy, y, ld_y, nullptr, dx, ld_dx, rows, cols, act, stream);
}

VJP_API int vjp_softmax_fwd_lse(const void* x, int64_t ld_x, void* y, int64_t ld_y,
                                float* row_lse, int64_t rows, int64_t cols, vjp_dtype_t act,
                                vjp_stream_t stream) {
  if (row_lse == nullptr && rows > 0) return fail(VJP_EINVAL, "row_lse is null");
  if (y == nullptr) ld_y = cols;   // ignored
  if (row_lse == nullptr && y == nullptr) return rows < 0 || cols < 0 ? fail(VJP_EINVAL, "negative size") : ok();
  return softmax_fwd_impl(x, ld_x, y, ld_y, row_lse, rows, cols, act, stream);
}

VJP_API int vjp_softmax_bwd_lse(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x,
                                const float* row_lse, void* dx, int64_t ld_dx, int64_t rows,
                                int64_t cols, vjp_dtype_t act, vjp_stream_t stream) {
  if (row_lse == nullptr && rows > 0) return fail(VJP_EINVAL, "row_lse is null");
  if (row_lse != nullptr && !aligned(row_lse, 4)) return fail(VJP_EALIGN, "row_lse is not 4-byte aligned");
  if (rows == 0) return softmax_bwd_impl(dy, ld_dy, x, ld_x, nullptr, dx, ld_dx, 0, cols, act, stream);
  return softmax_bwd_impl(dy, ld_dy, x, ld_x, row_lse, dx, ld_dx, rows, cols, act, stream);
}

// ------------------------------------------------------------------ softmax cross-entropy

VJP_API size_t vjp_softmax_xent_workspace_size(int64_t rows) {
  return rows > 0 ? size_t(rows) * sizeof(float) : 0;
}

VJP_API int vjp_softmax_xent_fwd_bwd(const void* logits, int64_t ld, const int32_t* targets,
                                     int64_t rows, int64_t classes, vjp_dtype_t act, float grad_scale,
                                     float* loss, float* row_max, float* row_lse, void* dlogits,
                                     int64_t ld_dlogits, int32_t* n_invalid, void* workspace,
                                     size_t workspace_bytes, vjp_stream_t stream) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (rows < 0 || classes < 0) return fail(VJP_EINVAL, "negative size");
  if (classes == 0) return fail(VJP_EINVAL, "cross-entropy over zero classes");
  if (classes > INT32_MAX) return fail(VJP_EINVAL, "classes beyond int32 targets");
  const int es = dtype_size(act);
  VJP_TRY(check_matrix("logits", logits, rows, classes, ld, es));
  VJP_TRY(check_vector("targets", targets, rows, 4));
  VJP_TRY(check_vector("loss", loss, 1, 4));
  VJP_TRY(check_vector("row_max", row_max, rows, 4));
  VJP_TRY(check_vector("row_lse", row_lse, rows, 4));
  VJP_TRY(check_matrix("dlogits", dlogits, rows, classes, ld_dlogits, es));
  if (n_invalid && !aligned(n_invalid, 4)) return fail(VJP_EALIGN, "n_invalid is not 4-byte aligned");
  const size_t need = vjp_softmax_xent_workspace_size(rows);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(VJP_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 4)) return fail(VJP_EALIGN, "workspace is not 4-byte aligned");
  }
  VJP_TRY(check_alias({span(loss, 4, "loss"), span(row_max, rows * 4, "row_max"),
                       span(row_lse, rows * 4, "row_lse"),
                       span(dlogits, mat_bytes(rows, classes, ld_dlogits, es), "dlogits"),
                       span(n_invalid, n_invalid ? 4 : 0, "n_invalid"),
                       span(workspace, int64_t(need), "workspace")},
                      {span(logits, mat_bytes(rows, classes, ld, es), "logits"),
                       span(targets, rows * 4, "targets")}));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  float* row_loss = static_cast<float*>(workspace);
  const bool vec = rows_vec_ok(logits, ld, es) && rows_vec_ok(dlogits, ld_dlogits, es);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
    const hipError_t e = launch_softmax_xent(
        static_cast<const char*>(logits) + r0 * ld * es, ld, targets + r0, nr, classes, act,
        grad_scale, row_max + r0, row_lse + r0, row_loss + r0,
        static_cast<char*>(dlogits) + r0 * ld_dlogits * es, ld_dlogits, vec, s);
    if (e != hipSuccess) return hip_status(e, "softmax_xent");
  }
  return hip_status(launch_xent_finalize(row_loss, targets, rows, classes, loss, n_invalid, s),
                    "softmax_xent finalize");
}

VJP_API int vjp_softmax_xent_fwd(const void* logits, int64_t ld, const int32_t* targets,
                                 int64_t rows, int64_t classes, vjp_dtype_t act, float* loss,
                                 float* row_max, float* row_lse, int32_t* n_invalid,
                                 void* workspace, size_t workspace_bytes, vjp_stream_t stream) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (rows < 0 || classes < 0) return fail(VJP_EINVAL, "negative size");
  if (classes == 0) return fail(VJP_EINVAL, "cross-entropy over zero classes");
  if (classes > INT32_MAX) return fail(VJP_EINVAL, "classes beyond int32 targets");
  const int es = dtype_size(act);
  VJP_TRY(check_matrix("logits", logits, rows, classes, ld, es));
  VJP_TRY(check_vector("targets", targets, rows, 4));
  VJP_TRY(check_vector("loss", loss, 1, 4));
  if (row_max != nullptr) VJP_TRY(check_vector("row_max", row_max, rows, 4));
  VJP_TRY(check_vector("row_lse", row_lse, rows, 4));
  if (n_invalid && !aligned(n_invalid, 4)) return fail(VJP_EALIGN, "n_invalid is not 4-byte aligned");
  const size_t need = vjp_softmax_xent_workspace_size(rows);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(VJP_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 4)) return fail(VJP_EALIGN, "workspace is not 4-byte aligned");
  }
  VJP_TRY(check_alias({span(loss, 4, "loss"), span(row_max, row_max ? rows * 4 : 0, "row_max"),
                       span(row_lse, rows * 4, "row_lse"),
                       span(n_invalid, n_invalid ? 4 : 0, "n_invalid"),
                       span(workspace, int64_t(need), "workspace")},
                      {span(logits, mat_bytes(rows, classes, ld, es), "logits"),
                       span(targets, rows * 4, "targets")}));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  float* row_loss = static_cast<float*>(workspace);
  const bool vec = rows_vec_ok(logits, ld, es);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
    const hipError_t e = launch_softmax_xent_stats(
        static_cast<const char*>(logits) + r0 * ld * es, ld, targets + r0, nr, classes, act,
        row_max ? row_max + r0 : nullptr, row_lse + r0, row_loss + r0, vec, s);
    if (e != hipSuccess) return hip_status(e, "softmax_xent_fwd");
  }
  return hip_status(launch_xent_finalize(row_loss, targets, rows, classes, loss, n_invalid, s),
                    "softmax_xent_fwd finalize");
}

VJP_API int vjp_softmax_xent_bwd(const void* logits, int64_t ld, const int32_t* targets,
                                 const float* row_lse, int64_t rows, int64_t classes, vjp_dtype_t act,
                                 const float* dloss, void* dlogits, int64_t ld_dlogits,
                                 vjp_stream_t stream) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (rows < 0 || classes < 0) return fail(VJP_EINVAL, "negative size");
  if (classes == 0) return fail(VJP_EINVAL, "cross-entropy over zero classes");
  if (classes > kXentBwdMaxClasses)
    return fail(VJP_EINVAL, "classes above %lld", (long long)kXentBwdMaxClasses);
  const int es = dtype_size(act);
  VJP_TRY(check_matrix("logits", logits, rows, classes, ld, es));
  VJP_TRY(check_vector("targets", targets, rows, 4));
  VJP_TRY(check_vector("row_lse", row_lse, rows, 4));
  VJP_TRY(check_vector("dloss", dloss, 1, 4));
  VJP_TRY(check_matrix("dlogits", dlogits, rows, classes, ld_dlogits, es));
  // In place (dlogits == logits, same leading dimension) is allowed; any
  // other overlap is rejected.
  const bool in_place = dlogits == logits && ld_dlogits == ld;
  VJP_TRY(check_alias({span(dlogits, mat_bytes(rows, classes, ld_dlogits, es), "dlogits")},
                      {span(targets, rows * 4, "targets"), span(row_lse, rows * 4, "row_lse"),
                       span(dloss, 4, "dloss"),
                       span(in_place ? nullptr : logits, mat_bytes(rows, classes, ld, es),
                            "logits")}));
  if (rows == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = rows_vec_ok(logits, ld, es) && rows_vec_ok(dlogits, ld_dlogits, es);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
    const hipError_t e = launch_softmax_xent_bwd(
        static_cast<const char*>(logits) + r0 * ld * es, ld, targets + r0, row_lse + r0, dloss,
        rows, nr, classes, act, static_cast<char*>(dlogits) + r0 * ld_dlogits * es, ld_dlogits,
        vec, s);
    if (e != hipSuccess) return hip_status(e, "softmax_xent_bwd");
  }
  return ok();
}

// ------------------------------------------------------------------ LayerNorm / RMSNorm

namespace {

// Backward tiles: rows are dealt round-robin to at most kNormTiles workgroups.
// Measured on MI355X for 32768 x 4096 bf16 (LayerNorm / RMSNorm, one process):
// 512 tiles of 8 waves x 1 vector per lane (two workgroups per CU)
// 143-154 / 132-133 us; 256, 768, 1024 and 1536 tiles 151-198 / 140-198 us;
// 4 waves x 2 vectors 155-176 / 141-153 us; 16 waves 189-207 us.  Again
// with the LayerNorm backward loading each row when it reaches it
// (medians of 39 interleaved runs): 384 / 512 / 640 / 768 / 1024 tiles
// 146.6 / 135.6 / 147.7 / 140.3 / 161.1 us.
constexpr int64_t kNormTiles = 512;

int64_t norm_tiles(int64_t rows) { return rows < kNormTiles ? rows : kNormTiles; }

bool eps_ok(float eps) { return eps >= 0.0f && eps < __builtin_inff(); }

int norm_check_cols(int64_t rows, int64_t cols, int act, bool vec) {
  if (rows > 0 && cols == 0) return fail(VJP_EINVAL, "normalisation over zero columns");
  const int64_t lim = norm_max_cols(act, vec);
  if (cols > lim)
    return fail(VJP_EINVAL, "%lld columns exceed the limit of %lld", (long long)cols,
                (long long)lim);
  return VJP_OK;
}

int norm_fwd_impl(bool rms, const void* x, int64_t ld_x, const void* w, const void* b, void* y,
                  int64_t ld_y, float* row_mean, float* row_rstd, int64_t rows, int64_t cols,
                  float eps, int act, int w_dtype, vjp_stream_t stream) {
  if (!dtype_ok(act) || !dtype_ok(w_dtype)) return fail(VJP_EDTYPE, "unknown dtype");
  if (rows < 0 || cols < 0) return fail(VJP_EINVAL, "negative size");
  if (!eps_ok(eps)) return fail(VJP_EINVAL, "eps must be finite and >= 0");
  const int es = dtype_size(act), ws = dtype_size(w_dtype);
  VJP_TRY(check_matrix("x", x, rows, cols, ld_x, es));
  VJP_TRY(check_matrix("y", y, rows, cols, ld_y, es));
  VJP_TRY(check_vector("w", w, rows > 0 ? cols : 0, ws));
  if (!rms) VJP_TRY(check_vector("b", b, rows > 0 ? cols : 0, ws));
  if (row_mean) VJP_TRY(check_vector("row_mean", row_mean, rows, 4));
  if (row_rstd) VJP_TRY(check_vector("row_rstd", row_rstd, rows, 4));
  VJP_TRY(check_alias({span(y, mat_bytes(rows, cols, ld_y, es), "y"),
                       span(row_mean, row_mean ? rows * 4 : 0, "row_mean"),
                       span(row_rstd, row_rstd ? rows * 4 : 0, "row_rstd")},
                      {span(x, mat_bytes(rows, cols, ld_x, es), "x"), span(w, cols * ws, "w"),
                       span(rms ? nullptr : b, cols * ws, "b")}));
  const bool vec = rows_vec_ok(x, ld_x, es) && rows_vec_ok(y, ld_y, es);
  VJP_TRY(norm_check_cols(rows, cols, act, vec));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = rows - r0 < kRowsPerLaunch ? rows - r0 : kRowsPerLaunch;
    const hipError_t e = launch_norm_fwd(
        rms, static_cast<const char*>(x) + r0 * ld_x * es, ld_x, w, b, w_dtype,
        static_cast<char*>(y) + r0 * ld_y * es, ld_y, row_mean ? row_mean + r0 : nullptr,
        row_rstd ? row_rstd + r0 : nullptr, nr, cols, eps, act, vec, s);
    if (e != hipSuccess) return hip_status(e, rms ? "rmsnorm_fwd" : "layernorm_fwd");
  }
  return ok();
}

int norm_bwd_impl(bool rms, const void* dy, int64_t ld_dy, const void* x, int64_t ld_x,
                  const void* w, const float* row_mean, const float* row_rstd, void* dx,
                  int64_t ld_dx, float* dw, float* db, int accumulate, int64_t rows, int64_t cols,
                  float eps, int act, int w_dtype, void* workspace, size_t workspace_bytes,
                  vjp_stream_t stream) {
  if (!dtype_ok(act) || !dtype_ok(w_dtype)) return fail(VJP_EDTYPE, "unknown dtype");
  if (rows < 0 || cols < 0) return fail(VJP_EINVAL, "negative size");
  if (!eps_ok(eps)) return fail(VJP_EINVAL, "eps must be finite and >= 0");
  if (accumulate != 0 && accumulate != 1) return fail(VJP_EINVAL, "accumulate must be 0 or 1");
  if (!rms && ((row_mean == nullptr) != (row_rstd == nullptr)))
    return fail(VJP_EINVAL, "row_mean and row_rstd must both be given or both be NULL");
  const int es = dtype_size(act), ws = dtype_size(w_dtype);
  VJP_TRY(check_matrix("dy", dy, rows, cols, ld_dy, es));
  VJP_TRY(check_matrix("x", x, rows, cols, ld_x, es));
  VJP_TRY(check_matrix("dx", dx, rows, cols, ld_dx, es));
  VJP_TRY(check_vector("w", w, rows > 0 ? cols : 0, ws));
  VJP_TRY(check_vector("dw", dw, cols, 4));
  if (!rms) VJP_TRY(check_vector("db", db, cols, 4));
  if (row_rstd) VJP_TRY(check_vector("row_rstd", row_rstd, rows, 4));
  if (row_mean) VJP_TRY(check_vector("row_mean", row_mean, rows, 4));
  const size_t need = rms ? vjp_rmsnorm_bwd_workspace_size(rows, cols)
                          : vjp_layernorm_bwd_workspace_size(rows, cols);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(VJP_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!aligned(workspace, 4)) return fail(VJP_EALIGN, "workspace is not 4-byte aligned");
  }
  VJP_TRY(check_alias({span(dx, mat_bytes(rows, cols, ld_dx, es), "dx"), span(dw, cols * 4, "dw"),
                       span(rms ? nullptr : db, cols * 4, "db"),
                       span(workspace, int64_t(need), "workspace")},
                      {span(dy, mat_bytes(rows, cols, ld_dy, es), "dy"),
                       span(x, mat_bytes(rows, cols, ld_x, es), "x"), span(w, cols * ws, "w"),
                       span(row_mean, row_mean ? rows * 4 : 0, "row_mean"),
                       span(row_rstd, row_rstd ? rows * 4 : 0, "row_rstd")}));
  const bool vec = rows_vec_ok(dy, ld_dy, es) && rows_vec_ok(x, ld_x, es) &&
                   rows_vec_ok(dx, ld_dx, es);
  VJP_TRY(norm_check_cols(rows, cols, act, vec));
  if (cols == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = norm_tiles(rows);
  float* P = static_cast<float*>(workspace);
  if (T > 0) {
    const hipError_t e = launch_norm_bwd_stage1(rms, dy, ld_dy, x, ld_x, w, w_dtype, row_mean,
                                                row_rstd, dx, ld_dx, P, rows, cols, T, eps, act,
                                                vec, s);
    if (e != hipSuccess) return hip_status(e, rms ? "rmsnorm_bwd stage 1" : "layernorm_bwd stage 1");
  }
  return hip_status(rms ? launch_reduce_partials(P, T, cols, dw, accumulate, s)
                        : launch_reduce_partials_split(P, T, 2 * cols, dw, db, cols, accumulate, s),
                    rms ? "rmsnorm_bwd stage 2" : "layernorm_bwd stage 2");
}

}  // namespace

VJP_API size_t vjp_layernorm_bwd_workspace_size(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return size_t(norm_tiles(rows)) * size_t(2 * cols) * sizeof(float);
}

VJP_API size_t vjp_rmsnorm_bwd_workspace_size(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return size_t(norm_tiles(rows)) * size_t(cols) * sizeof(float);
}

VJP_API int64_t vjp_norm_max_cols(vjp_dtype_t act, int aligned16) {
  if (!dtype_ok(act)) return -1;
  return norm_max_cols(act, aligned16 != 0);
}

VJP_API int vjp_layernorm_fwd(const void* x, int64_t ld_x, const void* w, const void* b, void* y,
                              int64_t ld_y, float* row_mean, float* row_rstd, int64_t rows,
                              int64_t cols, float eps, vjp_dtype_t act, vjp_dtype_t w_dtype,
                              vjp_stream_t stream) {
  return norm_fwd_impl(false, x, ld_x, w, b, y, ld_y, row_mean, row_rstd, rows, cols, eps, act,
                       w_dtype, stream);
}

VJP_API int vjp_layernorm_bwd(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x,
                              const void* w, const float* row_mean, const float* row_rstd,
                              void* dx, int64_t ld_dx, float* dw, float* db, int accumulate,
                              int64_t rows, int64_t cols, float eps, vjp_dtype_t act, vjp_dtype_t w_dtype,
                              void* workspace, size_t workspace_bytes, vjp_stream_t stream) {
  return norm_bwd_impl(false, dy, ld_dy, x, ld_x, w, row_mean, row_rstd, dx, ld_dx, dw, db,
                       accumulate, rows, cols, eps, act, w_dtype, workspace, workspace_bytes,
                       stream);
}

VJP_API int vjp_rmsnorm_fwd(const void* x, int64_t ld_x, const void* w, void* y, int64_t ld_y,
                            float* row_rstd, int64_t rows, int64_t cols, float eps, vjp_dtype_t act,
                            vjp_dtype_t w_dtype, vjp_stream_t stream) {
  return norm_fwd_impl(true, x, ld_x, w, nullptr, y, ld_y, nullptr, row_rstd, rows, cols, eps,
                       act, w_dtype, stream);
}

VJP_API int vjp_rmsnorm_bwd(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x,
                            const void* w, const float* row_rstd, void* dx, int64_t ld_dx,
                            float* dw, int accumulate, int64_t rows, int64_t cols, float eps,
                            vjp_dtype_t act, vjp_dtype_t w_dtype, void* workspace, size_t workspace_bytes,
                            vjp_stream_t stream) {
  return norm_bwd_impl(true, dy, ld_dy, x, ld_x, w, nullptr, row_rstd, dx, ld_dx, dw, nullptr,
                       accumulate, rows, cols, eps, act, w_dtype, workspace, workspace_bytes,
                       stream);
}

// ------------------------------------------------------------------ gather / scatter-add

VJP_API size_t vjp_gather_rows_bwd_workspace_size(int64_t M, int64_t V, int64_t D) {
  if (M < 0 || V < 0 || D < 0) return 0;
  return size_t(gather_workspace_ints(M, V, D)) * sizeof(int32_t);
}

VJP_API int vjp_gather_rows_fwd(const void* table, int64_t ld_t, int64_t V, int64_t D,
                                const int32_t* idx, int64_t M, void* y, int64_t ld_y, vjp_dtype_t act,
                                vjp_stream_t stream) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (V < 0 || D < 0 || M < 0) return fail(VJP_EINVAL, "negative size");
  if (M > INT32_MAX || V >= INT32_MAX) return fail(VJP_EINVAL, "M or V beyond int32");
  if (D > kGatherMaxCols) return fail(VJP_EINVAL, "D above %lld", (long long)kGatherMaxCols);
  const int es = dtype_size(act);
  VJP_TRY(check_matrix("table", table, V, D, ld_t, es));
  VJP_TRY(check_vector("idx", idx, M, 4));
  VJP_TRY(check_matrix("y", y, M, D, ld_y, es));
  VJP_TRY(check_alias({span(y, mat_bytes(M, D, ld_y, es), "y")},
                      {span(table, mat_bytes(V, D, ld_t, es), "table"), span(idx, M * 4, "idx")}));
  if (M == 0 || D == 0) return ok();
  const bool vec = rows_vec_ok(table, ld_t, es) && rows_vec_ok(y, ld_y, es);
  return hip_status(launch_gather_rows_fwd(table, ld_t, idx, M, V, D, y, ld_y, act, vec,
                                           static_cast<hipStream_t>(stream)),
                    "gather_rows_fwd");
}

VJP_API int vjp_gather_rows_bwd(const void* dy, int64_t ld_dy, const int32_t* idx, int64_t M,
                                int64_t V, int64_t D, float* dtable, int64_t ld_dt,
                                int accumulate, int32_t* n_invalid, vjp_dtype_t act, void* workspace,
                                size_t workspace_bytes, vjp_stream_t stream) {
  if (!dtype_ok(act)) return fail(VJP_EDTYPE, "unknown dtype");
  if (V < 0 || D < 0 || M < 0) return fail(VJP_EINVAL, "negative size");
  if (M > INT32_MAX || V >= INT32_MAX) return fail(VJP_EINVAL, "M or V beyond int32");
  if (D > kGatherMaxCols) return fail(VJP_EINVAL, "D above %lld", (long long)kGatherMaxCols);
  if (accumulate != 0 && accumulate != 1) return fail(VJP_EINVAL, "accumulate must be 0 or 1");
  const int es = dtype_size(act);
  VJP_TRY(check_matrix("dy", dy, M, D, ld_dy, es));
  VJP_TRY(check_vector("idx", idx, M, 4));
  VJP_TRY(check_matrix("dtable", dtable, V, D, ld_dt, 4));
  if (n_invalid && !aligned(n_invalid, 4)) return fail(VJP_EALIGN, "n_invalid is not 4-byte aligned");
  const size_t need = vjp_gather_rows_bwd_workspace_size(M, V, D);
  if (!workspace || workspace_bytes < need)
    return fail(VJP_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned(workspace, 16)) return fail(VJP_EALIGN, "workspace is not 16-byte aligned");
  VJP_TRY(check_alias({span(dtable, mat_bytes(V, D, ld_dt, 4), "dtable"),
                       span(n_invalid, n_invalid ? 4 : 0, "n_invalid"),
                       span(workspace, int64_t(need), "workspace")},
                      {span(dy, mat_bytes(M, D, ld_dy, es), "dy"), span(idx, M * 4, "idx")}));
  const bool vec = rows_vec_ok(dy, ld_dy, es);
  const bool pvec = aligned(dtable, 16) && ld_dt % 4 == 0;
  return hip_status(launch_gather_rows_bwd(dy, ld_dy, idx, M, V, D, dtable, ld_dt, accumulate,
                                           n_invalid, static_cast<int32_t*>(workspace), act, vec,
                                           pvec, static_cast<hipStream_t>(stream)),
                    "gather_rows_bwd");
}
