/*
 * libvjp -- paired forward / backward (vector-Jacobian product) kernels for
 * small fused ops on AMD Instinct MI355X (gfx950).
 *
 * A backward call reads the upstream gradient plus what its forward saved
 * and returns one gradient per differentiable input, never forming the
 * Jacobian ("Backprop for kernel writers", section 01 "The only idea";
 * "Backward in Triton -- autograd.Function and the backward grid", section
 * "The mental model: two kernels, one node").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory      Every pointer argument is a DEVICE pointer owned by the caller,
 *             except where a comment says otherwise.  The library allocates
 *             no device memory and keeps no state between calls; tensors
 *             saved by a forward for its backward (x, w, y, row_lse, ...) are
 *             the caller's buffers.
 * Layout      Matrices are row-major with unit stride along a row and a
 *             leading dimension ld (in elements, ld >= number of columns)
 *             between rows.  Vectors are contiguous.
 * Dtypes      `act` names the storage type of activations and of their
 *             gradients (x, y, dy, dx, logits, dlogits): VJP_F32, VJP_F16
 *             or VJP_BF16.  All arithmetic is fp32; every reduction
 *             accumulates in fp32.  Parameter gradients (dw, grad_w) and
 *             row statistics are always fp32 ("Backward in Triton", section
 *             "fp32 accumulation, and why gradients use +=").
 * Reductions  Parameter gradients are reduced in two stages with no float
 *             atomics: stage 1 writes one fp32 partial per tile into the
 *             caller's workspace, a second kernel sums the partials in a
 *             fixed order.  The tile count depends only on the problem
 *             size, so results are bitwise reproducible run to run.
 *             ("Writing Triton Kernels with Autograd: A Minimal End-to-End
 *             Example", section 3; "Backward in Triton", section "The
 *             backward grid is not the forward grid").
 * accumulate  0: the parameter gradient is overwritten.  1: the new gradient
 *             is added into the existing fp32 value ("Backward in Triton",
 *             section "fp32 accumulation, and why gradients use +=").
 * Streams     Every call is asynchronous on `stream` (a hipStream_t; NULL is
 *             the default stream) and never synchronises the host.  A call
 *             only launches kernels on that stream (no allocation, copy or
 *             memset; the only device queries are host-side: the scatter-add
 *             backward reads the current device and, on its first call on a
 *             device, its compute-unit count, and the no-allocation entry
 *             point reads the current device and, once per device, its
 *             scratch address), so calls may be captured in a HIP graph and
 *             replayed; a replay with the same inputs gives the same bits as
 *             an eager call.
 * Errors      Every call returns VJP_OK or a VJP_E* code.  On an error
 *             detected before launch nothing is launched and no output is
 *             touched; vjp_last_error() gives a per-thread message.
 *             VJP_EHIP means a launch failed; outputs are then undefined.
 * Empty       n = 0 or rows = 0 is valid: nothing is read, parameter
 *             gradients become 0 (or stay unchanged with accumulate = 1),
 *             the cross-entropy mean loss of zero rows is NaN.
 * Alignment   Pointers must be aligned to their element size (fp32 outputs
 *             and workspaces to 4 bytes).  16-byte alignment of base
 *             pointers and of ld * element size selects 128-bit loads;
 *             anything else runs the same algorithm with element loads.
 * Aliasing    An output range that overlaps an input range or another output
 *             is rejected with VJP_EALIAS.
 */
#ifndef LIBVJP_H
#define LIBVJP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VJP_VERSION 1

/* Storage dtype of activations (act) and parameters (w_dtype).  Passed as
   this int-sized enum; a value outside it returns VJP_EDTYPE. */
typedef enum { VJP_F32 = 0, VJP_F16 = 1, VJP_BF16 = 2 } vjp_dtype_t;

typedef enum {
  VJP_OK = 0,
  VJP_EINVAL = 1,     /* bad size, null pointer, ld < cols, bad flag value */
  VJP_EDTYPE = 2,     /* unknown dtype code */
  VJP_EALIGN = 3,     /* pointer not aligned to its element size */
  VJP_EWORKSPACE = 4, /* workspace missing or smaller than the *_workspace_size query */
  VJP_EALIAS = 5,     /* an output overlaps an input or another output */
  VJP_EHIP = 6        /* the HIP runtime reported an error at launch */
} vjp_status_t;

typedef void* vjp_stream_t; /* hipStream_t */

/* Library version (VJP_VERSION). */
int vjp_version(void);
/* Static text for a status code. */
const char* vjp_status_string(int status);
/* Text of the calling thread's last error ("" if none). */
const char* vjp_last_error(void);

/* Streaming device copy of `bytes` bytes from src to dst (device pointers,
 * any alignment; 16-byte aligned pointers take 16-byte nontemporal accesses).
 * Not an operation of the method: it is the measurement reference, the rate
 * at which this chip reads and writes each byte once, against which the
 * kernels below are judged (each of them moves its bytes once as well).
 * bytes = 0 is valid; overlapping ranges give VJP_EALIAS. */
int vjp_copy(const void* src, void* dst, int64_t bytes, vjp_stream_t stream);

/* vjp_copy with its launch shape given: vectors_per_lane 16-byte vectors in
 * flight per lane (1, 2, 4 or 8; vjp_copy uses 4) and a grid of at most
 * max_workgroups workgroups of 256 lanes looping over the data (vjp_copy:
 * 32768).  For sweeps of the copy reference over launch shapes; other values
 * give VJP_EINVAL.  Same pointers, alignment and aliasing rules as vjp_copy. */
int vjp_copy_shaped(const void* src, void* dst, int64_t bytes, int vectors_per_lane,
                    int64_t max_workgroups, vjp_stream_t stream);

/* ---------------------------------------------------------------- weighted sum
 * y[i] = sum_j x[i, j] * w[j];  x [n_rows, d] (ld_x), w [d], y [n_rows].
 * Backward: grad_x[i, j] = dy[i] * w[j]   (elementwise map, same shape as x)
 *           grad_w[j]    = sum_i x[i, j] * dy[i]   (reduction over the batch)
 * Source: "Writing Triton Kernels with Autograd: A Minimal End-to-End
 * Example", sections 1-4 (problem setup, forward tiled over rows with a loop
 * over D, gradients, two-stage grad_w: one partial row per tile of rows).
 */

/* x, y, dy, dx in `act`; w in `w_dtype`.  y has n_rows elements in `act`. */
int vjp_weighted_sum_fwd(const void* x, int64_t ld_x, const void* w, void* y,
                         int64_t n_rows, int64_t d, vjp_dtype_t act, vjp_dtype_t w_dtype,
                         vjp_stream_t stream);

/* Row tiling of the backward's stage 1.  The rows are cut into blocks of
 * block_rows consecutive rows (the last one may be shorter) and tile t holds
 * blocks t, t + tiles, t + 2 * tiles, ...
 *   rows_per_tile > 0: block_rows = rows_per_tile, tiles = ceil(n_rows /
 *     rows_per_tile), so tile t is the contiguous rows [t * rows_per_tile,
 *     (t + 1) * rows_per_tile); rows_per_tile must not exceed 2^30.
 *   rows_per_tile = 0 (automatic, a function of n_rows only): block_rows =
 *     32, tiles = min(1024, ceil(n_rows / 32)); the blocks are dealt to the
 *     tiles round-robin.
 * block_rows and tiles are HOST pointers written on success.  Returns VJP_OK,
 * or VJP_EINVAL for negative sizes, rows_per_tile > 2^30 or NULL outputs. */
int vjp_weighted_sum_tiling(int64_t n_rows, int64_t rows_per_tile, int64_t* block_rows,
                            int64_t* tiles);

/* Workspace bytes for vjp_weighted_sum_bwd: tiles * d * 4 (tiles as above;
 * 0 for invalid arguments).  Layout: fp32 partials P[tiles][d] row-major at
 * offset 0, where P[t][j] = sum over the rows i of tile t of x[i, j] * dy[i]. */
size_t vjp_weighted_sum_bwd_workspace_size(int64_t n_rows, int64_t d, int64_t rows_per_tile);

/* dy [n_rows] (act), x [n_rows, d] (ld_x, act), w [d] (w_dtype) ->
 * dx [n_rows, d] (ld_dx, act), dw [d] fp32 (overwritten or, with
 * accumulate = 1, added into).  workspace: see the size query.
 * grad_w[j] = sum over t = 0..tiles-1 of P[t][j] in this fixed order (d >= 2):
 * 128 row lanes r each sum P[r][j], P[r + 128][j], P[r + 256][j], ... in
 * increasing t, starting from 0, then a pairwise tree v[r] += v[r + s] for
 * s = 64, 32, ..., 1; finally dw[j] = v[0] (or dw[j] + v[0]).  For d = 1 the
 * order of vjp_scaled_silu_bwd's dw applies.  Within a tile each partial is
 * accumulated in fp32 in an order fixed by the tiling, so the whole result is
 * bitwise reproducible.  d at most 4194240 (VJP_EINVAL beyond). */
int vjp_weighted_sum_bwd(const void* dy, const void* x, int64_t ld_x, const void* w,
                         void* dx, int64_t ld_dx, float* dw, int accumulate,
                         int64_t n_rows, int64_t d, int64_t rows_per_tile,
                         vjp_dtype_t act, vjp_dtype_t w_dtype, void* workspace, size_t workspace_bytes,
                         vjp_stream_t stream);

/* ---------------------------------------------------------------- scaled SiLU
 * y = w * x * sigmoid(x), elementwise over n elements; w is ONE fp32 value
 * held in device memory (read by the kernels, no host synchronisation).
 * Backward (sigmoid recomputed from x, not saved):
 *   dx = dy * w * (s + x s (1 - s)),  s = sigmoid(x)
 *   dw = sum over all elements of dy * x * s   (fp32)
 * Source: "Backward in Triton -- autograd.Function and the backward grid",
 * sections "A complete minimal example -- fused scaled-SiLU, end to end" and
 * "Save vs recompute -- the decision at the Triton level".  The page's
 * single-cell atomic add of per-block partials is replaced by the two-stage
 * reduction described above.
 */
int vjp_scaled_silu_fwd(const void* x, const float* w, void* y, int64_t n, vjp_dtype_t act,
                        vjp_stream_t stream);

/* Elements per dw tile: max(2048, 2048 * ceil(ceil(n / 4096) / 2048)), a
 * function of n only (4096 tiles of 4096 elements for n = 2^24).  -1 if n < 0. */
int64_t vjp_scaled_silu_elems_per_tile(int64_t n);

/* Workspace bytes: T * 4, T = ceil(n / elems_per_tile).  Layout: fp32
 * partials P[T] at offset 0, P[t] = sum over elements k of tile t of
 * dy[k] * x[k] * s[k]. */
size_t vjp_scaled_silu_bwd_workspace_size(int64_t n);

/* dy, x [n] (act), w [1] fp32 -> dx [n] (act), dw [1] fp32.  dw is the
 * fixed-order sum of P: 1024 threads, thread r summing P[r], P[r + 1024],
 * ... in increasing t; each wave's 64 sums combined by a fixed DPP tree
 * (neighbour swap, pair swap, half-row mirror, row mirror, then 16-lane rows
 * (0 + 1) + (2 + 3)); the sixteen wave sums added in wave order. */
int vjp_scaled_silu_bwd(const void* dy, const void* x, const float* w, void* dx, float* dw,
                        int accumulate, int64_t n, vjp_dtype_t act, void* workspace,
                        size_t workspace_bytes, vjp_stream_t stream);

/* vjp_scaled_silu_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid hipMalloc).  It allocates nothing and calls no allocating routine:
 * the stage-1 partials go to a 16 KB buffer the library holds in device
 * memory, one per GPU it runs on, kept until the process ends.  That buffer
 * holds at most 4096 partials, which covers every n (the backward never forms
 * more than 4096 tiles); a larger need would return VJP_EINVAL.  Every call on
 * one GPU uses the same buffer: calls that overlap on one GPU (different
 * streams, no ordering between them) race and give wrong dw; calls ordered on
 * one stream are safe.  Nothing in the buffer needs clearing between calls
 * (each call writes every partial it reads).  Arguments, results, summation
 * order and errors are those of vjp_scaled_silu_bwd. */
int vjp_scaled_silu_bwd_noalloc(const void* dy, const void* x, const float* w, void* dx,
                                float* dw, int accumulate, int64_t n, vjp_dtype_t act,
                                vjp_stream_t stream);

/* ---------------------------------------------------------------- row softmax
 * y[r, j] = exp(x[r, j] - m_r) / sum_k exp(x[r, k] - m_r), m_r = max_k x[r, k].
 * The backward needs only the saved y: with s_r = sum_j dy[r, j] y[r, j],
 * dx[r, j] = y[r, j] (dy[r, j] - s_r); the cols x cols Jacobian is never
 * formed.  Source: "Backprop for kernel writers", section 01 and the softmax
 * section after 04 "The duality" (one row scalar, O(cols) time, O(1) extra
 * memory; the max shift adds no backward term).
 */
int vjp_softmax_fwd(const void* x, int64_t ld_x, void* y, int64_t ld_y, int64_t rows,
                    int64_t cols, vjp_dtype_t act, vjp_stream_t stream);

int vjp_softmax_bwd(const void* dy, int64_t ld_dy, const void* y, int64_t ld_y, void* dx,
                    int64_t ld_dx, int64_t rows, int64_t cols, vjp_dtype_t act, vjp_stream_t stream);

/* Save-the-statistics form ("Backprop for kernel writers", the softmax
 * section after 04: y can be recomputed from the saved max and logsumexp;
 * section 07 "Fusion": keep only L = m + log l per row, rebuild any
 * probability as exp(x - L)).
 * vjp_softmax_fwd_lse: as vjp_softmax_fwd and also row_lse[r] = L_r (fp32,
 * [rows], required).  y may be NULL (then ld_y is ignored): the call computes
 * the row logsumexp alone, reading x once.
 * vjp_softmax_bwd_lse: dx from dy, the forward's INPUT x and row_lse; y is
 * rebuilt in fp32 as exp(x - L) (never rounded to the storage type), then
 * dx = y (dy - s), s = sum_j dy_j y_j.  Reads dy and x, writes dx. */
int vjp_softmax_fwd_lse(const void* x, int64_t ld_x, void* y, int64_t ld_y, float* row_lse,
                        int64_t rows, int64_t cols, vjp_dtype_t act, vjp_stream_t stream);

int vjp_softmax_bwd_lse(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x,
                        const float* row_lse, void* dx, int64_t ld_dx, int64_t rows,
                        int64_t cols, vjp_dtype_t act, vjp_stream_t stream);

/* ---------------------------------------------------------------- softmax + cross-entropy
 * Fused forward and backward of the mean cross-entropy of a row softmax:
 *   row_max[r] = m_r = max_j z[r, j]
 *   row_lse[r] = m_r + log sum_j exp(z[r, j] - m_r)
 *   loss       = (1 / rows) * sum_r (row_lse[r] - z[r, t_r])        (fp32, [1])
 *   dlogits    = grad_scale * (exp(z - row_lse) - onehot(t_r))       (act)
 * grad_scale is the upstream gradient of the mean loss divided by rows
 * (1 / rows for a unit upstream gradient).  The probabilities are rebuilt
 * on chip from the row statistics and never written to memory.
 * Source: "Backprop for kernel writers", section 02 "See it move" (softmax
 * and cross-entropy derivatives cancel into softmax minus one-hot) and
 * section 07 "Fusion" (keep only m and log-sum-exp per row, rebuild P).
 * targets [rows] int32.  A target outside [0, classes) is not an error: that
 * row's loss is NaN (so is the mean), its dlogits row has no one-hot term,
 * and it is counted in *n_invalid (int32, optional: NULL skips the count).
 * workspace: vjp_softmax_xent_workspace_size(rows) bytes; layout: fp32 row
 * losses [rows] at offset 0.  The mean is their fixed-order sum (the order
 * of the dw sum of vjp_scaled_silu_bwd) divided by rows.
 */
size_t vjp_softmax_xent_workspace_size(int64_t rows);

int vjp_softmax_xent_fwd_bwd(const void* logits, int64_t ld, const int32_t* targets,
                             int64_t rows, int64_t classes, vjp_dtype_t act, float grad_scale,
                             float* loss, float* row_max, float* row_lse, void* dlogits,
                             int64_t ld_dlogits, int32_t* n_invalid, void* workspace,
                             size_t workspace_bytes, vjp_stream_t stream);

/* Split form of the above ("Backprop for kernel writers", section 07
 * "Fusion": the forward keeps only the row statistics, the backward rebuilds
 * p = exp(z - L) from them):
 * vjp_softmax_xent_fwd: loss, row_lse (required), row_max (optional, NULL
 * skips it), n_invalid (optional), exactly as vjp_softmax_xent_fwd_bwd but
 * without the logit gradient; the logits are read once.  Same workspace.
 * vjp_softmax_xent_bwd: dlogits[r, j] = (dloss[0] / rows) * (exp(z[r, j] -
 * row_lse[r]) - [j == t_r]); dloss is ONE fp32 value in DEVICE memory (the
 * upstream gradient of the mean loss, read by the kernel: no host
 * synchronisation), divided by rows in fp32.  Rows with an invalid target
 * get no one-hot term.  dlogits may be the logits buffer itself (same
 * pointer and leading dimension: computed in place); any other overlap is
 * VJP_EALIAS.  classes at most 268431360 (65535 blocks of 4096 columns),
 * else VJP_EINVAL. */
int vjp_softmax_xent_fwd(const void* logits, int64_t ld, const int32_t* targets, int64_t rows,
                         int64_t classes, vjp_dtype_t act, float* loss, float* row_max, float* row_lse,
                         int32_t* n_invalid, void* workspace, size_t workspace_bytes,
                         vjp_stream_t stream);

int vjp_softmax_xent_bwd(const void* logits, int64_t ld, const int32_t* targets,
                         const float* row_lse, int64_t rows, int64_t classes, vjp_dtype_t act,
                         const float* dloss, void* dlogits, int64_t ld_dlogits,
                         vjp_stream_t stream);

/* ---------------------------------------------------------------- LayerNorm / RMSNorm
 * Over the last dimension of x [rows, cols] (ld_x); w, b [cols] in w_dtype.
 *   LayerNorm: mu = mean(x), rstd = 1 / sqrt(mean((x - mu)^2) + eps)
 *              (biased variance, computed as the mean of squared deviations),
 *              xhat = (x - mu) rstd, y = xhat w + b
 *   RMSNorm:   rstd = 1 / sqrt(mean(x^2) + eps), xhat = x rstd, y = xhat w
 * Backward, with g = dy w, a = mean(g) (LayerNorm only), c = mean(g xhat):
 *   dx = rstd (g - a - xhat c),  dw = sum over rows of dy xhat (fp32),
 *   db = sum over rows of dy (fp32, LayerNorm only).
 * Source: "Backprop for kernel writers", the LayerNorm passage after 04 "The
 * duality" (the backward collapses to two row scalars; the parameter
 * gradients reduce over the batch axis) and section 07 (normalisation
 * constants are worth saving: one float per row); "Backward in Triton",
 * sections "Save vs recompute" and "The backward grid is not the forward
 * grid" (RMSNorm's dw partials summed by a deterministic second pass).
 * row_mean / row_rstd (fp32 [rows]) are optional outputs of the forward
 * (NULL: not written) and optional inputs of the backward (NULL: recomputed
 * from x with eps; LayerNorm takes both or neither).  eps must be finite and
 * >= 0.  cols may not exceed vjp_norm_max_cols(act, aligned16) = 16384 for
 * every dtype and alignment (a row lives in the registers of at most 1024
 * lanes, 16 values each); wider rows are VJP_EINVAL.
 * Backward stage 1: rows are dealt round-robin to tiles = min(512, rows)
 * workgroups; tile t holds rows t, t + tiles, ... and writes its fp32
 * partial row P[t][0 .. cols) = sum dy xhat and, for LayerNorm,
 * P[t][cols .. 2 cols) = sum dy (workspace layout, row width cols or
 * 2 cols).  Stage 2 sums the partial rows in the order documented for
 * vjp_weighted_sum_bwd (d = 2 cols for LayerNorm, split into dw and db).
 * accumulate = 1 adds into dw (and db). */
int64_t vjp_norm_max_cols(vjp_dtype_t act, int aligned16);

size_t vjp_layernorm_bwd_workspace_size(int64_t rows, int64_t cols);
size_t vjp_rmsnorm_bwd_workspace_size(int64_t rows, int64_t cols);

int vjp_layernorm_fwd(const void* x, int64_t ld_x, const void* w, const void* b, void* y,
                      int64_t ld_y, float* row_mean, float* row_rstd, int64_t rows,
                      int64_t cols, float eps, vjp_dtype_t act, vjp_dtype_t w_dtype, vjp_stream_t stream);

int vjp_layernorm_bwd(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x, const void* w,
                      const float* row_mean, const float* row_rstd, void* dx, int64_t ld_dx,
                      float* dw, float* db, int accumulate, int64_t rows, int64_t cols,
                      float eps, vjp_dtype_t act, vjp_dtype_t w_dtype, void* workspace, size_t workspace_bytes,
                      vjp_stream_t stream);

int vjp_rmsnorm_fwd(const void* x, int64_t ld_x, const void* w, void* y, int64_t ld_y,
                    float* row_rstd, int64_t rows, int64_t cols, float eps, vjp_dtype_t act,
                    vjp_dtype_t w_dtype, vjp_stream_t stream);

int vjp_rmsnorm_bwd(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x, const void* w,
                    const float* row_rstd, void* dx, int64_t ld_dx, float* dw, int accumulate,
                    int64_t rows, int64_t cols, float eps, vjp_dtype_t act, vjp_dtype_t w_dtype,
                    void* workspace, size_t workspace_bytes, vjp_stream_t stream);

/* ---------------------------------------------------------------- gather / scatter-add
 * Row gather (embedding lookup): y[m, :] = table[idx[m], :] for m < M;
 * table [V, D] (ld_t), idx [M] int32, y [M, D] (ld_y), all activations in
 * `act`.  An index outside [0, V) selects nothing: its y row is zero.
 * Backward, a scatter-add: dtable[v, :] = sum over m with idx[m] = v of
 * dy[m, :], fp32 [V, D] (ld_dt); rows never selected are 0 (or unchanged with
 * accumulate = 1); invalid indices contribute nothing and are counted in
 * *n_invalid (optional).
 * Source: "Backprop for kernel writers", section 06 "Top-k & routing"
 * (selection sends gradient only to the selected slots; repeated indices
 * must all be summed, and atomic adds make the result order-dependent) and
 * section 04 "The duality" (a value read by many outputs sums their
 * gradients).
 * Deterministic order: the indices are sorted stably (invalid last); a table
 * row selected at most 32 times sums its contributions in increasing m; a
 * row selected more often sums them in consecutive chunks of 32 (in
 * increasing m within a chunk) and then the chunk sums in order; all in
 * fp32, no float atomics, results bitwise reproducible.
 * Workspace (16-byte aligned): int32 sorted keys [M] at offset 0 (invalid
 * indices as V) and the positions m in sorted order [M] right after them,
 * then sort buffers, a digit table, run bounds, chunk bookkeeping and fp32
 * chunk sums; size from vjp_gather_rows_bwd_workspace_size.  M and V must be
 * below 2^31 - 1, D at most 16776960. */
size_t vjp_gather_rows_bwd_workspace_size(int64_t M, int64_t V, int64_t D);

int vjp_gather_rows_fwd(const void* table, int64_t ld_t, int64_t V, int64_t D,
                        const int32_t* idx, int64_t M, void* y, int64_t ld_y, vjp_dtype_t act,
                        vjp_stream_t stream);

int vjp_gather_rows_bwd(const void* dy, int64_t ld_dy, const int32_t* idx, int64_t M, int64_t V,
                        int64_t D, float* dtable, int64_t ld_dt, int accumulate,
                        int32_t* n_invalid, vjp_dtype_t act, void* workspace, size_t workspace_bytes,
                        vjp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBVJP_H */
