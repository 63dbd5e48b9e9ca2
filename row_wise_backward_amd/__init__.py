"""Python binding of libvjp (include/libvjp.h) -- argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU (PyTorch supplies device memory and the current
stream); their data pointers, leading dimensions and dtypes are passed to the
C ABI, which launches the HIP kernels.  Outputs not supplied by the caller
are allocated with ``torch.empty``.  Nothing is computed in Python, and there
is no fallback: importing this package fails if ``libvjp.so`` has not been
built (``python row_wise_backward_amd/build.py`` or
``__graft_entry__.build()``).

Inputs must have unit stride along their last dimension (call
``.contiguous()`` first); a 2-D tensor's row stride becomes the C ABI's
leading dimension.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvjp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python row_wise_backward_amd/build.py); "
        "there is no fallback path")

lib = ctypes.CDLL(LIB_PATH)

VJP_F32, VJP_F16, VJP_BF16 = 0, 1, 2
STATUS = {0: "VJP_OK", 1: "VJP_EINVAL", 2: "VJP_EDTYPE", 3: "VJP_EALIGN",
          4: "VJP_EWORKSPACE", 5: "VJP_EALIAS", 6: "VJP_EHIP"}

_vp, _i64, _int, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "vjp_version": ([], _int),
    "vjp_status_string": ([_int], ctypes.c_char_p),
    "vjp_last_error": ([], ctypes.c_char_p),
    "vjp_copy": ([_vp, _vp, _i64, _vp], _int),
    "vjp_copy_shaped": ([_vp, _vp, _i64, _int, _i64, _vp], _int),
    "vjp_weighted_sum_fwd": ([_vp, _i64, _vp, _vp, _i64, _i64, _int, _int, _vp], _int),
    "vjp_weighted_sum_tiling": ([_i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)], ctypes.c_int),
    "vjp_weighted_sum_bwd_workspace_size": ([_i64, _i64, _i64], _sz),
    "vjp_weighted_sum_bwd": ([_vp, _vp, _i64, _vp, _vp, _i64, _vp, _int, _i64, _i64, _i64,
                              _int, _int, _vp, _sz, _vp], _int),
    "vjp_scaled_silu_fwd": ([_vp, _vp, _vp, _i64, _int, _vp], _int),
    "vjp_scaled_silu_elems_per_tile": ([_i64], _i64),
    "vjp_scaled_silu_bwd_workspace_size": ([_i64], _sz),
    "vjp_scaled_silu_bwd": ([_vp, _vp, _vp, _vp, _vp, _int, _i64, _int, _vp, _sz, _vp], _int),
    "vjp_scaled_silu_bwd_noalloc": ([_vp, _vp, _vp, _vp, _vp, _int, _i64, _int, _vp], _int),
    "vjp_softmax_fwd": ([_vp, _i64, _vp, _i64, _i64, _i64, _int, _vp], _int),
    "vjp_softmax_bwd": ([_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _int, _vp], _int),
    "vjp_softmax_fwd_lse": ([_vp, _i64, _vp, _i64, _vp, _i64, _i64, _int, _vp], _int),
    "vjp_softmax_bwd_lse": ([_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _int, _vp], _int),
    "vjp_softmax_xent_workspace_size": ([_i64], _sz),
    "vjp_softmax_xent_fwd": ([_vp, _i64, _vp, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                             _int),
    "vjp_softmax_xent_bwd": ([_vp, _i64, _vp, _vp, _i64, _i64, _int, _vp, _vp, _i64, _vp], _int),
    "vjp_norm_max_cols": ([_int, _int], _i64),
    "vjp_gather_rows_bwd_workspace_size": ([_i64, _i64, _i64], _sz),
    "vjp_gather_rows_fwd": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _vp], _int),
    "vjp_gather_rows_bwd": ([_vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _int, _vp, _int, _vp, _sz,
                             _vp], _int),
    "vjp_layernorm_bwd_workspace_size": ([_i64, _i64], _sz),
    "vjp_rmsnorm_bwd_workspace_size": ([_i64, _i64], _sz),
    "vjp_layernorm_fwd": ([_vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _f32, _int, _int,
                           _vp], _int),
    "vjp_layernorm_bwd": ([_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _int, _i64,
                           _i64, _f32, _int, _int, _vp, _sz, _vp], _int),
    "vjp_rmsnorm_fwd": ([_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _f32, _int, _int, _vp], _int),
    "vjp_rmsnorm_bwd": ([_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _int, _i64, _i64, _f32,
                         _int, _int, _vp, _sz, _vp], _int),
    "vjp_softmax_xent_fwd_bwd": ([_vp, _i64, _vp, _i64, _i64, _int, _f32, _vp, _vp, _vp, _vp,
                                  _i64, _vp, _vp, _sz, _vp], _int),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret

EXPORTED = tuple(_SIGS)

_DT = {torch.float32: VJP_F32, torch.float16: VJP_F16, torch.bfloat16: VJP_BF16}


class VjpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.vjp_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise VjpError(status, where)


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("last dimension must have unit stride (call .contiguous())")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError("rows overlap (row stride < columns); call .contiguous()")
    return max(int(t.stride(0)), int(t.shape[1]))


def _flat(t: torch.Tensor) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous (call .contiguous())")
    return t


def _expect(t, shape, dtype, device, name):
    """Host-side guard: the C ABI trusts the sizes it is given, so every tensor
    is checked against them before a kernel can touch it."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return t


def _stream(t: torch.Tensor):
    if t.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {t.device}")
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(nbytes: int, like: torch.Tensor, workspace):
    if workspace is not None:
        if workspace.device != like.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        return workspace
    return torch.empty(max(int(nbytes), 0), dtype=torch.uint8, device=like.device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def vjp_version() -> int:
    return lib.vjp_version()


def vjp_status_string(status: int) -> str:
    return lib.vjp_status_string(status).decode()


def vjp_last_error() -> str:
    return lib.vjp_last_error().decode()


def vjp_copy(src, dst):
    """Copy the bytes of contiguous src into contiguous dst (same byte size,
    same device): the streaming copy the kernels are measured against."""
    n = _nbytes(_flat(src))
    if _nbytes(_flat(dst)) != n:
        raise ValueError(f"dst holds {_nbytes(dst)} bytes, src {n}")
    if dst.device != src.device:
        raise ValueError("src and dst must be on the same device")
    _check(lib.vjp_copy(_ptr(src), _ptr(dst), n, _stream(src)), "vjp_copy")
    return dst


def vjp_copy_shaped(src, dst, vectors_per_lane=4, max_workgroups=32768):
    """vjp_copy with its launch shape given (for sweeps of the copy reference)."""
    n = _nbytes(_flat(src))
    if _nbytes(_flat(dst)) != n:
        raise ValueError(f"dst holds {_nbytes(dst)} bytes, src {n}")
    if dst.device != src.device:
        raise ValueError("src and dst must be on the same device")
    _check(lib.vjp_copy_shaped(_ptr(src), _ptr(dst), n, int(vectors_per_lane), int(max_workgroups),
                               _stream(src)), "vjp_copy_shaped")
    return dst


# ----------------------------------------------------------------- weighted sum

def vjp_weighted_sum_fwd(x, w, y=None):
    """y[i] = sum_j x[i, j] w[j]; x [N, D] (row stride = ld), w [D], y [N] in x's dtype."""
    n, d = x.shape
    if y is None:
        y = torch.empty(n, dtype=x.dtype, device=x.device)
    _expect(w, (d,), None, x.device, "w")
    _expect(y, (n,), x.dtype, x.device, "y")
    _check(lib.vjp_weighted_sum_fwd(_ptr(x), _ld(x), _ptr(_flat(w)), _ptr(_flat(y)), n, d,
                                    _dt(x), _dt(w), _stream(x)), "vjp_weighted_sum_fwd")
    return y


def vjp_weighted_sum_tiling(n_rows: int, rows_per_tile: int = 0):
    """(block_rows, tiles): tile t holds row blocks t, t + tiles, ... of block_rows rows."""
    br, tl = _i64(), _i64()
    _check(lib.vjp_weighted_sum_tiling(n_rows, rows_per_tile, ctypes.byref(br), ctypes.byref(tl)),
           "vjp_weighted_sum_tiling")
    return int(br.value), int(tl.value)


def vjp_weighted_sum_bwd_workspace_size(n_rows: int, d: int, rows_per_tile: int = 0) -> int:
    return int(lib.vjp_weighted_sum_bwd_workspace_size(n_rows, d, rows_per_tile))


def vjp_weighted_sum_bwd(dy, x, w, dx=None, dw=None, accumulate=False, rows_per_tile=0,
                         workspace=None):
    """(dx, dw): dx = dy outer w (x's dtype), dw [D] fp32 (added into when accumulate)."""
    n, d = x.shape
    if dx is None:
        dx = torch.empty_like(x)
    if dw is None:
        dw = torch.empty(d, dtype=torch.float32, device=x.device)
    _expect(dy, (n,), x.dtype, x.device, "dy")
    _expect(w, (d,), None, x.device, "w")
    _expect(dx, (n, d), x.dtype, x.device, "dx")
    _expect(dw, (d,), torch.float32, x.device, "dw")
    need = vjp_weighted_sum_bwd_workspace_size(n, d, rows_per_tile)
    ws = _workspace(need, x, workspace)
    _check(lib.vjp_weighted_sum_bwd(_ptr(_flat(dy)), _ptr(x), _ld(x), _ptr(_flat(w)), _ptr(dx),
                                    _ld(dx), _ptr(_flat(dw)), int(bool(accumulate)), n, d,
                                    rows_per_tile, _dt(x), _dt(w), _ptr(ws), _nbytes(ws),
                                    _stream(x)), "vjp_weighted_sum_bwd")
    return dx, dw


# ----------------------------------------------------------------- scaled SiLU

def vjp_scaled_silu_fwd(x, w, y=None):
    """y = w x sigmoid(x); w is a one-element fp32 device tensor."""
    x = _flat(x)
    if y is None:
        y = torch.empty_like(x)
    _expect(w, (1,), torch.float32, x.device, "w")
    _expect(y, x.shape, x.dtype, x.device, "y")
    _check(lib.vjp_scaled_silu_fwd(_ptr(x), _ptr(w), _ptr(_flat(y)), x.numel(), _dt(x),
                                   _stream(x)), "vjp_scaled_silu_fwd")
    return y


def vjp_scaled_silu_elems_per_tile(n: int) -> int:
    return int(lib.vjp_scaled_silu_elems_per_tile(n))


def vjp_scaled_silu_bwd_workspace_size(n: int) -> int:
    return int(lib.vjp_scaled_silu_bwd_workspace_size(n))


def vjp_scaled_silu_bwd(dy, x, w, dx=None, dw=None, accumulate=False, workspace=None):
    """(dx, dw): dx in x's dtype, dw one fp32 (added into when accumulate)."""
    x = _flat(x)
    if dx is None:
        dx = torch.empty_like(x)
    if dw is None:
        dw = torch.empty(1, dtype=torch.float32, device=x.device)
    _expect(dy, x.shape, x.dtype, x.device, "dy")
    _expect(w, (1,), torch.float32, x.device, "w")
    _expect(dx, x.shape, x.dtype, x.device, "dx")
    _expect(dw, (1,), torch.float32, x.device, "dw")
    ws = _workspace(vjp_scaled_silu_bwd_workspace_size(x.numel()), x, workspace)
    _check(lib.vjp_scaled_silu_bwd(_ptr(_flat(dy)), _ptr(x), _ptr(w), _ptr(_flat(dx)), _ptr(dw),
                                   int(bool(accumulate)), x.numel(), _dt(x), _ptr(ws),
                                   _nbytes(ws), _stream(x)), "vjp_scaled_silu_bwd")
    return dx, dw


def vjp_scaled_silu_bwd_noalloc(dy, x, w, dx, dw, accumulate=False):
    """vjp_scaled_silu_bwd for callers that cannot allocate: dx and dw are the
    caller's; the partials go to the library's per-GPU scratch (no workspace,
    nothing allocated).  Calls that overlap on one GPU race."""
    x = _flat(x)
    _expect(dy, x.shape, x.dtype, x.device, "dy")
    _expect(w, (1,), torch.float32, x.device, "w")
    _expect(dx, x.shape, x.dtype, x.device, "dx")
    _expect(dw, (1,), torch.float32, x.device, "dw")
    _check(lib.vjp_scaled_silu_bwd_noalloc(_ptr(_flat(dy)), _ptr(x), _ptr(w), _ptr(_flat(dx)),
                                           _ptr(dw), int(bool(accumulate)), x.numel(), _dt(x),
                                           _stream(x)), "vjp_scaled_silu_bwd_noalloc")
    return dx, dw


# ----------------------------------------------------------------- softmax

def vjp_softmax_fwd(x, y=None):
    rows, cols = x.shape
    if y is None:
        y = torch.empty_like(x)
    _expect(y, (rows, cols), x.dtype, x.device, "y")
    _check(lib.vjp_softmax_fwd(_ptr(x), _ld(x), _ptr(y), _ld(y), rows, cols, _dt(x), _stream(x)),
           "vjp_softmax_fwd")
    return y


def vjp_softmax_bwd(dy, y, dx=None):
    rows, cols = y.shape
    if dx is None:
        dx = torch.empty_like(y)
    _expect(dy, (rows, cols), y.dtype, y.device, "dy")
    _expect(dx, (rows, cols), y.dtype, y.device, "dx")
    _check(lib.vjp_softmax_bwd(_ptr(dy), _ld(dy), _ptr(y), _ld(y), _ptr(dx), _ld(dx), rows, cols,
                               _dt(y), _stream(y)), "vjp_softmax_bwd")
    return dx


def vjp_softmax_fwd_lse(x, y=None, row_lse=None, write_y=True):
    """(y, row_lse): softmax and the row logsumexp L = m + log l (fp32 [rows]).

    write_y=False computes row_lse alone (y is returned as None)."""
    rows, cols = x.shape
    if write_y and y is None:
        y = torch.empty_like(x)
    if row_lse is None:
        row_lse = torch.empty(rows, dtype=torch.float32, device=x.device)
    if y is not None:
        _expect(y, (rows, cols), x.dtype, x.device, "y")
    _expect(row_lse, (rows,), torch.float32, x.device, "row_lse")
    _check(lib.vjp_softmax_fwd_lse(_ptr(x), _ld(x), _ptr(y), _ld(y) if y is not None else 0,
                                   _ptr(row_lse), rows, cols, _dt(x), _stream(x)),
           "vjp_softmax_fwd_lse")
    return y, row_lse


def vjp_softmax_bwd_lse(dy, x, row_lse, dx=None):
    """dx from dy, the forward's input x and its row logsumexp (y rebuilt on chip)."""
    rows, cols = x.shape
    if dx is None:
        dx = torch.empty_like(x)
    _expect(dy, (rows, cols), x.dtype, x.device, "dy")
    _expect(row_lse, (rows,), torch.float32, x.device, "row_lse")
    _expect(dx, (rows, cols), x.dtype, x.device, "dx")
    _check(lib.vjp_softmax_bwd_lse(_ptr(dy), _ld(dy), _ptr(x), _ld(x), _ptr(row_lse), _ptr(dx),
                                   _ld(dx), rows, cols, _dt(x), _stream(x)),
           "vjp_softmax_bwd_lse")
    return dx


# ----------------------------------------------------------------- softmax cross-entropy

def vjp_softmax_xent_workspace_size(rows: int) -> int:
    return int(lib.vjp_softmax_xent_workspace_size(rows))


def vjp_softmax_xent_fwd_bwd(logits, targets, grad_scale=None, dlogits=None, loss=None,
                             row_max=None, row_lse=None, n_invalid=None, count_invalid=True,
                             workspace=None):
    """Mean cross-entropy of softmax(logits) and its logit gradient.

    Returns dict(loss [1] fp32, row_max [R] fp32, row_lse [R] fp32,
    dlogits [R, C] in the logits' dtype, n_invalid [1] int32 or None).
    grad_scale defaults to 1 / R (unit upstream gradient of the mean).
    """
    rows, classes = logits.shape
    dev = logits.device
    if grad_scale is None:
        grad_scale = 1.0 / rows if rows > 0 else 0.0
    if dlogits is None:
        dlogits = torch.empty_like(logits)
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32) if loss is None else loss
    row_max = torch.empty(rows, **f32) if row_max is None else row_max
    row_lse = torch.empty(rows, **f32) if row_lse is None else row_lse
    if count_invalid and n_invalid is None:
        n_invalid = torch.empty(1, dtype=torch.int32, device=dev)
    _expect(targets, (rows,), torch.int32, dev, "targets")
    _expect(dlogits, (rows, classes), logits.dtype, dev, "dlogits")
    _expect(loss, (1,), torch.float32, dev, "loss")
    _expect(row_max, (rows,), torch.float32, dev, "row_max")
    _expect(row_lse, (rows,), torch.float32, dev, "row_lse")
    if n_invalid is not None:
        _expect(n_invalid, (1,), torch.int32, dev, "n_invalid")
    ws = _workspace(vjp_softmax_xent_workspace_size(rows), logits, workspace)
    _check(lib.vjp_softmax_xent_fwd_bwd(_ptr(logits), _ld(logits), _ptr(_flat(targets)), rows,
                                        classes, _dt(logits), float(grad_scale), _ptr(loss),
                                        _ptr(row_max), _ptr(row_lse), _ptr(dlogits),
                                        _ld(dlogits), _ptr(n_invalid), _ptr(ws), _nbytes(ws),
                                        _stream(logits)), "vjp_softmax_xent_fwd_bwd")
    return {"loss": loss, "row_max": row_max, "row_lse": row_lse, "dlogits": dlogits,
            "n_invalid": n_invalid}


def vjp_softmax_xent_fwd(logits, targets, loss=None, row_lse=None, row_max=None, want_max=False,
                         n_invalid=None, count_invalid=True, workspace=None):
    """Forward of the split form: dict(loss [1], row_lse [R], row_max [R] or None,
    n_invalid [1] int32 or None).  The logits are read once; no gradient is formed."""
    rows, classes = logits.shape
    dev = logits.device
    f32 = dict(dtype=torch.float32, device=dev)
    loss = torch.empty(1, **f32) if loss is None else loss
    row_lse = torch.empty(rows, **f32) if row_lse is None else row_lse
    if want_max and row_max is None:
        row_max = torch.empty(rows, **f32)
    if count_invalid and n_invalid is None:
        n_invalid = torch.empty(1, dtype=torch.int32, device=dev)
    _expect(targets, (rows,), torch.int32, dev, "targets")
    _expect(loss, (1,), torch.float32, dev, "loss")
    _expect(row_lse, (rows,), torch.float32, dev, "row_lse")
    if row_max is not None:
        _expect(row_max, (rows,), torch.float32, dev, "row_max")
    if n_invalid is not None:
        _expect(n_invalid, (1,), torch.int32, dev, "n_invalid")
    ws = _workspace(vjp_softmax_xent_workspace_size(rows), logits, workspace)
    _check(lib.vjp_softmax_xent_fwd(_ptr(logits), _ld(logits), _ptr(_flat(targets)), rows, classes,
                                    _dt(logits), _ptr(loss), _ptr(row_max), _ptr(row_lse),
                                    _ptr(n_invalid), _ptr(ws), _nbytes(ws), _stream(logits)),
           "vjp_softmax_xent_fwd")
    return {"loss": loss, "row_lse": row_lse, "row_max": row_max, "n_invalid": n_invalid}


def vjp_softmax_xent_bwd(logits, targets, row_lse, dloss, dlogits=None):
    """dlogits = (dloss / R) (exp(z - row_lse) - onehot); dloss is a one-element
    fp32 device tensor.  dlogits may be ``logits`` itself (in place)."""
    rows, classes = logits.shape
    dev = logits.device
    if dlogits is None:
        dlogits = torch.empty_like(logits)
    _expect(targets, (rows,), torch.int32, dev, "targets")
    _expect(row_lse, (rows,), torch.float32, dev, "row_lse")
    _expect(dloss, (1,), torch.float32, dev, "dloss")
    _expect(dlogits, (rows, classes), logits.dtype, dev, "dlogits")
    _check(lib.vjp_softmax_xent_bwd(_ptr(logits), _ld(logits), _ptr(_flat(targets)),
                                    _ptr(row_lse), rows, classes, _dt(logits), _ptr(_flat(dloss)),
                                    _ptr(dlogits), _ld(dlogits), _stream(logits)),
           "vjp_softmax_xent_bwd")
    return dlogits


# ----------------------------------------------------------------- LayerNorm / RMSNorm

def vjp_norm_max_cols(dtype=torch.bfloat16, aligned16=True) -> int:
    return int(lib.vjp_norm_max_cols(_DT[dtype], int(bool(aligned16))))


def vjp_layernorm_bwd_workspace_size(rows: int, cols: int) -> int:
    return int(lib.vjp_layernorm_bwd_workspace_size(rows, cols))


def vjp_rmsnorm_bwd_workspace_size(rows: int, cols: int) -> int:
    return int(lib.vjp_rmsnorm_bwd_workspace_size(rows, cols))


def _stats(t, rows, dev, name):
    if t is not None:
        _expect(t, (rows,), torch.float32, dev, name)
    return t


def vjp_layernorm_fwd(x, w, b, eps=1e-5, y=None, row_mean=None, row_rstd=None, save_stats=True):
    """(y, row_mean, row_rstd): LayerNorm over the last dim of x [rows, cols];
    the statistics are fp32 [rows] (None when save_stats is False)."""
    rows, cols = x.shape
    dev = x.device
    if y is None:
        y = torch.empty_like(x)
    if save_stats:
        row_mean = torch.empty(rows, dtype=torch.float32, device=dev) if row_mean is None else row_mean
        row_rstd = torch.empty(rows, dtype=torch.float32, device=dev) if row_rstd is None else row_rstd
    _expect(y, (rows, cols), x.dtype, dev, "y")
    _expect(w, (cols,), None, dev, "w")
    _expect(b, (cols,), w.dtype, dev, "b")
    _stats(row_mean, rows, dev, "row_mean")
    _stats(row_rstd, rows, dev, "row_rstd")
    _check(lib.vjp_layernorm_fwd(_ptr(x), _ld(x), _ptr(_flat(w)), _ptr(_flat(b)), _ptr(y), _ld(y),
                                 _ptr(row_mean), _ptr(row_rstd), rows, cols, float(eps), _dt(x),
                                 _dt(w), _stream(x)), "vjp_layernorm_fwd")
    return y, row_mean, row_rstd


def vjp_layernorm_bwd(dy, x, w, row_mean=None, row_rstd=None, eps=1e-5, dx=None, dw=None, db=None,
                      accumulate=False, workspace=None):
    """(dx, dw, db); dw, db fp32 [cols].  Without saved statistics they are
    recomputed from x."""
    rows, cols = x.shape
    dev = x.device
    if dx is None:
        dx = torch.empty_like(x)
    f32 = dict(dtype=torch.float32, device=dev)
    dw = torch.empty(cols, **f32) if dw is None else dw
    db = torch.empty(cols, **f32) if db is None else db
    _expect(dy, (rows, cols), x.dtype, dev, "dy")
    _expect(w, (cols,), None, dev, "w")
    _expect(dx, (rows, cols), x.dtype, dev, "dx")
    _expect(dw, (cols,), torch.float32, dev, "dw")
    _expect(db, (cols,), torch.float32, dev, "db")
    _stats(row_mean, rows, dev, "row_mean")
    _stats(row_rstd, rows, dev, "row_rstd")
    ws = _workspace(vjp_layernorm_bwd_workspace_size(rows, cols), x, workspace)
    _check(lib.vjp_layernorm_bwd(_ptr(dy), _ld(dy), _ptr(x), _ld(x), _ptr(_flat(w)), _ptr(row_mean),
                                 _ptr(row_rstd), _ptr(dx), _ld(dx), _ptr(dw), _ptr(db),
                                 int(bool(accumulate)), rows, cols, float(eps), _dt(x), _dt(w),
                                 _ptr(ws), _nbytes(ws), _stream(x)), "vjp_layernorm_bwd")
    return dx, dw, db


def vjp_rmsnorm_fwd(x, w, eps=1e-6, y=None, row_rstd=None, save_stats=True):
    """(y, row_rstd): RMSNorm over the last dim of x [rows, cols]."""
    rows, cols = x.shape
    dev = x.device
    if y is None:
        y = torch.empty_like(x)
    if save_stats and row_rstd is None:
        row_rstd = torch.empty(rows, dtype=torch.float32, device=dev)
    _expect(y, (rows, cols), x.dtype, dev, "y")
    _expect(w, (cols,), None, dev, "w")
    _stats(row_rstd, rows, dev, "row_rstd")
    _check(lib.vjp_rmsnorm_fwd(_ptr(x), _ld(x), _ptr(_flat(w)), _ptr(y), _ld(y), _ptr(row_rstd),
                               rows, cols, float(eps), _dt(x), _dt(w), _stream(x)),
           "vjp_rmsnorm_fwd")
    return y, row_rstd


def vjp_rmsnorm_bwd(dy, x, w, row_rstd=None, eps=1e-6, dx=None, dw=None, accumulate=False,
                    workspace=None):
    """(dx, dw); dw fp32 [cols]."""
    rows, cols = x.shape
    dev = x.device
    if dx is None:
        dx = torch.empty_like(x)
    dw = torch.empty(cols, dtype=torch.float32, device=dev) if dw is None else dw
    _expect(dy, (rows, cols), x.dtype, dev, "dy")
    _expect(w, (cols,), None, dev, "w")
    _expect(dx, (rows, cols), x.dtype, dev, "dx")
    _expect(dw, (cols,), torch.float32, dev, "dw")
    _stats(row_rstd, rows, dev, "row_rstd")
    ws = _workspace(vjp_rmsnorm_bwd_workspace_size(rows, cols), x, workspace)
    _check(lib.vjp_rmsnorm_bwd(_ptr(dy), _ld(dy), _ptr(x), _ld(x), _ptr(_flat(w)), _ptr(row_rstd),
                               _ptr(dx), _ld(dx), _ptr(dw), int(bool(accumulate)), rows, cols,
                               float(eps), _dt(x), _dt(w), _ptr(ws), _nbytes(ws), _stream(x)),
           "vjp_rmsnorm_bwd")
    return dx, dw


# ----------------------------------------------------------------- gather / scatter-add

def vjp_gather_rows_bwd_workspace_size(M: int, V: int, D: int) -> int:
    return int(lib.vjp_gather_rows_bwd_workspace_size(M, V, D))


def vjp_gather_rows_fwd(table, idx, y=None):
    """y[m] = table[idx[m]] (zero row for an index outside [0, V))."""
    V, D = table.shape
    M = idx.numel()
    if y is None:
        y = torch.empty((M, D), dtype=table.dtype, device=table.device)
    _expect(idx, (M,), torch.int32, table.device, "idx")
    _expect(y, (M, D), table.dtype, table.device, "y")
    _check(lib.vjp_gather_rows_fwd(_ptr(table), _ld(table), V, D, _ptr(_flat(idx)), M, _ptr(y),
                                   _ld(y), _dt(table), _stream(table)), "vjp_gather_rows_fwd")
    return y


def vjp_gather_rows_bwd(dy, idx, V, dtable=None, accumulate=False, n_invalid=None,
                        count_invalid=True, workspace=None):
    """(dtable fp32 [V, D], n_invalid int32 [1] or None): the scatter-add of dy rows."""
    M, D = dy.shape
    dev = dy.device
    if dtable is None:
        dtable = torch.empty((V, D), dtype=torch.float32, device=dev)
    if count_invalid and n_invalid is None:
        n_invalid = torch.empty(1, dtype=torch.int32, device=dev)
    _expect(idx, (M,), torch.int32, dev, "idx")
    _expect(dtable, (V, D), torch.float32, dev, "dtable")
    if n_invalid is not None:
        _expect(n_invalid, (1,), torch.int32, dev, "n_invalid")
    ws = _workspace(vjp_gather_rows_bwd_workspace_size(M, V, D), dy, workspace)
    _check(lib.vjp_gather_rows_bwd(_ptr(dy), _ld(dy), _ptr(_flat(idx)), M, V, D, _ptr(dtable),
                                   _ld(dtable), int(bool(accumulate)), _ptr(n_invalid), _dt(dy),
                                   _ptr(ws), _nbytes(ws), _stream(dy)), "vjp_gather_rows_bwd")
    return dtable, n_invalid
