"""Property-based argument fuzzing of the C ABI, on a host with no GPU.

Random sizes (negative, small, near the int32 and 2^46 limits, up to
2^63 - 1), leading dimensions, dtype codes and fake device addresses (null,
aligned, misaligned, overlapping, near the top of the address space) go
through the entry points.  Every call must return one of the documented
status codes without crashing, and a negative size or an unknown dtype must
be rejected (never VJP_OK, never a launch).  A call whose arguments are all
valid reaches a launch, which fails with VJP_EHIP on a host without a GPU;
so the test runs only where no GPU is visible (on a GPU host a launch on
fake addresses would fault)."""
import ctypes

import pytest

import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import row_wise_backward_amd as rwb

# device_count() counts devices without initialising them
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fuzzing launches on fake addresses: only without a GPU")

L = rwb.lib
P = ctypes.c_void_p
OK, EDTYPE, EHIP = 0, 2, 6
A = 0x10000000

size = st.one_of(st.integers(-4, 70), st.integers(0, 1 << 62),
                 st.sampled_from([(1 << 31) - 1, 1 << 31, 1 << 32, 1 << 46, (1 << 46) + 1,
                                  (1 << 63) - 1, -(1 << 63), 65535 * 256, 65535 * 256 + 1]))
ptr = st.sampled_from([0, A, A + 1, A + 2, A + 8, A + 64, 2 * A, 3 * A, 4 * A, 5 * A,
                       (1 << 63) - 16, (1 << 64) - 16])
dtype = st.integers(-2, 4)
flag = st.integers(-1, 2)
SETTINGS = settings(max_examples=300, deadline=None, derandomize=True)


def _check(status, sizes, dtypes):
    assert 0 <= status <= 6, status
    if any(s < 0 for s in sizes) or any(d not in (0, 1, 2) for d in dtypes):
        assert status not in (OK, EHIP), (status, rwb.vjp_last_error())


@SETTINGS
@given(ptr, size, ptr, ptr, size, size, dtype, dtype)
def test_weighted_sum_fwd(x, ld, w, y, n, d, act, wdt):
    s = L.vjp_weighted_sum_fwd(P(x), ld, P(w), P(y), n, d, act, wdt, None)
    _check(s, (n, d), (act, wdt))


@SETTINGS
@given(ptr, ptr, size, ptr, ptr, size, ptr, flag, size, size, size, dtype, dtype, ptr, size)
def test_weighted_sum_bwd(dy, x, ld, w, dx, ldd, dw, acc, n, d, rpt, act, wdt, ws, wsb):
    s = L.vjp_weighted_sum_bwd(P(dy), P(x), ld, P(w), P(dx), ldd, P(dw), acc, n, d, rpt, act, wdt,
                               P(ws), max(wsb, 0), None)
    _check(s, (n, d, rpt), (act, wdt))


@SETTINGS
@given(ptr, ptr, ptr, ptr, ptr, flag, size, dtype, ptr, size)
def test_scaled_silu_bwd(dy, x, w, dx, dw, acc, n, act, ws, wsb):
    s = L.vjp_scaled_silu_bwd(P(dy), P(x), P(w), P(dx), P(dw), acc, n, act, P(ws), max(wsb, 0), None)
    _check(s, (n,), (act,))


@SETTINGS
@given(ptr, size, ptr, size, size, size, dtype)
def test_softmax_fwd(x, ldx, y, ldy, rows, cols, act):
    s = L.vjp_softmax_fwd(P(x), ldx, P(y), ldy, rows, cols, act, None)
    _check(s, (rows, cols), (act,))


@SETTINGS
@given(ptr, size, ptr, size, size, dtype, ptr, ptr, ptr, ptr, size, ptr, ptr, size)
def test_softmax_xent_fwd_bwd(z, ld, t, rows, classes, act, loss, rmax, rlse, dz, ldz, ninv, ws, wsb):
    s = L.vjp_softmax_xent_fwd_bwd(P(z), ld, P(t), rows, classes, act, ctypes.c_float(0.5), P(loss),
                                   P(rmax), P(rlse), P(dz), ldz, P(ninv), P(ws), max(wsb, 0), None)
    _check(s, (rows, classes), (act,))


@SETTINGS
@given(ptr, size, ptr, ptr, ptr, size, ptr, ptr, size, size, dtype, dtype)
def test_layernorm_fwd(x, ldx, w, b, y, ldy, mean, rstd, rows, cols, act, wdt):
    s = L.vjp_layernorm_fwd(P(x), ldx, P(w), P(b), P(y), ldy, P(mean), P(rstd), rows, cols,
                            ctypes.c_float(1e-5), act, wdt, None)
    _check(s, (rows, cols), (act, wdt))


@SETTINGS
@given(ptr, size, ptr, size, size, size, ptr, size, flag, ptr, dtype, ptr, size)
def test_gather_rows_bwd(dy, ldy, idx, M, V, D, dt, ldt, acc, ninv, act, ws, wsb):
    s = L.vjp_gather_rows_bwd(P(dy), ldy, P(idx), M, V, D, P(dt), ldt, acc, P(ninv), act, P(ws),
                              max(wsb, 0), None)
    _check(s, (M, V, D), (act,))


@SETTINGS
@given(ptr, ptr, size, st.integers(-1, 9), size)
def test_copy_shaped(src, dst, nbytes, vpl, wg):
    s = L.vjp_copy_shaped(P(src), P(dst), nbytes, vpl, wg, None)
    _check(s, (nbytes,), ())


@SETTINGS
@given(size, size, size)
def test_workspace_queries(n, d, rpt):
    # size queries never crash; negative sizes give 0 (or -1 for the tile query)
    L.vjp_weighted_sum_bwd_workspace_size(n, d, rpt)
    L.vjp_scaled_silu_bwd_workspace_size(n)
    L.vjp_softmax_xent_workspace_size(n)
    L.vjp_gather_rows_bwd_workspace_size(n, d, rpt)
    L.vjp_layernorm_bwd_workspace_size(n, d)
    L.vjp_rmsnorm_bwd_workspace_size(n, d)
    assert (L.vjp_scaled_silu_elems_per_tile(n) == -1) == (n < 0)


@SETTINGS
@given(ptr, ptr, ptr, size, dtype)
def test_scaled_silu_fwd(x, w, y, n, act):
    _check(L.vjp_scaled_silu_fwd(P(x), P(w), P(y), n, act, None), (n,), (act,))


@SETTINGS
@given(ptr, ptr, ptr, ptr, ptr, flag, size, dtype)
def test_scaled_silu_bwd_noalloc(dy, x, w, dx, dw, acc, n, act):
    _check(L.vjp_scaled_silu_bwd_noalloc(P(dy), P(x), P(w), P(dx), P(dw), acc, n, act, None),
           (n,), (act,))


@SETTINGS
@given(ptr, size, ptr, size, ptr, size, size, size, dtype)
def test_softmax_bwd(dy, ldg, y, ldy, dx, ldd, rows, cols, act):
    _check(L.vjp_softmax_bwd(P(dy), ldg, P(y), ldy, P(dx), ldd, rows, cols, act, None),
           (rows, cols), (act,))


@SETTINGS
@given(ptr, size, ptr, size, ptr, size, size, dtype)
def test_softmax_fwd_lse(x, ldx, y, ldy, lse, rows, cols, act):
    _check(L.vjp_softmax_fwd_lse(P(x), ldx, P(y), ldy, P(lse), rows, cols, act, None),
           (rows, cols), (act,))


@SETTINGS
@given(ptr, size, ptr, size, ptr, ptr, size, size, size, dtype)
def test_softmax_bwd_lse(dy, ldg, x, ldx, lse, dx, ldd, rows, cols, act):
    _check(L.vjp_softmax_bwd_lse(P(dy), ldg, P(x), ldx, P(lse), P(dx), ldd, rows, cols, act, None),
           (rows, cols), (act,))


@SETTINGS
@given(ptr, size, ptr, size, size, dtype, ptr, ptr, ptr, ptr, ptr, size)
def test_softmax_xent_fwd(z, ld, t, rows, classes, act, loss, rmax, rlse, ninv, ws, wsb):
    _check(L.vjp_softmax_xent_fwd(P(z), ld, P(t), rows, classes, act, P(loss), P(rmax), P(rlse),
                                  P(ninv), P(ws), max(wsb, 0), None), (rows, classes), (act,))


@SETTINGS
@given(ptr, size, ptr, ptr, size, size, dtype, ptr, ptr, size)
def test_softmax_xent_bwd(z, ld, t, lse, rows, classes, act, dloss, dz, ldz):
    _check(L.vjp_softmax_xent_bwd(P(z), ld, P(t), P(lse), rows, classes, act, P(dloss), P(dz), ldz,
                                  None), (rows, classes), (act,))


@SETTINGS
@given(ptr, size, ptr, size, ptr, ptr, ptr, ptr, size, ptr, ptr, flag, size, size, dtype, dtype,
       ptr, size)
def test_layernorm_bwd(dy, ldg, x, ldx, w, mean, rstd, dx, ldd, dw, db, acc, rows, cols, act, wdt,
                       ws, wsb):
    _check(L.vjp_layernorm_bwd(P(dy), ldg, P(x), ldx, P(w), P(mean), P(rstd), P(dx), ldd, P(dw),
                               P(db), acc, rows, cols, ctypes.c_float(1e-5), act, wdt, P(ws),
                               max(wsb, 0), None), (rows, cols), (act, wdt))


@SETTINGS
@given(ptr, size, ptr, ptr, size, ptr, size, size, dtype, dtype)
def test_rmsnorm_fwd(x, ldx, w, y, ldy, rstd, rows, cols, act, wdt):
    _check(L.vjp_rmsnorm_fwd(P(x), ldx, P(w), P(y), ldy, P(rstd), rows, cols, ctypes.c_float(1e-6),
                             act, wdt, None), (rows, cols), (act, wdt))


@SETTINGS
@given(ptr, size, ptr, size, ptr, ptr, ptr, size, ptr, flag, size, size, dtype, dtype, ptr, size)
def test_rmsnorm_bwd(dy, ldg, x, ldx, w, rstd, dx, ldd, dw, acc, rows, cols, act, wdt, ws, wsb):
    _check(L.vjp_rmsnorm_bwd(P(dy), ldg, P(x), ldx, P(w), P(rstd), P(dx), ldd, P(dw), acc, rows,
                             cols, ctypes.c_float(1e-6), act, wdt, P(ws), max(wsb, 0), None),
           (rows, cols), (act, wdt))


@SETTINGS
@given(ptr, size, size, size, ptr, size, ptr, size, dtype)
def test_gather_rows_fwd(tab, ldt, V, D, idx, M, y, ldy, act):
    _check(L.vjp_gather_rows_fwd(P(tab), ldt, V, D, P(idx), M, P(y), ldy, act, None),
           (V, D, M), (act,))


@SETTINGS
@given(ptr, ptr, size)
def test_copy(src, dst, nbytes):
    _check(L.vjp_copy(P(src), P(dst), nbytes, None), (nbytes,), ())


@SETTINGS
@given(size, size, dtype, flag)
def test_tiling_and_norm_queries(n, rpt, act, aligned):
    br, tiles = ctypes.c_int64(0), ctypes.c_int64(0)
    s = L.vjp_weighted_sum_tiling(n, rpt, ctypes.byref(br), ctypes.byref(tiles))
    assert s in (0, 1)
    if s == 0:
        assert br.value >= 1 and tiles.value >= 0
    L.vjp_norm_max_cols(act, aligned)
