"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, sizes workspaces as documented, and rejects bad arguments
before launching anything (every call here returns before any HIP call).
Fake device addresses are used only for argument checking and are never
dereferenced."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libvjp.h")


def _ensure_built():
    lib = os.path.join(ROOT, "row_wise_backward_amd", "libvjp.so")
    if not os.path.exists(lib):
        subprocess.run(["python", os.path.join(ROOT, "row_wise_backward_amd", "build.py"), "-q"],
                       check=True)


def _load_build():
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "_libvjp_build_for_tests", os.path.join(ROOT, "row_wise_backward_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_ensure_built()
import row_wise_backward_amd as rwb  # noqa: E402

L = rwb.lib
P = ctypes.c_void_p
OK, EINVAL, EDTYPE, EALIGN, EWORKSPACE, EALIAS = 0, 1, 2, 3, 4, 5
A, B, C, D = 0x10000000, 0x20000000, 0x30000000, 0x40000000  # fake, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vjp_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ["vjp_weighted_sum_fwd", "vjp_weighted_sum_bwd", "vjp_scaled_silu_fwd",
              "vjp_scaled_silu_bwd", "vjp_softmax_fwd", "vjp_softmax_bwd",
              "vjp_softmax_xent_fwd_bwd"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in libvjp.h but not exported"
    nm = subprocess.run(["nm", "-D", "--defined-only", rwb.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (vjp_\w+)", nm))
    assert exported == set(declared_functions()), exported ^ set(declared_functions())


def test_binding_covers_every_entry_point():
    for n in declared_functions():
        assert n in rwb.EXPORTED and callable(getattr(rwb, n))


def test_version_and_strings():
    assert rwb.vjp_version() == 1
    assert rwb.vjp_status_string(OK) == "ok"
    assert "alias" in rwb.vjp_status_string(EALIAS) or "overlap" in rwb.vjp_status_string(EALIAS)


def test_tiling_queries():
    # the worked example: 100 rows in tiles of 32 -> 4 partial rows of 64 fp32
    assert rwb.vjp_weighted_sum_tiling(100, 32) == (32, 4)
    assert rwb.vjp_weighted_sum_bwd_workspace_size(100, 64, 32) == 4 * 64 * 4
    # automatic tiling depends only on the row count: blocks of 32 rows dealt
    # round-robin to at most 1024 tiles
    assert rwb.vjp_weighted_sum_tiling(100, 0) == (32, 4)
    assert rwb.vjp_weighted_sum_tiling(32768, 0) == (32, 1024)
    assert rwb.vjp_weighted_sum_tiling(32767, 0) == (32, 1024)
    assert rwb.vjp_weighted_sum_tiling(32736, 0) == (32, 1023)
    assert rwb.vjp_weighted_sum_tiling(1 << 20, 0) == (32, 1024)
    assert rwb.vjp_weighted_sum_tiling(0, 0) == (32, 0)
    assert rwb.vjp_weighted_sum_bwd_workspace_size(1 << 20, 256, 0) == 1024 * 256 * 4
    assert rwb.vjp_weighted_sum_tiling(7, 1 << 30) == (1 << 30, 1)
    assert L.vjp_weighted_sum_tiling(-1, 0, None, None) == EINVAL
    i64 = ctypes.c_int64
    assert L.vjp_weighted_sum_tiling(10, (1 << 30) + 1, ctypes.byref(i64()), ctypes.byref(i64())) == EINVAL
    assert L.vjp_weighted_sum_tiling(10, 0, None, ctypes.byref(i64())) == EINVAL
    assert rwb.vjp_weighted_sum_bwd_workspace_size(10, 4, (1 << 30) + 1) == 0
    assert rwb.vjp_scaled_silu_elems_per_tile(1 << 24) == 4096
    assert rwb.vjp_scaled_silu_bwd_workspace_size(1 << 24) == 4096 * 4
    assert rwb.vjp_scaled_silu_elems_per_tile(7) == 2048
    assert rwb.vjp_scaled_silu_bwd_workspace_size(0) == 0
    assert rwb.vjp_softmax_xent_workspace_size(16384) == 16384 * 4


def _ws_fwd(**kw):
    a = dict(x=A, ld=64, w=B, y=C, n=10, d=64, act=0, wdt=0)
    a.update(kw)
    return L.vjp_weighted_sum_fwd(P(a["x"]), a["ld"], P(a["w"]), P(a["y"]), a["n"], a["d"],
                                  a["act"], a["wdt"], None)


def test_weighted_sum_fwd_rejections():
    assert _ws_fwd(n=-1) == EINVAL
    assert _ws_fwd(ld=63) == EINVAL
    assert _ws_fwd(act=3) == EDTYPE
    assert _ws_fwd(wdt=-1) == EDTYPE
    assert _ws_fwd(x=0) == EINVAL
    assert _ws_fwd(x=A + 2) == EALIGN
    assert _ws_fwd(act=1, x=A + 1) == EALIGN
    assert _ws_fwd(y=A + 64) == EALIAS                    # y inside x
    assert _ws_fwd(y=B + 8) == EALIAS                     # y inside w
    assert "overlaps" in rwb.vjp_last_error()
    assert _ws_fwd(n=1 << 62, d=0, ld=0) == EINVAL        # no byte count can overflow
    assert _ws_bwd(n=1, d=65535 * 64 + 1, ld=65535 * 64 + 1, ldd=65535 * 64 + 1) == EINVAL
    assert "d above" in rwb.vjp_last_error()


def _ws_bwd(**kw):
    a = dict(dy=A, x=B, ld=64, w=C, dx=D, ldd=64, dw=D + 0x1000000, acc=0, n=100, d=64, rpt=32,
             act=0, wdt=0, ws=D + 0x2000000, wsb=1024)
    a.update(kw)
    return L.vjp_weighted_sum_bwd(P(a["dy"]), P(a["x"]), a["ld"], P(a["w"]), P(a["dx"]), a["ldd"],
                                  P(a["dw"]), a["acc"], a["n"], a["d"], a["rpt"], a["act"],
                                  a["wdt"], P(a["ws"]), a["wsb"], None)


def test_weighted_sum_bwd_rejections():
    assert _ws_bwd(wsb=1023) == EWORKSPACE
    assert _ws_bwd(ws=0) == EWORKSPACE
    assert _ws_bwd(ws=D + 0x2000002) == EALIGN
    assert _ws_bwd(acc=2) == EINVAL
    assert _ws_bwd(rpt=-3) == EINVAL
    assert _ws_bwd(dw=0) == EINVAL
    assert _ws_bwd(dw=D + 0x1000002) == EALIGN
    assert _ws_bwd(ldd=10) == EINVAL
    assert _ws_bwd(dx=B + 4) == EALIAS                    # dx over x
    assert _ws_bwd(dw=D + 8) == EALIAS                    # dw inside dx
    assert _ws_bwd(ws=A) == EALIAS                        # workspace over dy


def _silu_bwd(**kw):
    a = dict(dy=A, x=B, w=C, dx=D, dw=D + 0x1000000, acc=0, n=1 << 20, act=1,
             ws=D + 0x2000000, wsb=1 << 20)
    a.update(kw)
    return L.vjp_scaled_silu_bwd(P(a["dy"]), P(a["x"]), P(a["w"]), P(a["dx"]), P(a["dw"]), a["acc"],
                                 a["n"], a["act"], P(a["ws"]), a["wsb"], None)


def test_scaled_silu_rejections():
    assert L.vjp_scaled_silu_fwd(P(A), P(B), P(A + 2), 100, 1, None) == EALIAS
    assert L.vjp_scaled_silu_fwd(P(A), P(B + 2), P(C), 100, 1, None) == EALIGN
    assert L.vjp_scaled_silu_fwd(P(A), P(B), P(C), -5, 1, None) == EINVAL
    assert L.vjp_scaled_silu_fwd(P(A), P(B), P(C), 5, 7, None) == EDTYPE
    assert _silu_bwd(wsb=4) == EWORKSPACE
    assert _silu_bwd(w=0) == EINVAL
    assert _silu_bwd(dx=A + 2) == EALIAS


def test_softmax_rejections():
    assert L.vjp_softmax_fwd(P(A), 100, P(A + 100), 100, 10, 100, 2, None) == EALIAS
    assert L.vjp_softmax_fwd(P(A), 99, P(B), 100, 10, 100, 2, None) == EINVAL
    assert L.vjp_softmax_fwd(P(A), 100, P(B), 100, 10, 0, 2, None) == EINVAL   # no columns
    assert L.vjp_softmax_bwd(P(A), 100, P(B), 100, P(B), 100, 10, 100, 2, None) == EALIAS
    assert L.vjp_softmax_bwd(P(A), 100, P(B), 100, P(C + 1), 100, 10, 100, 2, None) == EALIGN


def _xent(**kw):
    a = dict(z=A, ld=1000, t=B, rows=10, C=1000, act=2, loss=C, rmax=C + 64, rlse=C + 128,
             dz=D, ldd=1000, ninv=C + 256, ws=C + 512, wsb=40)
    a.update(kw)
    return L.vjp_softmax_xent_fwd_bwd(P(a["z"]), a["ld"], P(a["t"]), a["rows"], a["C"], a["act"],
                                      ctypes.c_float(0.1), P(a["loss"]), P(a["rmax"]), P(a["rlse"]),
                                      P(a["dz"]), a["ldd"], P(a["ninv"]), P(a["ws"]), a["wsb"],
                                      None)


def test_softmax_xent_rejections():
    assert _xent(C=0) == EINVAL
    assert _xent(wsb=39) == EWORKSPACE
    assert _xent(rlse=C + 64 + 8) == EALIAS               # row_lse over row_max
    assert _xent(ninv=C + 2) == EALIGN
    assert _xent(dz=A + 10) == EALIAS
    assert _xent(t=0) == EINVAL
    assert _xent(rmax=0) == EINVAL


def test_softmax_lse_rejections():
    assert L.vjp_softmax_fwd_lse(P(A), 100, P(B), 100, None, 10, 100, 2, None) == EINVAL   # no row_lse
    assert L.vjp_softmax_fwd_lse(P(A), 100, P(B), 100, P(A + 8), 10, 100, 2, None) == EALIAS
    assert L.vjp_softmax_fwd_lse(P(A), 100, P(B), 100, P(B + 64), 10, 100, 2, None) == EALIAS
    assert L.vjp_softmax_fwd_lse(P(A), 100, P(B), 100, P(C + 2), 10, 100, 2, None) == EALIGN
    assert L.vjp_softmax_bwd_lse(P(A), 100, P(B), 100, None, P(C), 100, 10, 100, 2, None) == EINVAL
    assert L.vjp_softmax_bwd_lse(P(A), 100, P(B), 100, P(D + 1), P(C), 100, 10, 100, 2, None) == EALIGN
    assert L.vjp_softmax_bwd_lse(P(A), 100, P(B), 100, P(D), P(D + 16), 100, 10, 100, 2, None) == EALIAS
    assert L.vjp_softmax_bwd_lse(P(A), 100, P(B), 100, P(D), P(B + 2), 100, 10, 100, 2, None) == EALIAS
    # empty problems are accepted and launch nothing
    assert L.vjp_softmax_fwd_lse(P(A), 100, None, 0, None, 0, 100, 2, None) == OK
    assert L.vjp_softmax_bwd_lse(P(A), 100, P(B), 100, None, P(C), 100, 0, 100, 2, None) == OK


def _xent_fwd(**kw):
    a = dict(z=A, ld=1000, t=B, rows=10, C=1000, act=2, loss=C, rmax=C + 64, rlse=C + 128,
             ninv=C + 256, ws=C + 512, wsb=40)
    a.update(kw)
    return L.vjp_softmax_xent_fwd(P(a["z"]), a["ld"], P(a["t"]), a["rows"], a["C"], a["act"],
                                  P(a["loss"]), P(a["rmax"]), P(a["rlse"]), P(a["ninv"]),
                                  P(a["ws"]), a["wsb"], None)


def _xent_bwd(**kw):
    a = dict(z=A, ld=1000, t=B, rlse=C, rows=10, C=1000, act=2, dloss=C + 64, dz=D, ldd=1000)
    a.update(kw)
    return L.vjp_softmax_xent_bwd(P(a["z"]), a["ld"], P(a["t"]), P(a["rlse"]), a["rows"], a["C"],
                                  a["act"], P(a["dloss"]), P(a["dz"]), a["ldd"], None)


def test_softmax_xent_split_rejections():
    assert _xent_fwd(rlse=0) == EINVAL
    assert _xent_fwd(wsb=39) == EWORKSPACE
    assert _xent_fwd(rmax=C + 128 + 8) == EALIAS          # row_max over row_lse
    assert _xent_fwd(C=0) == EINVAL
    assert _xent_fwd(act=5) == EDTYPE
    assert _xent_bwd(dloss=0) == EINVAL
    assert _xent_bwd(dloss=C + 2) == EALIGN
    assert _xent_bwd(dz=A + 2) == EALIAS                  # partial overlap with the logits
    assert _xent_bwd(dz=A, ldd=1008) == EALIAS            # same base, other leading dimension
    assert _xent_bwd(dz=C) == EALIAS                      # over row_lse
    assert _xent_bwd(rlse=0) == EINVAL
    assert _xent_bwd(rows=0) == OK                        # nothing to do, nothing launched
    wide = 65535 * 4096                                   # 65535 column blocks of 4096
    assert _xent_bwd(rows=0, C=wide, ld=wide, ldd=wide) == OK
    assert _xent_bwd(rows=0, C=wide + 1, ld=wide + 1, ldd=wide + 1) == EINVAL


def test_binding_host_guards():
    """The binding checks shapes, dtypes and devices before calling the C ABI."""
    import torch

    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        rwb.vjp_weighted_sum_fwd(x, torch.zeros(8))        # host tensors never reach a kernel
    with pytest.raises(ValueError):
        rwb._ld(torch.zeros(1, 8).expand(4, 8))            # overlapping rows
    with pytest.raises(ValueError):
        rwb._ld(torch.zeros(8, 4).t())                     # non-unit inner stride
    with pytest.raises(ValueError):
        rwb._expect(torch.zeros(3), (4,), None, torch.device("cpu"), "y")


def test_autograd_layer_rejects_host_tensors():
    """The autograd wrappers call the same guarded binding: CPU tensors never
    reach a kernel, and there is no CPU fallback."""
    import torch

    from row_wise_backward_amd import autograd as ag

    x = torch.zeros(4, 8, requires_grad=True)
    with pytest.raises(ValueError):
        ag.weighted_sum(x, torch.zeros(8))
    with pytest.raises(ValueError):
        ag.softmax(x)
    with pytest.raises(ValueError):
        ag.softmax_cross_entropy(x, torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError):
        ag.softmax(x, save="nothing")


def _ln_fwd(**kw):
    a = dict(x=A, ld=64, w=B, b=B + 0x1000, y=C, ldy=64, mean=D, rstd=D + 0x1000, rows=10, cols=64,
             eps=1e-5, act=2, wdt=2)
    a.update(kw)
    return L.vjp_layernorm_fwd(P(a["x"]), a["ld"], P(a["w"]), P(a["b"]), P(a["y"]), a["ldy"],
                               P(a["mean"]), P(a["rstd"]), a["rows"], a["cols"],
                               ctypes.c_float(a["eps"]), a["act"], a["wdt"], None)


def _ln_bwd(**kw):
    a = dict(dy=A, x=B, w=C, mean=D, rstd=D + 0x1000, dx=D + 0x100000, dw=D + 0x200000,
             db=D + 0x201000, acc=0, rows=10, cols=64, eps=1e-5, act=2, wdt=2, ws=D + 0x300000,
             wsb=10 * 128 * 4)
    a.update(kw)
    return L.vjp_layernorm_bwd(P(a["dy"]), 64, P(a["x"]), 64, P(a["w"]), P(a["mean"]), P(a["rstd"]),
                               P(a["dx"]), 64, P(a["dw"]), P(a["db"]), a["acc"], a["rows"], a["cols"],
                               ctypes.c_float(a["eps"]), a["act"], a["wdt"], P(a["ws"]), a["wsb"], None)


def test_norm_queries_and_rejections():
    assert rwb.vjp_norm_max_cols() == 16384
    assert L.vjp_norm_max_cols(0, 0) == 16384 and L.vjp_norm_max_cols(9, 1) == -1
    # round-robin tiles: min(512, rows) partial rows of 2 cols (LayerNorm) or cols (RMSNorm)
    assert rwb.vjp_layernorm_bwd_workspace_size(10, 64) == 10 * 128 * 4
    assert rwb.vjp_layernorm_bwd_workspace_size(32768, 4096) == 512 * 8192 * 4
    assert rwb.vjp_rmsnorm_bwd_workspace_size(5000, 100) == 512 * 100 * 4
    assert _ln_fwd(eps=-1.0) == EINVAL
    assert _ln_fwd(eps=float("inf")) == EINVAL
    assert _ln_fwd(cols=16385, ld=16385, ldy=16385) == EINVAL        # wider than the resident limit
    assert "16384" in rwb.vjp_last_error()
    assert _ln_fwd(cols=0, ld=0, ldy=0) == EINVAL
    assert _ln_fwd(b=0) == EINVAL
    assert _ln_fwd(y=A + 64) == EALIAS
    assert _ln_fwd(rstd=D + 4) == EALIAS                             # rstd over mean
    assert _ln_fwd(act=4) == EDTYPE
    assert _ln_bwd(wsb=10 * 128 * 4 - 1) == EWORKSPACE
    assert _ln_bwd(mean=0) == EINVAL                                 # mean without rstd
    assert _ln_bwd(acc=3) == EINVAL
    assert _ln_bwd(db=D + 0x200000 + 8) == EALIAS                    # db over dw
    assert _ln_bwd(dx=B + 2) == EALIAS
    assert L.vjp_rmsnorm_fwd(P(A), 64, P(B), P(A + 2), 64, None, 10, 64, ctypes.c_float(1e-6), 2, 2, None) == EALIAS


def test_gather_queries_and_rejections():
    n = rwb.vjp_gather_rows_bwd_workspace_size(1000, 50, 64)
    assert n > 0 and n % 4 == 0
    assert rwb.vjp_gather_rows_bwd_workspace_size(-1, 5, 5) == 0
    fwd = lambda **k: L.vjp_gather_rows_fwd(P(k.get("t", A)), k.get("ldt", 64), k.get("V", 10), 64,
                                            P(k.get("idx", B)), k.get("M", 20), P(k.get("y", C)),
                                            64, k.get("act", 2), None)
    assert fwd(y=A + 128) == EALIAS
    assert fwd(ldt=63) == EINVAL
    assert fwd(idx=B + 2) == EALIGN
    assert fwd(act=7) == EDTYPE
    assert fwd(V=1 << 31) == EINVAL
    assert L.vjp_gather_rows_fwd(P(A), 1 << 24, 1, (1 << 24), P(B), 1, P(C), 1 << 24, 2,
                                 None) == EINVAL                   # D above 65535 * 256
    assert fwd(M=0) == OK                                   # nothing to do
    bwd = lambda **k: L.vjp_gather_rows_bwd(P(A), 64, P(B), 20, 10, 64, P(k.get("dt", C)), 64,
                                            k.get("acc", 0), P(k.get("ninv", None)), 2,
                                            P(k.get("ws", D)), k.get("wsb", 1 << 20), None)
    assert bwd(wsb=16) == EWORKSPACE
    assert bwd(ws=D + 4) == EALIGN                          # 16-byte alignment required
    assert bwd(dt=A + 64) == EALIAS
    assert bwd(acc=5) == EINVAL
    assert bwd(ninv=C + 2) == EALIGN
    assert bwd(ninv=D + 8) == EALIAS                        # count inside the workspace


def test_copy_rejections():
    assert L.vjp_copy(P(A), P(B), -1, None) == EINVAL
    assert L.vjp_copy(None, P(B), 16, None) == EINVAL
    assert L.vjp_copy(P(A), None, 16, None) == EINVAL
    assert L.vjp_copy(P(A), P(A + 8), 16, None) == EALIAS      # overlapping ranges
    assert L.vjp_copy(P(A + 8), P(A), 16, None) == EALIAS
    assert L.vjp_copy(None, None, 0, None) == OK               # nothing to do
    sh = lambda **k: L.vjp_copy_shaped(P(k.get("src", A)), P(k.get("dst", B)), k.get("n", 64),
                                       k.get("vpl", 4), k.get("wg", 32768), None)
    for vpl in (0, 3, 5, 16, -4):
        assert sh(vpl=vpl) == EINVAL
    assert sh(wg=0) == EINVAL and sh(wg=1 << 31) == EINVAL
    assert sh(n=-1) == EINVAL and sh(src=None) == EINVAL
    assert sh(dst=A + 8) == EALIAS
    assert sh(src=None, dst=None, n=0) == OK


def test_header_compiles_as_plain_c99():
    """include/libvjp.h is plain C: the C consumer of the ABI compiles with gcc
    -std=c99 -Wall -Wextra against it (and the HIP runtime's C API), with no
    diagnostics from either file of ours."""
    import subprocess

    build = _load_build()
    r = subprocess.run(build.consumer_cmd(link=False), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    ours = [ln for ln in r.stderr.splitlines() if "libvjp.h" in ln or "c_abi_consumer.c" in ln]
    assert not ours, ours
