"""torch.autograd.gradcheck on every autograd Function of the library.

"Backprop for kernel writers" (closing list of exercises) asks that a
derived backward be checked with torch.autograd.gradcheck: the analytical
Jacobian the Function's backward delivers (through the C ABI's backward
kernels) against central finite differences of its forward (the forward
kernels), column by column, on small inputs.  The kernels compute in fp32
and take fp32 inputs here (there is no fp64 kernel), so the differences
use eps = 1e-3 and the comparison atol = rtol = 2e-3: the finite-difference
noise of an O(1) fp32 function is about u / eps = 6e-5, its truncation
error eps^2 |f'''| / 6 about 1e-6.  nondet_tol = 0: repeated backward calls
must agree bit for bit.
"""
import warnings

import pytest
import torch

from gpu_util import DEV

pytestmark = pytest.mark.gpu
TOL = dict(eps=1e-3, atol=2e-3, rtol=2e-3, nondet_tol=0.0)


def _gradcheck(fn, inputs):
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")          # "inputs are not double precision"
        assert torch.autograd.gradcheck(fn, inputs, **TOL)


def _t(shape, seed, scale=1.0, shift=0.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32) * scale + shift
    return x.to(DEV).requires_grad_(True)


def test_weighted_sum(gpu_lib):
    from row_wise_backward_amd.autograd import weighted_sum
    _gradcheck(weighted_sum, (_t((5, 7), 1), _t((7,), 2)))


def test_scaled_silu(gpu_lib):
    from row_wise_backward_amd.autograd import scaled_silu
    _gradcheck(scaled_silu, (_t((13,), 3, scale=2.0), _t((1,), 4)))


@pytest.mark.parametrize("save", ["y", "lse"])
def test_softmax(gpu_lib, save):
    from row_wise_backward_amd.autograd import softmax
    _gradcheck(lambda x: softmax(x, save), (_t((4, 9), 5, scale=2.0),))


def test_softmax_cross_entropy(gpu_lib):
    from row_wise_backward_amd.autograd import softmax_cross_entropy
    t = torch.tensor([3, 0, 10, 7], dtype=torch.int64, device=DEV)
    _gradcheck(lambda z: softmax_cross_entropy(z, t), (_t((4, 11), 6, scale=2.0),))


def test_layer_norm(gpu_lib):
    from row_wise_backward_amd.autograd import layer_norm
    _gradcheck(lambda x, w, b: layer_norm(x, w, b, 1e-5),
               (_t((3, 8), 7), _t((8,), 8, 0.1, 1.0), _t((8,), 9, 0.1)))


def test_rms_norm(gpu_lib):
    from row_wise_backward_amd.autograd import rms_norm
    _gradcheck(lambda x, w: rms_norm(x, w, 1e-6), (_t((3, 8), 10), _t((8,), 11, 0.1, 1.0)))


def test_gather_rows(gpu_lib):
    """Repeated indices: the backward's scatter-add sums their gradients."""
    from row_wise_backward_amd.autograd import gather_rows
    idx = torch.tensor([2, 0, 2, 5, 2, 1, 0, 4, 2], dtype=torch.int64, device=DEV)
    _gradcheck(lambda tab: gather_rows(tab, idx), (_t((6, 5), 12),))
