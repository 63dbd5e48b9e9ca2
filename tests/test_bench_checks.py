"""The output checks that bench.py runs after timing: on correct outputs
(torch fp32 on the CPU, rounded to the storage dtypes) every check passes,
and a planted mistake in one output fails the check that covers it."""
import pytest
import torch

import bench

BF, F16 = torch.bfloat16, torch.float16


class _Outputs(bench.Workbench):
    """The step's tensors under the names the checks read (no GPU)."""

    def __init__(self, seed=0):
        g = torch.Generator().manual_seed(seed)
        rn = lambda *s, sd=1.0: torch.randn(*s, generator=g) * sd  # noqa: E731
        t = {}
        t["wx"], t["ww"], t["wg"] = rn(2000, 64).to(BF), rn(64, sd=0.1).to(BF), rn(2000).to(BF)
        x, w, dy = t["wx"].float(), t["ww"].float(), t["wg"].float()
        t["wy"] = (x * w).sum(1).to(BF)
        t["wdx"] = (dy[:, None] * w).to(BF)
        t["wdw"] = torch.mv(x.t(), dy)
        t["sx"], t["sg"] = rn(5000, sd=2.0).to(F16), rn(5000).to(F16)
        t["sw"] = torch.tensor([0.75])
        x, dy, s = t["sx"].float(), t["sg"].float(), torch.sigmoid(t["sx"].float())
        t["sy"] = (0.75 * x * s).to(F16)
        t["sdx"] = (dy * 0.75 * (s + x * s * (1 - s))).to(F16)
        t["sdw"] = (dy * x * s).sum().reshape(1)
        t["mx"], t["mg"] = rn(300, 100, sd=3.0).to(BF), rn(300, 100).to(BF)
        t["my"] = torch.softmax(t["mx"].float(), 1).to(BF)
        y, dy = t["my"].float(), t["mg"].float()
        t["mdx"] = (y * (dy - (dy * y).sum(1, keepdim=True))).to(BF)
        t["z"] = rn(200, 50, sd=2.0).to(BF)
        t["tg"] = torch.randint(0, 50, (200,), generator=g, dtype=torch.int32)
        z = t["z"].float()
        t["rmax"], t["rlse"] = z.max(1).values, torch.logsumexp(z, 1)
        t["loss"] = (t["rlse"] - z[torch.arange(200), t["tg"].long()]).mean().reshape(1)
        p = torch.softmax(z, 1)
        p[torch.arange(200), t["tg"].long()] -= 1.0
        self.scale = 1.0 / 200
        t["dz"] = (self.scale * p).to(BF)
        t["ninv"] = torch.zeros(1, dtype=torch.int32)
        self.t, self.torch = t, torch


def test_correct_outputs_pass():
    checks = _Outputs().check_step()
    assert len(checks) == 15
    assert all(v <= 1.0 for v in checks.values()), checks


@pytest.mark.parametrize("name, plant", [
    ("weighted_sum_y", lambda t: t["wy"].__setitem__(0, -t["wy"][0] + 1)),
    ("weighted_sum_grad_x_exact", lambda t: t["wdx"].__setitem__((0, 3), t["wdx"][0, 3] * 2 + 1)),
    ("weighted_sum_grad_w", lambda t: t["wdw"].__setitem__(5, t["wdw"][5] + 1.0)),
    ("scaled_silu_y", lambda t: t["sy"].__setitem__(7, t["sy"][7] * 1.5 + 1)),
    ("scaled_silu_dx", lambda t: t["sdx"].__setitem__(9, -t["sdx"][9] - 1)),
    ("scaled_silu_dw", lambda t: t["sdw"].mul_(1.01)),
    ("softmax_y_row_sums", lambda t: t["my"][3].mul_(1.1)),
    ("softmax_dx_rows", lambda t: t["mdx"][0].add_(0.1)),
    ("softmax_xent_loss", lambda t: t["loss"].add_(0.01)),
    ("softmax_xent_lse_bounds", lambda t: t["rlse"].__setitem__(4, t["rmax"][4] - 1)),
    ("softmax_xent_dlogits_row_sums", lambda t: t["dz"].__setitem__((5, 7), t["dz"][5, 7] + 0.005)),
    ("softmax_xent_dlogits_rows", lambda t: t["dz"][0].neg_()),
    ("softmax_xent_n_invalid", lambda t: t["ninv"].fill_(1)),
])
def test_planted_mistake_fails_its_check(name, plant):
    o = _Outputs()
    plant(o.t)
    checks = o.check_step()
    assert not checks[name] <= 1.0, (name, checks[name])
