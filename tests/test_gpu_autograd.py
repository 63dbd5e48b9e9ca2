"""torch.autograd.Function layer over libvjp on the GPU: gradients that the
autograd engine delivers (arity, order, accumulation into .grad, inputs that
need no gradient, non-contiguous inputs, chains of ops) against the CPU
oracle.  Tolerances are the per-op rules of the parity tests, checked here
on fp32 activations (16-bit cases are covered op by op elsewhere)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, to_host
from oracle.compare import pointwise, reduced

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ag(gpu_lib):
    from row_wise_backward_amd import autograd
    return autograd


def _t(a, dtype="f32", grad=True):
    t = synth.to_torch(a, dtype, DEV).clone()
    return t.requires_grad_(grad)


def test_weighted_sum_grads_and_accumulation(ag):
    n, d = 7, 33
    x = synth.normal((n, d), 1.0, "f32", 300, 0)
    w = synth.normal((d,), 1.0, "f32", 300, 1)
    g = synth.normal((n,), 1.0, "f32", 300, 2)
    xt, wt = _t(x), _t(w)
    for rep in range(2):                       # the second pass accumulates into .grad
        y = ag.weighted_sum(xt, wt)
        y.backward(synth.to_torch(g, "f32", DEV))
    gx, gw = oracle.weighted_sum.bwd(synth.to_f64(g, "f32"), synth.to_f64(x, "f32"), synth.to_f64(w, "f32"))
    r1 = pointwise(to_host(xt.grad, "f32"), 2 * gx, "f32", name="x.grad")
    r2 = reduced(to_host(wt.grad, "f32"), 2 * gw, name="w.grad")
    print("   ", r1, "\n   ", r2)
    assert r1.ok and r2.ok


def test_weighted_sum_needs_input_grad_and_layout(ag):
    """Only w needs a gradient; x is a non-contiguous view (every other column)."""
    n, d = 9, 16
    base = synth.normal((n, 2 * d), 1.0, "f32", 301, 0)
    w = synth.normal((d,), 1.0, "f32", 301, 1)
    xt = synth.to_torch(base, "f32", DEV)[:, ::2]
    assert not xt.is_contiguous()
    wt = _t(w)
    ag.weighted_sum(xt, wt).sum().backward()
    x64 = synth.to_f64(base, "f32")[:, ::2]
    _, gw = oracle.weighted_sum.bwd(np.ones(n), x64, synth.to_f64(w, "f32"))
    r = reduced(to_host(wt.grad, "f32"), gw, name="w.grad")
    assert r.ok and xt.grad is None


def test_weighted_sum_bf16_parameter_grad_dtype(ag):
    x = _t(synth.normal((5, 8), 1.0, "bf16", 302, 0), "bf16")
    w = _t(synth.normal((8,), 1.0, "bf16", 302, 1), "bf16")
    ag.weighted_sum(x, w).float().sum().backward()
    assert w.grad.dtype == torch.bfloat16 and x.grad.dtype == torch.bfloat16


def test_scaled_silu_grads(ag):
    x = synth.normal((4, 1000), 2.0, "f32", 303, 0)
    g = synth.normal((4, 1000), 1.0, "f32", 303, 2)
    xt = _t(x)
    wt = torch.tensor([0.75], device=DEV, requires_grad=True)
    y = ag.scaled_silu(xt, wt)
    assert y.shape == (4, 1000)
    y.backward(synth.to_torch(g, "f32", DEV))
    x64, g64 = synth.to_f64(x, "f32"), synth.to_f64(g, "f32")
    dx, dw = oracle.scaled_silu.bwd(g64, x64, 0.75)
    s = oracle.scaled_silu.sigmoid(x64)
    S = np.abs(g64 * 0.75) * (s + np.abs(x64) * s)   # s + x s (1 - s) cancels near x = -1.28
    r1 = pointwise(to_host(xt.grad, "f32"), dx, "f32", S=S, name="x.grad")
    r2 = reduced(to_host(wt.grad, "f32"), np.array([dw]), name="w.grad")
    print("   ", r1, "\n   ", r2)
    assert r1.ok and r2.ok and wt.grad.shape == (1,)


@pytest.mark.parametrize("save", ["y", "lse"])
def test_softmax_grads(ag, save):
    x = synth.normal((2, 3, 257), 3.0, "f32", 304, 0)      # leading dims flattened into rows
    g = synth.normal((2, 3, 257), 1.0, "f32", 304, 2)
    xt = _t(x)
    y = ag.softmax(xt, save=save)
    y.backward(synth.to_torch(g, "f32", DEV))
    x64, g64 = synth.to_f64(x, "f32").reshape(6, 257), synth.to_f64(g, "f32").reshape(6, 257)
    y_ref = oracle.softmax.fwd(x64)
    r0 = pointwise(to_host(y.detach(), "f32").reshape(6, 257), y_ref, "f32", name="y")
    dx_ref = oracle.softmax.bwd_from_x(g64, x64)
    s = np.sum(g64 * y_ref, axis=-1, keepdims=True)
    S = np.abs(y_ref) * (np.abs(g64) + np.abs(s) + np.sum(np.abs(g64 * y_ref), axis=-1, keepdims=True))
    r1 = pointwise(to_host(xt.grad, "f32").reshape(6, 257), dx_ref, "f32", S=S * 4, name="x.grad")
    print("   ", r0, "\n   ", r1)
    assert r0.ok and r1.ok


def test_softmax_cross_entropy_grads(ag):
    R, C = 7, 3000
    z = synth.normal((R, C), 2.0, "f32", 305, 0)
    t = synth.targets(R, C, 305)
    zt = _t(z)
    loss = ag.softmax_cross_entropy(zt, torch.from_numpy(t.astype(np.int64)).to(DEV))
    assert loss.dim() == 0
    (loss * -2.5).backward()                  # upstream gradient other than 1
    z64 = synth.to_f64(z, "f32")
    ref = oracle.softmax_xent.fwd(z64, t)
    r0 = reduced(to_host(loss.detach().reshape(1), "f32"), np.array([ref["loss"]]), name="loss")
    dz = oracle.softmax_xent.bwd(z64, t, -2.5)
    p = np.exp(z64 - ref["row_lse"][:, None])
    r1 = pointwise(to_host(zt.grad, "f32"), dz, "f32", S=2.5 / R * (p + 1) * 4, name="logits.grad")
    print("   ", r0, "\n   ", r1)
    assert r0.ok and r1.ok


def test_chain_silu_into_cross_entropy(ag):
    """loss = xent(scaled_silu(x, w), t): the gradient flows through both ops."""
    R, C = 5, 700
    x = synth.normal((R, C), 2.0, "f32", 306, 0)
    t = synth.targets(R, C, 306)
    xt = _t(x)
    wt = torch.tensor([1.5], device=DEV, requires_grad=True)
    loss = ag.softmax_cross_entropy(ag.scaled_silu(xt, wt), torch.from_numpy(t).to(DEV))
    loss.backward()
    x64 = synth.to_f64(x, "f32")
    z = oracle.scaled_silu.fwd(x64, 1.5)
    dz = oracle.softmax_xent.bwd(z, t, 1.0)
    dx, dw = oracle.scaled_silu.bwd(dz, x64, 1.5)
    r1 = reduced(to_host(xt.grad, "f32").reshape(-1), dx.reshape(-1), name="x.grad")
    r2 = reduced(to_host(wt.grad, "f32"), np.array([dw]), name="w.grad")
    print("   ", r1, "\n   ", r2)
    assert r1.ok and r2.ok


def test_chain_weighted_sum_into_softmax(ag):
    """softmax over a [B, N] matrix of weighted sums: rows of x are grouped."""
    B, N, d = 3, 50, 24
    x = synth.normal((B * N, d), 1.0, "f32", 307, 0)
    w = synth.normal((d,), 1.0, "f32", 307, 1)
    g = synth.normal((B, N), 1.0, "f32", 307, 2)
    xt, wt = _t(x), _t(w)
    y = ag.softmax(ag.weighted_sum(xt, wt).reshape(B, N), save="lse")
    y.backward(synth.to_torch(g, "f32", DEV))
    x64, w64, g64 = synth.to_f64(x, "f32"), synth.to_f64(w, "f32"), synth.to_f64(g, "f32")
    s = oracle.weighted_sum.fwd(x64, w64).reshape(B, N)
    ds = oracle.softmax.bwd_from_x(g64, s).reshape(-1)
    dx, dw = oracle.weighted_sum.bwd(ds, x64, w64)
    r1 = reduced(to_host(xt.grad, "f32").reshape(-1), dx.reshape(-1), name="x.grad")
    r2 = reduced(to_host(wt.grad, "f32"), dw, name="w.grad")
    print("   ", r1, "\n   ", r2)
    assert r1.ok and r2.ok


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_norm_grads(ag, kind):
    x = synth.normal((2, 5, 300), 1.0, "f32", 308, 0)
    g = synth.normal((2, 5, 300), 1.0, "f32", 308, 2)
    rng = np.random.default_rng(308)
    w = (1 + 0.1 * rng.standard_normal(300)).astype(np.float32)
    b = (0.1 * rng.standard_normal(300)).astype(np.float32)
    xt, wt, bt = _t(x), _t(w), _t(b)
    y = ag.layer_norm(xt, wt, bt) if kind == "ln" else ag.rms_norm(xt, wt)
    y.backward(synth.to_torch(g, "f32", DEV))
    x64, g64 = synth.to_f64(x, "f32").reshape(10, 300), synth.to_f64(g, "f32").reshape(10, 300)
    if kind == "ln":
        dx, dw, db = oracle.norms.layernorm_bwd(g64, x64, w.astype(np.float64), 1e-5)
        r3 = reduced(to_host(bt.grad, "f32"), db, name="b.grad")
    else:
        dx, dw = oracle.norms.rmsnorm_bwd(g64, x64, w.astype(np.float64), 1e-6)
        r3 = None
        assert bt.grad is None
    r1 = reduced(to_host(xt.grad, "f32").reshape(-1), dx.reshape(-1), name="x.grad")
    r2 = reduced(to_host(wt.grad, "f32"), dw, name="w.grad")
    for r in (r1, r2, r3):
        if r is not None:
            print("   ", r)
    assert r1.ok and r2.ok and (r3 is None or r3.ok)


def test_gather_rows_grads(ag):
    """Embedding lookup with repeated ids ([2, 50] index tensor), two backward
    passes accumulating into table.grad."""
    V, D = 40, 24
    table = synth.normal((V, D), 1.0, "f32", 309, 0)
    idx = synth.zipf_indices(100, V, 309)
    g = synth.normal((100, D), 1.0, "f32", 309, 2)
    tt = _t(table)
    it = torch.from_numpy(idx.astype(np.int64)).to(DEV).reshape(2, 50)
    for _ in range(2):
        y = ag.gather_rows(tt, it)
        assert y.shape == (2, 50, D)
        y.backward(synth.to_torch(g, "f32", DEV).reshape(2, 50, D))
    dt, _ = oracle.gather.bwd(synth.to_f64(g, "f32"), idx, V)
    S, _ = oracle.gather.bwd(np.abs(synth.to_f64(g, "f32")), idx, V)
    r = pointwise(to_host(tt.grad, "f32"), 2 * dt, "f32", S=2 * S, name="table.grad")
    print("   ", r)
    assert r.ok


def test_training_steps_against_oracle_chain(ag):
    """Five SGD steps of a small model built from the autograd layer
    (embedding gather -> RMSNorm -> scaled SiLU -> a projection -> softmax
    cross-entropy; the projection is a plain fp32 matmul, not part of the
    library) against the same steps in fp64 on the CPU, with every gradient
    chained by hand through the oracle functions.  The losses of every step
    and the parameters after the last must agree to 1e-4 (relative L2): the
    gradients reach every parameter, with the right sign and scale, through
    every op's backward."""
    B, V, D, C, lr, eps = 48, 40, 64, 19, 0.5, 1e-6
    g = np.random.default_rng(4242)
    ids = g.integers(0, V, size=B).astype(np.int32)
    ids[:6] = 3                                  # repeated rows in the scatter-add
    tgt = g.integers(0, C, size=B).astype(np.int32)
    p64 = {"table": g.standard_normal((V, D)), "gamma": 1 + 0.1 * g.standard_normal(D),
           "s": np.array([0.75]), "W": 0.2 * g.standard_normal((D, C))}
    params = {k: torch.tensor(v, dtype=torch.float32, device=DEV, requires_grad=True)
              for k, v in p64.items()}
    ids_d = torch.from_numpy(ids).to(DEV)
    tgt_d = torch.from_numpy(tgt).to(DEV)
    gpu_losses, ref_losses = [], []
    for _ in range(5):
        # GPU: the autograd layer
        for t in params.values():
            t.grad = None
        h = ag.gather_rows(params["table"], ids_d)
        n = ag.rms_norm(h, params["gamma"], eps)
        a = ag.scaled_silu(n, params["s"])
        z = a @ params["W"]
        loss = ag.softmax_cross_entropy(z, tgt_d)
        loss.backward()
        gpu_losses.append(float(loss.item()))
        with torch.no_grad():
            for t in params.values():
                t -= lr * t.grad
        # CPU: the oracle, chained by hand
        P = {k: v.astype(np.float64) for k, v in p64.items()}
        h64 = oracle.gather.fwd(P["table"], ids)
        n64, _ = oracle.norms.rmsnorm_fwd(h64, P["gamma"], eps)
        a64 = oracle.scaled_silu.fwd(n64, P["s"][0])
        z64 = a64 @ P["W"]
        out = oracle.softmax_xent.fwd_bwd(z64, tgt, 1.0 / B)
        ref_losses.append(out["loss"])
        dz = out["dz"]
        dW = a64.T @ dz
        da = dz @ P["W"].T
        dn, ds = oracle.scaled_silu.bwd(da, n64, P["s"][0])
        dh, dgamma = oracle.norms.rmsnorm_bwd(dn, h64, P["gamma"], eps)
        dtable, _ = oracle.gather.bwd(dh, ids, V)
        grads = {"table": dtable, "gamma": dgamma, "s": np.array([ds]), "W": dW}
        p64 = {k: P[k] - lr * grads[k] for k in P}
    print("\n    losses gpu", np.round(gpu_losses, 6), "\n    losses ref", np.round(ref_losses, 6),
          flush=True)
    assert ref_losses[-1] < ref_losses[0]       # the steps do train
    reps = [reduced(np.array(gpu_losses), np.array(ref_losses), name="losses")]
    for k in p64:
        reps.append(reduced(params[k].detach().cpu().numpy().astype(np.float64).reshape(-1),
                            p64[k].reshape(-1), name=k))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


def test_training_steps_norm_softmax_weighted_sum(ag):
    """Five SGD steps through LayerNorm -> softmax (saving the row logsumexp)
    -> weighted sum under a mean squared error against fixed targets r,
    against the same steps chained by hand through the oracle in fp64: the
    losses and the LayerNorm weight and bias and the weighted-sum weights
    agree to 1e-4 (relative L2)."""
    B, D, lr, eps = 64, 96, 0.5, 1e-5
    g = np.random.default_rng(4343)
    X = g.standard_normal((B, D)) * 2 + 0.5
    r = g.standard_normal(B)
    p64 = {"w": 1 + 0.1 * g.standard_normal(D), "b": 0.1 * g.standard_normal(D),
           "v": g.standard_normal(D)}
    params = {k: torch.tensor(v, dtype=torch.float32, device=DEV, requires_grad=True)
              for k, v in p64.items()}
    Xd = torch.tensor(X, dtype=torch.float32, device=DEV)
    X32 = Xd.cpu().numpy().astype(np.float64)   # the oracle sees the same fp32 input
    rd = torch.tensor(r, dtype=torch.float32, device=DEV)
    r32 = rd.cpu().numpy().astype(np.float64)
    gpu_losses, ref_losses = [], []
    for _ in range(5):
        for t in params.values():
            t.grad = None
        h = ag.layer_norm(Xd, params["w"], params["b"], eps)
        p = ag.softmax(h, save="lse")
        y = ag.weighted_sum(p, params["v"])
        loss = ((y - rd) ** 2).mean()
        loss.backward()
        gpu_losses.append(float(loss.item()))
        with torch.no_grad():
            for t in params.values():
                t -= lr * t.grad
        P = {k: v.astype(np.float64) for k, v in p64.items()}
        h64, _, _ = oracle.norms.layernorm_fwd(X32, P["w"], P["b"], eps)
        y_sm = oracle.softmax.fwd(h64)
        y64 = oracle.weighted_sum.fwd(y_sm, P["v"])
        ref_losses.append(float(np.mean((y64 - r32) ** 2)))
        dp, dv = oracle.weighted_sum.bwd(2.0 * (y64 - r32) / B, y_sm, P["v"])
        dh = oracle.softmax.bwd(dp, y_sm)
        _, dw, db = oracle.norms.layernorm_bwd(dh, X32, P["w"], eps)
        grads = {"w": dw, "b": db, "v": dv}
        p64 = {k: P[k] - lr * grads[k] for k in P}
    print("\n    losses gpu", np.round(gpu_losses, 6), "\n    losses ref", np.round(ref_losses, 6),
          flush=True)
    assert ref_losses[-1] < ref_losses[0]
    reps = [reduced(np.array(gpu_losses), np.array(ref_losses), name="losses")]
    for k in p64:
        reps.append(reduced(params[k].detach().cpu().numpy().astype(np.float64), p64[k], name=k))
    for r_ in reps:
        print("   ", r_, flush=True)
    assert all(r_.ok for r_ in reps), [str(r_) for r_ in reps if not r_.ok]


def test_readme_example(ag):
    """The Python example of README.md, run as written (full-size logits):
    the loss equals the mean of lse - z_t, and each row of the logit gradient
    sums to about zero."""
    import os
    import re

    readme = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")
    code = re.search(r"```python\n(.*?)```", open(readme).read(), re.S).group(1)
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    logits, targets, loss = env["logits"], env["targets"], env["loss"]
    z = logits.detach().float()
    ref = (torch.logsumexp(z, 1) - z[torch.arange(z.shape[0], device=z.device), targets]).mean()
    print(f"\n[readme] loss {loss.item():.6f} ref {ref.item():.6f}", flush=True)
    assert abs(loss.item() - ref.item()) <= 1e-5 * abs(ref.item())
    g = logits.grad
    assert g.shape == logits.shape and g.dtype == logits.dtype
    assert float(g.float().sum(1).abs().max()) <= 2e-2 / z.shape[0]
