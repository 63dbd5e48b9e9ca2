"""Host-side pieces of bench.py: the one-GPU guard, the byte models and the
CPU oracle baseline (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for an unsupported run


@pytest.mark.parametrize("es", [2, 4])
def test_byte_models_count_each_tensor_once(es):
    # Every model is at least the bytes of the tensors the op must read and
    # write once, and at most that plus its small fp32 side arrays.
    r, c = 16384, 32000
    big = 2 * r * c * es                            # logits read + dlogits written
    assert big <= bench.bytes_xent(r, c, es) <= big + 64 * r
    assert r * c * es <= bench.bytes_xent_fwd(r, c, es) <= r * c * es + 64 * r
    assert big <= bench.bytes_xent_bwd(r, c, es) <= big + 64 * r
    assert bench.bytes_softmax_fwd(r, c, es) == 2 * r * c * es
    assert bench.bytes_softmax_bwd(r, c, es) == 3 * r * c * es
    n, d, T = 1 << 20, 256, 2048
    base = 2 * n * d * es                           # x read, grad_x written
    wsb = bench.bytes_weighted_sum_bwd(n, d, T, es, es)
    assert base + 2 * T * d * 4 <= wsb <= base + 2 * T * d * 4 + 8 * n + 8 * d
    M, V, D = 65536, 128000, 1024
    assert bench.bytes_gather_bwd(M, V, D, es) == M * D * es + V * D * 4 + 4 * M


def test_cpu_baseline_small_sample():
    """Both legs: all cores (one worker process per core) and one core."""
    out = bench.cpu_baseline(scale=0.01, min_seconds=0.0, cores=2)
    assert out["kind"] == "oracle" and out["unit"] == "GB/s"
    assert out["value"] > 0 and out["cores"] == 2
    assert "2 worker processes" in out["sample"] and "passes" in out["sample"]
    assert out["one_core"]["cores"] == 1 and out["one_core"]["value"] > 0
    json.dumps(out)                                  # serialisable into the bench line


def test_cpu_cores_is_bounded():
    assert 1 <= bench.cpu_cores() <= 16


def test_protocol_trace_parsing(tmp_path):
    """Launch groups open at every fill kernel after the marker copy; each
    label's groups are its 3 + 20 repetitions; a group's time is the sum of
    its kernel durations; medians over the last 20."""
    labels = ["op_a", "op_b"]
    rows = [("torch_setup_kernel", 0, 5), ("vjp::copy_bytes(...)", 10, 11)]
    t = 100
    per = bench.PROTOCOL_WARM + bench.PROTOCOL_REPS
    for k, lab in enumerate(labels):
        for r in range(per):
            rows.append(("at::native::FillFunctor<unsigned char>", t, t + 50))
            t += 60
            d1 = 1000 + 10 * r + 5000 * k           # stage 1 grows with r: median is r = 12.5
            rows.append((f"stage1_{lab}", t, t + d1))
            t += d1 + 5
            rows.append((f"stage2_{lab}", t, t + 4))
            t += 10
    path = tmp_path / "trace.csv"
    with open(path, "w") as f:
        f.write('"Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for name, a, b in rows:
            f.write(f'"{name}",{a},{b}\n')
    res = bench.parse_protocol_trace(str(path), labels)
    for k, lab in enumerate(labels):
        med_r = (bench.PROTOCOL_WARM + (bench.PROTOCOL_WARM + bench.PROTOCOL_REPS - 1)) / 2
        want_ns = 1000 + 10 * med_r + 5000 * k + 4
        assert abs(res[lab]["ms"] - want_ns * 1e-6) < 1e-12
        assert res[lab]["kernels"][f"stage2_{lab}"]["launches"] == bench.PROTOCOL_REPS
    with pytest.raises(RuntimeError):
        bench.parse_protocol_trace(str(path), labels + ["missing"])
