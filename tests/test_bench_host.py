"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the FLOP
conventions, the traffic record's source check, and the per-workload oracle
timing leg."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from io_aware_exact_15_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_flop_conventions():
    # forward 4 B H N^2 d, backward 10 B H N^2 d, both halved by the causal mask
    assert bench._flops(1, 32, 16384, 128, True, "fwd") == 2 * 32 * 16384 ** 2 * 128
    assert bench._flops(2, 16, 4096, 128, False, "bwd") == 10 * 2 * 16 * 4096 ** 2 * 128
    assert bench._flops(2, 16, 4096, 128, True, "bwd") == 5 * 2 * 16 * 4096 ** 2 * 128


def _fake_root(tmp_path):
    """A scratch root holding a copy of the kernel sources and an empty profiles folder."""
    csrc = tmp_path / "io_aware_exact_15_amd" / "csrc"
    csrc.mkdir(parents=True)
    for n in set(bench.KERNEL_SOURCES["fwd"] + bench.KERNEL_SOURCES["bwd"]):
        shutil.copy(os.path.join(ROOT, "io_aware_exact_15_amd", "csrc", n), csrc / n)
    (tmp_path / "profiles").mkdir()
    return tmp_path


@pytest.mark.parametrize("sha_ok", [True, False])
def test_recorded_traffic_follows_the_sources(tmp_path, monkeypatch, sha_ok):
    root = _fake_root(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    sha = bench._source_sha(bench.KERNEL_SOURCES["fwd"]) if sha_ok else "0" * 64
    (root / "profiles" / bench.TRAFFIC_FILES["fwd"]).write_text(
        f"# summary\n\ntraffic_bytes_per_launch: 123456789 source_sha256: {sha}\n")
    assert bench._recorded_traffic("fwd") == (123456789 if sha_ok else None)
    assert bench._recorded_traffic("bwd") is None  # no record at all


def test_cpu_baseline_sample_reports_what_it_timed():
    w = dict(seed=5, B=1, H=2, N=300, d=64, dtype="bf16", causal=(True,), backward=True)
    inp = inputs.make_inputs(1, 2, 300, 64, 5, "bf16", with_do=True)
    for kind in ("fwd", "bwd"):
        r = bench.cpu_baseline_sample(kind, w, inp, True, target_flop=1e6)
        assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
        assert r["cores"] == len(os.sched_getaffinity(0))
        assert "s wall" in r["sample"]


def _tiny_step_outputs(w):
    """What a correct step of workload w produces, from the oracle (float64)."""
    import math

    import oracle
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "bf16", with_do=True)
    q, k, v, do = (inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, scale, w["causal"])
    dq, dk, dv = oracle.backward(q, k, v, do, scale, w["causal"])
    return {"o_bf16": o, "lse_bf16": lse, "o32": o, "lse32": lse, "dq": dq, "dk": dk, "dv": dv}


def test_parity_of_step_accepts_the_exact_result_and_flags_a_wrong_one():
    w = dict(name="tiny", B=1, H=2, N=96, d=64, causal=True, seed=3)
    outs = _tiny_step_outputs(w)
    r = bench.parity_of_step(w, outs, rows_per_head=16, tail=8)
    assert r["ok"] and max(r[k] for k in bench.PARITY_TOL) < 1e-12
    for name in ("o32", "dq", "dk", "dv", "lse_bf16"):
        bad = {n: a.copy() for n, a in outs.items()}
        if name in ("dk", "dv"):
            bad[name][0, 1, -1, 3] += 0.02  # a tail key
        else:
            bad[name][0, 1] += 0.02  # every row of head 1 (sampled rows included)
        r = bench.parity_of_step(w, bad, rows_per_head=16, tail=8)
        assert not r["ok"], name


def test_headline_cpu_baseline_times_forward_and_backward():
    w = dict(name="tiny", B=1, H=4, N=128, d=64, causal=True, seed=3)
    r = bench.cpu_baseline(w, heads=1)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert "forward + backward of 1 of 4 heads" in r["sample"]
    assert r["blas"] and r["full_step_extrapolated_s"] > 0


def test_workload_table_names_every_workload():
    t = bench.workload_table()
    for group in (inputs.WORKLOADS, inputs.GQA_WORKLOADS, inputs.FP8_BWD_WORKLOADS, inputs.DECODE_WORKLOADS,
                  inputs.FP8_E5M2_WORKLOADS):
        assert set(group) <= set(t)
