"""FP8 E4M3 forward parity against the oracle on the dequantised inputs (code * scale)."""
import numpy as np
import pytest

from io_aware_exact_15_amd import inputs
from parity import assert_close, assert_lse, gather_rows, gpu_forward, oracle_forward

pytestmark = pytest.mark.gpu


def test_workload_fp8_causal_n65536_d128_sampled():
    """B=1 H=8 N=65536 d=128 causal, E4M3 with per-tensor scales, bf16 O: 256 seeded rows per head."""
    w = inputs.WORKLOADS["fwd_fp8_causal_b1h8_n65536_d128"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    print(f"case {w}", flush=True)
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "fp8")
    rows = inputs.sample_rows(w["seed"], B, H, N, w["sample"])
    o, lse = gpu_forward(inp, "fp8", True)
    ro, rl = oracle_forward(inp, "fp8", True, rows=rows)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    mx, rms = assert_close(gather_rows(o, rows), ro, "fp8", "O")
    le = assert_lse(gather_rows(lse, rows), rl, "lse")
    print(f"  max|dO|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)


EDGE = [(1, 1, 1, 128), (1, 1, 33, 64), (1, 2, 200, 128), (2, 3, 129, 64), (1, 8, 1000, 128), (1, 4, 4096, 128)]


@pytest.mark.parametrize("shape", EDGE, ids=[f"B{b}H{h}N{n}d{d}" for b, h, n, d in EDGE])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_fp8(shape, causal):
    B, H, N, d = shape
    print(f"case B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    inp = inputs.make_inputs(B, H, N, d, 400 + N, "fp8")
    o, lse = gpu_forward(inp, "fp8", causal)
    ro, rl = oracle_forward(inp, "fp8", causal)
    mx, rms = assert_close(o, ro, "fp8", "O")
    le = assert_lse(lse, rl, "lse")
    print(f"  max|dO|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)


def test_workload_fp8_e5m2_causal_n65536_d128_sampled():
    """The same shape with E5M2 inputs (per-tensor scales), bf16 O: 256 seeded rows per head."""
    w = inputs.FP8_E5M2_WORKLOADS["fwd_fp8e5m2_causal_b1h8_n65536_d128"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    print(f"case {w}", flush=True)
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "fp8e5m2")
    rows = inputs.sample_rows(w["seed"], B, H, N, w["sample"])
    o, lse = gpu_forward(inp, "fp8e5m2", True)
    ro, rl = oracle_forward(inp, "fp8e5m2", True, rows=rows)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    mx, rms = assert_close(gather_rows(o, rows), ro, "fp8e5m2", "O")
    le = assert_lse(gather_rows(lse, rows), rl, "lse")
    print(f"  max|dO|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)


@pytest.mark.parametrize("shape", EDGE, ids=[f"B{b}H{h}N{n}d{d}" for b, h, n, d in EDGE])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_fp8_e5m2(shape, causal):
    B, H, N, d = shape
    print(f"case e5m2 B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    inp = inputs.make_inputs(B, H, N, d, 500 + N, "fp8e5m2")
    o, lse = gpu_forward(inp, "fp8e5m2", causal)
    ro, rl = oracle_forward(inp, "fp8e5m2", causal)
    mx, rms = assert_close(o, ro, "fp8e5m2", "O")
    le = assert_lse(lse, rl, "lse")
    print(f"  max|dO|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)
