"""Forward parity: HIP path (through the C ABI) vs the float64 oracle."""
import math

import numpy as np
import pytest
import torch

from io_aware_exact_15_amd import inputs
from parity import assert_close, assert_lse, gather_rows, gpu_forward, oracle_forward

pytestmark = pytest.mark.gpu


def _run_full(B, H, N, d, seed, dtype, causal, o_dtype="bf16"):
    inp = inputs.make_inputs(B, H, N, d, seed, dtype)
    print(f"case B={B} H={H} N={N} d={d} seed={seed} {dtype} causal={causal} o={o_dtype}", flush=True)
    o, lse = gpu_forward(inp, dtype, causal, o_dtype)
    ro, rl = oracle_forward(inp, dtype, causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    tol_dtype = "f32" if (dtype == "f32" and o_dtype == "f32") else ("bf16" if dtype != "fp8" else "fp8")
    mx, rms = assert_close(o, ro, tol_dtype, "O", o_bf16=(o_dtype == "bf16"))
    le = assert_lse(lse, rl, "lse")
    print(f"  max|O err|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)


def test_workload_f32_n256_d64():
    """fp32 operands, B=1 H=1 N=256 d=64, non-causal: every output element."""
    w = inputs.WORKLOADS["fwd_f32_b1h1_n256_d64"]
    _run_full(w["B"], w["H"], w["N"], w["d"], w["seed"], "f32", False, o_dtype="f32")


@pytest.mark.parametrize("causal", [False, True])
def test_workload_bf16_b4h16_n2048_d64(causal):
    """bf16 operands, B=4 H=16 N=2048 d=64, non-causal and causal: every element."""
    w = inputs.WORKLOADS["fwd_bf16_b4h16_n2048_d64"]
    _run_full(w["B"], w["H"], w["N"], w["d"], w["seed"], "bf16", causal)


@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
def test_workload_bf16_causal_n16384_d128_sampled(o_dtype):
    """bf16, B=1 H=32 N=16384 d=128 causal: 512 seeded query rows per head vs
    the oracle over all keys, with the bf16 O of the headline forward and the
    float32 O of the forward that feeds the backward (both timed by bench.py)."""
    w = inputs.WORKLOADS["fwd_bf16_causal_b1h32_n16384_d128"]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "bf16")
    rows = inputs.sample_rows(w["seed"], B, H, N, w["sample"])
    print(f"case {w} sampled o={o_dtype}", flush=True)
    o, lse = gpu_forward(inp, "bf16", True, o_dtype)
    ro, rl = oracle_forward(inp, "bf16", True, rows=rows)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    mx, rms = assert_close(gather_rows(o, rows), ro, "bf16", "O", o_bf16=(o_dtype == "bf16"))
    le = assert_lse(gather_rows(lse, rows), rl, "lse")
    print(f"  max|O err|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)


# Ragged and small shapes: tails shorter than a tile, a single row, head
# counts that do and do not fill the 8 XCDs evenly, both head sizes.
EDGE = [
    (1, 1, 1, 64), (1, 1, 1, 128), (1, 1, 17, 64), (1, 2, 63, 128), (2, 3, 100, 64), (1, 1, 129, 128),
    (1, 8, 255, 64), (2, 8, 257, 128), (1, 3, 640, 128), (1, 16, 1000, 64),
]


@pytest.mark.parametrize("shape", EDGE, ids=[f"B{b}H{h}N{n}d{d}" for b, h, n, d in EDGE])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_bf16(shape, causal):
    B, H, N, d = shape
    _run_full(B, H, N, d, 100 + N, "bf16", causal)


@pytest.mark.parametrize("shape", [(1, 1, 1, 64), (1, 2, 77, 64), (2, 1, 300, 128), (1, 8, 129, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_f32(shape, causal):
    B, H, N, d = shape
    _run_full(B, H, N, d, 200 + N, "f32", causal, o_dtype="f32")


@pytest.mark.parametrize("B", [2, 3])
def test_resident_grid_pass_order(B):
    """Causal d = 64 grids that the CUs hold at once, in 2 and 3 passes of one
    workgroup per CU (512 and 768 workgroups on 256 CUs), where odd passes run
    in reverse order: every element against the oracle (the B = 4 workload
    covers 4 passes)."""
    _run_full(B, 16, 2048, 64, 16 + B, "bf16", True)


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_operands_f32_output(causal):
    """bf16 operands with a float32 O (the form the backward pass consumes)."""
    _run_full(2, 4, 300, 128, 7, "bf16", causal, o_dtype="f32")


# Score ranges that move the running max after the first key block, or that
# would underflow or overflow without it: keys from row 300 on scaled by
# `grow` (their scores exceed every earlier one by up to ~16, ~40 and ~260 in
# log2 units; the last overflows float32 unless the max moves), and keys and
# queries shifted apart so that every score of every row lies near -260 in
# log2 units (exp2 of them underflows unless the max is subtracted).
#
# Such rows are sharp (a few keys carry the weight), so the bf16 rounding of
# P is not averaged away and the flat 1e-2 bound of the N(0,1) workloads is no
# yardstick. The bound follows from the arithmetic instead: the matrix cores
# see bf16(p_j) = p_j (1 + e_j) with |e_j| <= 2^-8 (8 significant bits,
# round to nearest), while l sums the unrounded p_j, so
# |O_gpu - O| <= 2^-8 sum_j P_j |v_j| per element; 2^-12 more covers the
# float32 scores and exp2 (the oracle gives sum_j P_j |v_j| as its forward
# with |V|). A stale running max that is never moved, or an overflow, misses
# it by orders of magnitude.
RANGE_CASES = [("grow2.5", 2.5), ("grow6", 6.0), ("grow40", 40.0), ("shifted", None)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", RANGE_CASES, ids=[c[0] for c in RANGE_CASES])
def test_score_range(case, causal, d):
    name, grow = case
    B, H, N = 1, 4, 700
    print(f"case score range {name} B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    q, k, v = inputs.normal_tensors(B, H, N, d, 15, 3)
    if grow is not None:
        k = k.clone()
        k[:, :, 300:] *= grow
    else:
        q, k = q - 4.0, k + 4.0
    inp = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16)}
    o, lse = gpu_forward(inp, "bf16", causal, o_dtype="f32")
    ro, rl = oracle_forward(inp, "bf16", causal)
    r_abs, _ = oracle_forward(dict(inp, v=inp["v"].abs()), "bf16", causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    err = np.abs(o - ro)
    bound = (2.0 ** -8 + 2.0 ** -12) * r_abs + 1e-5
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"O: error {worst:.3g}x the bf16-P bound (max|err| {err.max():.3g})"
    le = assert_lse(lse, rl, "lse")  # lse reaches ~|180| here; float32 holds it to ~1e-5
    print(f"  max|O err|={err.max():.3g} ({worst:.2f} of the bound) lse={le:.3g}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_invariant_constant_value_column(causal):
    """A constant V column comes back as that constant (independent of the oracle)."""
    B, H, N, d = 1, 4, 700, 128
    inp = inputs.make_inputs(B, H, N, d, 11, "bf16")
    v = inp["v"].clone()
    v[..., 3] = 1.5
    inp["v"] = v
    o, _ = gpu_forward(inp, "bf16", causal, o_dtype="f32")
    # P is rounded to bf16 (relative error <= 2^-8: 8 significant bits, round
    # to nearest) for P.V while l sums the unrounded p, so the column is
    # 1.5 * sum(p_hat) / sum(p), within 1.5 * 2^-8 of 1.5 (plus float32
    # accumulation).
    assert np.max(np.abs(o[..., 3] - 1.5)) <= 1.5 * 2.0 ** -8 + 1e-5


def test_invariant_uniform_scores():
    """Q = 0: non-causal rows are the mean of V, causal rows the prefix means, lse = ln(#keys)."""
    B, H, N, d = 1, 2, 513, 64
    inp = inputs.make_inputs(B, H, N, d, 12, "bf16")
    inp["q"] = torch.zeros_like(inp["q"])
    v = inp["v"].to(torch.float64).numpy()
    o, lse = gpu_forward(inp, "bf16", False, o_dtype="f32")
    assert np.max(np.abs(o - v.mean(axis=2, keepdims=True))) <= 1e-4
    assert np.max(np.abs(lse - math.log(N))) <= 1e-5
    o, lse = gpu_forward(inp, "bf16", True, o_dtype="f32")
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.max(np.abs(o - prefix)) <= 1e-4
    assert np.max(np.abs(lse - np.log(np.arange(1, N + 1)))) <= 1e-5


def test_deterministic():
    """Two runs give bitwise-identical outputs."""
    inp = inputs.make_inputs(1, 8, 1024, 128, 13, "bf16")
    o1, l1 = gpu_forward(inp, "bf16", True)
    o2, l2 = gpu_forward(inp, "bf16", True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("side_stream", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_plain_entry_point(causal, side_stream):
    """fa_forward itself (bf16 in and out, the plain signature), on the
    current stream or on a caller-made stream: the same bits as
    fa_forward_typed(BF16, BF16) and the oracle's values."""
    from io_aware_exact_15_amd import binding as fa
    B, H, N, d = 2, 4, 777, 128
    print(f"case fa_forward B={B} H={H} N={N} d={d} causal={causal} side_stream={side_stream}", flush=True)
    inp = inputs.make_inputs(B, H, N, d, 14, "bf16")
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in "qkv")
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    if side_stream:
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        fa.fa_forward(q, k, v, o, lse, 1.0 / math.sqrt(d), causal, stream=st)
        st.synchronize()
    else:
        fa.fa_forward(q, k, v, o, lse, 1.0 / math.sqrt(d), causal)
        torch.cuda.synchronize()
    got_o, got_l = o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()
    typed_o, typed_l = gpu_forward(inp, "bf16", causal)
    assert np.array_equal(got_o, typed_o) and np.array_equal(got_l, typed_l)
    ro, rl = oracle_forward(inp, "bf16", causal)
    mx, rms = assert_close(got_o, ro, "bf16", "O", o_bf16=True)
    le = assert_lse(got_l, rl, "lse")
    print(f"  max|O err|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)
