"""Wave-specialised forward (fa_forward_ws) through the C ABI vs the float64
oracle: the full-size workloads, ragged and tiny shapes, grouped-query heads,
score ranges that move the running max (the rescale factor travels from the
producer waves to the consumer waves), scales other than 1/sqrt(d), and
agreement with fa_forward."""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs
from parity import FA_DT, assert_close, assert_lse, gather_rows, gpu_forward, oracle_forward

pytestmark = pytest.mark.gpu


def gpu_forward_ws(inp, causal, o_dtype="bf16", scale=None):
    B, H, N, d = inp["q"].shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dev = torch.device("cuda:0")
    qd, kd, vd = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16 if o_dtype == "bf16" else torch.float32,
                   device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_forward_ws(FA_DT[o_dtype], qd, kd, vd, o, lse, scale, causal)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def _check(inp, causal, o_dtype="bf16", rows=None, scale=None, what=""):
    B, H, N, d = inp["q"].shape
    Hkv = inp["k"].shape[1]
    print(f"case ws B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} o={o_dtype} scale={scale} {what}", flush=True)
    o, lse = gpu_forward_ws(inp, causal, o_dtype, scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v = (inputs.to_numpy(inp[n]) for n in "qkv")
    if Hkv == H:
        ro, rl = oracle.forward(q, k, v, sc, causal, rows)
    else:
        ro, rl = oracle.forward_gqa(q, k, v, sc, causal, rows)
    if rows is not None:
        o, lse = gather_rows(o, rows), gather_rows(lse, rows)
    mx, rms = assert_close(o, ro, "bf16", "O", o_bf16=(o_dtype == "bf16"))
    le = assert_lse(lse, rl, "lse")
    print(f"  max|O err|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)


@pytest.mark.parametrize("o_dtype", ["bf16", "f32"])
def test_workload_causal_n16384_d128_sampled(o_dtype):
    """B=1 H=32 N=16384 d=128 causal: 512 seeded query rows per head."""
    w = inputs.WORKLOADS["fwd_bf16_causal_b1h32_n16384_d128"]
    inp = inputs.make_inputs(w["B"], w["H"], w["N"], w["d"], w["seed"], "bf16")
    rows = inputs.sample_rows(w["seed"], w["B"], w["H"], w["N"], w["sample"])
    _check(inp, True, o_dtype, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
def test_workload_b4h16_n2048_d64(causal):
    """B=4 H=16 N=2048 d=64: every element."""
    w = inputs.WORKLOADS["fwd_bf16_b4h16_n2048_d64"]
    _check(inputs.make_inputs(w["B"], w["H"], w["N"], w["d"], w["seed"], "bf16"), causal)


def test_workload_gqa_n16384_sampled():
    """B=1 H=32 Hkv=8 N=16384 d=128 causal: 512 seeded rows per query head."""
    w = inputs.GQA_WORKLOADS["fwd_bf16_gqa_causal_b1h32kv8_n16384_d128"]
    inp = inputs.make_inputs_heads(w["B"], w["H"], w["Hkv"], w["N"], w["N"], w["d"], w["seed"], "bf16")
    rows = inputs.sample_rows(w["seed"], w["B"], w["H"], w["N"], w["sample"])
    _check(inp, True, rows=rows)


# Ragged and tiny shapes: one row, tails shorter than a 64-key block or a
# 128-row workgroup, key-block counts of 1 to 16 (the tick loop is unrolled
# by six), and head counts that do and do not fill the 8 XCDs.
EDGE = [
    (1, 1, 1, 64), (1, 1, 1, 128), (1, 1, 17, 64), (1, 2, 63, 128), (1, 1, 64, 128), (1, 1, 65, 64),
    (2, 3, 100, 64), (1, 1, 129, 128), (1, 8, 255, 64), (2, 8, 257, 128), (1, 2, 320, 128), (1, 3, 384, 64),
    (1, 3, 640, 128), (1, 16, 1000, 64),
]


@pytest.mark.parametrize("shape", EDGE, ids=[f"B{b}H{h}N{n}d{d}" for b, h, n, d in EDGE])
@pytest.mark.parametrize("causal", [False, True])
def test_edge(shape, causal):
    B, H, N, d = shape
    _check(inputs.make_inputs(B, H, N, d, 300 + N, "bf16"), causal)


@pytest.mark.parametrize("shape", [(1, 4, 1, 1, 64), (1, 4, 2, 17, 128), (2, 6, 3, 100, 64), (1, 8, 2, 257, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_gqa(shape, causal):
    B, H, Hkv, N, d = shape
    _check(inputs.make_inputs_heads(B, H, Hkv, N, N, d, 400 + N, "bf16"), causal)


@pytest.mark.parametrize("scale", [0.05, 1.0])
@pytest.mark.parametrize("d", [64, 128])
def test_scale(scale, d):
    """A scale other than 1/sqrt(d) reaches the exponent. For scale 1.0 the
    queries and keys have standard deviation 0.3 (before the cast), so the
    scores stay moderate and the ordinary bf16 bound applies."""
    q, k, v = inputs.normal_tensors(1, 4, 333, d, 17, 3)
    if scale == 1.0:
        q, k = 0.3 * q, 0.3 * k
    inp = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16)}
    _check(inp, True, "f32", scale=scale)
    _check(inp, False, "f32", scale=scale)


# Score ranges that move the running max after the first key block, or that
# would overflow or underflow without it (the cases of the fa_forward score
# range tests). The bound: the matrix cores see bf16(p_j) = p_j (1 + e_j) with
# |e_j| <= 2^-8 while l sums the unrounded p_j, so |O_gpu - O| <=
# 2^-8 sum_j P_j |v_j| per element, plus 2^-12 for the float32 scores and
# exponentials.
RANGE_CASES = [("grow2.5", 2.5), ("grow6", 6.0), ("grow40", 40.0), ("shifted", None)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", RANGE_CASES, ids=[c[0] for c in RANGE_CASES])
def test_score_range(case, causal, d):
    name, grow = case
    B, H, N = 1, 4, 700
    print(f"case ws score range {name} B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    q, k, v = inputs.normal_tensors(B, H, N, d, 15, 3)
    if grow is not None:
        k = k.clone()
        k[:, :, 300:] *= grow
    else:
        q, k = q - 4.0, k + 4.0
    inp = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16)}
    o, lse = gpu_forward_ws(inp, causal, "f32")
    ro, rl = oracle_forward(inp, "bf16", causal)
    r_abs, _ = oracle_forward(dict(inp, v=inp["v"].abs()), "bf16", causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    err = np.abs(o - ro)
    bound = (2.0 ** -8 + 2.0 ** -12) * r_abs + 1e-5
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"O: error {worst:.3g}x the bf16-P bound (max|err| {err.max():.3g})"
    le = assert_lse(lse, rl, "lse")
    print(f"  max|O err|={err.max():.3g} ({worst:.2f} of the bound) lse={le:.3g}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_invariant_uniform_scores(causal):
    """Q = 0: non-causal rows are the mean of V, causal rows the prefix means, lse = ln(#keys)."""
    B, H, N, d = 1, 2, 513, 128
    inp = inputs.make_inputs(B, H, N, d, 12, "bf16")
    inp["q"] = torch.zeros_like(inp["q"])
    v = inp["v"].to(torch.float64).numpy()
    o, lse = gpu_forward_ws(inp, causal, "f32")
    if causal:
        ref = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        lref = np.log(np.arange(1, N + 1))
    else:
        ref, lref = v.mean(axis=2, keepdims=True), math.log(N)
    assert np.max(np.abs(o - ref)) <= 1e-4
    assert np.max(np.abs(lse - lref)) <= 1e-5


@pytest.mark.parametrize("causal", [False, True])
def test_agrees_with_fa_forward(causal):
    """Same inputs through fa_forward_typed and fa_forward_ws: float32 outputs
    within the bf16 rounding of P of each other, lse within float32 noise."""
    inp = inputs.make_inputs(2, 8, 1500, 128, 19, "bf16")
    o1, l1 = gpu_forward(inp, "bf16", causal, "f32")
    o2, l2 = gpu_forward_ws(inp, causal, "f32")
    # Each is within (2^-8 + 2^-12) sum_j P_j |v_j| of the exact O (the bound
    # of the score-range tests), so they are within twice that of each other.
    r_abs, _ = oracle_forward(dict(inp, v=inp["v"].abs()), "bf16", causal)
    worst = float(np.max(np.abs(o1 - o2) / (2 * (2.0 ** -8 + 2.0 ** -12) * r_abs + 1e-5)))
    print(f"  fa_forward vs fa_forward_ws: max|dO|={np.max(np.abs(o1 - o2)):.3g} ({worst:.2f} of the bound) "
          f"max|dlse|={np.max(np.abs(l1 - l2)):.3g}", flush=True)
    assert worst <= 1.0
    assert np.max(np.abs(l1 - l2)) <= 1e-4


def test_deterministic():
    """Two runs give bitwise-identical outputs."""
    inp = inputs.make_inputs(1, 8, 1024, 128, 13, "bf16")
    o1, l1 = gpu_forward_ws(inp, True)
    o2, l2 = gpu_forward_ws(inp, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_long_sequence_offsets():
    """N = 2^20 + 77 (ragged), two heads, d=128, causal, float32 O: sampled
    rows far into each head (both sides of 2^16 and 2^20, the last rows)
    against the oracle, with the per-row relative bound of the long-sequence
    test of the other kernels."""
    from test_gpu_large import B, D, H, N, SEED, _relative, _rows
    scale = 1.0 / math.sqrt(D)
    rows = _rows()
    print(f"case ws long sequence B={B} H={H} N={N} d={D} seed={SEED} rows/head={rows.shape[-1]}", flush=True)
    inp = inputs.make_inputs(B, H, N, D, SEED, "bf16")
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_forward_ws(fa.FA_F32, q, k, v, o, lse, scale, True)
    torch.cuda.synchronize()
    idx = torch.tensor(rows[0], device=dev)
    pick = lambda t: torch.stack([t[0, h][idx[h]] for h in range(H)])[None].double().cpu().numpy()  # noqa: E731
    g_o, g_lse = pick(o), pick(lse)
    finite = bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    assert finite
    cq, ck, cv = (inputs.to_numpy(inp[n]) for n in "qkv")
    r_o, r_lse = oracle.forward(cq, ck, cv, scale, True, rows)
    mx, rms = assert_close(g_o, r_o, "bf16", "O")
    rel = _relative(g_o, r_o, "O", 2e-2)
    le = assert_lse(g_lse, r_lse, "lse")
    print(f"  O max={mx:.3g} rms={rms:.3g} of-allowed={rel:.3g} lse={le:.3g}", flush=True)


def test_caller_stream():
    """On a caller-made stream the results are the bits of the default-stream call."""
    B, H, N, d = 2, 4, 777, 128
    inp = inputs.make_inputs(B, H, N, d, 14, "bf16")
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in "qkv")
    outs = []
    for side in (False, True):
        o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
        if side:
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            fa.fa_forward_ws(fa.FA_BF16, q, k, v, o, lse, 1.0 / math.sqrt(d), True, stream=st)
            st.synchronize()
        else:
            fa.fa_forward_ws(fa.FA_BF16, q, k, v, o, lse, 1.0 / math.sqrt(d), True)
            torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert bool(torch.isfinite(outs[0][0].float()).all())
