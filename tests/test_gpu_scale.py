"""The `scale` argument on the GPU: every entry point at scales other than
1/sqrt(d), against the oracle at the same scale.

A kernel that ignored `scale` and used 1/sqrt(d) would fail each of these:
at 0.05 and 1.0 the scores differ from the 1/sqrt(d) ones by factors of
1.8-20. For scale 1.0 the queries and keys are drawn with standard deviation
0.3 (before the cast), so the scores stay moderate and the bounds are the
ordinary ones of each dtype, except for the gradients: the matrix-core
operands of the backward pass are rounded relative to their size, and a
larger scale enlarges dQ and dK by the same factor, so their bound is
max(1e-2, 2e-3 max|ref|) (RMS max(2e-3, 4e-4 max|ref|)), i.e. the absolute
bf16 bound for gradients of unit size and a relative one beyond that.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs
from parity import assert_close, assert_lse, gpu_backward, gpu_forward, oracle_backward, oracle_forward

pytestmark = pytest.mark.gpu

SCALES = (0.05, 1.0)


def _grad_close(got, ref, name):
    top = float(np.max(np.abs(ref)))
    tol, rtol = max(1e-2, 2e-3 * top), max(2e-3, 4e-4 * top)
    err = np.abs(got - ref)
    mx, rms = float(err.max()), float(np.sqrt(np.mean(err ** 2)))
    print(f"  {name} max={mx:.3g} rms={rms:.3g} (bound {tol:.3g}, max|ref| {top:.3g})", flush=True)
    assert mx <= tol, f"{name}: max|err| {mx:.3g} > {tol:.3g}"
    assert rms <= rtol, f"{name}: rms {rms:.3g} > {rtol:.3g}"


def _xs(shapes, seed, scale):
    g = torch.Generator(device="cpu").manual_seed(seed)
    xs = [torch.randn(*sh, dtype=torch.float32, generator=g) for sh in shapes]
    if scale == 1.0:
        xs[0], xs[1] = 0.3 * xs[0], 0.3 * xs[1]
    return xs


def _cast(names, xs, dtype):
    out = {}
    for n, x in zip(names, xs):
        if dtype == "f32":
            out[n] = x
        elif dtype == "bf16" or n == "do":
            out[n] = x.to(torch.bfloat16)
        else:
            out[n], out["s" + n] = inputs.quantize_e4m3(x)
    return out


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64), ("fp8", 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward(scale, dtype, d, causal):
    B, H, N = 1, 2, 300
    print(f"case forward {dtype} d={d} causal={causal} scale={scale}", flush=True)
    inp = _cast("qkv", _xs([(B, H, N, d)] * 3, 31, scale), dtype)
    o_dtype = "f32" if dtype == "f32" else "bf16"
    o, lse = gpu_forward(inp, dtype, causal, o_dtype=o_dtype, scale=scale)
    ro, rl = oracle_forward(inp, dtype, causal, scale=scale)
    mx, rms = assert_close(o, ro, dtype, "O", o_bf16=(o_dtype == "bf16"))
    le = assert_lse(lse, rl, "lse")
    print(f"  max|O err|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward(scale, d, causal):
    B, H, N = 1, 2, 300
    print(f"case backward d={d} causal={causal} scale={scale}", flush=True)
    inp = _cast(["q", "k", "v", "do"], _xs([(B, H, N, d)] * 4, 32, scale), "bf16")
    got = gpu_backward(inp, causal, scale=scale)
    ref = oracle_backward(inp, causal, scale=scale)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        _grad_close(g, r, name)


@pytest.mark.parametrize("scale", SCALES)
def test_grouped_heads(scale):
    B, H, Hkv, N, d = 1, 4, 2, 200, 128
    print(f"case grouped heads scale={scale}", flush=True)
    inp = _cast(["q", "k", "v", "do"], _xs([(B, H, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, H, N, d)], 33, scale),
                "bf16")
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    fa.fa_forward_gqa(fa.FA_BF16, fa.FA_F32, q, k, v, None, o, lse, scale, True)
    ws = torch.empty(fa.fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device=dev)
    dq = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    dk, dv = (torch.empty(B, Hkv, N, d, dtype=torch.float32, device=dev) for _ in range(2))
    fa.fa_backward_gqa(q, k, v, o, fa.FA_F32, do, lse, dq, dk, dv, ws, scale, True)
    torch.cuda.synchronize()
    arr = [inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do")]
    ro, rl = oracle.forward_gqa(*arr[:3], scale, True)
    assert_close(o.cpu().double().numpy(), ro, "bf16", "O")
    assert_lse(lse.cpu().double().numpy(), rl, "lse")
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), oracle.backward_gqa(*arr, scale, True)):
        _grad_close(g.cpu().double().numpy(), r, name)


@pytest.mark.parametrize("scale", SCALES)
def test_decode(scale):
    B, H, Hkv, Nq, Nk, d = 1, 8, 2, 3, 500, 128
    print(f"case decode scale={scale}", flush=True)
    inp = _cast("qkv", _xs([(B, H, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)], 34, scale), "bf16")
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in "qkv")
    o = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), dtype=torch.uint8, device=dev)
    fa.fa_decode(q, k, v, o, fa.FA_BF16, lse, ws, scale, True)
    torch.cuda.synchronize()
    ro, rl = oracle.forward_decode(*(inputs.to_numpy(inp[n]) for n in "qkv"), scale, True)
    mx, rms = assert_close(o.cpu().double().numpy(), ro, "bf16", "O", o_bf16=True)
    assert_lse(lse.cpu().double().numpy(), rl, "lse")
    print(f"  max|O err|={mx:.3g} rms={rms:.3g}", flush=True)


@pytest.mark.parametrize("scale", SCALES)
def test_fp8_backward(scale):
    B, H, N, d = 1, 2, 200, 128
    print(f"case fp8 backward scale={scale}", flush=True)
    xs = _xs([(B, H, N, d)] * 4, 35, scale)
    inp = {}
    for n, x in zip(("q", "k", "v", "do"), xs):
        inp[n], inp["s" + n] = (inputs.quantize_e5m2 if n == "do" else inputs.quantize_e4m3)(x)
    dev = torch.device("cuda:0")
    deq = {n: (inp[n].to(torch.float32) * float(inp["s" + n])).to(dev) for n in ("q", "k", "v")}
    o = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    fa.fa_forward_gqa(fa.FA_F32, fa.FA_F32, deq["q"], deq["k"], deq["v"], None, o, lse, scale, True)
    codes = {n: inp[n].to(dev) for n in ("q", "k", "v", "do")}
    desc = torch.tensor([inp["sq"], inp["sk"], inp["sv"], inp["sdo"]], dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_backward_gqa_workspace_bytes(B, H, H, N, d), dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.empty(B, H, N, d, dtype=torch.float32, device=dev) for _ in range(3))
    fa.fa_backward_typed(fa.FA_FP8_E4M3, fa.FA_FP8_E5M2, codes["q"], codes["k"], codes["v"], codes["do"], desc, o,
                         fa.FA_F32, lse, dq, dk, dv, ws, scale, True)
    torch.cuda.synchronize()
    ref = oracle.backward_quantized(*(inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do")), inp["sq"], inp["sk"],
                                    inp["sv"], inp["sdo"], scale, True)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _grad_close(g.cpu().double().numpy(), r, name)
