"""Helpers for GPU-vs-oracle parity: run the HIP path through the C ABI and
compare with the float64 oracle element by element.

Tolerances (absolute, over every compared element):
  float32 operands: max |err| <= 1e-5
  bf16 operands:    max |err| <= 1e-2 and RMS <= 2e-3
  fp8 E4M3 / E5M2:  max |err| <= 6e-2 (against the dequantised inputs)
  log-sum-exp:      max |err| <= 1e-3 (every dtype)
"""
import math

import numpy as np
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs

TOL = {"f32": dict(max=1e-5, rms=None), "bf16": dict(max=1e-2, rms=2e-3), "fp8": dict(max=6e-2, rms=None)}
TOL["fp8e5m2"] = TOL["fp8"]  # the oracle sees the same quantised inputs; P is E4M3 in both paths
LSE_TOL = 1e-3
FA_DT = {"f32": fa.FA_F32, "bf16": fa.FA_BF16, "fp8": fa.FA_FP8_E4M3, "fp8e5m2": fa.FA_FP8_E5M2}


def gpu_forward(inp, dtype, causal, o_dtype="bf16", scale=None):
    """Runs fa_forward_typed on device copies of the CPU inputs; returns CPU (o float64, lse float64)."""
    q = inp["q"]
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dev = torch.device("cuda:0")
    qd, kd, vd = (inp[n].to(dev) for n in ("q", "k", "v"))
    odt = torch.bfloat16 if o_dtype == "bf16" else torch.float32
    o = torch.empty(B, H, N, d, dtype=odt, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    descale = None
    if dtype in ("fp8", "fp8e5m2"):
        descale = torch.tensor([inp["sq"], inp["sk"], inp["sv"]], dtype=torch.float32, device=dev)
    fa.fa_forward_typed(FA_DT[dtype], FA_DT[o_dtype], qd, kd, vd, descale, o, lse, scale, causal)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def oracle_forward(inp, dtype, causal, rows=None, scale=None):
    d = inp["q"].shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if dtype in ("fp8", "fp8e5m2"):
        return oracle.forward_quantized(inputs.to_numpy(inp["q"]), inputs.to_numpy(inp["k"]), inputs.to_numpy(inp["v"]),
                                        inp["sq"], inp["sk"], inp["sv"], scale, causal, rows,
                                        fmt="e4m3" if dtype == "fp8" else "e5m2")
    return oracle.forward(inputs.to_numpy(inp["q"]), inputs.to_numpy(inp["k"]), inputs.to_numpy(inp["v"]),
                          scale, causal, rows)


def gather_rows(x, rows):
    """x: [B,H,N,...] -> [B,H,R,...] at rows [B,H,R]."""
    B, H = rows.shape[:2]
    return np.stack([np.stack([x[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])


def errors(got, ref):
    diff = np.abs(got - ref)
    return float(diff.max()) if diff.size else 0.0, float(np.sqrt(np.mean(diff ** 2))) if diff.size else 0.0


def assert_close(got, ref, dtype, what, o_bf16=None):
    tol = TOL[dtype]
    mx, rms = errors(got, ref)
    if o_bf16:
        floor = float(np.max(np.abs(torch.tensor(ref).to(torch.bfloat16).to(torch.float64).numpy() - ref))) if ref.size else 0.0
        assert floor < tol["max"], f"{what}: tolerance unachievable at this seed (bf16 rounding floor {floor:.3g})"
    assert mx <= tol["max"], f"{what}: max|err| {mx:.3g} > {tol['max']}"
    if tol["rms"] is not None:
        assert rms <= tol["rms"], f"{what}: rms {rms:.3g} > {tol['rms']}"
    return mx, rms


def assert_lse(got, ref, what):
    mx = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert mx <= LSE_TOL, f"{what}: lse max|err| {mx:.3g} > {LSE_TOL}"
    return mx


def gpu_backward(inp, causal, o_dtype="f32", scale=None):
    """Forward (saving O in o_dtype and lse) then fa_backward; returns CPU float64 (dq, dk, dv)."""
    q = inp["q"]
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    odt = torch.float32 if o_dtype == "f32" else torch.bfloat16
    o = torch.empty(B, H, N, d, dtype=odt, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    fa.fa_forward_typed(fa.FA_BF16, FA_DT[o_dtype], qd, kd, vd, None, o, lse, scale, causal)
    ws = torch.empty(max(fa.fa_backward_workspace_bytes(B, H, N, d), 1), dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device=dev) for _ in range(3))
    fa.fa_backward(qd, kd, vd, o, FA_DT[o_dtype], dod, lse, dq, dk, dv, ws, scale, causal)
    torch.cuda.synchronize()
    return tuple(t.cpu().to(torch.float64).numpy() for t in (dq, dk, dv))


def oracle_backward(inp, causal, scale=None, heads=None):
    d = inp["q"].shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return oracle.backward(*(inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do")), scale, causal, heads=heads)
