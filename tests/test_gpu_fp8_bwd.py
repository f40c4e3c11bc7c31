"""FP8 backward: fa_backward_typed with E4M3 Q, K, V and an E5M2 (or E4M3) dO,
per-tensor scales, through the C ABI vs the float64 oracle on the
dequantised values. O and lse come from the float32 forward on the same
dequantised values, so the comparison isolates the backward pass; the bound
is the bf16 one (the matrix-core operands are the exact fp16 codes)."""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs
from parity import assert_close

pytestmark = pytest.mark.gpu

FMT = {"e4m3": fa.FA_FP8_E4M3, "e5m2": fa.FA_FP8_E5M2}


def _inputs(B, H, Hkv, N, d, seed, fmt_in, fmt_do):
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shapes = [(B, H, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, H, N, d)]
    xs = [torch.randn(*sh, dtype=torch.float32, generator=g) for sh in shapes]
    quant = {"e4m3": inputs.quantize_e4m3, "e5m2": inputs.quantize_e5m2}
    out = {}
    for n, x in zip(("q", "k", "v", "do"), xs):
        codes, s = quant[fmt_do if n == "do" else fmt_in](x)
        out[n], out["s" + n] = codes, s
    return out


def _run(inp, fmt_in, fmt_do, causal):
    B, H, N, d = inp["q"].shape
    Hkv = inp["k"].shape[1]
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    # The forward's float32 inputs are the dequantised values, formed by
    # torch's own (exact) FP8 -> float32 conversion, not by the oracle.
    deq = {n: inp[n].to(torch.float32) * float(inp["s" + n]) for n in ("q", "k", "v")}
    o = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    fa.fa_forward_gqa(fa.FA_F32, fa.FA_F32, deq["q"].to(dev), deq["k"].to(dev), deq["v"].to(dev), None, o, lse,
                      scale, causal)
    codes = {n: inp[n].to(dev) for n in ("q", "k", "v", "do")}
    desc = torch.tensor([inp["sq"], inp["sk"], inp["sv"], inp["sdo"]], dtype=torch.float32, device=dev)
    ws = torch.empty(max(fa.fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d), 1), dtype=torch.uint8, device=dev)
    dq = torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device=dev)
    dk, dv = (torch.full((B, Hkv, N, d), float("nan"), dtype=torch.float32, device=dev) for _ in range(2))
    fa.fa_backward_typed(FMT[fmt_in], FMT[fmt_do], codes["q"], codes["k"], codes["v"], codes["do"], desc, o,
                         fa.FA_F32, lse, dq, dk, dv, ws, scale, causal)
    torch.cuda.synchronize()
    return tuple(t.cpu().to(torch.float64).numpy() for t in (dq, dk, dv))


def _check(B, H, Hkv, N, d, seed, causal, fmt_in="e4m3", fmt_do="e5m2", inp=None):
    print(f"case fp8 bwd B={B} H={H} Hkv={Hkv} N={N} d={d} seed={seed} causal={causal} {fmt_in}/{fmt_do}", flush=True)
    inp = inp or _inputs(B, H, Hkv, N, d, seed, fmt_in, fmt_do)
    got = _run(inp, fmt_in, fmt_do, causal)
    ref = oracle.backward_quantized(*(inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do")), inp["sq"], inp["sk"],
                                    inp["sv"], inp["sdo"], 1.0 / math.sqrt(d), causal, fmt_in=fmt_in, fmt_do=fmt_do)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), name
        mx, rms = assert_close(g, r, "bf16", name)
        print(f"  {name}: max={mx:.3g} rms={rms:.3g}", flush=True)


def test_workload_bwd_fp8_causal_b2h16_n4096_d128():
    """B=2 H=16 N=4096 d=128 causal, E4M3 Q/K/V and E5M2 dO: every element of dQ, dK, dV."""
    w = inputs.FP8_BWD_WORKLOADS["bwd_fp8_causal_b2h16_n4096_d128"]
    inp = inputs.make_inputs(w["B"], w["H"], w["N"], w["d"], w["seed"], "fp8bwd", with_do=True)
    _check(w["B"], w["H"], w["Hkv"], w["N"], w["d"], w["seed"], True, inp=inp)


EDGE = [(1, 1, 1, 1, 64), (1, 2, 1, 17, 128), (2, 4, 2, 129, 64), (1, 8, 2, 300, 128), (1, 4, 4, 1000, 128)]


@pytest.mark.parametrize("shape", EDGE, ids=[f"B{b}H{h}kv{g}N{n}d{d}" for b, h, g, n, d in EDGE])
@pytest.mark.parametrize("causal", [False, True])
def test_edge(shape, causal):
    B, H, Hkv, N, d = shape
    _check(B, H, Hkv, N, d, 1300 + N, causal)


@pytest.mark.parametrize("fmts", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e5m2", "e4m3")], ids=lambda f: "-".join(f))
def test_formats(fmts):
    _check(1, 4, 2, 500, 128, 61, True, fmt_in=fmts[0], fmt_do=fmts[1])
