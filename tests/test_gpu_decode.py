"""Decode step (split-K forward): fa_decode through the C ABI vs the float64
oracle (rows are the last Nq positions; causal row i sees keys <= Nk - Nq + i)."""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs
from parity import assert_close, assert_lse

pytestmark = pytest.mark.gpu


def gpu_decode(inp, causal, o_dtype="bf16"):
    B, H, Nq, d = inp["q"].shape
    Hkv, Nk = inp["k"].shape[1], inp["k"].shape[2]
    dev = torch.device("cuda:0")
    qd, kd, vd = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16 if o_dtype == "bf16" else torch.float32,
                   device=dev)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fa.fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), 1), dtype=torch.uint8, device=dev)
    fa.fa_decode(qd, kd, vd, o, fa.FA_BF16 if o_dtype == "bf16" else fa.FA_F32, lse, ws, 1.0 / math.sqrt(d), causal)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def _check(B, H, Hkv, Nq, Nk, d, seed, causal, o_dtype="bf16"):
    print(f"case B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} seed={seed} causal={causal} o={o_dtype}", flush=True)
    inp = inputs.make_inputs_heads(B, H, Hkv, Nq, Nk, d, seed, "bf16")
    o, lse = gpu_decode(inp, causal, o_dtype)
    ro, rl = oracle.forward_decode(*(inputs.to_numpy(inp[n]) for n in "qkv"), 1.0 / math.sqrt(d), causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    mx, rms = assert_close(o, ro, "bf16", "O", o_bf16=(o_dtype == "bf16"))
    lmx = assert_lse(lse, rl, "lse")
    print(f"  O max={mx:.3g} rms={rms:.3g} lse={lmx:.3g}", flush=True)


@pytest.mark.parametrize("name", sorted(inputs.DECODE_WORKLOADS))
def test_workload(name):
    w = inputs.DECODE_WORKLOADS[name]
    _check(w["B"], w["H"], w["Hkv"], w["Nq"], w["Nk"], w["d"], w["seed"], w["causal"])


EDGE = [
    (1, 1, 1, 1, 1, 64), (1, 4, 1, 1, 100, 128), (2, 8, 2, 3, 129, 64), (1, 32, 8, 1, 1000, 128),
    (1, 8, 8, 7, 257, 128), (1, 16, 2, 5, 300, 64), (2, 4, 4, 16, 16, 128), (1, 8, 1, 4, 5000, 128),
    # one 32-row tile, medium caches: a handful of splits of 18 blocks each
    (1, 4, 1, 1, 20000, 128), (1, 2, 1, 2, 9000, 64),
    # one 32-row tile and long caches: 92 and 65 splits, so the merge walks its
    # partials in chunks of 64 with a ragged last chunk (of 28 and of 1)
    (1, 4, 1, 1, 200003, 128), (1, 2, 1, 2, 140000, 64),
]


@pytest.mark.parametrize("shape", EDGE, ids=[f"B{b}H{h}kv{g}q{nq}k{nk}d{d}" for b, h, g, nq, nk, d in EDGE])
@pytest.mark.parametrize("causal", [False, True])
def test_edge(shape, causal):
    B, H, Hkv, Nq, Nk, d = shape
    _check(B, H, Hkv, Nq, Nk, d, 1000 + Nk + Nq, causal)


def test_f32_output():
    _check(1, 8, 2, 2, 777, 128, 51, True, o_dtype="f32")


def test_decode_matches_forward_tail():
    """Independent of the oracle: decode rows equal the last rows of the
    causal forward on the same tensors (two different kernels)."""
    B, H, Hkv, N, d, nq = 1, 8, 2, 1500, 128, 3
    full = inputs.make_inputs_heads(B, H, Hkv, N, N, d, 52, "bf16")
    dev = torch.device("cuda:0")
    qd, kd, vd = (full[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    fa.fa_forward_gqa(fa.FA_BF16, fa.FA_F32, qd, kd, vd, None, o, lse, 1.0 / math.sqrt(d), True)
    dec = dict(q=full["q"][:, :, N - nq:].contiguous(), k=full["k"], v=full["v"])
    od, ld = gpu_decode(dec, True, "f32")
    torch.cuda.synchronize()
    assert np.max(np.abs(od - o[:, :, N - nq:].cpu().double().numpy())) <= 1e-2
    assert np.max(np.abs(ld - lse[:, :, N - nq:].cpu().double().numpy())) <= 1e-3


def test_determinism():
    inp = inputs.make_inputs_heads(1, 8, 2, 2, 3000, 128, 53, "bf16")
    a = gpu_decode(inp, True)
    b = gpu_decode(inp, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
