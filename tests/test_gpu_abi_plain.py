"""The C ABI without torch: a child process that never imports torch
(tests/abi_plain_client.py) allocates device memory and copies with the HIP
runtime through ctypes, runs fa_forward and fa_backward on plain device
pointers, and hands the results back; here they are checked against the
float64 oracle at the bf16 bounds of the other parity tests."""
import math
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs
from parity import assert_close, assert_lse

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_backward_without_torch(tmp_path, causal):
    B, H, N, d, seed = 1, 2, 333, 128, 41
    scale = 1.0 / math.sqrt(d)
    print(f"case plain-pointer client B={B} H={H} N={N} d={d} seed={seed} causal={causal}", flush=True)
    inp = inputs.make_inputs(B, H, N, d, seed, "bf16", with_do=True)
    bits = {n: inp[n].contiguous().view(torch.int16).numpy().view(np.uint16) for n in ("q", "k", "v", "do")}
    src, dst = tmp_path / "in.npz", tmp_path / "out.npz"
    np.savez(src, B=B, H=H, N=N, d=d, scale=np.float32(scale), causal=int(causal), **bits)
    fa.lib()  # the library this process tests is the one the child loads
    r = subprocess.run([sys.executable, os.path.join(HERE, "abi_plain_client.py"), fa._LIB_PATH, str(src), str(dst)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"client failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    out = np.load(dst)
    print(f"  client HIP runtime: {list(out['runtime'])}", flush=True)
    assert len(out["runtime"]) == 1 and "torch" not in str(out["runtime"][0])

    q, k, v, do = (_bf16_to_f64(bits[n]) for n in ("q", "k", "v", "do"))
    r_o, r_lse = oracle.forward(q, k, v, scale, causal)
    o = _bf16_to_f64(out["o"])
    mx, rms = assert_close(o, r_o, "bf16", "O", o_bf16=True)
    le = assert_lse(out["lse"].astype(np.float64), r_lse, "lse")
    # The backward is fed the bf16 O of the forward, as a caller holding only
    # that output would; D = rowsum(dO o O) then carries O's bf16 rounding.
    r_dq, r_dk, r_dv = oracle.backward(q, k, v, do, scale, causal)
    errs = []
    for name, g, ref in (("dQ", out["dq"], r_dq), ("dK", out["dk"], r_dk), ("dV", out["dv"], r_dv)):
        errs.append(assert_close(g.astype(np.float64), ref, "bf16", name))
    print(f"  O max={mx:.3g} rms={rms:.3g} lse={le:.3g} grads max={[f'{e[0]:.3g}' for e in errs]}", flush=True)
