"""fa_decode_noalloc (the decode entry point that allocates nothing: its
partials live in the library's static per-GPU scratch array) against
fa_decode with a caller workspace and against the oracle, on two calls in a
row, the second smaller than the first."""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs
from parity import assert_close, assert_lse

pytestmark = pytest.mark.gpu

CASES = [  # (B, H, Hkv, Nq, Nk, d, causal, seed): the first a decode workload, then a smaller one
    (8, 32, 8, 1, 32768, 128, True, 8),
    (1, 8, 2, 3, 1000, 64, True, 41),
]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    dev = torch.device("cuda:0")
    for B, H, Hkv, Nq, Nk, d, causal, seed in CASES:
        print(f"case fa_decode_noalloc B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}", flush=True)
        assert fa.fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d) <= fa.FA_DECODE_NOALLOC_MAX_WORKSPACE
        inp = inputs.make_inputs_heads(B, H, Hkv, Nq, Nk, d, seed, "bf16")
        q, k, v = (inp[n].to(dev) for n in "qkv")
        scale = 1.0 / math.sqrt(d)
        o_ref = torch.full((B, H, Nq, d), float("nan"), dtype=torch.bfloat16, device=dev)
        lse_ref = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), dtype=torch.uint8, device=dev)
        fa.fa_decode(q, k, v, o_ref, fa.FA_BF16, lse_ref, ws, scale, causal)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        fa.fa_decode_noalloc(q, k, v, o, fa.FA_BF16, lse, scale, causal)
        torch.cuda.synchronize()
        # same kernels, same split: the results are identical
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
        ro, rl = oracle.forward_decode(*(inputs.to_numpy(inp[n]) for n in "qkv"), scale, causal)
        mx, rms = assert_close(o.cpu().double().numpy(), ro, "bf16", "O", o_bf16=True)
        le = assert_lse(lse.cpu().double().numpy(), rl, "lse")
        print(f"  identical to fa_decode; max|O err|={mx:.3g} rms={rms:.3g} lse={le:.3g}", flush=True)
