"""A long sequence: N = 2^20 + 77 (ragged), two heads, d=128, causal.

Checks offsets far into each head (the last key and query blocks of a head
more than a GiB into the float32 outputs) on every kernel of the path:
- forward O and lse on sampled rows, including the first and last rows and
  rows on both sides of 2^16 and 2^20;
- backward dQ on the same rows (the oracle's row-restricted backward);
- dK and dV of the last 64 keys (under the causal mask only the last 64 rows
  reach them, so the oracle computes them exactly from those rows);
- the gradient-sum identities sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 over
  all keys.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_15_amd import binding as fa
from io_aware_exact_15_amd import inputs
from parity import assert_close, assert_lse

pytestmark = pytest.mark.gpu

B, H, N, D, SEED, TAIL = 1, 2, (1 << 20) + 77, 128, 700, 64


def _rows():
    fixed = [0, 1, 127, 128, 255, 256, 65535, 65536, (1 << 20) - 1, 1 << 20, N - 2, N - 1]
    g = np.random.default_rng([SEED, 1])
    per_head = []
    for _ in range(H):
        extra = []
        while len(extra) < 4:
            x = int(g.integers(N))
            if x not in fixed and x not in extra:
                extra.append(x)
        per_head.append(sorted(fixed + extra))
    return np.array([per_head])


def _relative(got, ref, what, frac, floor=1e-5):
    """Far along the sequence the rows are small (attention spreads over up to
    2^20 keys), so the absolute bound alone would say little there: every row
    must also be within `frac` of its own largest reference magnitude, plus a
    floor far below the absolute bound for rows whose exact value vanishes
    (row 0 sees only key 0, where dS = P (dP - D) is exactly 0).
    Returns the worst error as a fraction of what is allowed."""
    err = np.abs(got - ref).max(axis=-1)
    allowed = frac * np.abs(ref).max(axis=-1) + floor
    worst = float((err / allowed).max())
    assert worst <= 1.0, f"{what}: row error {worst:.3g} x the allowed {frac} of the row's magnitude + {floor}"
    return worst


def test_long_sequence_offsets():
    scale = 1.0 / math.sqrt(D)
    rows = _rows()
    print(f"case long sequence B={B} H={H} N={N} d={D} seed={SEED} causal rows/head={rows.shape[-1]}", flush=True)
    inp = inputs.make_inputs(B, H, N, D, SEED, "bf16", with_do=True)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty(B, H, N, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    fa.fa_forward_typed(fa.FA_BF16, fa.FA_F32, q, k, v, None, o, lse, scale, True)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=dev) for _ in range(3))
    fa.fa_backward(q, k, v, o, fa.FA_F32, do, lse, dq, dk, dv, ws, scale, True)
    torch.cuda.synchronize()
    idx = torch.tensor(rows[0], device=dev)
    pick = lambda t: torch.stack([t[0, h][idx[h]] for h in range(H)])[None].double().cpu().numpy()  # noqa: E731
    g_o, g_lse, g_dq = pick(o), pick(lse), pick(dq)
    g_dk, g_dv = (t[:, :, N - TAIL:].double().cpu().numpy() for t in (dk, dv))
    sum_dk = dk.double().sum(dim=2).cpu().numpy()
    sum_dv = dv.double().sum(dim=2).cpu().numpy()
    finite = all(bool(torch.isfinite(t).all()) for t in (o, lse, dq, dk, dv))
    del q, k, v, do, o, lse, ws, dq, dk, dv
    torch.cuda.empty_cache()
    assert finite

    cq, ck, cv, cdo = (inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do"))
    r_o, r_lse = oracle.forward(cq, ck, cv, scale, True, rows)
    mx, rms = assert_close(g_o, r_o, "bf16", "O")
    rel = _relative(g_o, r_o, "O", 2e-2)
    le = assert_lse(g_lse, r_lse, "lse")
    print(f"  O max={mx:.3g} rms={rms:.3g} of-allowed={rel:.3g} lse={le:.3g}", flush=True)
    r_dq = oracle.backward_rows(cq, ck, cv, cdo, scale, True, rows)
    mx, rms = assert_close(g_dq, r_dq, "bf16", "dQ rows")
    rel = _relative(g_dq, r_dq, "dQ rows", 2e-2)
    print(f"  dQ rows max={mx:.3g} rms={rms:.3g} of-allowed={rel:.3g}", flush=True)
    r_dk, r_dv = oracle.backward_causal_tail(cq, ck, cv, cdo, scale, TAIL)
    for name, g, r in (("dK tail", g_dk, r_dk), ("dV tail", g_dv, r_dv)):
        mx, rms = assert_close(g, r, "bf16", name)
        rel = _relative(g, r, name, 2e-2)
        print(f"  {name} max={mx:.3g} rms={rms:.3g} of-allowed={rel:.3g}", flush=True)
    # Identities over all 2^20 keys. The residuals come from rounding P and dS
    # to fp16 and from the float32 O that D is formed from; they shrink like
    # 1/sqrt(row) along the sequence, so they stay far below these bounds.
    r_dv_sum = np.abs(sum_dv - cdo.astype(np.float64).sum(axis=2)).max()
    r_dk_sum = np.abs(sum_dk).max()
    print(f"  |sum dV - sum dO|={r_dv_sum:.3g} |sum dK|={r_dk_sum:.3g}", flush=True)
    assert r_dv_sum <= 5e-2
    assert r_dk_sum <= 2e-1
