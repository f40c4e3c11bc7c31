"""Seeded synthetic workloads for the attention path.

This module only draws inputs: normal samples, their casts to the operand
dtype, the per-tensor FP8 quantisation that the FP8 workload prescribes, and
seeded samples of query rows. It holds none of the attention arithmetic and
serves both the GPU path and the float64 oracle, which never import each
other.

Recipe (the five workloads of the exact-attention path):
  * Q, K, V (and dO for the backward workload), in that order, are
    `torch.randn(B, H, N, d, dtype=float32)` from one CPU generator seeded
    with the workload's seed, then cast to the operand dtype (bf16: round to
    nearest even) or quantised to FP8 E4M3 with a per-tensor scale
    s = amax|x| / 448 and codes e4m3fn(x / s) rounded to nearest even.
  * Sampled rows: per (b, h), `sorted(default_rng([seed, b, h]).choice(N,
    size, replace=False))`.
  * Grouped-query workloads: Q [B,H,N,d], then K and V [B,Hkv,N,d], then dO
    [B,H,N,d], drawn in that order from one generator seeded with the
    workload's seed (same casts as above).
  * Decode workloads: Q [B,H,Nq,d], then K and V [B,Hkv,Nk,d], same recipe.
"""
import numpy as np
import torch

E4M3_MAX = 448.0
E5M2_MAX = 57344.0

# name -> workload description (sizes as in the exact-attention workloads)
WORKLOADS = {
    "fwd_f32_b1h1_n256_d64": dict(seed=1, B=1, H=1, N=256, d=64, dtype="f32", causal=(False,),
                                  sample=None, backward=False),
    "fwd_bf16_b4h16_n2048_d64": dict(seed=2, B=4, H=16, N=2048, d=64, dtype="bf16", causal=(False, True),
                                     sample=None, backward=False),
    "fwd_bf16_causal_b1h32_n16384_d128": dict(seed=3, B=1, H=32, N=16384, d=128, dtype="bf16", causal=(True,),
                                              sample=512, backward=False),
    "bwd_bf16_causal_b2h16_n4096_d128": dict(seed=4, B=2, H=16, N=4096, d=128, dtype="bf16", causal=(True,),
                                             sample=None, backward=True),
    "fwd_fp8_causal_b1h8_n65536_d128": dict(seed=5, B=1, H=8, N=65536, d=128, dtype="fp8", causal=(True,),
                                            sample=256, backward=False),
}

# Grouped-query workloads: the 16K forward and the 4K backward shapes above
# with 4 query heads per key/value head.
GQA_WORKLOADS = {
    "fwd_bf16_gqa_causal_b1h32kv8_n16384_d128": dict(seed=6, B=1, H=32, Hkv=8, N=16384, d=128, dtype="bf16",
                                                     causal=(True,), sample=512, backward=False),
    "bwd_bf16_gqa_causal_b2h16kv4_n4096_d128": dict(seed=7, B=2, H=16, Hkv=4, N=4096, d=128, dtype="bf16",
                                                    causal=(True,), sample=None, backward=True),
}


def normal_tensors(B, H, N, d, seed, count=3):
    """`count` float32 N(0,1) tensors [B,H,N,d] drawn in order from one seeded CPU generator."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return [torch.randn(B, H, N, d, dtype=torch.float32, generator=g) for _ in range(count)]


def quantize_e4m3(x):
    """Per-tensor FP8 E4M3 quantisation: returns (codes float8_e4m3fn, scale float32).

    scale = amax|x| / 448 in float32; codes = e4m3fn(x / scale), round to
    nearest even (torch's cast). The dequantised value is codes * scale.
    """
    x = x.to(torch.float32)
    amax = x.abs().max()
    scale = (amax / E4M3_MAX).to(torch.float32)
    if float(scale) == 0.0:
        scale = torch.tensor(1.0, dtype=torch.float32)
    codes = (x / scale).to(torch.float8_e4m3fn)
    return codes, np.float32(scale.item())


def quantize_e5m2(x):
    """Per-tensor FP8 E5M2 quantisation: scale = amax|x| / 57344 in float32;
    codes = e5m2(x / scale), round to nearest even (torch's cast)."""
    x = x.to(torch.float32)
    amax = x.abs().max()
    scale = (amax / E5M2_MAX).to(torch.float32)
    if float(scale) == 0.0:
        scale = torch.tensor(1.0, dtype=torch.float32)
    codes = (x / scale).to(torch.float8_e5m2)
    return codes, np.float32(scale.item())


# FP8 backward: the 4K backward shape with E4M3 Q, K, V and an E5M2 dO.
FP8_BWD_WORKLOADS = {
    "bwd_fp8_causal_b2h16_n4096_d128": dict(seed=11, B=2, H=16, Hkv=16, N=4096, d=128, dtype="fp8bwd",
                                            causal=(True,), sample=None, backward=True),
}

# FP8 E5M2 variant of the 64K FP8 workload.
FP8_E5M2_WORKLOADS = {
    "fwd_fp8e5m2_causal_b1h8_n65536_d128": dict(seed=10, B=1, H=8, N=65536, d=128, dtype="fp8e5m2",
                                                causal=(True,), sample=256, backward=False),
}


# Decode workloads: Nq new rows per query head against an Nk-row cache of
# Hkv key/value heads (4 query heads per key/value head).
DECODE_WORKLOADS = {
    "decode_bf16_b8h32kv8_nq1_nk32768_d128": dict(seed=8, B=8, H=32, Hkv=8, Nq=1, Nk=32768, d=128, dtype="bf16",
                                                  causal=True),
    "decode_bf16_b4h32kv8_nq4_nk16384_d128": dict(seed=9, B=4, H=32, Hkv=8, Nq=4, Nk=16384, d=128, dtype="bf16",
                                                  causal=True),
}


def make_inputs(B, H, N, d, seed, dtype, with_do=False):
    """Seeded CPU inputs of one workload.

    dtype: "f32" | "bf16" | "fp8" (E4M3) | "fp8e5m2". Returns a dict with q,
    k, v (and do) as CPU tensors of the operand dtype; for the FP8 dtypes
    also the scales sq, sk, sv.
    """
    xs = normal_tensors(B, H, N, d, seed, 4 if with_do else 3)
    return _cast({}, ["q", "k", "v", "do"][: len(xs)], xs, dtype)


def _cast(out, names, xs, dtype):
    if dtype == "f32":
        out.update(zip(names, xs))
    elif dtype == "bf16":
        out.update((n, x.to(torch.bfloat16)) for n, x in zip(names, xs))
    elif dtype in ("fp8", "fp8e5m2"):
        quant = quantize_e4m3 if dtype == "fp8" else quantize_e5m2
        for n, x in zip(names, xs):
            if n == "do":
                out[n] = x.to(torch.bfloat16)
                continue
            codes, s = quant(x)
            out[n] = codes
            out["s" + n] = s
    elif dtype == "fp8bwd":  # E4M3 Q, K, V and an E5M2 gradient dO, per-tensor scales
        for n, x in zip(names, xs):
            codes, s = (quantize_e5m2 if n == "do" else quantize_e4m3)(x)
            out[n] = codes
            out["s" + n] = s
    else:
        raise ValueError(f"unknown dtype {dtype}")
    return out


def make_inputs_heads(B, H, Hkv, Nq, Nk, d, seed, dtype, with_do=False):
    """Seeded CPU inputs with H query heads of Nq rows and Hkv key/value heads
    of Nk rows (grouped-query and decode workloads). Same dict as make_inputs."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shapes = [(B, H, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)] + ([(B, H, Nq, d)] if with_do else [])
    xs = [torch.randn(*sh, dtype=torch.float32, generator=g) for sh in shapes]
    return _cast({}, ["q", "k", "v", "do"][: len(xs)], xs, dtype)


def sample_rows(seed, B, H, N, size):
    """Seeded query-row sample [B, H, size] (sorted, without replacement, per head)."""
    size = min(size, N)
    rows = np.empty((B, H, size), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            rows[b, h] = np.sort(np.random.default_rng([seed, b, h]).choice(N, size, replace=False))
    return rows


def to_numpy(t):
    """CPU tensor -> numpy array that the oracle reads (exact for f32/bf16; uint8 codes for fp8)."""
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8).numpy()
    return t.to(torch.float32).numpy()
