"""Throughput of the exact-attention hot path on one MI355X.

Workload: causal attention, bf16 operands, B=1 H=32 N=16384 d=128, scale
1/sqrt(d), synthetic N(0,1) inputs resident in HBM. One step is the whole
path: the forward pass (saving O and lse) followed by the backward pass
(D = rowsum(dO*O), dK/dV, dQ). Algorithmic FLOP: forward 4*B*H*N^2*d,
backward 10*B*H*N^2*d, both halved for the causal mask.

Prints one JSON line. Per-kernel durations come from HIP events recorded on
the launch stream around every launch of the timed region.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
  python bench.py --configs      # one JSON line per workload and pass (not the bench line)
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0
WORKLOAD = dict(name="fwd_bwd_bf16_causal_b1h32_n16384_d128", B=1, H=32, N=16384, d=128, causal=True, seed=3)


def _flops(B, H, N, d, causal, kind):
    f = {"fwd": 4, "bwd": 10}[kind] * B * H * N * N * d
    return f / 2 if causal else f


def _source_sha(names):
    """sha256 over the kernel sources (and the build script, which holds the
    compiler flags) that a measurement depends on."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "io_aware_exact_15_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


KERNEL_SOURCES = {"fwd": ["fa_fwd.hip", "fa_device.hpp", "../build.py"],
                  "bwd": ["fa_bwd.hip", "fa_device.hpp", "../build.py"]}
TRAFFIC_FILES = {"fwd": "fwd_bf16_causal_b1h32_n16384_d128_traffic.md",
                 "bwd": "bwd_bf16_causal_b1h32_n16384_d128_traffic.md"}


def _recorded_traffic(kind):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    (profiles/), or None when absent or taken on a different kernel source."""
    import re
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILES[kind])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)\s+source_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(2) != _source_sha(KERNEL_SOURCES[kind]):
        return None
    return int(m.group(1))


def _roofline(kernel, kind, flops, mean_ms):
    achieved = flops / (mean_ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": _recorded_traffic(kind),
            "algorithmic_flop_per_launch": flops, "mean_launch_ms": mean_ms}


def cpu_baseline(w, rows_per_head=4096):
    """The float64 oracle on host cores, on a bounded sample of the same workload.

    Sample: `rows_per_head` seeded query rows of every head, each against all
    keys (forward only). Value: the algorithmic causal FLOP of those rows
    (4*d*(i+1) for row i) per second of oracle wall time.
    """
    import numpy as np

    import oracle
    from io_aware_exact_15_amd import inputs

    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "bf16")
    q, k, v = (inputs.to_numpy(inp[n]) for n in ("q", "k", "v"))
    rows = inputs.sample_rows(w["seed"], B, H, N, rows_per_head)
    t0 = time.perf_counter()
    oracle.forward(q, k, v, 1.0 / math.sqrt(d), True, rows=rows)
    dt = time.perf_counter() - t0
    flops = float(np.sum(4.0 * d * (rows + 1)))
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"forward, {rows_per_head} seeded query rows per head x {B * H} heads against all {N} keys, "
                  f"float64 numpy ({dt:.2f} s wall, OMP_NUM_THREADS={os.environ.get('OMP_NUM_THREADS', 'unset')})",
    }


def cpu_baseline_sample(kind, w, inp, causal, target_flop=5e10):
    """The float64 oracle timed on a bounded sample of one workload, for the
    per-workload lines of --configs (a few seconds each).

    kind: "fwd" (seeded query rows of every head against all their keys),
    "bwd" (the full backward of the first head group), or "decode" (the whole
    decode step). Value: the algorithmic FLOP of what was computed per second
    of oracle wall time.
    """
    import numpy as np

    import oracle
    from io_aware_exact_15_amd import inputs

    B, H, d = w["B"], w["H"], w["d"]
    Hkv = w.get("Hkv", H)
    G = H // Hkv
    scale = 1.0 / math.sqrt(d)
    dtype = w["dtype"]
    arr = {n: inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do") if n in inp}
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    if kind == "decode":
        Nq, Nk = w["Nq"], w["Nk"]
        oracle.forward_decode(arr["q"], arr["k"], arr["v"], scale, causal)
        pos = np.arange(Nk - Nq, Nk)
        keys = np.minimum(pos + 1, Nk) if causal else np.full(Nq, Nk)
        flop = 4.0 * d * B * H * float(np.sum(keys))
        sample = f"the whole decode step ({B * H * Nq} rows against {Nk} keys)"
    elif kind == "fwd":
        N = w["N"]
        per_row = 4.0 * d * N * B * H
        R = int(min(N, max(1, target_flop // per_row)))
        rows = inputs.sample_rows(w["seed"], B, H, N, R)
        if dtype == "fp8":
            oracle.forward_quantized(arr["q"], arr["k"], arr["v"], inp["sq"], inp["sk"], inp["sv"], scale, causal, rows)
        elif G > 1:
            oracle.forward_gqa(arr["q"], arr["k"], arr["v"], scale, causal, rows)
        else:
            oracle.forward(arr["q"], arr["k"], arr["v"], scale, causal, rows)
        flop = float(np.sum(4.0 * d * (rows + 1))) if causal else 4.0 * d * N * rows.size
        sample = f"{R} seeded query rows per head x {B * H} heads against all their keys"
    else:  # bwd: the first head group (G query heads and their key/value head) of batch 0
        N = w["N"]
        sl = lambda x, h: x[:1, :h]  # noqa: E731
        if dtype == "fp8bwd":
            oracle.backward_quantized(sl(arr["q"], 1), sl(arr["k"], 1), sl(arr["v"], 1), sl(arr["do"], 1),
                                      inp["sq"], inp["sk"], inp["sv"], inp["sdo"], scale, causal)
            heads = 1
        elif G > 1:
            oracle.backward_gqa(sl(arr["q"], G), sl(arr["k"], 1), sl(arr["v"], 1), sl(arr["do"], G), scale, causal)
            heads = G
        else:
            oracle.backward(sl(arr["q"], 1), sl(arr["k"], 1), sl(arr["v"], 1), sl(arr["do"], 1), scale, causal)
            heads = 1
        flop = _flops(1, heads, N, d, causal, "bwd")
        sample = f"full backward of {heads} head(s)"
    dt = time.perf_counter() - t0
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample}, float64 numpy ({dt:.2f} s wall)"}


PEAK_FP8_TFLOPS = 5033.2
PEAK_F32_MFMA_TFLOPS = 157.3


def _median_ms(torch, fn, iters, warmup):
    """Median and min of the per-call GPU time: the calls are enqueued back to
    back (as in the headline loop), each between its own pair of events, and
    the host synchronises once at the end, so host launch latency does not
    land inside the timed intervals."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return ts[len(ts) // 2], ts[0]


def run_configs(iters=20, warmup=3, with_cpu=True):
    """Times every workload of the path (one JSON line per workload and pass)."""
    import torch

    from io_aware_exact_15_amd import binding as fa
    from io_aware_exact_15_amd import inputs

    dev = torch.device("cuda:0")
    allw = [(n, dict(w, Hkv=w["H"])) for n, w in inputs.WORKLOADS.items()] + list(inputs.GQA_WORKLOADS.items())
    for name, w in allw:
        B, H, Hkv, N, d = w["B"], w["H"], w["Hkv"], w["N"], w["d"]
        scale = 1.0 / math.sqrt(d)
        inp = inputs.make_inputs_heads(B, H, Hkv, N, N, d, w["seed"], w["dtype"], with_do=w["backward"])
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        if w["dtype"] == "fp8":
            in_t, o_t, peak, odt = fa.FA_FP8_E4M3, fa.FA_BF16, PEAK_FP8_TFLOPS, torch.bfloat16
            desc = torch.tensor([inp["sq"], inp["sk"], inp["sv"]], dtype=torch.float32, device=dev)
        elif w["dtype"] == "f32":
            in_t, o_t, peak, odt, desc = fa.FA_F32, fa.FA_F32, PEAK_F32_MFMA_TFLOPS, torch.float32, None
        else:
            in_t, o_t, peak, odt, desc = fa.FA_BF16, fa.FA_BF16, PEAK_BF16_TFLOPS, torch.bfloat16, None
        if w["backward"]:
            o_t, odt = fa.FA_F32, torch.float32  # the forward that feeds the backward writes float32 O
        o = torch.empty(B, H, N, d, dtype=odt, device=dev)
        for causal in w["causal"]:
            fwd = lambda: fa.fa_forward_gqa(in_t, o_t, q, k, v, desc, o, lse, scale, causal)
            med, mn = _median_ms(torch, fwd, iters, warmup)
            f = _flops(B, H, N, d, causal, "fwd")
            line = {"workload": name, "pass": "fwd", "causal": causal, "dtype": w["dtype"],
                    "ms_median": med, "ms_min": mn, "tflops": f / (med * 1e-3) / 1e12,
                    "frac_of_peak": f / (med * 1e-3) / 1e12 / peak, "peak_tflops": peak}
            if with_cpu:
                line["cpu_baseline"] = cpu_baseline_sample("fwd", w, inp, causal)
            print(json.dumps(line), flush=True)
            if w["backward"]:
                do = inp["do"].to(dev)
                dq = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
                dk, dv = (torch.empty(B, Hkv, N, d, dtype=torch.float32, device=dev) for _ in range(2))
                ws = torch.empty(fa.fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device=dev)
                fwd()
                bwd = lambda: fa.fa_backward_gqa(q, k, v, o, fa.FA_F32, do, lse, dq, dk, dv, ws, scale, causal)
                bmed, bmn = _median_ms(torch, bwd, iters, warmup)
                bf = _flops(B, H, N, d, causal, "bwd")
                line = {"workload": name, "pass": "bwd", "causal": causal, "dtype": w["dtype"],
                        "ms_median": bmed, "ms_min": bmn, "tflops": bf / (bmed * 1e-3) / 1e12,
                        "frac_of_peak": bf / (bmed * 1e-3) / 1e12 / peak, "peak_tflops": peak}
                if with_cpu:
                    line["cpu_baseline"] = cpu_baseline_sample("bwd", w, inp, causal)
                print(json.dumps(line), flush=True)
                print(json.dumps({"workload": name, "pass": "fwd+bwd", "causal": causal, "dtype": w["dtype"],
                                  "ms_median": med + bmed,
                                  "tflops": (f + bf) / ((med + bmed) * 1e-3) / 1e12,
                                  "frac_of_peak": (f + bf) / ((med + bmed) * 1e-3) / 1e12 / peak}), flush=True)


def run_fp8_bwd_configs(iters=20, warmup=3, with_cpu=True):
    """Times the FP8 backward workloads (E4M3 Q, K, V; E5M2 dO). The forward
    that feeds them runs in float32 on the dequantised values (untimed)."""
    import numpy as np
    import torch

    from io_aware_exact_15_amd import binding as fa
    from io_aware_exact_15_amd import inputs

    dev = torch.device("cuda:0")
    for name, w in inputs.FP8_BWD_WORKLOADS.items():
        B, H, Hkv, N, d = w["B"], w["H"], w["Hkv"], w["N"], w["d"]
        scale = 1.0 / math.sqrt(d)
        inp = inputs.make_inputs(B, H, N, d, w["seed"], "fp8bwd", with_do=True)
        codes = {n: inp[n].to(dev) for n in ("q", "k", "v", "do")}
        deq = {n: (inp[n].to(torch.float32) * float(inp["s" + n])).to(dev) for n in ("q", "k", "v")}
        desc = torch.tensor([inp["sq"], inp["sk"], inp["sv"], inp["sdo"]], dtype=torch.float32, device=dev)
        o = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        for causal in w["causal"]:
            fa.fa_forward_gqa(fa.FA_F32, fa.FA_F32, deq["q"], deq["k"], deq["v"], None, o, lse, scale, causal)
            dq = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
            dk, dv = (torch.empty(B, Hkv, N, d, dtype=torch.float32, device=dev) for _ in range(2))
            ws = torch.empty(fa.fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device=dev)
            fn = lambda: fa.fa_backward_typed(fa.FA_FP8_E4M3, fa.FA_FP8_E5M2, codes["q"], codes["k"], codes["v"],
                                              codes["do"], desc, o, fa.FA_F32, lse, dq, dk, dv, ws, scale, causal)
            med, mn = _median_ms(torch, fn, iters, warmup)
            bf = _flops(B, H, N, d, causal, "bwd")
            line = {"workload": name, "pass": "bwd", "causal": causal, "dtype": "fp8 e4m3 / e5m2 dO",
                    "ms_median": med, "ms_min": mn, "tflops": bf / (med * 1e-3) / 1e12,
                    "frac_of_peak": bf / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                    "peak_tflops": PEAK_BF16_TFLOPS, "note": "fp16 matrix-core operands"}
            if with_cpu:
                line["cpu_baseline"] = cpu_baseline_sample("bwd", w, inp, causal)
            print(json.dumps(line), flush=True)


def run_decode_configs(iters=20, warmup=3, with_cpu=True):
    """Times the decode workloads (HBM-bound: reported as GB/s of the
    algorithmic bytes, the K/V cache read once plus Q, O and lse)."""
    import torch

    from io_aware_exact_15_amd import binding as fa
    from io_aware_exact_15_amd import inputs

    dev = torch.device("cuda:0")
    for name, w in inputs.DECODE_WORKLOADS.items():
        B, H, Hkv, Nq, Nk, d = w["B"], w["H"], w["Hkv"], w["Nq"], w["Nk"], w["d"]
        inp = inputs.make_inputs_heads(B, H, Hkv, Nq, Nk, d, w["seed"], "bf16")
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), dtype=torch.uint8, device=dev)
        fn = lambda: fa.fa_decode(q, k, v, o, fa.FA_BF16, lse, ws, 1.0 / math.sqrt(d), w["causal"])
        med, mn = _median_ms(torch, fn, iters, warmup)
        nbytes = 2 * B * Hkv * Nk * d * 2 + 2 * B * H * Nq * d * 2 + B * H * Nq * 4
        gbs = nbytes / (med * 1e-3) / 1e9
        line = {"workload": name, "pass": "decode", "causal": w["causal"], "dtype": "bf16",
                "ms_median": med, "ms_min": mn, "algorithmic_bytes": nbytes, "GB_per_s": gbs,
                "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}
        if with_cpu:
            line["cpu_baseline"] = cpu_baseline_sample("decode", w, inp, w["causal"])
        print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload (fwd, and bwd where it has one); one JSON line each")
    ap.add_argument("--counters", action="store_true",
                    help="untimed: one float32 copy-kernel launch of known size (512 MiB read + 512 MiB written, "
                         "the traffic calibration) and one step, for hardware-counter runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build runs on a single "
              "MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.configs:
        run_configs(with_cpu=not args.no_cpu)
        run_fp8_bwd_configs(with_cpu=not args.no_cpu)
        run_decode_configs(with_cpu=not args.no_cpu)
        return

    import torch

    from io_aware_exact_15_amd import binding as fa
    from io_aware_exact_15_amd import inputs

    w = WORKLOAD
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "bf16", with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    o_bf = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    lse_bf = torch.empty_like(lse)
    torch.cuda.synchronize()

    # Backward availability (the step is forward-only until it is built).
    have_bwd = True
    dq = dk = dv = ws = None
    try:
        dq, dk, dv = (torch.empty(B, H, N, d, dtype=torch.float32, device=dev) for _ in range(3))
        ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        fa.fa_forward_typed(fa.FA_BF16, fa.FA_F32, q, k, v, None, o, lse, scale, causal)
        fa.fa_backward(q, k, v, o, fa.FA_F32, do, lse, dq, dk, dv, ws, scale, causal)
    except fa.FAError as e:
        if e.status != fa.FA_ERR_UNSUPPORTED:
            raise
        have_bwd = False
    torch.cuda.synchronize()

    def step(ev):
        # headline forward: bf16 O
        ev[0].record()
        fa.fa_forward_typed(fa.FA_BF16, fa.FA_BF16, q, k, v, None, o_bf, lse_bf, scale, causal)
        ev[1].record()
        if have_bwd:
            fa.fa_forward_typed(fa.FA_BF16, fa.FA_F32, q, k, v, None, o, lse, scale, causal)
            ev[2].record()
            fa.fa_backward(q, k, v, o, fa.FA_F32, do, lse, dq, dk, dv, ws, scale, causal)
            ev[3].record()

    if args.counters:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # copy kernel: reads 512 MiB, writes 512 MiB
        torch.cuda.synchronize()
        warm = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(warm)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "copy_bytes_each_way": src.numel() * 4}), flush=True)
        return

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(args.warmup):
        step(warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    fwd_med = sorted(fwd_ms)[len(fwd_ms) // 2]
    fwd_mean = sum(fwd_ms) / len(fwd_ms)
    fwd_f = _flops(B, H, N, d, causal, "fwd")
    fwd_tf = fwd_f / (fwd_med * 1e-3) / 1e12
    res_fwd = {"ms_median": fwd_med, "ms_mean": fwd_mean, "ms_min": min(fwd_ms), "tflops": fwd_tf,
               "frac_of_bf16_peak": fwd_tf / PEAK_BF16_TFLOPS}
    roof_fwd = _roofline("fwd_bf16_kernel (bf16 O)", "fwd", fwd_f, fwd_mean)
    step_flops = fwd_f
    roofline = roof_fwd
    if have_bwd:
        fwd32_ms = [e[1].elapsed_time(e[2]) for e in evs]
        bwd_ms = [e[2].elapsed_time(e[3]) for e in evs]
        bwd_med = sorted(bwd_ms)[len(bwd_ms) // 2]
        bwd_mean = sum(bwd_ms) / len(bwd_ms)
        bwd_f = _flops(B, H, N, d, causal, "bwd")
        res_bwd = {"ms_median": bwd_med, "ms_mean": bwd_mean, "ms_min": min(bwd_ms),
                   "tflops": bwd_f / (bwd_med * 1e-3) / 1e12}
        fb_ms = sorted(a + b for a, b in zip(fwd32_ms, bwd_ms))[len(bwd_ms) // 2]
        res_fb = {"ms_median": fb_ms, "tflops": (fwd_f + bwd_f) / (fb_ms * 1e-3) / 1e12}
        step_flops = fwd_f + fwd_f + bwd_f
        if bwd_mean > fwd_mean:  # the backward pass dominates the step
            roofline = _roofline("fa_backward (bwd_pre + bwd_dkdv + bwd_dq)", "bwd", bwd_f, bwd_mean)
    ms_per_step = wall / args.steps * 1e3

    out = {
        "metric": "attention TFLOP/s (fwd, fwd+bwd) and % of MFMA peak, causal bf16 N=16K d=128",
        "value": (res_fb["tflops"] if have_bwd else fwd_tf),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"] if have_bwd else "fwd_bf16_causal_b1h32_n16384_d128",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "scale": scale,
                   "value_is": "fwd+bwd TFLOP/s (fwd with fp32 O, then bwd)" if have_bwd else "fwd TFLOP/s (backward not built)"},
        "fwd": res_fwd,
        "roofline": roofline,
        "roofline_fwd": roof_fwd,
    }
    if have_bwd:
        out["bwd"] = res_bwd
        out["fwd_bwd"] = res_fb
    out["step_flops"] = step_flops
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
