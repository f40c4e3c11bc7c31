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
                  "bwd": ["fa_bwd.hip", "fa_bwd_dq.hip", "fa_bwd_common.hpp", "fa_device.hpp", "../build.py"]}
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


def _blas():
    """Name and version of the BLAS library numpy uses (the oracle's matmuls)."""
    import numpy as np
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # pragma: no cover - older numpy
        return "unknown"


def cpu_baseline(w, heads=4):
    """The float64 oracle on host cores, on a bounded sample of the same workload.

    Sample: the full forward and backward (every query row against all keys,
    the N x N matrices materialised) of the first `heads` head(s) of the
    headline workload. Value: the algorithmic causal FLOP of that forward and
    backward ((4 + 10) * N^2 * d / 2 per head) per second of oracle wall time.
    Heads are independent, so the whole step would take H / heads times as
    long; that extrapolation is reported too.
    """
    import numpy as np

    import oracle
    from io_aware_exact_15_amd import inputs

    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "bf16", with_do=True)
    q, k, v, do = (inputs.to_numpy(inp[n])[:1, :heads] for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    t0 = time.perf_counter()
    oracle.forward(q, k, v, scale, w["causal"])
    oracle.backward(q, k, v, do, scale, w["causal"])
    dt = time.perf_counter() - t0
    flops = _flops(1, heads, N, d, w["causal"], "fwd") + _flops(1, heads, N, d, w["causal"], "bwd")
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"forward + backward of {heads} of {B * H} heads, every query row against all {N} keys, "
                  f"float64 numpy ({dt:.2f} s wall)",
        "blas": _blas(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS", "unset"),
        "full_step_extrapolated_s": dt * B * H / heads,
    }


# Parity bounds of the bench's own check (absolute, over every compared element).
PARITY_TOL = {"o_max": 1e-2, "o_rms": 2e-3, "lse_max": 1e-3, "dq_max": 1e-2, "dk_max": 1e-2, "dv_max": 1e-2}


def parity_of_step(w, outs, rows_per_head=64, tail=64):
    """Compares what the timed step produced with the oracle on a sample.

    outs: CPU float64 arrays of the last timed step: o_bf16, lse_bf16 (the
    headline forward), o32, lse32 (the forward that feeds the backward), dq,
    dk, dv. Compared: O and lse of `rows_per_head` seeded query rows of every
    head (both forwards), dQ at the same rows, and dK, dV of the last `tail`
    keys of every head (which, under the causal mask, only the last `tail`
    query rows reach). Returns the max / RMS errors and whether all are
    within PARITY_TOL.
    """
    import numpy as np

    import oracle
    from io_aware_exact_15_amd import inputs

    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    scale = 1.0 / math.sqrt(d)
    inp = inputs.make_inputs(B, H, N, d, w["seed"], "bf16", with_do=True)
    q, k, v, do = (inputs.to_numpy(inp[n]) for n in ("q", "k", "v", "do"))
    rows = inputs.sample_rows(w["seed"], B, H, N, rows_per_head)
    ro, rl = oracle.forward(q, k, v, scale, w["causal"], rows=rows)
    rdq = oracle.backward_rows(q, k, v, do, scale, w["causal"], rows)
    rdk, rdv = oracle.backward_causal_tail(q, k, v, do, scale, tail)

    def gather(x):
        return np.stack([np.stack([x[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])

    def mx(a, b):
        return float(np.max(np.abs(a - b)))

    res = {"rows_per_head": rows_per_head, "tail_keys": tail}
    o_err = np.concatenate([(gather(outs["o_bf16"]) - ro).ravel(), (gather(outs["o32"]) - ro).ravel()])
    res["o_max"] = float(np.max(np.abs(o_err)))
    res["o_rms"] = float(np.sqrt(np.mean(o_err ** 2)))
    res["lse_max"] = max(mx(gather(outs["lse_bf16"]), rl), mx(gather(outs["lse32"]), rl))
    res["dq_max"] = mx(gather(outs["dq"]), rdq)
    res["dk_max"] = mx(outs["dk"][:, :, N - tail:], rdk)
    res["dv_max"] = mx(outs["dv"][:, :, N - tail:], rdv)
    res["ok"] = all(res[key] <= tol for key, tol in PARITY_TOL.items())
    return res


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
        if dtype in ("fp8", "fp8e5m2"):
            oracle.forward_quantized(arr["q"], arr["k"], arr["v"], inp["sq"], inp["sk"], inp["sv"], scale, causal, rows,
                                     fmt="e4m3" if dtype == "fp8" else "e5m2")
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


# Forward traffic against sequence length: causal bf16 forward, d = 128, the
# same 524288 query rows (and so the same algorithmic bytes) at every N.
SWEEP_NS = (2048, 4096, 8192, 16384, 32768, 65536)


def sweep_table():
    return {f"fwd_sweep_bf16_causal_b1h{524288 // n}_n{n}_d128": (
        "std", dict(B=1, H=524288 // n, Hkv=524288 // n, N=n, d=128, seed=70 + i, dtype="bf16", causal=[True],
                    backward=False)) for i, n in enumerate(SWEEP_NS)}


def workload_table(sweep=False):
    """name -> (kind, workload) for every workload of the path except the
    headline step: "std" (forward, plus backward where it has one), "fp8bwd"
    (FP8 backward), "decode" and "ws" (the wave-specialised forward); with
    `sweep`, the forward traffic sweep instead."""
    from io_aware_exact_15_amd import inputs

    if sweep:
        return sweep_table()

    t = {n: ("std", dict(w, Hkv=w["H"])) for n, w in inputs.WORKLOADS.items()}
    t.update((n, ("std", dict(w, Hkv=w["H"]))) for n, w in inputs.FP8_E5M2_WORKLOADS.items())
    t.update((n, ("std", w)) for n, w in inputs.GQA_WORKLOADS.items())
    t.update((n, ("fp8bwd", w)) for n, w in inputs.FP8_BWD_WORKLOADS.items())
    t.update((n, ("decode", w)) for n, w in inputs.DECODE_WORKLOADS.items())
    # The wave-specialised forward (fa_forward_ws) on the bf16 forward workloads.
    for n in ("fwd_bf16_causal_b1h32_n16384_d128", "fwd_bf16_b4h16_n2048_d64"):
        t["ws_" + n] = ("ws", dict(inputs.WORKLOADS[n], Hkv=inputs.WORKLOADS[n]["H"]))
    return t


def workload_calls(name, kind, w, dev):
    """Device inputs of one workload and its calls, in order: a list of dicts
    with pass, causal, fn (one enqueued call), setup (what must run before fn,
    or None), the algorithmic flop (or bytes for decode) and the peak."""
    import torch

    from io_aware_exact_15_amd import binding as fa
    from io_aware_exact_15_amd import inputs

    calls = []
    B, H, Hkv, d = w["B"], w["H"], w["Hkv"], w["d"]
    scale = 1.0 / math.sqrt(d)
    if kind == "decode":
        Nq, Nk = w["Nq"], w["Nk"]
        inp = inputs.make_inputs_heads(B, H, Hkv, Nq, Nk, d, w["seed"], "bf16")
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), dtype=torch.uint8, device=dev)
        nbytes = 2 * B * Hkv * Nk * d * 2 + 2 * B * H * Nq * d * 2 + B * H * Nq * 4
        calls.append(dict(pass_="decode", causal=w["causal"], setup=None, bytes=nbytes,
                          fn=lambda: fa.fa_decode(q, k, v, o, fa.FA_BF16, lse, ws, scale, w["causal"])))
        return inp, calls
    N = w["N"]
    if kind == "fp8bwd":
        inp = inputs.make_inputs(B, H, N, d, w["seed"], "fp8bwd", with_do=True)
        codes = {n: inp[n].to(dev) for n in ("q", "k", "v", "do")}
        deq = {n: (inp[n].to(torch.float32) * float(inp["s" + n])).to(dev) for n in ("q", "k", "v")}
        desc = torch.tensor([inp["sq"], inp["sk"], inp["sv"], inp["sdo"]], dtype=torch.float32, device=dev)
        o = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        dq = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
        dk, dv = (torch.empty(B, Hkv, N, d, dtype=torch.float32, device=dev) for _ in range(2))
        ws = torch.empty(fa.fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device=dev)
        for causal in w["causal"]:
            # the forward that feeds it runs in float32 on the dequantised values (untimed)
            setup = (lambda c=causal: fa.fa_forward_gqa(fa.FA_F32, fa.FA_F32, deq["q"], deq["k"], deq["v"], None,
                                                        o, lse, scale, c))
            calls.append(dict(pass_="bwd", causal=causal, setup=setup, flop=_flops(B, H, N, d, causal, "bwd"),
                              peak=PEAK_BF16_TFLOPS, dtype="fp8 e4m3 / e5m2 dO", note="fp16 matrix-core operands",
                              fn=(lambda c=causal: fa.fa_backward_typed(
                                  fa.FA_FP8_E4M3, fa.FA_FP8_E5M2, codes["q"], codes["k"], codes["v"], codes["do"],
                                  desc, o, fa.FA_F32, lse, dq, dk, dv, ws, scale, c))))
        return inp, calls
    inp = inputs.make_inputs_heads(B, H, Hkv, N, N, d, w["seed"], w["dtype"], with_do=w["backward"])
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    if kind == "ws":
        o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
        for causal in w["causal"]:
            calls.append(dict(pass_="fwd", causal=causal, setup=None, peak=PEAK_BF16_TFLOPS, dtype="bf16",
                              flop=_flops(B, H, N, d, causal, "fwd"), note="wave-specialised schedule (fa_forward_ws)",
                              fn=(lambda c=causal: fa.fa_forward_ws(fa.FA_BF16, q, k, v, o, lse, scale, c))))
        return inp, calls
    desc = None
    if w["dtype"] in ("fp8", "fp8e5m2"):
        in_t = fa.FA_FP8_E4M3 if w["dtype"] == "fp8" else fa.FA_FP8_E5M2
        o_t, peak, odt = fa.FA_BF16, PEAK_FP8_TFLOPS, torch.bfloat16
        desc = torch.tensor([inp["sq"], inp["sk"], inp["sv"]], dtype=torch.float32, device=dev)
    elif w["dtype"] == "f32":
        in_t, o_t, peak, odt = fa.FA_F32, fa.FA_F32, PEAK_F32_MFMA_TFLOPS, torch.float32
    else:
        in_t, o_t, peak, odt = fa.FA_BF16, fa.FA_BF16, PEAK_BF16_TFLOPS, torch.bfloat16
    if w["backward"]:
        o_t, odt = fa.FA_F32, torch.float32  # the forward that feeds the backward writes float32 O
    o = torch.empty(B, H, N, d, dtype=odt, device=dev)
    if w["backward"]:
        do = inp["do"].to(dev)
        dq = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
        dk, dv = (torch.empty(B, Hkv, N, d, dtype=torch.float32, device=dev) for _ in range(2))
        ws = torch.empty(fa.fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device=dev)
    for causal in w["causal"]:
        fwd = (lambda c=causal: fa.fa_forward_gqa(in_t, o_t, q, k, v, desc, o, lse, scale, c))
        calls.append(dict(pass_="fwd", causal=causal, setup=None, fn=fwd, peak=peak,
                          flop=_flops(B, H, N, d, causal, "fwd"), dtype=w["dtype"]))
        if w["backward"]:
            calls.append(dict(pass_="bwd", causal=causal, setup=fwd, peak=peak, dtype=w["dtype"],
                              flop=_flops(B, H, N, d, causal, "bwd"),
                              fn=(lambda c=causal: fa.fa_backward_gqa(q, k, v, o, fa.FA_F32, do, lse, dq, dk, dv,
                                                                      ws, scale, c))))
    return inp, calls


def run_configs(iters=20, warmup=3, with_cpu=True, only=None, sweep=False):
    """Times every workload of the path (one JSON line per workload and pass)."""
    import torch

    dev = torch.device("cuda:0")
    for name, (kind, w) in workload_table(sweep).items():
        if only and name not in only:
            continue
        inp, calls = workload_calls(name, kind, w, dev)
        fwd_ms = {}
        for c in calls:
            if c["setup"] is not None:
                c["setup"]()
            med, mn = _median_ms(torch, c["fn"], iters, warmup)
            line = {"workload": name, "pass": c["pass_"], "causal": c["causal"], "dtype": c.get("dtype", "bf16"),
                    "ms_median": med, "ms_min": mn}
            if "bytes" in c:
                gbs = c["bytes"] / (med * 1e-3) / 1e9
                line.update(algorithmic_bytes=c["bytes"], GB_per_s=gbs, frac_of_hbm_peak=gbs / PEAK_HBM_GBS)
            else:
                tf = c["flop"] / (med * 1e-3) / 1e12
                line.update(tflops=tf, frac_of_peak=tf / c["peak"], peak_tflops=c["peak"])
            if "note" in c:
                line["note"] = c["note"]
            if with_cpu:
                line["cpu_baseline"] = cpu_baseline_sample(c["pass_"], w, inp, c["causal"])
            print(json.dumps(line), flush=True)
            if c["pass_"] == "fwd":
                fwd_ms[c["causal"]] = (med, c["flop"])
            elif kind == "std" and c["pass_"] == "bwd":
                fm, ff = fwd_ms[c["causal"]]
                tot = (ff + c["flop"]) / ((fm + med) * 1e-3) / 1e12
                print(json.dumps({"workload": name, "pass": "fwd+bwd", "causal": c["causal"], "dtype": w["dtype"],
                                  "ms_median": fm + med, "tflops": tot, "frac_of_peak": tot / c["peak"]}), flush=True)


def run_counters(only, sweep=False):
    """Untimed, for hardware-counter runs: one float32 copy-kernel launch of
    known size (512 MiB read + 512 MiB written, the traffic calibration),
    then one call of every pass of the named workloads (the headline step
    when `only` is empty; every sweep point with `sweep`)."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)  # copy kernel: reads 512 MiB, writes 512 MiB
    torch.cuda.synchronize()
    del src, dst
    table = workload_table(sweep)
    if sweep and not only:
        only = list(table)
    if not only:
        return False
    for name in only:
        if name not in table:
            raise SystemExit(f"unknown workload {name}; known: {', '.join(table)}")
        kind, w = table[name]
        _, calls = workload_calls(name, kind, w, dev)
        for c in calls:
            if c["setup"] is not None:
                c["setup"]()
            c["fn"]()
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": name, "calls": [c["pass_"] for c in calls]}), flush=True)
    return True


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle leg (its timing and the parity check of what was timed)")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload (fwd, and bwd where it has one); one JSON line each")
    ap.add_argument("--only", action="append", default=[],
                    help="with --configs or --counters: only this workload (repeatable)")
    ap.add_argument("--sweep", action="store_true",
                    help="with --configs or --counters: the forward traffic sweep (causal bf16, d=128, "
                         "N = 2048 ... 65536, 524288 query rows each) instead of the workloads")
    ap.add_argument("--counters", action="store_true",
                    help="untimed: one float32 copy-kernel launch of known size (512 MiB read + 512 MiB written, "
                         "the traffic calibration) and one step (or one call of each pass of the --only "
                         "workloads), for hardware-counter runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build runs on a single "
              "MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.configs:
        run_configs(with_cpu=not args.no_cpu, only=args.only, sweep=args.sweep)
        return
    if args.counters and run_counters(args.only, args.sweep):
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
    dq, dk, dv = (torch.empty(B, H, N, d, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev):
        # headline forward: bf16 O
        ev[0].record()
        fa.fa_forward_typed(fa.FA_BF16, fa.FA_BF16, q, k, v, None, o_bf, lse_bf, scale, causal)
        ev[1].record()
        # the forward that feeds the backward (float32 O), then the backward
        fa.fa_forward_typed(fa.FA_BF16, fa.FA_F32, q, k, v, None, o, lse, scale, causal)
        ev[2].record()
        fa.fa_backward(q, k, v, o, fa.FA_F32, do, lse, dq, dk, dv, ws, scale, causal)
        ev[3].record()

    if args.counters:  # the calibration copy ran in run_counters; one untimed step
        step([torch.cuda.Event(enable_timing=True) for _ in range(4)])
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "copy_bytes_each_way": 512 << 20}), flush=True)
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
    fwd32_ms = [e[1].elapsed_time(e[2]) for e in evs]
    bwd_ms = [e[2].elapsed_time(e[3]) for e in evs]
    bwd_med = sorted(bwd_ms)[len(bwd_ms) // 2]
    bwd_mean = sum(bwd_ms) / len(bwd_ms)
    bwd_f = _flops(B, H, N, d, causal, "bwd")
    res_bwd = {"ms_median": bwd_med, "ms_mean": bwd_mean, "ms_min": min(bwd_ms),
               "tflops": bwd_f / (bwd_med * 1e-3) / 1e12}
    fb_ms = sorted(a + b for a, b in zip(fwd32_ms, bwd_ms))[len(bwd_ms) // 2]
    res_fb = {"ms_median": fb_ms, "tflops": (fwd_f + bwd_f) / (fb_ms * 1e-3) / 1e12}
    roofline = roof_fwd
    if bwd_mean > fwd_mean:  # the backward pass dominates the step
        roofline = _roofline("fa_backward (bwd_prep + bwd_dkdv + bwd_dq)", "bwd", bwd_f, bwd_mean)
    ms_per_step = wall / args.steps * 1e3

    out = {
        "metric": "attention TFLOP/s (fwd, fwd+bwd) and % of MFMA peak, causal bf16 N=16K d=128",
        "value": res_fb["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "B": B, "H": H, "N": N, "d": d, "causal": causal, "scale": scale,
                   "value_is": "fwd+bwd TFLOP/s (fwd with fp32 O, then bwd)"},
        "fwd": res_fwd,
        "bwd": res_bwd,
        "fwd_bwd": res_fb,
        "roofline": roofline,
        "roofline_fwd": roof_fwd,
        "step_flops": fwd_f + fwd_f + bwd_f,
    }
    ok = True
    if not args.no_cpu:
        # The oracle leg, after the timed region: what the last timed step
        # produced is checked against the oracle on a sample, then the oracle
        # itself is timed.
        outs = {"o_bf16": o_bf, "lse_bf16": lse_bf, "o32": o, "lse32": lse, "dq": dq, "dk": dk, "dv": dv}
        outs = {n: t.cpu().to(torch.float64).numpy() for n, t in outs.items()}
        out["parity"] = parity_of_step(w, outs)
        ok = out["parity"]["ok"]
        del outs
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    if not ok:
        print(f"bench.py: the timed step's outputs are outside the parity bounds {PARITY_TOL}", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
