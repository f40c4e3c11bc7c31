"""A client of libfa.so that does not use torch: device memory and copies go
through the HIP runtime called with ctypes, and plain device pointers go into
the C ABI declared in include/fa.h.

Usage: python abi_plain_client.py LIBFA INPUT.npz OUTPUT.npz
INPUT.npz holds q, k, v, do as bf16 bit patterns (uint16, [B,H,N,d]) and
B, H, N, d, scale, causal. OUTPUT.npz receives o (bf16 bits), lse, dq, dk, dv
(float32) from fa_forward and fa_backward, and the HIP runtime's path.
Run by tests/test_gpu_abi_plain.py in a process of its own.
"""
import ctypes
import sys

import numpy as np

FA_OK, FA_BF16 = 0, 1
H2D, D2H = 1, 2  # hipMemcpyHostToDevice, hipMemcpyDeviceToHost


def main(lib_path, in_path, out_path):
    fa = ctypes.CDLL(lib_path)  # brings in the HIP runtime it was linked against
    hip = ctypes.CDLL("libamdhip64.so.7")
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    hip.hipMalloc.argtypes = [ctypes.POINTER(vp), sz]
    hip.hipMemcpy.argtypes = [vp, vp, sz, i]
    hip.hipFree.argtypes = [vp]
    fa.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    fa.fa_backward_workspace_bytes.argtypes = [i, i, i, i]
    fa.fa_backward_workspace_bytes.restype = sz
    fa.fa_backward.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]

    def check(rc, what):
        if rc != 0:
            raise SystemExit(f"{what} returned {rc}")

    z = np.load(in_path)
    B, H, N, d = (int(z[n]) for n in ("B", "H", "N", "d"))
    scale, causal = float(z["scale"]), int(z["causal"])
    bufs = []

    def dev(nbytes, host=None):
        p = vp()
        check(hip.hipMalloc(ctypes.byref(p), max(int(nbytes), 1)), "hipMalloc")
        bufs.append(p)
        if host is not None:
            h = np.ascontiguousarray(host)
            check(hip.hipMemcpy(p, h.ctypes.data, h.nbytes, H2D), "hipMemcpy H2D")
        return p

    def host(p, dtype, shape):
        h = np.empty(shape, dtype=dtype)
        check(hip.hipMemcpy(h.ctypes.data, p, h.nbytes, D2H), "hipMemcpy D2H")
        return h

    shape, rows = (B, H, N, d), (B, H, N)
    q, k, v, do = (dev(z[n].nbytes, z[n]) for n in ("q", "k", "v", "do"))
    o = dev(B * H * N * d * 2)
    lse = dev(B * H * N * 4)
    check(fa.fa_forward(q, k, v, o, lse, B, H, N, d, scale, causal, None), "fa_forward")
    ws_bytes = fa.fa_backward_workspace_bytes(B, H, N, d)
    ws = dev(ws_bytes)
    dq, dk, dv = (dev(B * H * N * d * 4) for _ in range(3))
    check(fa.fa_backward(q, k, v, o, FA_BF16, do, lse, dq, dk, dv, ws, ws_bytes, B, H, N, d, scale, causal, None),
          "fa_backward")
    out = dict(o=host(o, np.uint16, shape), lse=host(lse, np.float32, rows), dq=host(dq, np.float32, shape),
               dk=host(dk, np.float32, shape), dv=host(dv, np.float32, shape))
    for p in bufs:
        check(hip.hipFree(p), "hipFree")
    if "torch" in sys.modules:
        raise SystemExit("torch was imported")
    maps = open("/proc/self/maps").read().split("\n")
    runtime = sorted({line.split()[-1] for line in maps if "libamdhip64" in line})
    np.savez(out_path, runtime=np.array(runtime), **out)


if __name__ == "__main__":
    main(*sys.argv[1:4])
