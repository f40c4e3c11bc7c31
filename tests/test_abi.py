"""The C-ABI library loads, exports what include/fa.h declares, and rejects
bad arguments before launching anything (no GPU needed for these)."""
import ctypes
import os
import re

import pytest

from io_aware_exact_15_amd import binding as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fa.lib()
    names = _header_functions()
    assert set(names) == set(fa.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_WORKSPACE, fa.FA_ERR_LAUNCH):
        assert fa.fa_status_string(code).startswith("FA_")
    assert fa.fa_status_string(12345) == "unknown fa_status"


def _fwd(**kw):
    a = dict(in_dtype=fa.FA_BF16, o_dtype=fa.FA_BF16, q=16, k=16, v=16, descale=None, o=16, lse=16,
             B=1, H=1, N=8, d=64, scale=0.125, causal=0)
    a.update(kw)
    return fa.lib().fa_forward_typed(a["in_dtype"], a["o_dtype"], a["q"], a["k"], a["v"], a["descale"], a["o"],
                                     a["lse"], a["B"], a["H"], a["N"], a["d"], ctypes.c_float(a["scale"]),
                                     a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(q=18), fa.FA_ERR_INVALID_ARG),  # misaligned
    (dict(in_dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(o_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),  # descale missing
    (dict(in_dtype=fa.FA_FP8_E4M3, o_dtype=fa.FA_F32, descale=16), fa.FA_ERR_UNSUPPORTED),
    (dict(descale=16), fa.FA_ERR_INVALID_ARG),  # descale given for bf16
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None), fa.FA_OK),  # empty batch: no-op
    (dict(H=0), fa.FA_OK),
    (dict(B=1 << 20, H=1 << 12, N=1 << 12), fa.FA_ERR_INVALID_ARG),  # grid overflow
    (dict(N=1 << 24, d=128), fa.FA_ERR_UNSUPPORTED),  # head larger than a 32-bit buffer range
])
def test_forward_validation(kw, status):
    assert _fwd(**kw) == status


def _bwd(ws_bytes=None, **kw):
    a = dict(q=16, k=16, v=16, o=16, o_dtype=fa.FA_F32, do=16, lse=16, dq=16, dk=16, dv=16, ws=16,
             B=1, H=2, N=40, d=128, scale=0.1, causal=1)
    a.update(kw)
    need = fa.fa_backward_workspace_bytes(a["B"], a["H"], a["N"], a["d"])
    ws_bytes = need if ws_bytes is None else ws_bytes
    return fa.lib().fa_backward(a["q"], a["k"], a["v"], a["o"], a["o_dtype"], a["do"], a["lse"], a["dq"], a["dk"],
                                a["dv"], a["ws"], ws_bytes, a["B"], a["H"], a["N"], a["d"], ctypes.c_float(a["scale"]),
                                a["causal"], None)


CTL = 4096 + 1024 * 4 * 4  # control block, then one 4-float magnitude record per prep workgroup


def test_workspace_size():
    rows = 2 * 16 * 4096
    assert fa.fa_backward_workspace_bytes(2, 16, 4096, 128) == CTL + 2 * rows * 4 + 4 * rows * 128 * 2
    # each of the six row regions rounds up to 256 bytes
    assert fa.fa_backward_workspace_bytes(1, 1, 3, 64) == CTL + 2 * 256 + 4 * 512
    assert fa.fa_backward_workspace_bytes(0, 1, 3, 64) == 0
    assert fa.fa_backward_workspace_bytes(1, 1, 3, 96) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dq=None), fa.FA_ERR_INVALID_ARG),
    (dict(o_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=8), fa.FA_ERR_WORKSPACE),
    (dict(B=0, q=None), fa.FA_OK),
])
def test_backward_validation(kw, status):
    assert _bwd(**kw) == status


def _fwd_gqa(**kw):
    a = dict(in_dtype=fa.FA_BF16, o_dtype=fa.FA_BF16, q=16, k=16, v=16, descale=None, o=16, lse=16,
             B=1, H=8, Hkv=2, N=8, d=64, scale=0.125, causal=0)
    a.update(kw)
    return fa.lib().fa_forward_gqa(a["in_dtype"], a["o_dtype"], a["q"], a["k"], a["v"], a["descale"], a["o"],
                                   a["lse"], a["B"], a["H"], a["Hkv"], a["N"], a["d"], ctypes.c_float(a["scale"]),
                                   a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=-2), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),   # does not divide H
    (dict(Hkv=16), fa.FA_ERR_INVALID_ARG),  # more key/value heads than query heads
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),  # descale missing
    (dict(H=0, Hkv=1), fa.FA_OK),
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None), fa.FA_OK),
])
def test_forward_gqa_validation(kw, status):
    assert _fwd_gqa(**kw) == status


def _fwd_ws(**kw):
    a = dict(o_dtype=fa.FA_BF16, q=16, k=16, v=16, o=16, lse=16, B=1, H=8, Hkv=2, N=8, d=64, scale=0.125, causal=0)
    a.update(kw)
    return fa.lib().fa_forward_ws(a["o_dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                                  a["N"], a["d"], ctypes.c_float(a["scale"]), a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),   # does not divide H
    (dict(Hkv=16), fa.FA_ERR_INVALID_ARG),  # more key/value heads than query heads
    (dict(o_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(o_dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=24), fa.FA_ERR_INVALID_ARG),  # misaligned
    (dict(H=0, Hkv=1), fa.FA_OK),
    (dict(B=0, q=None, k=None, v=None, o=None, lse=None), fa.FA_OK),
    (dict(N=1 << 24, d=128), fa.FA_ERR_UNSUPPORTED),  # head larger than a 32-bit buffer range
])
def test_forward_ws_validation(kw, status):
    assert _fwd_ws(**kw) == status


def test_gqa_workspace_size():
    q_rows, kv_rows = 2 * 16 * 4096, 2 * 4 * 4096
    assert fa.fa_backward_gqa_workspace_bytes(2, 16, 4, 4096, 128) == \
        CTL + 2 * q_rows * 4 + 2 * q_rows * 128 * 2 + 2 * kv_rows * 128 * 2 + 2 * q_rows * 128 * 4
    assert fa.fa_backward_gqa_workspace_bytes(2, 16, 16, 4096, 128) == fa.fa_backward_workspace_bytes(2, 16, 4096, 128)
    assert fa.fa_backward_gqa_workspace_bytes(1, 6, 4, 64, 64) == 0  # 4 does not divide 6
    assert fa.fa_backward_gqa_workspace_bytes(1, 6, 0, 64, 64) == 0


def _bwd_gqa(ws_bytes=None, **kw):
    a = dict(q=16, k=16, v=16, o=16, o_dtype=fa.FA_F32, do=16, lse=16, dq=16, dk=16, dv=16, ws=16,
             B=1, H=4, Hkv=2, N=40, d=128, scale=0.1, causal=1)
    a.update(kw)
    need = fa.fa_backward_gqa_workspace_bytes(a["B"], a["H"], a["Hkv"], a["N"], a["d"])
    ws_bytes = need if ws_bytes is None else ws_bytes
    return fa.lib().fa_backward_gqa(a["q"], a["k"], a["v"], a["o"], a["o_dtype"], a["do"], a["lse"], a["dq"],
                                    a["dk"], a["dv"], a["ws"], ws_bytes, a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                                    ctypes.c_float(a["scale"]), a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=64), fa.FA_ERR_WORKSPACE),
    (dict(B=0, q=None), fa.FA_OK),
])
def test_backward_gqa_validation(kw, status):
    assert _bwd_gqa(**kw) == status


def _dec(ws_bytes=None, **kw):
    a = dict(q=16, k=16, v=16, o=16, o_dtype=fa.FA_BF16, lse=16, ws=16, B=1, H=8, Hkv=2, Nq=1, Nk=100, d=128,
             scale=0.1, causal=1)
    a.update(kw)
    need = fa.fa_decode_workspace_bytes(a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"])
    ws_bytes = need if ws_bytes is None else ws_bytes
    return fa.lib().fa_decode(a["q"], a["k"], a["v"], a["o"], a["o_dtype"], a["lse"], a["ws"], ws_bytes, a["B"],
                              a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], ctypes.c_float(a["scale"]), a["causal"],
                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=101), fa.FA_ERR_INVALID_ARG),  # more new rows than cache rows
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(o_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(Nk=1 << 24, Nq=1, d=128), fa.FA_ERR_UNSUPPORTED),  # cache head larger than a 32-bit buffer range
    (dict(B=0, q=None), fa.FA_OK),
])
def test_decode_validation(kw, status):
    assert _dec(**kw) == status


def test_decode_workspace_size():
    assert fa.fa_decode_workspace_bytes(1, 8, 2, 1, 100, 128) > 0
    assert fa.fa_decode_workspace_bytes(1, 8, 3, 1, 100, 128) == 0
    assert fa.fa_decode_workspace_bytes(1, 8, 2, 5, 4, 128) == 0


def _bwd_typed(**kw):
    a = dict(in_dtype=fa.FA_FP8_E4M3, do_dtype=fa.FA_FP8_E5M2, q=16, k=16, v=16, do=16, desc=16, o=16,
             o_dtype=fa.FA_F32, lse=16, dq=16, dk=16, dv=16, ws=16, B=1, H=4, Hkv=2, N=40, d=128, scale=0.1,
             causal=1)
    a.update(kw)
    need = fa.fa_backward_gqa_workspace_bytes(a["B"], a["H"], a["Hkv"], a["N"], a["d"])
    return fa.lib().fa_backward_typed(a["in_dtype"], a["do_dtype"], a["q"], a["k"], a["v"], a["do"], a["desc"],
                                      a["o"], a["o_dtype"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                                      kw.get("ws_bytes", need), a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                                      ctypes.c_float(a["scale"]), a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(desc=None), fa.FA_ERR_INVALID_ARG),                       # FP8 needs the scales
    (dict(in_dtype=fa.FA_BF16, do_dtype=fa.FA_BF16), fa.FA_ERR_INVALID_ARG),  # bf16 must not pass scales
    (dict(do_dtype=fa.FA_BF16), fa.FA_ERR_UNSUPPORTED),             # mixed bf16 / FP8
    (dict(in_dtype=fa.FA_F32), fa.FA_ERR_INVALID_ARG),
    (dict(do_dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=8), fa.FA_ERR_WORKSPACE),
    (dict(B=0, q=None), fa.FA_OK),
])
def test_backward_typed_validation(kw, status):
    assert _bwd_typed(**kw) == status


@pytest.mark.gpu
def test_caller_stale_hip_error_is_not_reported_or_consumed():
    """An error left by the caller's own earlier HIP call (a refused
    oversized allocation, which launches nothing) must not come back as a
    launch error of a valid call: each launch reports its own status."""
    import torch

    dev = torch.device("cuda:0")
    B, H, N, d = 1, 2, 130, 64
    q, k, v = (torch.randn(B, H, N, d, device=dev).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(B, H, N, d, dtype=torch.float32, device=dev) for _ in range(3))
    o32 = torch.empty(B, H, N, d, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
    hip = ctypes.CDLL(path)  # the runtime this process already uses
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipMalloc.restype = ctypes.c_int
    hip.hipGetLastError.restype = ctypes.c_int
    ptr = ctypes.c_void_p()
    refused = hip.hipMalloc(ctypes.byref(ptr), ctypes.c_size_t(1 << 62))
    assert refused != 0
    try:
        # no torch work between the refused call and these: torch checks the
        # thread's last error after its own launches
        fa.fa_forward(q, k, v, o, lse, 1 / 8, True)
        fa.fa_forward_typed(fa.FA_BF16, fa.FA_F32, q, k, v, None, o32, lse, 1 / 8, True)
        fa.fa_backward(q, k, v, o32, fa.FA_F32, q, lse, dq, dk, dv, ws, 1 / 8, True)
    finally:
        left = hip.hipGetLastError()  # clears the caller's error before torch runs again
    assert left == refused
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(o.float()).all()


def test_decode_noalloc_validation_and_size_limit():
    """Arguments are checked as for fa_decode; a problem whose partials
    exceed the static buffer is refused with FA_ERR_TOO_LARGE before any
    device work (so this runs without a GPU)."""
    L = fa.lib()

    def call(B=1, H=8, Hkv=2, Nq=1, Nk=1000, d=128, o_dtype=fa.FA_BF16, q=16):
        return L.fa_decode_noalloc(q, 16, 16, 16, o_dtype, 16, B, H, Hkv, Nq, Nk, d, ctypes.c_float(0.1), 1, None)

    assert call(Nq=0) == fa.FA_ERR_INVALID_ARG
    assert call(Nk=0) == fa.FA_ERR_INVALID_ARG
    assert call(Hkv=3) == fa.FA_ERR_INVALID_ARG
    assert call(d=96) == fa.FA_ERR_UNSUPPORTED
    assert call(q=None) == fa.FA_ERR_INVALID_ARG
    assert call(B=0) == fa.FA_OK
    big = dict(B=64, H=64, Hkv=64, Nq=1, Nk=128, d=128)
    assert fa.fa_decode_workspace_bytes(*(big[x] for x in ("B", "H", "Hkv", "Nq", "Nk", "d"))) > \
        fa.FA_DECODE_NOALLOC_MAX_WORKSPACE
    assert call(**big) == fa.FA_ERR_TOO_LARGE
    assert "FA_ERR_TOO_LARGE" in fa.fa_status_string(fa.FA_ERR_TOO_LARGE)
    h = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_DECODE_NOALLOC_MAX_WORKSPACE \(\(size_t\)\((\d+)u << (\d+)\) \+ \(size_t\)\((\d+)u << (\d+)\)\)", h)
    assert m and (int(m[1]) << int(m[2])) + (int(m[3]) << int(m[4])) == fa.FA_DECODE_NOALLOC_MAX_WORKSPACE
