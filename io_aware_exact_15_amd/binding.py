"""Thin ctypes binding of libfa.so: same entry points as include/fa.h.

Argument marshalling only: tensors become device pointers and sizes, the
stream becomes the current torch stream's handle. Every arithmetic step runs
inside the HIP library; if it is missing this module raises instead of
computing anything another way.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_LAUNCH = -4
FA_ERR_TOO_LARGE = -5

FA_DECODE_NOALLOC_MAX_WORKSPACE = (16 << 20) + (256 << 10)  # include/fa.h

FA_F32 = 0
FA_BF16 = 1
FA_FP8_E4M3 = 3
FA_FP8_E5M2 = 4

_TORCH_DTYPE = {FA_F32: torch.float32, FA_BF16: torch.bfloat16, FA_FP8_E4M3: torch.float8_e4m3fn,
                FA_FP8_E5M2: torch.float8_e5m2}

EXPORTS = ("fa_forward", "fa_forward_typed", "fa_backward", "fa_backward_workspace_bytes", "fa_forward_gqa",
           "fa_backward_gqa_workspace_bytes", "fa_backward_gqa", "fa_backward_typed", "fa_decode_workspace_bytes",
           "fa_decode", "fa_decode_noalloc", "fa_forward_ws",
           "fa_status_string")


class FAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lib().fa_status_string(status).decode()} ({status})")


def lib():
    """Loads libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m io_aware_exact_15_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        L.fa_forward.restype = i
        L.fa_forward_typed.argtypes = [i, i, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        L.fa_forward_typed.restype = i
        L.fa_backward.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, vp]
        L.fa_backward.restype = i
        L.fa_backward_workspace_bytes.argtypes = [i, i, i, i]
        L.fa_backward_workspace_bytes.restype = sz
        L.fa_forward_gqa.argtypes = [i, i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.fa_forward_gqa.restype = i
        L.fa_backward_gqa.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, vp]
        L.fa_backward_gqa.restype = i
        L.fa_backward_gqa_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_backward_gqa_workspace_bytes.restype = sz
        L.fa_backward_typed.argtypes = [i, i, vp, vp, vp, vp, vp, vp, i, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i,
                                        vp]
        L.fa_backward_typed.restype = i
        L.fa_decode.argtypes = [vp, vp, vp, vp, i, vp, vp, sz, i, i, i, i, i, i, f, i, vp]
        L.fa_decode.restype = i
        L.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, i, vp, i, i, i, i, i, i, f, i, vp]
        L.fa_decode_noalloc.restype = i
        L.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.fa_decode_workspace_bytes.restype = sz
        L.fa_forward_ws.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        L.fa_forward_ws.restype = i
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise TypeError("tensors must be device tensors")
    if not t.is_contiguous():
        raise TypeError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dims(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _check(status, where):
    if status != FA_OK:
        raise FAError(status, where)


def fa_forward(q, k, v, o, lse, scale, causal, stream=None):
    """bf16 forward: o <- softmax(scale q k^T) v, lse <- row log-sum-exp."""
    B, H, N, d = _dims(q)
    _check(lib().fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                            int(bool(causal)), _stream(stream)), "fa_forward")


def fa_forward_typed(in_dtype, o_dtype, q, k, v, descale, o, lse, scale, causal, stream=None):
    """Forward with in_dtype in {FA_F32, FA_BF16, FA_FP8_E4M3, FA_FP8_E5M2}; descale: device float32[3] or None."""
    B, H, N, d = _dims(q)
    _check(lib().fa_forward_typed(int(in_dtype), int(o_dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(descale),
                                  _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
                                  _stream(stream)), "fa_forward_typed")


def fa_backward_workspace_bytes(B, H, N, d):
    return int(lib().fa_backward_workspace_bytes(int(B), int(H), int(N), int(d)))


def fa_backward(q, k, v, o, o_dtype, do, lse, dq, dk, dv, workspace, scale, causal, stream=None):
    """Backward: dq, dk, dv (float32) <- gradients of <O, dO>; workspace: device buffer (uint8)."""
    B, H, N, d = _dims(q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(o_dtype), _ptr(do), _ptr(lse), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(workspace), nbytes, B, H, N, d, float(scale),
                             int(bool(causal)), _stream(stream)), "fa_backward")


def fa_forward_gqa(in_dtype, o_dtype, q, k, v, descale, o, lse, scale, causal, stream=None):
    """Grouped-query forward: q, o [B,H,N,d]; k, v [B,Hkv,N,d] (Hkv divides H)."""
    B, H, N, d = _dims(q)
    Hkv = _dims(k)[1]
    _check(lib().fa_forward_gqa(int(in_dtype), int(o_dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(descale),
                                _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale), int(bool(causal)),
                                _stream(stream)), "fa_forward_gqa")


def fa_forward_ws(o_dtype, q, k, v, o, lse, scale, causal, stream=None):
    """bf16 forward under the wave-specialised schedule: q, o [B,H,N,d]; k, v [B,Hkv,N,d]."""
    B, H, N, d = _dims(q)
    Hkv = _dims(k)[1]
    _check(lib().fa_forward_ws(int(o_dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                               float(scale), int(bool(causal)), _stream(stream)), "fa_forward_ws")


def fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d):
    return int(lib().fa_backward_gqa_workspace_bytes(int(B), int(H), int(Hkv), int(N), int(d)))


def fa_backward_gqa(q, k, v, o, o_dtype, do, lse, dq, dk, dv, workspace, scale, causal, stream=None):
    """Grouped-query backward: dq [B,H,N,d]; dk, dv [B,Hkv,N,d] summed over each head group."""
    B, H, N, d = _dims(q)
    Hkv = _dims(k)[1]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fa_backward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(o_dtype), _ptr(do), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), nbytes, B, H, Hkv, N, d,
                                 float(scale), int(bool(causal)), _stream(stream)), "fa_backward_gqa")


def fa_backward_typed(in_dtype, do_dtype, q, k, v, do, descale, o, o_dtype, lse, dq, dk, dv, workspace, scale, causal,
                      stream=None):
    """Backward with bf16 or FP8 operands (descale: device float32[4] {s_q, s_k, s_v, s_dO} for FP8)."""
    B, H, N, d = _dims(q)
    Hkv = _dims(k)[1]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fa_backward_typed(int(in_dtype), int(do_dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(descale),
                                   _ptr(o), int(o_dtype), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                   nbytes, B, H, Hkv, N, d, float(scale), int(bool(causal)), _stream(stream)),
           "fa_backward_typed")


def fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d):
    return int(lib().fa_decode_workspace_bytes(int(B), int(H), int(Hkv), int(Nq), int(Nk), int(d)))


def fa_decode(q, k, v, o, o_dtype, lse, workspace, scale, causal, stream=None):
    """Decode step: q, o [B,H,Nq,d]; k, v [B,Hkv,Nk,d] cache; lse [B,H,Nq]."""
    B, H, Nq, d = _dims(q)
    Hkv, Nk = _dims(k)[1], _dims(k)[2]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(o_dtype), _ptr(lse), _ptr(workspace), nbytes,
                           B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _stream(stream)), "fa_decode")


def fa_decode_noalloc(q, k, v, o, o_dtype, lse, scale, causal, stream=None):
    """Decode step without a workspace: the partials use the library's static per-GPU buffer."""
    B, H, Nq, d = _dims(q)
    Hkv, Nk = _dims(k)[1], _dims(k)[2]
    _check(lib().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(o_dtype), _ptr(lse), B, H, Hkv, Nq, Nk, d,
                                   float(scale), int(bool(causal)), _stream(stream)), "fa_decode_noalloc")


def fa_status_string(status):
    return lib().fa_status_string(int(status)).decode()
