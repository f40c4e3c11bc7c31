// C ABI of the attention library: argument validation, then dispatch to the
// kernel launchers. No allocation and no exceptions across the ABI; the only
// state is fa_decode_noalloc's per-device scratch address (fa_decode.hip).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks. Returns FA_OK, or the status to report.
int check_shape(int B, int H, int N, int d, float scale) {
  if (B < 0 || H < 0 || N < 1) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // grid = B*H*ceil(N/32) must fit in an int; element offsets use size_t.
  const long long bh = (long long)B * H;
  if (bh > 0 && bh * ((N + 31) / 32) > INT_MAX) return FA_ERR_INVALID_ARG;
  // One head of K or V must be addressable by a 32-bit buffer offset.
  if ((long long)N * d * 4 > 0xffffffffLL) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head size or dtype not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: the problem needs more scratch than the library's static buffer holds "
             "(FA_DECODE_NOALLOC_MAX_WORKSPACE bytes); use fa_decode with a workspace";
    default: return "unknown fa_status";
  }
}

int fa_forward_gqa(int in_dtype, int o_dtype, const void* q, const void* k, const void* v, const float* descale,
                   void* o, float* lse, int B, int H, int Hkv, int N, int d, float scale, int causal,
                   void* stream) {
  int st = check_shape(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (Hkv < 1 || (H > 0 && (Hkv > H || H % Hkv != 0))) return FA_ERR_INVALID_ARG;
  if (in_dtype != FA_F32 && in_dtype != FA_BF16 && in_dtype != FA_FP8_E4M3 && in_dtype != FA_FP8_E5M2)
    return FA_ERR_INVALID_ARG;
  if (o_dtype != FA_F32 && o_dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (in_dtype == FA_FP8_E4M3 || in_dtype == FA_FP8_E5M2) {
    if (o_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!descale) return FA_ERR_INVALID_ARG;
  } else if (descale) {
    return FA_ERR_INVALID_ARG;
  }
  if ((long long)B * H == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_INVALID_ARG;
  return fa::launch_forward(in_dtype, o_dtype, q, k, v, descale, o, lse, B, H, Hkv, N, d, scale, causal,
                            (hipStream_t)stream);
}

int fa_forward_ws(int o_dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Hkv, int N, int d, float scale, int causal, void* stream) {
  int st = check_shape(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (Hkv < 1 || (H > 0 && (Hkv > H || H % Hkv != 0))) return FA_ERR_INVALID_ARG;
  if (o_dtype != FA_F32 && o_dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if ((long long)B * H == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_INVALID_ARG;
  return fa::launch_forward_ws(o_dtype, q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, (hipStream_t)stream);
}

int fa_forward_typed(int in_dtype, int o_dtype, const void* q, const void* k, const void* v,
                     const float* descale, void* o, float* lse, int B, int H, int N, int d,
                     float scale, int causal, void* stream) {
  return fa_forward_gqa(in_dtype, o_dtype, q, k, v, descale, o, lse, B, H, H > 0 ? H : 1, N, d, scale, causal,
                        stream);
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
               int d, float scale, int causal, void* stream) {
  return fa_forward_typed(FA_BF16, FA_BF16, q, k, v, nullptr, o, lse, B, H, N, d, scale, causal, stream);
}

size_t fa_backward_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return 0;
  return fa::backward_workspace_bytes((size_t)B * H * N, (size_t)B * Hkv * N, d);
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  return fa_backward_gqa_workspace_bytes(B, H, H, N, d);
}

int fa_backward_typed(int in_dtype, int do_dtype, const void* q, const void* k, const void* v, const void* dO,
                      const float* descale, const void* o, int o_dtype, const float* lse, float* dq, float* dk,
                      float* dv, void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N, int d,
                      float scale, int causal, void* stream) {
  int st = check_shape(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (Hkv < 1 || (H > 0 && (Hkv > H || H % Hkv != 0))) return FA_ERR_INVALID_ARG;
  if (o_dtype != FA_F32 && o_dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  auto fmt = [](int t) { return t == FA_BF16 ? 0 : t == FA_FP8_E4M3 ? 1 : t == FA_FP8_E5M2 ? 2 : -1; };
  const int fin = fmt(in_dtype), fdo = fmt(do_dtype);
  if (fin < 0 || fdo < 0) return FA_ERR_INVALID_ARG;
  if ((fin == 0) != (fdo == 0)) return FA_ERR_UNSUPPORTED;  // both bf16 or both FP8
  if ((fin != 0) != (descale != nullptr)) return FA_ERR_INVALID_ARG;
  if ((long long)B * H == 0) return FA_OK;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(lse) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_backward_gqa_workspace_bytes(B, H, Hkv, N, d) || !aligned16(workspace))
    return FA_ERR_WORKSPACE;
  return fa::launch_backward(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, B, H, Hkv, N, d, scale, causal,
                             fin, fdo, descale, (hipStream_t)stream);
}

int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                    const float* lse, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                    int B, int H, int Hkv, int N, int d, float scale, int causal, void* stream) {
  return fa_backward_typed(FA_BF16, FA_BF16, q, k, v, dO, nullptr, o, o_dtype, lse, dq, dk, dv, workspace,
                           workspace_bytes, B, H, Hkv, N, d, scale, causal, stream);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                const float* lse, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                int B, int H, int N, int d, float scale, int causal, void* stream) {
  return fa_backward_gqa(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, workspace_bytes, B, H,
                         H > 0 ? H : 1, N, d, scale, causal, stream);
}

size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk < Nq || (d != 64 && d != 128)) return 0;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return 0;
  return fa::decode_workspace_bytes(B, H, Hkv, Nq, Nk, d);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points (workspace aside).
int check_decode(const void* q, const void* k, const void* v, const void* o, int o_dtype, const float* lse, int B,
                 int H, int Hkv, int Nq, int Nk, int d, float scale) {
  if (B < 0 || H < 0 || Nq < 1 || Nk < Nq) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (Hkv < 1 || (H > 0 && (Hkv > H || H % Hkv != 0))) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (o_dtype != FA_F32 && o_dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  // One head of K or V must be addressable by a 32-bit buffer offset; the
  // grid (at most one workgroup per 128 keys per row tile) must fit an int.
  if ((long long)Nk * d * 2 > 0xffffffffLL) return FA_ERR_UNSUPPORTED;
  const long long R = (long long)(H > 0 ? H / Hkv : 0) * Nq;
  if ((long long)B * Hkv * ((R + 31) / 32) * ((Nk + 127) / 128) > INT_MAX) return FA_ERR_INVALID_ARG;
  if ((long long)B * H == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, void* workspace,
              size_t workspace_bytes, int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
              void* stream) {
  const int st = check_decode(q, k, v, o, o_dtype, lse, B, H, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK || (long long)B * H == 0) return st;
  if (!workspace || workspace_bytes < fa_decode_workspace_bytes(B, H, Hkv, Nq, Nk, d) || !aligned16(workspace))
    return FA_ERR_WORKSPACE;
  return fa::launch_decode(q, k, v, o, o_dtype, lse, workspace, B, H, Hkv, Nq, Nk, d, scale, causal,
                           (hipStream_t)stream);
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, int B, int H,
                      int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  const int st = check_decode(q, k, v, o, o_dtype, lse, B, H, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK || (long long)B * H == 0) return st;
  return fa::launch_decode_noalloc(q, k, v, o, o_dtype, lse, B, H, Hkv, Nq, Nk, d, scale, causal,
                                   (hipStream_t)stream);
}

}  // extern "C"
