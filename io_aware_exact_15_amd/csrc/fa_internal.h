// Internal entry points between the C ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Forward launch; arguments already validated by the ABI layer. H query
// heads share Hkv key/value heads (H % Hkv == 0; query head h reads key/value
// head h / (H / Hkv)).
int launch_forward(int in_dtype, int o_dtype, const void* q, const void* k, const void* v,
                   const float* descale, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                   float scale, int causal, hipStream_t stream);

// FP8 forward launch (descale: device pointer to {s_q, s_k, s_v}); inputs
// E4M3 (e5m2 = 0) or E5M2 (e5m2 = 1); G = query heads per key/value head.
hipError_t launch_forward_fp8(const void* q, const void* k, const void* v, const float* descale, void* o, float* lse,
                              int BH, int G, int N, int d, float scale, int causal, int e5m2, hipStream_t stream);

// Backward launch; arguments already validated by the ABI layer. `workspace`
// holds at least backward_workspace_bytes(B*H*N, B*Hkv*N, d) bytes.
// in_fmt / do_fmt: element format of Q, K, V / of dO: 0 = bf16, 1 = FP8
// E4M3, 2 = FP8 E5M2 (both 0 or both FP8); desc = device {s_q, s_k, s_v,
// s_dO} for FP8, unused for bf16.
int launch_backward(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                    const void* dO, const float* lse, float* dq, float* dk, float* dv,
                    void* workspace, int B, int H, int Hkv, int N, int d, float scale, int causal,
                    int in_fmt, int do_fmt, const float* desc, hipStream_t stream);

// Backward workspace: D and -lse*log2(e) (float32 per query row), fp16
// copies of Q and dO (per query row) and of K and V (per key/value row),
// each region 256-byte aligned.
size_t backward_workspace_bytes(size_t q_rows, size_t kv_rows, int d);

// Decode (split-K) launch; arguments already validated. q [B,H,Nq,d],
// k, v [B,Hkv,Nk,d]; workspace >= decode_workspace_bytes(...).
int launch_decode(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, void* workspace,
                  int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream);

// Decode workspace: per split and wave, the unnormalised partial output
// (32 x d float32) and its running max and denominator (2 x 32 float32).
size_t decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d);

}  // namespace fa
