// Internal entry points between the C ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <tuple>
#include <utility>

namespace fa {

// Enqueues kernel<<<grid, block, 0, stream>>>(args...) through hipLaunchKernel
// and returns the runtime's status for this launch alone. The calling
// thread's last-error state is neither read nor cleared, so an error left by
// the caller's own earlier HIP calls is not reported (or consumed) here.
template <typename... P, size_t... I>
hipError_t launch_kernel_impl(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                              std::index_sequence<I...>, std::tuple<P...>& args) {
  void* argv[] = {static_cast<void*>(&std::get<I>(args))..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> conv(std::forward<A>(args)...);
  return launch_kernel_impl(kernel, grid, block, stream, std::index_sequence_for<P...>{}, conv);
}

// Compute units of the current device (0 if the runtime cannot say).
int device_cu_count();

// Forward launch; arguments already validated by the ABI layer. H query
// heads share Hkv key/value heads (H % Hkv == 0; query head h reads key/value
// head h / (H / Hkv)).
int launch_forward(int in_dtype, int o_dtype, const void* q, const void* k, const void* v,
                   const float* descale, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                   float scale, int causal, hipStream_t stream);

// Wave-specialised bf16 forward (fa_fwd_ws.hip); arguments already validated.
int launch_forward_ws(int o_dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int Hkv, int N, int d, float scale, int causal, hipStream_t stream);

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

// dQ kernel of the backward pass (fa_bwd_dq.hip), after the dK/dV kernel
// has chosen the copies' exponents; `grid` persistent workgroups.
hipError_t launch_bwd_dq(int d, int causal, void* workspace, const float* desc, int fin, int fdo, float* dq, int BH,
                         int G, int N, float c, float scale, int grid, hipStream_t st);

// Backward workspace: D and -lse*log2(e) (float32 per query row), fp16
// copies of Q and dO (per query row) and of K and V (per key/value row),
// each region 256-byte aligned.
size_t backward_workspace_bytes(size_t q_rows, size_t kv_rows, int d);

// Decode (split-K) launch; arguments already validated. q [B,H,Nq,d],
// k, v [B,Hkv,Nk,d]; workspace >= decode_workspace_bytes(...).
int launch_decode(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, void* workspace,
                  int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream);

// Decode with the library's static scratch array instead of a caller
// workspace (FA_ERR_TOO_LARGE when the partials do not fit in it).
int launch_decode_noalloc(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, int B, int H,
                          int Hkv, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream);

// Decode workspace: per split and wave, the unnormalised partial output
// (32 x d float32) and its running max and denominator (2 x 32 float32).
size_t decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d);

}  // namespace fa
