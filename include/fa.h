/*
 * fa.h -- C ABI of the exact IO-aware attention library (libfa.so, gfx950).
 *
 * Operation. Exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V
 * per (batch, head), as defined on the page "Walk through what
 * FlashAttention does differently from standard attention ..." (zenaique.com,
 * FlashAttention family short answer), answer paragraph 1, and on the card
 * "FlashAttention Kernel & Online Softmax", definition paragraph. The library
 * computes it tile by tile with an online softmax (running max, running
 * denominator, rescaled output accumulator; same card, definition paragraph;
 * "FlashAttention" explainer by A. Tiwari) so that no N x N matrix is ever
 * written to device memory. The forward pass saves O and one log-sum-exp
 * per row (the pages save the running max m and denominator l; here
 * lse = m + ln l over the scaled scores, natural log). The backward pass
 * recomputes the score blocks from Q, K, V and lse (short-answer page,
 * answer paragraph 2; card, history paragraph).
 *
 * Conventions common to every entry point:
 *   - Tensors are dense, row-major [B, H, N, d] (d fastest), 16-byte
 *     aligned; lse and the backward workspace are [B, H, N] float32.
 *   - All tensor pointers are DEVICE pointers owned by the caller. The
 *     library never allocates or frees device memory and keeps no state
 *     between calls, except for the static scratch buffer of
 *     fa_decode_noalloc (see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and is asynchronous. The return value reports argument
 *     validation and launch errors only; a device fault surfaces at the
 *     caller's next synchronisation.
 *   - Errors. FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED and FA_ERR_WORKSPACE
 *     come from validation, before anything is enqueued: nothing has been
 *     launched and no output has been written. FA_ERR_LAUNCH is the HIP
 *     runtime refusing one of the call's kernel launches (the status that
 *     hipLaunchKernel returned for that launch); kernels of the same call
 *     enqueued before it still run, and the outputs are then unspecified.
 *     An error left by the caller's own earlier HIP calls is neither
 *     reported nor cleared.
 *   - Supported head sizes: d = 64 or d = 128. Any N >= 1 (ragged tails are
 *     masked). B = 0 or H = 0 is a no-op that returns FA_OK.
 *   - causal != 0 applies the lower-triangular mask: key j is visible to
 *     query i iff j <= i.
 *   - No C++ exception crosses this interface.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad enum  */
  FA_ERR_UNSUPPORTED = -2, /* head size or dtype combination not built   */
  FA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  FA_ERR_LAUNCH = -4,      /* the HIP runtime rejected a kernel launch   */
  FA_ERR_TOO_LARGE = -5    /* fa_decode_noalloc: scratch would not fit   */
} fa_status;

typedef enum {
  FA_F32 = 0,      /* IEEE float32                                       */
  FA_BF16 = 1,     /* bfloat16                                           */
  FA_FP8_E4M3 = 3, /* OCP FP8 E4M3 ("fn": finite only, max 448), inputs only */
  FA_FP8_E5M2 = 4  /* OCP FP8 E5M2 (max finite 57344), inputs only          */
} fa_dtype;

/*
 * fa_forward -- bf16 forward.
 *   q, k, v : bf16 [B,H,N,d] inputs.
 *   o       : bf16 [B,H,N,d] output, fully overwritten.
 *   lse     : float32 [B,H,N] output, lse_i = ln sum_j exp(scale * q_i.k_j)
 *             over the visible keys.
 *   scale   : multiplier of Q K^T (1/sqrt(d) for standard attention).
 * Same as fa_forward_typed(FA_BF16, FA_BF16, ..., descale = NULL, ...).
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_forward_typed -- forward with a choice of operand and output dtype.
 *   in_dtype : FA_F32 (float32 operands, P kept float32),
 *              FA_BF16 (bf16 operands, P rounded to bf16 for P.V),
 *              FA_FP8_E4M3 (E4M3 codes; P quantised to E4M3 for P.V; the
 *              FP8 path of the version table on the FlashAttention-family
 *              multiple-choice page),
 *              FA_FP8_E5M2 (E5M2 codes, the other FP8 format the pages name
 *              for that path; P is still quantised to E4M3).
 *   o_dtype  : FA_F32 or FA_BF16 (FA_F32 with an FP8 input is unsupported).
 *   descale  : FP8 inputs only: DEVICE pointer to 3 float32 per-tensor
 *              scales {s_q, s_k, s_v}; the inputs stand for code * s.
 *              Must be NULL for the other dtypes.
 * Accumulation is float32 for every dtype; the softmax runs in float32 and
 * the denominator is summed from the unrounded float32 probabilities.
 */
int fa_forward_typed(int in_dtype, int o_dtype, const void* q, const void* k, const void* v,
                     const float* descale, void* o, float* lse, int B, int H, int N, int d,
                     float scale, int causal, void* stream);

/*
 * fa_backward_workspace_bytes -- device workspace that fa_backward needs:
 * a 4 KiB control block (work-list counters) and 16 KiB of per-workgroup
 * magnitude records, two float32 per row (D_i = sum_t dO_it O_it and
 * -lse_i*log2(e)) and fp16 copies of Q, K, V and dO (the matrix-core
 * operands of the backward pass), each region rounded up to 256 bytes. 0
 * for an empty batch or an unsupported head size.
 */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_backward -- gradients of <O, dO> with respect to Q, K, V.
 *   q, k, v, dO : bf16 [B,H,N,d].
 *   o           : [B,H,N,d] output of the forward pass, dtype o_dtype
 *                 (FA_F32 or FA_BF16; FA_F32 is the accurate choice because
 *                 D = rowsum(dO * O) is formed from it).
 *   lse         : float32 [B,H,N] from the same forward call.
 *   dq, dk, dv  : float32 [B,H,N,d] outputs, fully overwritten.
 *   workspace   : device buffer of at least fa_backward_workspace_bytes();
 *                 its contents on entry are ignored and on return unspecified.
 * The probabilities are recomputed block by block from Q, K and lse; no
 * N x N buffer exists at any time. The matrix-core operands are fp16 copies
 * of q, k, v and dO, each multiplied by a power of two chosen per tensor from
 * its largest magnitude, and dS is formed in the units of the dO and V
 * copies; the powers of two are undone in float32 on dq, dk, dv. So any
 * finite bf16 inputs are supported, gradients of training size (dO near
 * 1e-6 or far below) included: a tensor keeps its values exactly in its copy
 * down to 2^-17 of its largest magnitude, and smaller values with fp16's
 * subnormal resolution relative to that magnitude. The softmax probabilities
 * enter the dV product scaled by 2^15, so they stay in fp16's normal range
 * for any sequence length.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                const void* dO, const float* lse, float* dq, float* dk, float* dv,
                void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                float scale, int causal, void* stream);

/*
 * fa_forward_gqa -- forward with grouped-query heads. The "FlashAttention"
 * explainer (A. Tiwari, lineage paragraph) pairs the method with
 * grouped-query attention: H query heads share Hkv key/value heads, and
 * query head h attends with key/value head h / (H / Hkv) (groups of
 * H / Hkv consecutive query heads). Hkv = H is fa_forward_typed; Hkv = 1 is
 * multi-query attention.
 *   q, o : [B,H,N,d];  k, v : [B,Hkv,N,d];  lse : float32 [B,H,N].
 *   Hkv  : >= 1 and a divisor of H, else FA_ERR_INVALID_ARG.
 * Every other argument, dtype rule and error is that of fa_forward_typed.
 */
int fa_forward_gqa(int in_dtype, int o_dtype, const void* q, const void* k, const void* v,
                   const float* descale, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                   float scale, int causal, void* stream);

/*
 * fa_forward_ws -- the bf16 forward of fa_forward_gqa under a
 * wave-specialised producer/consumer schedule. In each workgroup, four
 * consumer waves run every matrix-core product (S = Q K^T and O += P V),
 * and four producer waves, one beside each consumer on its SIMD, stream the
 * K and V tiles into on-chip memory and turn scores into probabilities,
 * handing them over through LDS. This is the warp-specialisation idea that
 * the card "FlashAttention Kernel & Online Softmax" (history paragraph) and
 * the FlashAttention-family short-answer page (answer paragraph 2) give for
 * FlashAttention-3 on Hopper, re-derived for CDNA4; fa_forward's schedule, in
 * which every wave does both kinds of work, is the faster one on gfx950.
 *   o_dtype : FA_BF16 or FA_F32 output.
 *   q       : bf16 [B,H,N,d]; k, v: bf16 [B,Hkv,N,d], Hkv divides H.
 *   o       : [B,H,N,d] in o_dtype; lse: float32 [B,H,N].
 * Same operation, layouts, sizes and error rules as fa_forward_gqa with
 * in_dtype = FA_BF16 and descale = NULL. Results agree with fa_forward to
 * rounding, not bit for bit: 64-key blocks change where the running max
 * moves and how the denominator's partial sums group.
 */
int fa_forward_ws(int o_dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Hkv, int N, int d, float scale, int causal, void* stream);

/*
 * fa_backward_gqa_workspace_bytes -- workspace of fa_backward_gqa: the 4 KiB
 * control block and 16 KiB of magnitude records (as for fa_backward), two
 * float32 per query row (D and the exponent offset of P), fp16 copies of Q
 * and dO per query row, fp16 copies of K and V per key/value row and, when
 * Hkv < H, float32 per-query-head dK and dV (B*H*N*d each), every region
 * rounded up to 256 bytes. 0 for an empty batch, an unsupported head size or
 * an Hkv that does not divide H.
 */
size_t fa_backward_gqa_workspace_bytes(int B, int H, int Hkv, int N, int d);

/*
 * fa_backward_gqa -- gradients for grouped-query heads (layouts as in
 * fa_forward_gqa). dq : float32 [B,H,N,d]. dk, dv : float32 [B,Hkv,N,d]: a
 * key/value head enters the output of each of the H / Hkv query heads that
 * share it, so its gradient is the sum of what those heads send it. The
 * per-query-head contributions are formed in the workspace and summed in
 * head order (deterministic, no atomics).
 * workspace >= fa_backward_gqa_workspace_bytes(). Every other argument,
 * rule and error is that of fa_backward.
 */
int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                    const void* dO, const float* lse, float* dq, float* dk, float* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N, int d,
                    float scale, int causal, void* stream);

/*
 * fa_backward_typed -- backward with a choice of operand formats: bf16 Q, K,
 * V and dO (as fa_backward_gqa), or FP8 ones: Q, K, V in in_dtype
 * (FA_FP8_E4M3 or FA_FP8_E5M2) and dO in do_dtype (FA_FP8_E5M2, the format
 * with the wider range, is the natural one for a gradient; FA_FP8_E4M3 is
 * accepted). This extends the FP8 path of the version table on the
 * FlashAttention-family multiple-choice page to the backward pass.
 *   descale : FP8 only: DEVICE pointer to 4 float32 per-tensor scales
 *             {s_q, s_k, s_v, s_dO}; the tensors stand for code * s. Must be
 *             NULL for bf16.
 * The FP8 codes become fp16 matrix-core operands times a per-tensor power of
 * two, as bf16 values do in fa_backward (by default 2^-6 for E4M3 and 2^-13
 * for E5M2, which keeps the largest code below 8), and the scales are
 * applied in float32: to the score exponent, to dP, and to dQ, dK, dV.
 * Mixing bf16 and
 * FP8 between the two dtypes returns FA_ERR_UNSUPPORTED. o, lse, dq, dk, dv,
 * the workspace (fa_backward_gqa_workspace_bytes) and every other rule are
 * those of fa_backward_gqa.
 */
int fa_backward_typed(int in_dtype, int do_dtype, const void* q, const void* k, const void* v,
                      const void* dO, const float* descale, const void* o, int o_dtype,
                      const float* lse, float* dq, float* dk, float* dv, void* workspace,
                      size_t workspace_bytes, int B, int H, int Hkv, int N, int d, float scale,
                      int causal, void* stream);

/*
 * fa_decode_workspace_bytes -- workspace of fa_decode: per split of the keys
 * and per wave, an unnormalised 32 x d float32 partial output and its running
 * max and denominator; 0 for invalid sizes (see fa_decode).
 */
size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d);

/*
 * fa_decode -- decode step: Nq new query rows per head against a key/value
 * cache of Nk rows (the decode step named in the prompts of the card
 * "FlashAttention Kernel & Online Softmax"), computed as a split-K forward:
 * each split of the keys keeps its own running max, denominator and output
 * (the online softmax of the card's definition paragraph) and a second
 * kernel merges the splits with the same rescale-and-add.
 *   q     : bf16 [B,H,Nq,d];   k, v : bf16 [B,Hkv,Nk,d] (Hkv divides H; query
 *           head h uses key/value head h / (H / Hkv)).
 *   o     : [B,H,Nq,d], o_dtype FA_BF16 or FA_F32, fully overwritten.
 *   lse   : float32 [B,H,Nq], natural log-sum-exp of the scaled scores.
 *   causal: the query rows are the last Nq positions of the sequence, so row
 *           i sees keys j <= Nk - Nq + i; causal = 0 lets every row see all
 *           Nk keys.
 *   workspace : device buffer of at least fa_decode_workspace_bytes().
 * Requires 1 <= Nq <= Nk (else FA_ERR_INVALID_ARG), d in {64, 128}, and
 * Nk * d * 2 < 2^32 (FA_ERR_UNSUPPORTED otherwise). Other conventions as
 * for the forward pass.
 */
int fa_decode(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
              void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int Nq, int Nk, int d,
              float scale, int causal, void* stream);

/* Bytes of the static scratch buffer behind fa_decode_noalloc. */
#define FA_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)(16u << 20) + (size_t)(256u << 10))

/*
 * fa_decode_noalloc -- fa_decode without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. It allocates nothing: the
 * split partials live in a file-scope device array of the library,
 * FA_DECODE_NOALLOC_MAX_WORKSPACE bytes per GPU, held until the process
 * ends. Arguments, layouts, results and the other errors are those of
 * fa_decode; the caller still passes q, k, v, o and lse.
 *   - Returns FA_ERR_TOO_LARGE, before launching anything, when
 *     fa_decode_workspace_bytes() of the sizes exceeds
 *     FA_DECODE_NOALLOC_MAX_WORKSPACE (about 1000 partials of 32 rows at
 *     d = 128: B * Hkv * ceil(G * Nq / 32) * splits); use fa_decode then.
 *   - The buffer of the current device is used (the device the stream
 *     belongs to must be current). Its address is looked up on the first
 *     call on each device.
 *   - Every call on one GPU shares that GPU's buffer: calls that overlap in
 *     time on one GPU (other streams, other host threads) race and must be
 *     serialised by the caller. Nothing in the buffer has to start at zero.
 */
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
                      int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
