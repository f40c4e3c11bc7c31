// Backward pass of exact attention: dQ, dK, dV of <O, dO>.
//
// The forward pass keeps only O and the per-row log-sum-exp; the backward
// pass recomputes each score block on chip from Q, K and lse instead of
// storing the N x N matrix (the short-answer FlashAttention-family page,
// answer paragraph 2; the card "FlashAttention Kernel & Online Softmax",
// history paragraph; the "FlashAttention" explainer). The gradients are the
// chain rule through O = P V and the row softmax:
//     P  = exp(scale * Q K^T - lse)        (recomputed)
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_t dO_it O_it
//     dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q
// Three kernels run in order on the caller's stream:
//   bwd_prep  per row: fp16 copies of Q, K, V, dO; D = rowsum(dO * O);
//             -lse * log2(e). Bandwidth-bound, one pass over the inputs.
//   bwd_dkdv  one workgroup per (query head, block of 128 keys), 8 waves:
//             wave w owns keys 32 (w mod 4) .. +31 and the query half w / 4
//             of every 64-query block. The K and V tiles stay in LDS for the
//             whole loop; Q / dO tiles and their per-row lse / D stream
//             HBM -> LDS by DMA. S = Q K^T is formed with keys along the lanes
//             so that P and dS leave the accumulators already in the operand
//             layout of dV += P^T dO and dK += dS^T Q. The two query halves of
//             a key group are summed through LDS at the end.
//   bwd_dq    one workgroup per block of 256 queries (8 waves x 32 queries,
//             two waves per SIMD); Q and dO stay in registers, K / V tiles
//             stream by DMA; S^T = K Q^T (queries along lanes) so dS^T feeds
//             dQ^T += K^T dS^T directly.
//   bwd_group_sum  grouped-query heads only: a key/value head shared by G
//             query heads gets dK, dV = the sum of the G per-query-head
//             results that bwd_dkdv leaves in the workspace (a fixed order,
//             so the result is deterministic).
// No buffer of size N x N exists. The workspace holds D, -lse*log2(e), the
// fp16 copies and, for grouped heads, the per-query-head dK / dV.
//
// Matrix-core operands are fp16: bf16 inputs convert exactly while their
// magnitude lies in fp16's normal range (2^-14 .. 65504; smaller values keep
// fp16's subnormal precision, 2^-24), and P and dS, which must be rounded
// for the products, keep 3 more significant bits than bf16 would give them.
// P enters dV = P^T dO multiplied by 2^15 (kPScale; P <= 1, so at most
// 32768): over long rows attention spreads thin (P ~ 1/N), and unscaled
// probabilities below 2^-14 would fall into fp16's subnormal range and lose
// relative precision. The factor rides in the exponent (the workspace holds
// NL = 15 - lse log2 e) and leaves dV with one multiply by 2^-15 at the end;
// D is stored times 2^-15 so that dS = 2^15 P (2^-15 dP - 2^-15 D) keeps its
// true scale at the same instruction count.
// Accumulation is float32 throughout.
//
// LDS tiles use the forward pass's XOR swizzle (16-byte chunk c of row r at
// c ^ swz(r)), which keeps both row reads (ds_read_b128) and transposing reads
// (ds_read_b64_tr_b16) free of bank conflicts.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 cat4h(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ s16x4 lds_read_tr16h(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 FA_LDS*)(p));
}

template <int D>
__device__ __forceinline__ int swz_b(int r) {
  if (D == 128) return (4 * (r & 3)) ^ ((r >> 2) & 3);
  return (4 * ((r >> 1) & 1)) ^ ((r >> 2) & 3);
}

// Same XCD-aware, heavy-first order as the forward pass; first_is_heavy
// selects whether block index 0 (dK/dV, causal) or nb-1 (dQ) is heaviest.
// Workspace layout (all offsets 256-byte aligned): D [q_rows] f32,
// NL = kPScale - lse*log2(e) [q_rows] f32 (D is stored times 2^-kPScale),
// Q [q_rows, d] fp16, K and V [kv_rows, d]
// fp16, dO [q_rows, d] fp16, and when q_rows > kv_rows (grouped heads)
// per-query-head dK and dV [q_rows, d] f32. q_rows = B*H*N, kv_rows = B*Hkv*N.
constexpr float kPScale = 15.f;            // P is scaled by 2^kPScale for the dV product
constexpr float kPScaleInv = 1.f / 32768.f;  // 2^-kPScale
struct BwdWs {
  float* Dv;
  float* NL;
  f16 *q, *k, *v, *dO;
  float *dKp, *dVp;
};
static inline size_t ws_align(size_t x) { return (x + 255) & ~(size_t)255; }
static inline BwdWs carve_ws(void* base, size_t q_rows, size_t kv_rows, int d) {
  char* p = (char*)base;
  BwdWs w;
  const size_t fbytes = ws_align(q_rows * sizeof(float));
  const size_t qbytes = ws_align(q_rows * (size_t)d * sizeof(f16));
  const size_t kvbytes = ws_align(kv_rows * (size_t)d * sizeof(f16));
  const size_t pbytes = ws_align(q_rows * (size_t)d * sizeof(float));
  w.Dv = (float*)p;
  w.NL = (float*)(p + fbytes);
  w.q = (f16*)(p + 2 * fbytes);
  w.k = (f16*)(p + 2 * fbytes + qbytes);
  w.v = (f16*)(p + 2 * fbytes + qbytes + kvbytes);
  w.dO = (f16*)(p + 2 * fbytes + qbytes + 2 * kvbytes);
  const bool grouped = q_rows > kv_rows;
  w.dKp = grouped ? (float*)(p + 2 * fbytes + 2 * qbytes + 2 * kvbytes) : nullptr;
  w.dVp = grouped ? (float*)(p + 2 * fbytes + 2 * qbytes + 2 * kvbytes + pbytes) : nullptr;
  return w;
}
size_t backward_workspace_bytes(size_t q_rows, size_t kv_rows, int d) {
  size_t b = 2 * ws_align(q_rows * sizeof(float)) + 2 * ws_align(q_rows * (size_t)d * sizeof(f16)) +
             2 * ws_align(kv_rows * (size_t)d * sizeof(f16));
  if (q_rows > kv_rows) b += 2 * ws_align(q_rows * (size_t)d * sizeof(float));
  return b;
}

// 8 bf16 (raw 16 bytes) -> 8 fp16 (exact in fp16's normal range); f gets the float values.
__device__ __forceinline__ f16x8 bf16x8_to_f16(i32x4 raw, float* f) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned w = (unsigned)raw[j];
    f[2 * j] = __builtin_bit_cast(float, w << 16);
    f[2 * j + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
    r[2 * j] = (f16)f[2 * j];
    r[2 * j + 1] = (f16)f[2 * j + 1];
  }
  return r;
}

// ---------------------------------------------------------------------------
// 8 FP8 codes (raw 8 bytes; E4M3 if E5M2 == false) -> 8 fp16 (exact: every
// E4M3 and E5M2 value is an fp16 value); f gets the float values.
template <bool E5M2, int SEL>
__device__ __forceinline__ float fp8_byte(int w) {
  return E5M2 ? __builtin_amdgcn_cvt_f32_bf8(w, SEL) : __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}
template <bool E5M2>
__device__ __forceinline__ f16x8 fp8x8_to_f16(i32x2 raw, float* f) {
  f[0] = fp8_byte<E5M2, 0>(raw[0]);
  f[1] = fp8_byte<E5M2, 1>(raw[0]);
  f[2] = fp8_byte<E5M2, 2>(raw[0]);
  f[3] = fp8_byte<E5M2, 3>(raw[0]);
  f[4] = fp8_byte<E5M2, 0>(raw[1]);
  f[5] = fp8_byte<E5M2, 1>(raw[1]);
  f[6] = fp8_byte<E5M2, 2>(raw[1]);
  f[7] = fp8_byte<E5M2, 3>(raw[1]);
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (f16)f[j];
  return r;
}

// Element format of a backward input: 0 = bf16, 1 = FP8 E4M3, 2 = FP8 E5M2.
template <int FMT>
__device__ __forceinline__ f16x8 load8_f16(const void* base, size_t elem, float* f) {
  if (FMT == 0) return bf16x8_to_f16(*(const i32x4*)((const bf16*)base + elem), f);
  return fp8x8_to_f16<FMT == 2>(*(const i32x2*)((const uint8_t*)base + elem), f);
}

// Per row: fp16 copies of the operands (FP8 codes are copied as their code
// values; the per-tensor scales are applied by the kernels that use them),
// D_i = sum_t dO_it * O_it (with dO's scale), NL_i = -lse_i * log2(e).
// One group of D/8 lanes per row, 8 elements of each input per lane.
template <int D, typename OT, int FIN, int FDO>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                       const void* __restrict__ V, const void* __restrict__ dO,
                                                       const OT* __restrict__ O, const float* __restrict__ LSE,
                                                       const float* __restrict__ desc, BwdWs ws, long rows,
                                                       long kv_rows) {
  constexpr int L = D / 8;
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / L;
  const int part = (int)(t % L);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + 8 * part;
    float tmp[8], dof[8];
    *(f16x8*)(ws.q + off) = load8_f16<FIN>(Q, off, tmp);
    if (row < kv_rows) {  // key/value heads: kv_rows <= rows
      *(f16x8*)(ws.k + off) = load8_f16<FIN>(K, off, tmp);
      *(f16x8*)(ws.v + off) = load8_f16<FIN>(V, off, tmp);
    }
    *(f16x8*)(ws.dO + off) = load8_f16<FDO>(dO, off, dof);
    const OT* o = O + off;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += dof[j] * (float)o[j];
  }
#pragma unroll
  for (int s = L / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && part == 0) {
    ws.Dv[row] = (FDO == 0 ? acc : acc * desc[3]) * kPScaleInv;
    ws.NL[row] = kPScale - LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV. 8 waves per workgroup of 128 keys: wave w owns key group w % 4
// (32 keys) and query half w / 4 of every 64-row query block, so two waves
// share each SIMD and each key group, and each keeps only its own partial
// dK, dV accumulators (128 registers). The workgroup's K and V tiles stay
// resident in LDS and are read as the B operands of S = Q K^T and
// dP = dO V^T. The two partial sums of a key group are added through LDS at
// the end. With grouped heads the workgroup belongs to one query head and
// reads its key/value head's K and V.
// SCALED: the operands are FP8 codes with per-tensor scales desc = {s_q, s_k,
// s_v, s_dO}: S gets s_q s_k (folded into the exponent), dP gets s_dO s_v,
// dV s_dO and dK s_q.
template <int D, bool CAUSAL, bool SCALED>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdWs ws, float* __restrict__ dK, float* __restrict__ dV,
                                                          int BH, int G, int N, int nkb, float c, float scale,
                                                          const float* __restrict__ desc) {
  constexpr int NW = 8, BKV = 128, BQ = 64;
  constexpr int ROWB = 2 * D, TILEB = BQ * ROWB, CPR = D / 8;
  constexpr int VTB = BKV * ROWB;           // resident K (and V) tile bytes
  constexpr int NPW = CPR * BQ / 64 / NW;   // 1024-byte DMA instructions per wave per Q (or dO) tile
  constexpr int NPV = CPR * BKV / 64 / NW;  // ... per wave for the V tile
  constexpr int NKS = D / 16, NDT = D / 32;
  constexpr int NST = 2;
  constexpr int STB = 2 * TILEB + 2 * BQ * 4;  // Q tile, dO tile, NL[BQ], D[BQ]
  static_assert(NPW >= 1 && NPV >= 1, "tile split");
  static_assert(NST * STB >= 4 * 32 * D * 4 * 2 / 2, "reduction buffer fits in the ring");
  __shared__ __attribute__((aligned(1024))) char lds_k[VTB];
  __shared__ __attribute__((aligned(1024))) char lds_v[VTB];
  __shared__ __attribute__((aligned(1024))) char lds[NST][STB];

  // p below is 2^15 P; sPV carries the matching 2^-15 (and the FP8 scales), fV undoes it on dV.
  float cS = c, sPV = kPScaleInv, fK = scale, fV = kPScaleInv;
  if (SCALED) {
    cS = c * desc[0] * desc[1];
    sPV = desc[3] * desc[2] * kPScaleInv;
    fK = scale * desc[0];
    fV = desc[3] * kPScaleInv;
  }
  int bh, kb;
  map_head_block(blockIdx.x, BH, G, nkb, CAUSAL, bh, kb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const int kg = wave & 3, qh = wave >> 2;  // key group, query half
  const size_t hoff = (size_t)bh * N * D;         // query head: Q, dO; dK, dV written here
  const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head: K, V
  const int k0w = kb * BKV + 32 * kg;  // first key of this wave
  const int key = k0w + col;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  const i32x4 qr = make_rsrc(ws.q + hoff, (unsigned)N * ROWB);
  const i32x4 orr = make_rsrc(ws.dO + hoff, (unsigned)N * ROWB);
  const i32x4 vr = make_rsrc(ws.v + kvoff, (unsigned)N * ROWB);
  const i32x4 kr = make_rsrc(ws.k + kvoff, (unsigned)N * ROWB);
  const i32x4 nlr = make_rsrc(ws.NL + (size_t)bh * N, (unsigned)N * 4);
  const i32x4 dr = make_rsrc(ws.Dv + (size_t)bh * N, (unsigned)N * 4);
  // DMA addressing: instruction n of this wave fills tile chunks 64 (NP wave + n) + lane.
  auto dma_off = [&](int n_global) {
    const int p = 64 * n_global + lane, row = p / CPR, pc = p % CPR;
    return (unsigned)(row * ROWB + 16 * (pc ^ swz_b<D>(row)));
  };
  unsigned goff[NPW];
#pragma unroll
  for (int n = 0; n < NPW; ++n) goff[n] = dma_off(NPW * wave + n);
  // Waves 0 and 1 also bring the block's 64 NL and 64 D values (4 bytes per lane).
  const bool row_loader = wave_u < 2;
  auto issue_loads = [&](int qb, int st) {
    const unsigned base = (unsigned)qb * TILEB;
    const unsigned la = lds_addr(lds[st]) + 1024u * NPW * wave_u;
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      load_lds16(qr, la + 1024u * n, base + goff[n]);
      load_lds16(orr, la + TILEB + 1024u * n, base + goff[n]);
    }
    if (row_loader) {
      const i32x4 r = wave_u == 0 ? nlr : dr;
      const unsigned dst = lds_addr(lds[st]) + 2 * TILEB + 256u * wave_u;
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                   :
                   : "s"(dst), "v"((unsigned)(qb * BQ + lane) * 4u), "s"(r)
                   : "memory", "m0");
    }
  };

  // K and V tiles of the workgroup, once (rows past N read as zeros).
  {
    const unsigned base = (unsigned)kb * VTB;
    const unsigned lk = lds_addr(lds_k) + 1024u * NPV * wave_u;
    const unsigned lv = lds_addr(lds_v) + 1024u * NPV * wave_u;
#pragma unroll
    for (int n = 0; n < NPV; ++n) {
      const unsigned off = base + dma_off(NPV * wave + n);
      load_lds16(kr, lk + 1024u * n, off);
      load_lds16(vr, lv + 1024u * n, off);
    }
  }
  // Row reads at row r, logical chunk 2 kk + hi; transposing reads at row
  // 4 hi + (j >> 2) + 8 sec, byte column 64 dt + 32 g + 8 (j & 3).
  int roff[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) roff[kk] = col * ROWB + 16 * ((2 * kk + hi) ^ swz_b<D>(col));
  int toff[NDT][2];
  {
    const int j = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int r = 4 * hi + (j >> 2) + 8 * sec;
        const int bcol = 64 * dt + 32 * g + 8 * (j & 3);
        toff[dt][sec] = r * ROWB + 16 * ((bcol >> 4) ^ swz_b<D>(r)) + (bcol & 15);
      }
  }
  const char* krow = lds_k + 32 * kg * ROWB;  // this wave's 32 K rows (B operand of S)
  const char* vrow = lds_v + 32 * kg * ROWB;  // this wave's 32 V rows (B operand of dP)

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = f32x16{};

  const int nqb = (N + BQ - 1) / BQ;
  const int qb0 = CAUSAL ? (kb * BKV) / BQ : 0;
  const int qb_unmasked = CAUSAL ? qb0 + BKV / BQ : 0;

  // This wave's 32-query tile of the block in stage st: S, dP -> P, dS -> dV, dK.
  auto tile = [&](const char* st, int q0, auto masked_c) {
    constexpr bool masked = decltype(masked_c)::value;
    const char* qs = st + 32 * qh * ROWB;
    const char* os = st + TILEB + 32 * qh * ROWB;
    const float* nl = (const float*)(st + 2 * TILEB) + 32 * qh;
    const float* dd = nl + BQ;
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      const f16x8 aq = *(const f16x8*)(qs + roff[kk]);
      const f16x8 ao = *(const f16x8*)(os + roff[kk]);
      const f16x8 bk = *(const f16x8*)(krow + roff[kk]);
      const f16x8 bv = *(const f16x8*)(vrow + roff[kk]);
      s = mfma_f16(aq, bk, s);
      dp = mfma_f16(ao, bv, dp);
      // Bound the look-ahead of the fragment reads: two k-steps in flight keep
      // the register budget at two waves per SIMD (the other wave hides latency).
      if (kk % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    // Accumulator rows: query q0 + 8 (i/4) + 4 hi + i % 4; lane = key.
    float pv[16], dsv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l4 = *(const f32x4*)(nl + 8 * g + 4 * hi);
      const f32x4 d4 = *(const f32x4*)(dd + 8 * g + 4 * hi);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[4 * g + r], cS, l4[r]));
        if (masked && key > q0 + 8 * g + 4 * hi + r) p = 0.f;
        pv[4 * g + r] = p;
        dsv[4 * g + r] = p * __builtin_fmaf(dp[4 * g + r], sPV, -d4[r]);  // P (dP - D)
      }
    }
    f16x8 pf[2], df[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      pf[h2] = f16x8{(f16)pv[8 * h2], (f16)pv[8 * h2 + 1], (f16)pv[8 * h2 + 2], (f16)pv[8 * h2 + 3],
                     (f16)pv[8 * h2 + 4], (f16)pv[8 * h2 + 5], (f16)pv[8 * h2 + 6], (f16)pv[8 * h2 + 7]};
      df[h2] = f16x8{(f16)dsv[8 * h2], (f16)dsv[8 * h2 + 1], (f16)dsv[8 * h2 + 2], (f16)dsv[8 * h2 + 3],
                     (f16)dsv[8 * h2 + 4], (f16)dsv[8 * h2 + 5], (f16)dsv[8 * h2 + 6], (f16)dsv[8 * h2 + 7]};
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int rb = 16 * h2 * ROWB;
        const f16x8 bo = cat4h(lds_read_tr16h(os + rb + toff[dt][0]), lds_read_tr16h(os + rb + toff[dt][1]));
        const f16x8 bq = cat4h(lds_read_tr16h(qs + rb + toff[dt][0]), lds_read_tr16h(qs + rb + toff[dt][1]));
        dv[dt] = mfma_f16(pf[h2], bo, dv[dt]);
        dk[dt] = mfma_f16(df[h2], bq, dk[dt]);
        if (h2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
  };

  // Ring of two stages, loads one block ahead; block qb0 + i lives in stage
  // i % 2. Steps come in pairs so that each stage index is a compile-time
  // constant (stage base addresses fold into the LDS instruction offsets).
  auto step = [&](int qb, auto stage_c, auto diag_c) {
    constexpr int st = decltype(stage_c)::value;
    constexpr bool diag = decltype(diag_c)::value;
    wait_vmem();  // this wave's loads of block qb (and, the first time, of the K/V tiles)
    __syncthreads();
    if (qb + 1 < nqb) issue_loads(qb + 1, st ^ 1);
    const int q0 = qb * BQ + 32 * qh;
    if (diag) {
      // Tiles whose queries all precede the wave's keys add nothing; tiles
      // crossing the diagonal are masked element-wise.
      if (q0 + 31 >= k0w) {
        if (q0 < k0w + 31) tile(lds[st], q0, std::true_type{});
        else tile(lds[st], q0, std::false_type{});
      }
    } else {
      tile(lds[st], q0, std::false_type{});
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (qb0 < nqb) issue_loads(qb0, 0);
  int qb = qb0;
  if (CAUSAL) {
    // the (at most) two query blocks that cross the workgroup's keys
    static_assert(BKV / BQ == 2, "two diagonal query blocks");
    if (qb < nqb) step(qb++, S0{}, std::true_type{});
    if (qb < nqb) step(qb++, S1{}, std::true_type{});
  }
  for (; qb + 1 < nqb; qb += 2) {
    step(qb, S0{}, std::false_type{});
    step(qb + 1, S1{}, std::false_type{});
  }
  if (qb < nqb) step(qb, S0{}, std::false_type{});

  // Sum the two query halves of each key group through LDS (the ring is free
  // once every wave has passed the barrier), then store.
  // Accumulator layout: lane holds dim 32 dt + col, keys 8 (i/4) + 4 hi + i % 4.
  float* red = (float*)lds[0];  // [4 key groups][NDT][16][64 lanes]
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* a = pass == 0 ? dk : dv;
    if (qh == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[((kg * NDT + dt) * 16 + i) * 64 + lane] = a[dt][i];
    }
    __syncthreads();
    if (qh == 0) {
      float* out = pass == 0 ? dK : dV;
      const float f = pass == 0 ? fK : fV;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = k0w + 8 * (i / 4) + 4 * hi + (i % 4);
          const float v = (a[dt][i] + red[((kg * NDT + dt) * 16 + i) * 64 + lane]) * f;
          if (kr < N) out[hoff + (size_t)kr * D + 32 * dt + col] = v;
        }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dQ. 8 waves x 32 queries (BR = 256), two waves per SIMD; key blocks of 64.
// SCALED as for bwd_dkdv: S gets s_q s_k, dP gets s_dO s_v, dQ gets s_k.
template <int D, bool CAUSAL, bool SCALED>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdWs ws, float* __restrict__ dQ, int BH, int G, int N, int nqb,
                                                        float c, float scale, const float* __restrict__ desc) {
  constexpr int NW = 8, BR = 32 * NW, BC = 64;
  constexpr int ROWB = 2 * D, TILEB = BC * ROWB, CPR = D / 8;
  constexpr int NPW = CPR * BC / 64 / NW;
  constexpr int NKS = D / 16, NDT = D / 32, NKT = BC / 32;
  static_assert(NPW >= 1, "tile split");
  __shared__ __attribute__((aligned(1024))) char lds[2][2 * TILEB];  // [stage][K | V]

  float cS = c, sPV = 1.f, fQ = scale;
  if (SCALED) {
    cS = c * desc[0] * desc[1];
    sPV = desc[3] * desc[2];
    fQ = scale * desc[1];
  }
  int bh, qb;
  map_head_block(blockIdx.x, BH, G, nqb, false, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;         // query head: Q, dO, dQ
  const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head: K, V
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qw = qb * BR + 32 * wave_u;  // wave-uniform: the mask test below is a scalar branch
  const int q = qw + col;

  const i32x4 kr = make_rsrc(ws.k + kvoff, (unsigned)N * ROWB);
  const i32x4 vr = make_rsrc(ws.v + kvoff, (unsigned)N * ROWB);
  unsigned goff[NPW];
#pragma unroll
  for (int n = 0; n < NPW; ++n) {
    const int p = 64 * (NPW * wave + n) + lane, row = p / CPR, pc = p % CPR;
    goff[n] = row * ROWB + 16 * (pc ^ swz_b<D>(row));
  }
  auto issue_loads = [&](int kb, char* st) {
    const unsigned base = (unsigned)kb * TILEB;
    const unsigned la = lds_addr(st) + 1024u * NPW * wave_u;
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      load_lds16(kr, la + 1024u * n, base + goff[n]);
      load_lds16(vr, la + TILEB + 1024u * n, base + goff[n]);
    }
  };
  int roff[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) roff[kk] = col * ROWB + 16 * ((2 * kk + hi) ^ swz_b<D>(col));
  int toff[NDT][2];
  {
    const int j = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int r = 4 * hi + (j >> 2) + 8 * sec;
        const int bcol = 64 * dt + 32 * g + 8 * (j & 3);
        toff[dt][sec] = r * ROWB + 16 * ((bcol >> 4) ^ swz_b<D>(r)) + (bcol & 15);
      }
  }

  // Q and dO as B operands: lane holds row q, dims 16 ks + 8 hi + 0..7.
  f16x8 qf[NKS], of[NKS];
  {
    const int qr = q < N ? q : 0;
    const f16x8* qsrc = (const f16x8*)(ws.q + hoff + (size_t)qr * D);
    const f16x8* osrc = (const f16x8*)(ws.dO + hoff + (size_t)qr * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f16x8 a = qsrc[2 * ks + hi], b = osrc[2 * ks + hi];
      qf[ks] = q < N ? a : f16x8{};
      of[ks] = q < N ? b : f16x8{};
    }
  }
  // The workspace's 2^15 on P and 2^-15 on D are for the dK/dV kernel; here P is unscaled.
  const float nl = q < N ? ws.NL[(size_t)bh * N + q] - kPScale : 0.f;
  const float dq_d = q < N ? ws.Dv[(size_t)bh * N + q] * 32768.f : 0.f;
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};

  const int nkb_all = (N + BC - 1) / BC;
  const int q_last = min(N - 1, qb * BR + BR - 1);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;

  auto compute = [&](int kb, const char* st) {
    const int k0 = kb * BC;
    if (CAUSAL && k0 > qw + 31) return;  // every key of the block follows every query of the wave
    const char* ks = st;
    const char* vs = st + TILEB;
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
    // S^T = K Q^T and dP^T = V dO^T for the 32-key tiles of the block, k-step
    // outer: the 2 NKT products of a step are independent and the next
    // step's fragments are read before them (the fences keep the scheduler
    // from sinking the reads next to their use).
    f32x16 s[NKT], dp[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt] = dp[kt] = f32x16{};
    f16x8 ak[2][NKT], av[2][NKT];
    auto kvread = [&](int kk, int b) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        ak[b][kt] = *(const f16x8*)(ks + 32 * kt * ROWB + roff[kk]);
        av[b][kt] = *(const f16x8*)(vs + 32 * kt * ROWB + roff[kk]);
      }
    };
    kvread(0, 0);
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      if (kk + 1 < NKS) kvread(kk + 1, (kk + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        s[kt] = mfma_f16(ak[kk & 1][kt], qf[kk], s[kt]);
        dp[kt] = mfma_f16(av[kk & 1][kt], of[kk], dp[kt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // P and dS^T -> fp16 B fragments. Only blocks that cross the diagonal or
    // the ragged tail take the masked copy (need_mask is wave-uniform).
    f16x8 df[NKT][2];
    auto ds_tiles = [&](auto masked_c) __attribute__((always_inline)) {
      constexpr bool masked = decltype(masked_c)::value;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        float dsv[16];
        // key k0 + 32 kt + 8 (i/4) + 4 hi + i % 4 is kept iff its offset 8 (i/4) + i % 4 <= lim
        const int lim = min(CAUSAL ? q : N - 1, N - 1) - (k0 + 32 * kt) - 4 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(__builtin_fmaf(s[kt][i], cS, nl));
          if (masked && 8 * (i / 4) + (i % 4) > lim) p = 0.f;
          dsv[i] = p * ((SCALED ? dp[kt][i] * sPV : dp[kt][i]) - dq_d);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          df[kt][h2] = f16x8{(f16)dsv[8 * h2], (f16)dsv[8 * h2 + 1], (f16)dsv[8 * h2 + 2], (f16)dsv[8 * h2 + 3],
                             (f16)dsv[8 * h2 + 4], (f16)dsv[8 * h2 + 5], (f16)dsv[8 * h2 + 6], (f16)dsv[8 * h2 + 7]};
      }
    };
    if (need_mask) ds_tiles(std::true_type{});
    else ds_tiles(std::false_type{});
    // dQ^T += K^T dS^T: K^T read transposed, key order of the accumulator
    // rows; 16-key steps outer with the next step's reads issued first.
    constexpr int NST = 2 * NKT;
    auto kread = [&](int st, int dt) __attribute__((always_inline)) {
      const int rb = 16 * st * ROWB;
      return cat4h(lds_read_tr16h(ks + rb + toff[dt][0]), lds_read_tr16h(ks + rb + toff[dt][1]));
    };
    f16x8 kf[2][NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) kf[0][dt] = kread(0, dt);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + 1 < NST) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) kf[(st + 1) & 1][dt] = kread(st + 1, dt);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = mfma_f16(kf[st & 1][dt], df[st >> 1][st & 1], acc[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  issue_loads(0, lds[0]);
  for (int kb = 0; kb < nkb; kb += 2) {
    wait_vmem();
    __syncthreads();
    if (kb + 1 < nkb) issue_loads(kb + 1, lds[1]);
    compute(kb, lds[0]);
    if (kb + 1 < nkb) {
      wait_vmem();
      __syncthreads();
      if (kb + 2 < nkb) issue_loads(kb + 2, lds[0]);
      compute(kb + 1, lds[1]);
    }
  }

  if (q < N) {
    float* dst = dQ + hoff + (size_t)q * D + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {acc[dt][4 * g] * fQ, acc[dt][4 * g + 1] * fQ, acc[dt][4 * g + 2] * fQ,
                   acc[dt][4 * g + 3] * fQ};
        *(f32x4*)(dst + 32 * dt + 8 * g) = v;
      }
  }
}

// ---------------------------------------------------------------------------
// Grouped heads: out[kv row] = sum over g < G of part[(kv head * G + g) row],
// 4 floats per lane, heads added in order g = 0, 1, ...
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                            long head_elems, int G, long total4) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= total4) return;
  const long e = 4 * t;                      // element of the [B*Hkv, N, d] output
  const long kvh = e / head_elems, r = e - kvh * head_elems;
  const float* src = part + kvh * G * head_elems + r;
  f32x4 acc = *(const f32x4*)src;
  for (int g = 1; g < G; ++g) acc += *(const f32x4*)(src + g * head_elems);
  *(f32x4*)(out + e) = acc;
}

template <int D, typename OT, int FIN, int FDO>
static hipError_t launch_prep(const void* q, const void* k, const void* v, const void* dO, const void* o,
                              const float* lse, const float* desc, const BwdWs& ws, long rows, long kv_rows,
                              hipStream_t st) {
  const long threads = rows * (D / 8);
  const int blocks = (int)((threads + 255) / 256);
  return launch_kernel(bwd_prep_kernel<D, OT, FIN, FDO>, dim3(blocks), dim3(256), st, q, k, v, dO, (const OT*)o, lse,
                       desc, ws, rows, kv_rows);
}

template <int D, typename OT>
static hipError_t launch_prep_fmt(int fin, int fdo, const void* q, const void* k, const void* v, const void* dO,
                                  const void* o, const float* lse, const float* desc, const BwdWs& ws, long rows,
                                  long kv_rows, hipStream_t st) {
  if (fin == 0) return launch_prep<D, OT, 0, 0>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, st);
  if (fin == 1 && fdo == 2) return launch_prep<D, OT, 1, 2>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, st);
  if (fin == 1) return launch_prep<D, OT, 1, 1>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, st);
  if (fdo == 2) return launch_prep<D, OT, 2, 2>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, st);
  return launch_prep<D, OT, 2, 1>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, st);
}

template <int D, bool CAUSAL, bool SCALED>
static hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                               const float* lse, float* dq, float* dk, float* dv, void* workspace, int BH, int G,
                               int N, float scale, int fin, int fdo, const float* desc, hipStream_t st) {
  const long rows = (long)BH * N, kv_rows = rows / G;
  const BwdWs ws = carve_ws(workspace, (size_t)rows, (size_t)kv_rows, D);
  hipError_t e = o_dtype == FA_F32
                     ? launch_prep_fmt<D, float>(fin, fdo, q, k, v, dO, o, lse, desc, ws, rows, kv_rows, st)
                     : launch_prep_fmt<D, bf16>(fin, fdo, q, k, v, dO, o, lse, desc, ws, rows, kv_rows, st);
  if (e != hipSuccess) return e;
  const float c = scale * kLog2e;
  const int nkb = (N + 127) / 128;
  float* dk_out = G > 1 ? ws.dKp : dk;  // grouped heads: per-query-head results, summed below
  float* dv_out = G > 1 ? ws.dVp : dv;
  e = launch_kernel(bwd_dkdv_kernel<D, CAUSAL, SCALED>, dim3(BH * nkb), dim3(512), st, ws, dk_out, dv_out, BH, G, N,
                    nkb, c, scale, desc);
  if (e != hipSuccess) return e;
  if (G > 1) {
    const long head_elems = (long)N * D, total4 = kv_rows * D / 4;
    const int blocks = (int)((total4 + 255) / 256);
    e = launch_kernel(bwd_group_sum_kernel, dim3(blocks), dim3(256), st, (const float*)ws.dKp, dk, head_elems, G,
                      total4);
    if (e != hipSuccess) return e;
    e = launch_kernel(bwd_group_sum_kernel, dim3(blocks), dim3(256), st, (const float*)ws.dVp, dv, head_elems, G,
                      total4);
    if (e != hipSuccess) return e;
  }
  const int nqb = (N + 255) / 256;
  return launch_kernel(bwd_dq_kernel<D, CAUSAL, SCALED>, dim3(BH * nqb), dim3(512), st, ws, dq, BH, G, N, nqb, c,
                       scale, desc);
}

template <bool SCALED>
static hipError_t launch_bwd_s(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                               const float* lse, float* dq, float* dk, float* dv, void* workspace, int BH, int G,
                               int N, int d, float scale, int causal, int fin, int fdo, const float* desc,
                               hipStream_t st) {
  if (d == 64)
    return causal ? launch_bwd_d<64, true, SCALED>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N,
                                                    scale, fin, fdo, desc, st)
                  : launch_bwd_d<64, false, SCALED>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N,
                                                     scale, fin, fdo, desc, st);
  return causal ? launch_bwd_d<128, true, SCALED>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N,
                                                   scale, fin, fdo, desc, st)
                : launch_bwd_d<128, false, SCALED>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N,
                                                    scale, fin, fdo, desc, st);
}

// in_fmt / do_fmt: 0 = bf16, 1 = FP8 E4M3, 2 = FP8 E5M2 (both bf16 or both
// FP8; desc = {s_q, s_k, s_v, s_dO} for FP8, else unused).
int launch_backward(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                    const float* lse, float* dq, float* dk, float* dv, void* workspace, int B, int H, int Hkv,
                    int N, int d, float scale, int causal, int in_fmt, int do_fmt, const float* desc,
                    hipStream_t stream) {
  const int BH = B * H, G = H / Hkv;
  const hipError_t e =
      in_fmt == 0 ? launch_bwd_s<false>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N, d, scale, causal,
                                        0, 0, nullptr, stream)
                  : launch_bwd_s<true>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N, d, scale, causal,
                                       in_fmt, do_fmt, desc, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
