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
// Kernels, in order on the caller's stream:
//   bwd_prep  per row: fp16 copies of Q, K, V, dO; D = rowsum(dO * O);
//             -lse * log2(e); per workgroup the largest magnitude of each of
//             Q, K, V, dO; the work-list counters of the next two kernels
//             set to zero. Bandwidth-bound, one pass over the inputs.
//   bwd_dkdv  persistent, one workgroup per CU, each taking (query head,
//             block of 128 keys) items from work lists. 8 waves: wave w owns
//             keys 32 (w mod 4) .. +31 and the query half w / 4 of every
//             64-query block. The K and V tiles stay in LDS for the whole
//             item; Q / dO tiles and their per-row lse / D stream HBM -> LDS
//             by DMA. S = Q K^T is formed with keys along the lanes so that P
//             and dS leave the accumulators already in the operand layout of
//             dV += P^T dO and dK += dS^T Q. The two query halves of a key
//             group are summed through LDS at the end of the item.
//   bwd_dq    persistent likewise, items (query head, block of 256 queries),
//             8 waves x 32 queries; Q and dO stay in registers, K / V tiles
//             stream by DMA; S^T = K Q^T (queries along lanes) so dS^T feeds
//             dQ^T += K^T dS^T directly.
//   bwd_group_sum  grouped-query heads only: a key/value head shared by G
//             query heads gets dK, dV = the sum of the G per-query-head
//             results that bwd_dkdv leaves in the workspace (a fixed order,
//             so the result is deterministic).
// No buffer of size N x N exists.
//
// Work lists. The items of a persistent kernel are dealt round-robin into 8
// lists, one per XCD, so that a list holds whole head groups (their K/V and
// Q/dO streams then share one L2), heaviest causal blocks first. A workgroup
// takes the next item of its own XCD's list and, once that list is empty,
// of the other lists in turn. The XCDs of one chip do not run equally fast
// (the same work measured up to 8 % apart); with a fixed share of the
// workgroups each, the slowest XCD would set the kernel's time.
//
// Matrix-core operands are fp16: P and dS, which must be rounded for the
// products, keep 3 more significant bits than bf16 would give them. Each
// tensor's fp16 copy holds its values times a power of two 2^-e chosen per
// tensor (the "units" of the copy): bf16 values keep e = 0 and FP8 codes
// e = 6 (E4M3) or 13 (E5M2) while the copy's largest magnitude stays where
// the fp16 products are safe; otherwise e is set from that magnitude (its
// copy then peaks in [4, 8)). Every dK/dV workgroup makes this choice, the
// same way, from the maxima bwd_prep recorded; if a tensor's exponent
// changes, the workgroups rewrite its copy together (and rescale D) before
// any item starts. dS is carried in units of the copies of dO and V, so a
// gradient dO of any magnitude, tiny or large, leaves dS in fp16's range;
// the exponents are undone in float32 on dQ, dK, dV.
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
#include <algorithm>
#include <type_traits>

#include "fa_bwd_common.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

size_t backward_workspace_bytes(size_t q_rows, size_t kv_rows, int d) {
  size_t b = kCtlWords * 4 + ws_align(kPrepWgs * 4 * sizeof(float)) + 2 * ws_align(q_rows * sizeof(float)) +
             2 * ws_align(q_rows * (size_t)d * sizeof(f16)) + 2 * ws_align(kv_rows * (size_t)d * sizeof(f16));
  if (q_rows > kv_rows) b += 2 * ws_align(q_rows * (size_t)d * sizeof(float));
  return b;
}


// ---------------------------------------------------------------------------
// Per row: fp16 copies of the operands at their format's default exponent,
// D_i = sum_t dO_it O_it (in units of the dO and V copies, times 2^-15),
// NL_i = kPScale - lse_i * log2(e); per workgroup the largest |value| of each
// input (amax); the work-list counters and the barrier set to zero. One group
// of D/8 lanes per row, 8 elements of each input per lane; the grid strides
// over the rows.
template <int D, typename OT, int FIN, int FDO>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                       const void* __restrict__ V, const void* __restrict__ dO,
                                                       const OT* __restrict__ O, const float* __restrict__ LSE,
                                                       const float* __restrict__ desc, BwdWs ws, long rows,
                                                       long kv_rows) {
  constexpr int L = D / 8;
  __shared__ float s_m[4][4];
  constexpr int ein = default_exp(FIN), edo = default_exp(FDO);
  const float in_mul = ldexpf(1.f, -ein), do_mul = ldexpf(1.f, -edo);
  // D in units of the dO and V copies, times 2^-kPScale: with dO's values f
  // (code values for FP8), D / (s_dO 2^e_dO s_v 2^e_v) = sum f o / (s_v 2^(e_dO + e_v)).
  const float s_v = FIN ? desc[2] : 1.f;
  const float d_mul = ldexpf(kPScaleInv / s_v, -(ein + edo));
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < kCtlWords; i += 256) ws.ctl[i] = 0u;
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  const long total = rows * L;
  for (long base = (long)blockIdx.x * 256; base < total; base += (long)gridDim.x * 256) {
    const long t = base + threadIdx.x;
    const bool live = t < total;
    const long row = live ? t / L : 0;
    const int part = (int)(t % L);
    float acc = 0.f;
    if (live) {
      const size_t off = (size_t)row * D + 8 * part;
      float f[8];
      load8<FIN>(Q, off, f);
      m[0] = fmaxf(m[0], amax8(f));
      *(f16x8*)(ws.q + off) = pack_f16(f, in_mul);
      if (row < kv_rows) {  // key/value heads: kv_rows <= rows
        load8<FIN>(K, off, f);
        m[1] = fmaxf(m[1], amax8(f));
        *(f16x8*)(ws.k + off) = pack_f16(f, in_mul);
        load8<FIN>(V, off, f);
        m[2] = fmaxf(m[2], amax8(f));
        *(f16x8*)(ws.v + off) = pack_f16(f, in_mul);
      }
      load8<FDO>(dO, off, f);
      m[3] = fmaxf(m[3], amax8(f));
      *(f16x8*)(ws.dO + off) = pack_f16(f, do_mul);
      const OT* o = O + off;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += f[j] * (float)o[j];
    }
#pragma unroll
    for (int s = L / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
    if (live && part == 0) {
      ws.Dv[row] = acc * d_mul;
      ws.NL[row] = kPScale - LSE[row] * kLog2e;
    }
  }
  // workgroup maxima -> this workgroup's record
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m[x] = fmaxf(m[x], __shfl_xor(m[x], s, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0)
#pragma unroll
    for (int x = 0; x < 4; ++x) s_m[wave][x] = m[x];
  __syncthreads();
  if (threadIdx.x < 4)
    ws.amax[4 * blockIdx.x + threadIdx.x] =
        fmaxf(fmaxf(s_m[0][threadIdx.x], s_m[1][threadIdx.x]), fmaxf(s_m[2][threadIdx.x], s_m[3][threadIdx.x]));
}

// Every workgroup of a launch: the largest magnitudes recorded by the
// nslots prep workgroups, then the exponents (identical in every workgroup).
__device__ __forceinline__ void gather_exps(const BwdWs& ws, int nslots, int fin, int fdo, float (*s_m)[4], int* e) {
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = threadIdx.x; i < nslots; i += blockDim.x) {
    const f32x4 a = *(const f32x4*)(ws.amax + 4 * i);
#pragma unroll
    for (int x = 0; x < 4; ++x) m[x] = fmaxf(m[x], a[x]);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m[x] = fmaxf(m[x], __shfl_xor(m[x], s, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0)
#pragma unroll
    for (int x = 0; x < 4; ++x) s_m[wave][x] = m[x];
  __syncthreads();
  float amax[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    amax[x] = 0.f;
    for (int w = 0; w < nw; ++w) amax[x] = fmaxf(amax[x], s_m[w][x]);
  }
  choose_exps(amax, fin, fdo, e);
}

// Rare path: the copies of the tensors whose exponent moved away from the
// default are rewritten at the new exponent (and D rescaled when the dO or
// V exponent moved), by all workgroups of the launch, striding over rows.
template <int D>
__device__ void rewrite_copies(const BwdWs& ws, const BwdIn& in, const int* e, const int* ed) {
  constexpr int L = D / 8;
  const long total = in.rows * L;
  const float dfix = ldexpf(1.f, ed[2] + ed[3] - e[2] - e[3]);
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (long)gridDim.x * blockDim.x) {
    const long row = t / L;
    const size_t off = (size_t)row * D + 8 * (t % L);
    float f[8];
    if (e[0] != ed[0]) {
      load8_fmt(in.fin, in.q, off, f);
      *(f16x8*)(ws.q + off) = pack_f16(f, ldexpf(1.f, -e[0]));
    }
    if (row < in.kv_rows && e[1] != ed[1]) {
      load8_fmt(in.fin, in.k, off, f);
      *(f16x8*)(ws.k + off) = pack_f16(f, ldexpf(1.f, -e[1]));
    }
    if (row < in.kv_rows && e[2] != ed[2]) {
      load8_fmt(in.fin, in.v, off, f);
      *(f16x8*)(ws.v + off) = pack_f16(f, ldexpf(1.f, -e[2]));
    }
    if (e[3] != ed[3]) {
      load8_fmt(in.fdo, in.dO, off, f);
      *(f16x8*)(ws.dO + off) = pack_f16(f, ldexpf(1.f, -e[3]));
    }
    if (t % L == 0 && dfix != 1.f) ws.Dv[row] *= dfix;
  }
}

// ---------------------------------------------------------------------------
// dK, dV. Persistent: one workgroup of 8 waves per CU takes (query head,
// block of 128 keys) items from the work lists. Wave w owns key group w % 4
// (32 keys) and query half w / 4 of every 64-row query block, so two waves
// share each SIMD and each key group, and each keeps only its own partial
// dK, dV accumulators (128 registers). The item's K and V tiles stay
// resident in LDS and are read as the B operands of S = Q K^T and
// dP = dO V^T. The two partial sums of a key group are added through LDS at
// the end of the item. With grouped heads an item belongs to one query head
// and reads its key/value head's K and V.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(void* wsb, BwdIn in, float* __restrict__ dK,
                                                          float* __restrict__ dV, int BH, int G, int N, int nkb,
                                                          float c, float scale, int nslots) {
  constexpr int NW = 8, BKV = 128, BQ = 64;
  constexpr int ROWB = 2 * D, TILEB = BQ * ROWB, CPR = D / 8;
  constexpr int VTB = BKV * ROWB;           // resident K (and V) tile bytes
  constexpr int NPW = CPR * BQ / 64 / NW;   // 1024-byte DMA instructions per wave per Q (or dO) tile
  constexpr int NPV = CPR * BKV / 64 / NW;  // ... per wave for the V tile
  constexpr int NKS = D / 16, NDT = D / 32;
  constexpr int STB = 2 * TILEB + 2 * BQ * 4;  // Q tile, dO tile, NL[BQ], D[BQ]
  static_assert(NPW >= 1 && NPV >= 1, "tile split");
  static_assert(STB >= 2 * NDT * 16 * 64 * 4, "dK partials of two key groups fit in a ring stage");
  static_assert(VTB >= 4 * (NDT / 2) * 16 * 64 * 4, "dV partials fit in the K and V tiles");
  __shared__ __attribute__((aligned(1024))) char lds_k[VTB];
  __shared__ __attribute__((aligned(1024))) char lds_v[VTB];
  // Ring stages (Q tile, dO tile, NL, D), one object each (see dma_to_lds).
  __shared__ __attribute__((aligned(1024))) char lds0[STB];
  __shared__ __attribute__((aligned(1024))) char lds1[STB];
  __shared__ float s_m[NW][4];
  __shared__ int s_next;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = wave & 3, qh = wave >> 2;  // key group, query half
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const BwdWs ws = carve_ws(wsb, in.rows, in.kv_rows, D);

  // Exponents of the copies; the rare rewrite, then one barrier, before any item.
  int e[4];
  gather_exps(ws, nslots, in.fin, in.fdo, s_m, e);
  const int ed[4] = {default_exp(in.fin), default_exp(in.fin), default_exp(in.fin), default_exp(in.fdo)};
  if (e[0] != ed[0] || e[1] != ed[1] || e[2] != ed[2] || e[3] != ed[3]) {
    rewrite_copies<D>(ws, in, e, ed);
    grid_barrier(ws.ctl + kBarrier, gridDim.x);
  }
  if (blockIdx.x == 0 && tid == 0) {
    float* ef = (float*)(ws.ctl + kExps);
    ef[0] = (float)e[0];
    ef[1] = (float)e[1];
    ef[2] = (float)e[2];
    ef[3] = (float)e[3];
  }
  // Scale of each copy: value * (FP8 scale) = copy * s.
  const float sq = (in.fin ? in.desc[0] : 1.f) * ldexpf(1.f, e[0]);
  const float sk = (in.fin ? in.desc[1] : 1.f) * ldexpf(1.f, e[1]);
  const float sv = (in.fin ? in.desc[2] : 1.f) * ldexpf(1.f, e[2]);
  const float sdo = (in.fdo ? in.desc[3] : 1.f) * ldexpf(1.f, e[3]);
  // p below is 2^15 P; dS is formed in units of sdo * sv (dP from the copies,
  // D stored in those units times 2^-15), fV undoes 2^15 and the dO units.
  const float cS = c * sq * sk, sPV = kPScaleInv;
  const float fK = scale * sq * sdo * sv, fV = kPScaleInv * sdo;

  const int nqb = (N + BQ - 1) / BQ;

  const int total = BH * nkb, xcd = xcd_id();
  int item = blockIdx.x;  // the grid never exceeds the items
  while (item >= 0) {
    // Per-item values are formed inside the loop from operands the compiler
    // cannot carry across items (an empty asm redefines them): keeping them
    // live across the whole persistent loop would spill registers.
    int ln = lane;
    void* wb = wsb;
    asm volatile("" : "+v"(ln));
    asm volatile("" : "+s"(wb));
    const BwdWs w = carve_ws(wb, (size_t)BH * N, (size_t)BH / G * N, D);
    const int hi = ln >> 5, col = ln & 31;
    // DMA addressing: instruction n of this wave fills tile chunks 64 (NP wave + n) + lane.
    auto dma_off = [&](int n_global) {
      const int p = 64 * n_global + ln, row = p / CPR, pc = p % CPR;
      return (unsigned)(row * ROWB + 16 * (pc ^ tile_swz<D>(row)));
    };
    unsigned goff[NPW];
#pragma unroll
    for (int n = 0; n < NPW; ++n) goff[n] = dma_off(NPW * wave + n);
    // Waves 0 and 1 also bring the block's 64 NL and 64 D values (4 bytes per lane).
    const bool row_loader = wave_u < 2;
    // Row reads at row r, logical chunk 2 kk + hi; transposing reads at row
    // 4 hi + (j >> 2) + 8 sec, byte column 64 dt + 32 g + 8 (j & 3).
    int roff[NKS];
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) roff[kk] = col * ROWB + 16 * ((2 * kk + hi) ^ tile_swz<D>(col));
    int toff[NDT][2];
    {
      const int j = ln & 15, g = (ln >> 4) & 1;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) {
          const int r = 4 * hi + (j >> 2) + 8 * sec;
          const int bcol = 64 * dt + 32 * g + 8 * (j & 3);
          toff[dt][sec] = r * ROWB + 16 * ((bcol >> 4) ^ tile_swz<D>(r)) + (bcol & 15);
        }
    }
    const char* krow = lds_k + 32 * kg * ROWB;  // this wave's 32 K rows (B operand of S)
    const char* vrow = lds_v + 32 * kg * ROWB;  // this wave's 32 V rows (B operand of dP)
    int bh, kb;
    map_head_block(item, BH, G, nkb, CAUSAL, bh, kb);
    const size_t hoff = (size_t)bh * N * D;         // query head: Q, dO; dK, dV written here
    const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head: K, V
    const int k0w = kb * BKV + 32 * kg;             // first key of this wave
    const int key = k0w + col;
    const rsrc_t qr = buffer_rsrc(w.q + hoff, (unsigned)N * ROWB);
    const rsrc_t orr = buffer_rsrc(w.dO + hoff, (unsigned)N * ROWB);
    const rsrc_t nlr = buffer_rsrc(w.NL + (size_t)bh * N, (unsigned)N * 4);
    const rsrc_t dr = buffer_rsrc(w.Dv + (size_t)bh * N, (unsigned)N * 4);
    auto issue_loads = [&](int qb, char* st) {
      const unsigned base = (unsigned)qb * TILEB;
      char* const la = st + 1024 * NPW * wave_u;
#pragma unroll
      for (int n = 0; n < NPW; ++n) {
        dma_to_lds<16>(qr, la + 1024 * n, base + goff[n]);
        dma_to_lds<16>(orr, la + TILEB + 1024 * n, base + goff[n]);
      }
      if (row_loader) {  // waves 0 and 1: NL and D of the block's rows
        char* const dst = st + 2 * TILEB + 256 * wave_u;
        const unsigned off = (unsigned)(qb * BQ + lane) * 4u;
        if (wave_u == 0) dma_to_lds<4>(nlr, dst, off);
        else dma_to_lds<4>(dr, dst, off);
      }
    };
    // K and V tiles of the item (rows past N read as zeros).
    {
      const rsrc_t kr = buffer_rsrc(w.k + kvoff, (unsigned)N * ROWB);
      const rsrc_t vr = buffer_rsrc(w.v + kvoff, (unsigned)N * ROWB);
      const unsigned base = (unsigned)kb * VTB;
      char* const lk = lds_k + 1024 * NPV * wave_u;
      char* const lv = lds_v + 1024 * NPV * wave_u;
#pragma unroll
      for (int n = 0; n < NPV; ++n) {
        const unsigned off = base + dma_off(NPV * wave + n);
        dma_to_lds<16>(kr, lk + 1024 * n, off);
        dma_to_lds<16>(vr, lv + 1024 * n, off);
      }
    }

    f32x16 dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = f32x16{};
    const int qb0 = CAUSAL ? (kb * BKV) / BQ : 0;

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
      if (qb + 1 < nqb) issue_loads(qb + 1, st == 0 ? lds1 : lds0);
      const int q0 = qb * BQ + 32 * qh;
      if (diag) {
        // Tiles whose queries all precede the wave's keys add nothing; tiles
        // crossing the diagonal are masked element-wise.
        if (q0 + 31 >= k0w) {
          if (q0 < k0w + 31) tile(st == 0 ? lds0 : lds1, q0, std::true_type{});
          else tile(st == 0 ? lds0 : lds1, q0, std::false_type{});
        }
      } else {
        tile(st == 0 ? lds0 : lds1, q0, std::false_type{});
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    issue_loads(qb0, lds0);  // qb0 < nqb: the item's keys start before N
    int qb = qb0;
    if (CAUSAL) {
      // the (at most) two query blocks that cross the item's keys
      static_assert(BKV / BQ == 2, "two diagonal query blocks");
      step(qb++, S0{}, std::true_type{});
      if (qb < nqb) step(qb++, S1{}, std::true_type{});
    }
    for (; qb + 1 < nqb; qb += 2) {
      step(qb, S0{}, std::false_type{});
      step(qb + 1, S1{}, std::false_type{});
    }
    if (qb < nqb) step(qb, S0{}, std::false_type{});

    // Sum the two query halves of each key group through LDS, then store. Once
    // every wave is past the loop the ring and the K/V tiles are free: the dK
    // partials of the second half go to the ring, the dV partials to the K/V
    // tiles, so one exchange serves both. The barriers order LDS only (the
    // global stores that follow need not complete before anything here).
    // Accumulator layout: lane holds dim 32 dt + col, keys 8 (i/4) + 4 hi + i % 4.
    // The next item is taken now: the atomic's latency overlaps the exchange.
    int next = -1;
    if (tid == 0) next = pop_item((unsigned*)wsb, 0, total, gridDim.x, xcd);
    // [4 key groups][NDT][16][64 lanes]: groups 0, 1 in stage 0, 2, 3 in stage 1
    float* red_k = (float*)(kg < 2 ? lds0 : lds1) + (kg & 1) * NDT * 16 * 64;
    auto red_v = [&](int dt) {      // [4 key groups][NDT / 2][16][64 lanes] in each of the K and V tiles
      return (float*)(dt < NDT / 2 ? lds_k : lds_v) + (kg * (NDT / 2) + dt % (NDT / 2)) * 16 * 64;
    };
    lds_barrier();
    if (qh == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          red_k[(dt * 16 + i) * 64 + lane] = dk[dt][i];
          red_v(dt)[i * 64 + lane] = dv[dt][i];
        }
    }
    lds_barrier();
    if (qh == 0) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = k0w + 8 * (i / 4) + 4 * hi + (i % 4);
          const float vk = (dk[dt][i] + red_k[(dt * 16 + i) * 64 + lane]) * fK;
          const float vv = (dv[dt][i] + red_v(dt)[i * 64 + lane]) * fV;
          if (kr < N) {
            dK[hoff + (size_t)kr * D + 32 * dt + col] = vk;
            dV[hoff + (size_t)kr * D + 32 * dt + col] = vv;
          }
        }
    }
    // The next item's DMA rewrites the K/V tiles and the ring: every wave has
    // read its partials once it is past this barrier (LDS only: this item's
    // stores stay in flight).
    if (tid == 0) s_next = next;
    lds_barrier();
    item = __builtin_amdgcn_readfirstlane(s_next);
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
                              int grid, hipStream_t st) {
  return launch_kernel(bwd_prep_kernel<D, OT, FIN, FDO>, dim3(grid), dim3(256), st, q, k, v, dO, (const OT*)o, lse,
                       desc, ws, rows, kv_rows);
}

template <int D, typename OT>
static hipError_t launch_prep_fmt(int fin, int fdo, const void* q, const void* k, const void* v, const void* dO,
                                  const void* o, const float* lse, const float* desc, const BwdWs& ws, long rows,
                                  long kv_rows, int grid, hipStream_t st) {
  if (fin == 0) return launch_prep<D, OT, 0, 0>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, grid, st);
  if (fin == 1 && fdo == 2) return launch_prep<D, OT, 1, 2>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, grid, st);
  if (fin == 1) return launch_prep<D, OT, 1, 1>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, grid, st);
  if (fdo == 2) return launch_prep<D, OT, 2, 2>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, grid, st);
  return launch_prep<D, OT, 2, 1>(q, k, v, dO, o, lse, desc, ws, rows, kv_rows, grid, st);
}

// Grid of a persistent launch: one workgroup per CU (these kernels take a
// whole CU each), no more than there are items.
static int persistent_grid(long items) {
  const int cus = device_cu_count();
  const long g = cus > 0 ? cus : 256;
  return (int)(items < g ? items : g);
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                               const float* lse, float* dq, float* dk, float* dv, void* workspace, int BH, int G,
                               int N, float scale, int fin, int fdo, const float* desc, hipStream_t st) {
  const long rows = (long)BH * N, kv_rows = rows / G;
  const BwdWs ws = carve_ws(workspace, (size_t)rows, (size_t)kv_rows, D);
  const long prep_threads = rows * (D / 8);
  const int prep_grid = (int)std::min<long>(kPrepWgs, (prep_threads + 255) / 256);
  hipError_t e = o_dtype == FA_F32
                     ? launch_prep_fmt<D, float>(fin, fdo, q, k, v, dO, o, lse, desc, ws, rows, kv_rows, prep_grid, st)
                     : launch_prep_fmt<D, bf16>(fin, fdo, q, k, v, dO, o, lse, desc, ws, rows, kv_rows, prep_grid, st);
  if (e != hipSuccess) return e;
  const float c = scale * kLog2e;
  const int nkb = (N + 127) / 128;
  float* dk_out = G > 1 ? ws.dKp : dk;  // grouped heads: per-query-head results, summed below
  float* dv_out = G > 1 ? ws.dVp : dv;
  // bf16 has no scales: the kernels then never read desc, which still points
  // at valid memory (the control block) rather than nowhere.
  const float* dsc = desc ? desc : (const float*)ws.ctl;
  const BwdIn in{q, k, v, dO, dsc, fin, fdo, rows, kv_rows};
  e = launch_kernel(bwd_dkdv_kernel<D, CAUSAL>, dim3(persistent_grid((long)BH * nkb)), dim3(512), st, workspace, in, dk_out,
                    dv_out, BH, G, N, nkb, c, scale, prep_grid);
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
  return launch_bwd_dq(D, CAUSAL, workspace, dsc, fin, fdo, dq, BH, G, N, c, scale,
                       persistent_grid((long)BH * nqb), st);
}

// in_fmt / do_fmt: 0 = bf16, 1 = FP8 E4M3, 2 = FP8 E5M2 (both bf16 or both
// FP8; desc = {s_q, s_k, s_v, s_dO} for FP8, else unused).
int launch_backward(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                    const float* lse, float* dq, float* dk, float* dv, void* workspace, int B, int H, int Hkv,
                    int N, int d, float scale, int causal, int in_fmt, int do_fmt, const float* desc,
                    hipStream_t stream) {
  const int BH = B * H, G = H / Hkv;
  hipError_t e;
  if (d == 64)
    e = causal ? launch_bwd_d<64, true>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N, scale, in_fmt,
                                        do_fmt, desc, stream)
               : launch_bwd_d<64, false>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N, scale, in_fmt,
                                         do_fmt, desc, stream);
  else
    e = causal ? launch_bwd_d<128, true>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N, scale, in_fmt,
                                         do_fmt, desc, stream)
               : launch_bwd_d<128, false>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, workspace, BH, G, N, scale,
                                          in_fmt, do_fmt, desc, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
