// Forward pass of exact attention: O = softmax(scale * Q K^T) V and the
// per-row log-sum-exp, one workgroup per (batch*head, block of query rows).
//
// The method: each workgroup owns a group of query rows and visits the key
// and value rows group by group in on-chip memory. Per query row it carries
// three running quantities, the largest score seen so far m, the sum l of
// exponentials taken against that maximum, and the matching unnormalised
// output, and corrects l and the output by exp(m - m_new) whenever a new
// group raises the maximum, so that no N x N matrix is ever stored (the
// short-answer page "Walk through what FlashAttention does differently ...",
// answer paragraph 1; the card "FlashAttention Kernel & Online Softmax",
// definition paragraph; the "FlashAttention" explainer by A. Tiwari). One
// division by l finishes each row.
//
// gfx950 mapping (per wave of 64 lanes, 32 query rows):
//   * Scores are formed transposed, S^T = K Q^T, on the matrix cores: the
//     accumulator layout then gives every lane one query column and 16 keys,
//     so the row max and row sum are in-lane loops plus one exchange with the
//     partner half-wave.
//   * The probabilities P^T, converted in place, are directly the B operand
//     of O^T += V^T P^T; V^T comes from the row-major V tile in LDS through
//     the transposing LDS read, with the contraction (key) order chosen to
//     match the accumulator layout.
//   * Q stays in registers for the whole kernel; K and V tiles go HBM -> LDS
//     by DMA one block ahead (double-buffered LDS), and each product reads
//     its LDS fragments one k-step ahead.
//   * Base-2 exponentials with scale*log2(e) folded into one FMA; the
//     denominator l is summed from the unrounded float32 probabilities.
//   * Causal: key blocks past the diagonal are never visited; only blocks
//     that cross the diagonal (or the ragged tail) are masked element-wise.
//   * Grid order: heaviest causal query blocks first; all query blocks of a
//     key/value head (of every query head that shares it) go to the same XCD
//     (workgroups are dealt round-robin to the 8 XCDs) so that its K/V
//     stream is shared through one L2.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

// Output stores of 4 consecutive elements in the output dtype.
template <typename T> struct OutStore;
template <> struct OutStore<bf16> {
  static __device__ __forceinline__ void store4(bf16* dst, float a, float b, float c, float d) {
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *(bf16x4*)dst = v;
  }
};
template <> struct OutStore<float> {
  static __device__ __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
    f32x4 v = {a, b, c, d};
    *(f32x4*)dst = v;
  }
};

// ---------------------------------------------------------------------------
// bf16 operands. NW waves x 32 query rows (BR = 32 NW) per workgroup, blocks
// of BC keys. d = 128: 8 waves, 128-key blocks, one workgroup per CU (two
// waves per SIMD, which is what the registers allow), so one wave's softmax
// overlaps the other's matrix-core work. d = 64 halves the matrix work per
// block but not the softmax, and needs fewer registers: 4 waves, 64-key
// blocks and four workgroups per CU, four waves per SIMD.
//
// K/V tiles go HBM -> LDS with buffer loads that write LDS directly (no
// staging registers; rows past N come back as zeros) into a 2-stage ring.
// Tiles are row-major, D*2 bytes per row, with the 16-byte chunks of row r
// XOR-permuted by tile_swz(r) so that both the row reads of K (ds_read_b128, 16
// rows at one column) and the transposing reads of V (ds_read_b64_tr_b16, 4
// rows x 64 bytes) hit distinct LDS banks.
//
// Lazy rescaling: the running max m that the exponentials subtract only
// guards them against overflow and underflow. l and the accumulator share it,
// so the final O = acc / l and lse do not depend on its value, and p =
// exp2(s*c - m) may exceed 1 (bf16 and the float32 accumulators hold such p
// without loss). Two forms:
//   * d = 128: m moves only when a block's max exceeds it by more than kTau
//     (log2 units). For typical data the max is settled by the first block,
//     and the per-block rescale of the 64 accumulator registers disappears.
//   * d = 64 (where the softmax weighs twice as much against the matrix work):
//     the block max is formed only on key block 0, which every row sees, so
//     every row's max gives p = 1 there and l >= 1 from then on (later
//     probabilities that underflow are negligible against it). On later
//     blocks p is taken with the m already held, and the lane's sum of its p
//     (which bounds each of them, all being non-negative) is checked against
//     kSumMax; a block that exceeds it (or overflows) is formed again with the
//     max path. This saves the row max of every later block. At d = 128 the
//     same form measured slower: with its extra code paths the loop spills
//     scalar registers, and their reloads cost more vector instructions than
//     the row max they replace.
constexpr float kTau = 8.f;
constexpr float kSumMax = 256.f;


template <int D, int BC, int NW, int LB, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(64 * NW, LB) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, int BH, int G, int N, int nqb, float c, int pass_wgs) {
  constexpr int BR = 32 * NW;
  constexpr int NKT = BC / 32;  // 32-key tiles per block
  constexpr int ROWB = 2 * D;          // bytes per tile row
  constexpr int TILEB = BC * ROWB;     // bytes per K (or V) tile
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int NI = CPR * BC / 64 / NW;  // load instructions per wave per tile
  constexpr int NDT = D / 32, NKS = D / 16;
  static_assert(NI >= 1 && CPR % NW == 0, "tile load split");
  // Ring stages [K | V], one object each (see dma_to_lds).
  __shared__ __attribute__((aligned(1024))) char lds0[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * TILEB];

  // pass_wgs > 0: the whole grid is resident at once, in passes of one
  // workgroup per CU (pass_wgs = the CU count). Workgroups are then placed
  // when the grid starts, not as CUs free up, so heaviest-first order alone
  // would give a CU the heaviest block of every pass. Odd passes run in
  // reverse order within each XCD (workgroup w goes to XCD w mod 8, which
  // the reversal keeps), pairing heavy blocks with light ones on each CU.
  int bid = blockIdx.x;
  if (pass_wgs > 0) {
    const int r = bid / pass_wgs, i = bid - r * pass_wgs;
    if (r & 1) bid = r * pass_wgs + 8 * (pass_wgs / 8 - 1 - (i >> 3)) + (i & 7);
  }
  int bh, qb;
  map_head_block(bid, BH, G, nqb, false, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;         // query head
  const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qw = qb * BR + 32 * wave_u;  // first query row of this wave (wave-uniform: scalar branches below)
  const int q = qw + col;

  const rsrc_t kr = buffer_rsrc(K + kvoff, (unsigned)N * ROWB);
  const rsrc_t vr = buffer_rsrc(V + kvoff, (unsigned)N * ROWB);

  // Load addressing: instruction n of this wave fills tile chunks
  // 64 (NI wave + n) + lane, i.e. row p / CPR, physical chunk p % CPR, which
  // holds logical chunk (p % CPR) ^ tile_swz(row).
  unsigned goff[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int p = 64 * (NI * wave + n) + lane, row = p / CPR, pc = p % CPR;  // row < BC
    goff[n] = row * ROWB + 16 * (pc ^ tile_swz<D>(row));
  }
  auto issue_loads = [&](int kb, char* st) {
    const unsigned base = (unsigned)kb * TILEB;
    char* const la = st + 1024 * NI * wave_u;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      dma_to_lds<16>(kr, la + 1024 * n, base + goff[n]);
      dma_to_lds<16>(vr, la + TILEB + 1024 * n, base + goff[n]);
    }
  };

  // Read addressing. The per-lane offsets are held as LDS addresses, one set
  // per stage (the second stage lies beyond the 16-bit immediate offset of
  // LDS reads), hidden from the optimiser, which would otherwise rebuild
  // them with one vector add per read. A read takes the stage object plus
  // (held address - address of the object): the compiler folds that back
  // to the held register and still knows which object is read.
  const int lds_at[2] = {(int)lds_addr(lds0), (int)lds_addr(lds1)};
  int koff[2][NKS];  // K row (32 kt + col), logical chunk 2 kk + hi; + kt * 32 * ROWB
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    const int o = col * ROWB + 16 * ((2 * kk + hi) ^ tile_swz<D>(col));
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      koff[st][kk] = o + lds_at[st];
      asm volatile("" : "+v"(koff[st][kk]));
    }
  }
  int voff[2][NDT][2];  // V row 4 hi + (j >> 2) + 8 sec, byte column 64 dt + 32 g + 8 (j & 3)
  {
    const int j = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int r = 4 * hi + (j >> 2) + 8 * sec;
        const int bcol = 64 * dt + 32 * g + 8 * (j & 3);
        const int o = TILEB + r * ROWB + 16 * ((bcol >> 4) ^ tile_swz<D>(r)) + (bcol & 15);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          voff[st][dt][sec] = o + lds_at[st];
          asm volatile("" : "+v"(voff[st][dt][sec]));
        }
      }
  }

  // Q^T fragments (B operand): lane holds Q[q][16 ks + 8 hi + 0..7].
  bf16x8 qf[NKS];
  {
    const bf16x8* src = (const bf16x8*)(Q + hoff + (size_t)(q < N ? q : 0) * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 x = src[2 * ks + hi];
      qf[ks] = q < N ? x : bf16x8{};
    }
  }

  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int nkb_all = (N + BC - 1) / BC;
  const int q_last = min(N - 1, qb * BR + BR - 1);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;

  // SUMCHECK selects the second form of the lazy rescale above. FIRST: key
  // block 0, which every row of the wave sees (at least key 0).
  constexpr bool SUMCHECK = D == 64;
  enum { kNoMax, kExactMax };
  auto compute = [&](int kb, auto stage, auto first) {
    constexpr int S = decltype(stage)::value;
    constexpr bool FIRST = decltype(first)::value;
    const char* const lb = (S == 0 ? lds0 : lds1) - lds_at[S];  // + a held address: inside the stage object
    const int k0 = kb * BC;
    if (CAUSAL && !FIRST && k0 > qw + 31) return;  // every key of the block is after every query of the wave
    auto scores = [&](f32x16 (&s)[NKT]) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};
      // k-step outer: the NKT products of one step are independent, and the
      // fragment reads of the next step are issued before them (the fences
      // keep the scheduler from sinking the reads next to their use).
      bf16x8 a[2][NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) a[0][kt] = *(const bf16x8*)(lb + koff[S][0] + kt * 32 * ROWB);
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        if (kk + 1 < NKS) {
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
            a[(kk + 1) & 1][kt] = *(const bf16x8*)(lb + koff[S][kk + 1] + kt * 32 * ROWB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) s[kt] = mfma_bf16(a[kk & 1][kt], qf[kk], s[kt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw)) {
        // key index of register i of tile kt: k0 + 32 kt + 8 (i / 4) + 4 hi + i % 4
        const int lim = min(CAUSAL ? q : N - 1, N - 1) - k0 - 4 * hi;  // keep iff offset <= lim
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + (i % 4) > lim) s[kt][i] = kNegInf;
      }
    };
    float rs0, rs1;
    bf16x8 pf[NKT][2];
    auto probs = [&](f32x16 (&s)[NKT], auto mode) __attribute__((always_inline)) {
      constexpr int MODE = decltype(mode)::value;
      if constexpr (MODE != kNoMax) {
        float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
        for (int kt = 0; kt < NKT; kt += 2)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            mx0 = fmaxf(fmaxf(mx0, s[kt][i]), s[kt][i + 1]);
            mx1 = fmaxf(fmaxf(mx1, s[kt + 1][i]), s[kt + 1][i + 1]);
          }
        const float mx = pair_max(fmaxf(mx0, mx1)) * c;
        const bool upd = mx > m;
        if (__builtin_amdgcn_ballot_w64(upd)) {  // wave-uniform, rare after the first block
          const float alpha = upd ? fast_exp2(m - mx) : 1.f;  // 0 while m is still -inf (l, acc are 0)
          if (upd) m = mx;
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
        }
      }
      const float nm = (m == kNegInf) ? 0.f : -m;
      rs0 = 0.f;
      rs1 = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) p[j] = fast_exp2(__builtin_fmaf(s[kt][8 * h2 + j], c, nm));
          rs0 += (p[0] + p[1]) + (p[2] + p[3]);
          rs1 += (p[4] + p[5]) + (p[6] + p[7]);
          pf[kt][h2] = bf16x8{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3],
                              (bf16)p[4], (bf16)p[5], (bf16)p[6], (bf16)p[7]};
        }
    };
    using Exact = std::integral_constant<int, kExactMax>;
    if constexpr (SUMCHECK) {
      {
        f32x16 s[NKT];
        scores(s);
        if constexpr (FIRST) probs(s, Exact{});
        else probs(s, std::integral_constant<int, kNoMax>{});
      }
      if (!FIRST && __builtin_amdgcn_ballot_w64(!(rs0 + rs1 <= kSumMax))) {  // rare; also catches +inf
        // Formed again with the max path, after which every p is at most 1.
        f32x16 s[NKT];
        scores(s);
        probs(s, Exact{});
      }
    } else {  // the scores and the per-block lazy max written out in place (as lambdas they cost SGPR spills)
      f32x16 s[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};
      bf16x8 a[2][NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) a[0][kt] = *(const bf16x8*)(lb + koff[S][0] + kt * 32 * ROWB);
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        if (kk + 1 < NKS) {
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
            a[(kk + 1) & 1][kt] = *(const bf16x8*)(lb + koff[S][kk + 1] + kt * 32 * ROWB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) s[kt] = mfma_bf16(a[kk & 1][kt], qf[kk], s[kt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw)) {
        const int lim = min(CAUSAL ? q : N - 1, N - 1) - k0 - 4 * hi;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + 8 * (i / 4) + (i % 4) > lim) s[kt][i] = kNegInf;
      }
      float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
      for (int kt = 0; kt < NKT; kt += 2)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          mx0 = fmaxf(fmaxf(mx0, s[kt][i]), s[kt][i + 1]);
          mx1 = fmaxf(fmaxf(mx1, s[kt + 1][i]), s[kt + 1][i + 1]);
        }
      const float mx = pair_max(fmaxf(mx0, mx1)) * c;
      const bool upd = mx > m + kTau;
      if (__builtin_amdgcn_ballot_w64(upd)) {  // wave-uniform, rare after the first block
        const float alpha = upd ? fast_exp2(m - mx) : 1.f;
        if (upd) m = mx;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
      }
      const float nm = (m == kNegInf) ? 0.f : -m;
      rs0 = 0.f;
      rs1 = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) p[j] = fast_exp2(__builtin_fmaf(s[kt][8 * h2 + j], c, nm));
          rs0 += (p[0] + p[1]) + (p[2] + p[3]);
          rs1 += (p[4] + p[5]) + (p[6] + p[7]);
          pf[kt][h2] = bf16x8{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3],
                              (bf16)p[4], (bf16)p[5], (bf16)p[6], (bf16)p[7]};
        }
    }
    l += pair_sum(rs0 + rs1);
    // O^T += V^T P^T; contraction slots per 16-key step: lanes 0-31 keys
    // {0-3, 8-11}, lanes 32-63 keys {4-7, 12-15} (the accumulator rows).
    // Step outer, as for the scores: the NDT products of a step are
    // independent and the next step's transposing reads are issued first.
    constexpr int NST = 2 * NKT;  // 16-key steps per block
    auto vread = [&](int st, int dt) __attribute__((always_inline)) {
      const int rb = 16 * st * ROWB;
      return cat4(lds_read_tr16((const bf16*)(lb + voff[S][dt][0] + rb)),
                  lds_read_tr16((const bf16*)(lb + voff[S][dt][1] + rb)));
    };
    bf16x8 vf[2][NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vf[0][dt] = vread(0, dt);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + 1 < NST) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vf[(st + 1) & 1][dt] = vread(st + 1, dt);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = mfma_bf16(vf[st & 1][dt], pf[st >> 1][st & 1], acc[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using Stage0 = std::integral_constant<int, 0>;
  using Stage1 = std::integral_constant<int, 1>;
  using Later = std::false_type;
  issue_loads(0, lds0);
  if constexpr (SUMCHECK) {  // key block 0 peeled: it alone forms the max
    wait_vmem();
    __syncthreads();
    if (1 < nkb) issue_loads(1, lds1);
    compute(0, Stage0{}, std::true_type{});
    for (int kb = 1; kb < nkb; kb += 2) {
      wait_vmem();
      __syncthreads();
      if (kb + 1 < nkb) issue_loads(kb + 1, lds0);
      compute(kb, Stage1{}, Later{});
      if (kb + 1 < nkb) {
        wait_vmem();
        __syncthreads();
        if (kb + 2 < nkb) issue_loads(kb + 2, lds1);
        compute(kb + 1, Stage0{}, Later{});
      }
    }
  } else {
    for (int kb = 0; kb < nkb; kb += 2) {
      wait_vmem();
      __syncthreads();
      if (kb + 1 < nkb) issue_loads(kb + 1, lds1);
      compute(kb, Stage0{}, Later{});
      if (kb + 1 < nkb) {
        wait_vmem();
        __syncthreads();
        if (kb + 2 < nkb) issue_loads(kb + 2, lds0);
        compute(kb + 1, Stage1{}, Later{});
      }
    }
  }

  // Epilogue: O = acc / l, lse = (m + log2 l) * ln 2 (m in log2 units of the scaled scores).
  if (q < N) {
    const float inv = 1.f / l;
    OutT* dst = O + hoff + (size_t)q * D + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        OutStore<OutT>::store4(dst + 32 * dt + 8 * g, acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv,
                               acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
    if (hi == 0) LSE[(size_t)bh * N + q] = (m + __log2f(l)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// float32 operands (P kept in float32), v_mfma_f32_32x32x2_f32. One
// workgroup per (batch*head, 32 query rows); its 4 waves split the key blocks
// of 32 (wave w takes blocks w, w + 4, ...), each keeping its own running
// max, denominator and output accumulator over its keys, and the 4 partial
// results are merged through LDS with the combine that the online softmax
// applies between blocks: m = max m_w, l = sum l_w 2^(m_w - m),
// O = sum acc_w 2^(m_w - m) / l. At float32 matrix-core rates this path is
// latency-bound at the sizes it serves, so the split shortens each wave's
// serial chain fourfold. K-step i of O^T += V^T P^T pairs accumulator
// register i of both half-waves, so P needs no conversion.
template <int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, int BH, int G, int N, int nqb, float c) {
  constexpr int NWV = 4, BC = 32;
  constexpr int KS = D + 4, VS = D + 4;  // padded rows: conflict-free column reads
  constexpr int KT = BC * KS, VT = BC * VS;
  constexpr int NDT = D / 32;
  // Per wave: its K and V tiles; reused at the end for its partial result
  // (acc as [d][32 rows], then m[32], l[32]).
  constexpr int WAVE_FLOATS = KT + VT;
  static_assert(D * 32 + 64 <= WAVE_FLOATS, "partial result fits in the wave's tiles");
  __shared__ __attribute__((aligned(16))) float smem[NWV * WAVE_FLOATS];

  int bh, qb;
  map_head_block(blockIdx.x, BH, G, nqb, false, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;         // query head
  const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head
  const int q0 = qb * 32;
  const int q = q0 + col;
  float* ks = smem + wave * WAVE_FLOATS;
  float* vs = ks + KT;

  float qf[D / 2];
  {
    const float* src = Q + hoff + (size_t)(q < N ? q : 0) * D;
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qf[kk] = (q < N) ? src[2 * kk + hi] : 0.f;
  }
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int nkb_all = (N + BC - 1) / BC;
  const int q_last = min(N - 1, q0 + 31);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;

  for (int kb = wave; kb < nkb; kb += NWV) {
    const int k0 = kb * BC;
    // The wave's own tiles: every earlier read of them has returned (its
    // values fed the products), so they can be overwritten; the wave-level
    // fences order these stores before the reads below.
    for (int idx = lane; idx < BC * D / 4; idx += 64) {
      const int row = idx / (D / 4), c4 = idx % (D / 4), key = k0 + row;
      f32x4 kx = {}, vx = {};
      if (key < N) {
        kx = *(const f32x4*)(K + kvoff + (size_t)key * D + 4 * c4);
        vx = *(const f32x4*)(V + kvoff + (size_t)key * D + 4 * c4);
      }
      *(f32x4*)(ks + row * KS + 4 * c4) = kx;
      *(f32x4*)(vs + row * VS + 4 * c4) = vx;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x16 s = {};
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) s = mfma_f32(ks[col * KS + 2 * kk + hi], qf[kk], s);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + 8 * (i / 4) + 4 * hi + (i % 4);
      if (key >= N || (CAUSAL && key > q)) s[i] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = fast_exp2(__builtin_fmaf(s[i], c, -m_use));
      rs += s[i];
    }
    rs += xor32(rs);
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      acc[dt] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i / 4) + 4 * hi + (i % 4);
        acc[dt] = mfma_f32(vs[key * VS + 32 * dt + col], s[i], acc[dt]);
      }
    }
  }

  // Merge. Register i of acc[dt] holds dimension 32 dt + 8 (i / 4) + 4 hi + i % 4
  // of query row col. Each wave stores its partial over its own tiles (its
  // reads of them have all returned); after the barrier, wave w < NDT
  // combines dimensions 32 w .. 32 w + 31 of all 32 rows (a wave whose keys
  // were all masked holds m = -inf and weighs 0).
  {
    float* part = ks;  // [d][32 rows], then m[32], l[32]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) part[(32 * dt + 8 * (i / 4) + 4 * hi + (i % 4)) * 32 + col] = acc[dt][i];
    if (hi == 0) {
      part[D * 32 + col] = m;
      part[D * 32 + 32 + col] = l;
    }
  }
  __syncthreads();
  if (wave < NDT && q < N) {
    float mw[NWV], M = kNegInf;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      mw[w] = smem[w * WAVE_FLOATS + D * 32 + col];
      M = fmaxf(M, mw[w]);
    }
    float fw[NWV], L = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      fw[w] = mw[w] == kNegInf ? 0.f : fast_exp2(mw[w] - M);
      L += smem[w * WAVE_FLOATS + D * 32 + 32 + col] * fw[w];
    }
    const float inv = 1.f / L;
    OutT* dst = O + hoff + (size_t)q * D + 32 * wave;
    // Lane (hi, col) writes dimensions 32 wave + 16 hi .. + 15 of row col.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float o4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int dd = 32 * wave + 16 * hi + 4 * g + r;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) v += smem[w * WAVE_FLOATS + dd * 32 + col] * fw[w];
        o4[r] = v * inv;
      }
      OutStore<OutT>::store4(dst + 16 * hi + 4 * g, o4[0], o4[1], o4[2], o4[3]);
    }
    if (wave == 0 && hi == 0) LSE[(size_t)bh * N + q] = (M + __log2f(L)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Host-side launch selection.

// Compute units of the current device (0 if the runtime cannot say).
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

template <int D, bool CAUSAL, typename OutT>
static hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                              int G, int N, float c, hipStream_t st) {
  constexpr int NW = D == 64 ? 4 : 8, BC = D == 64 ? 64 : 128, LB = D == 64 ? 4 : 1;
  const int nqb = (N + 32 * NW - 1) / (32 * NW);
  const long wgs = (long)BH * nqb;
  // Causal grids that the CUs hold at once, in two or more whole passes, get
  // the alternating pass order (unequal blocks, no dynamic balancing).
  int pass_wgs = 0;
  if (CAUSAL && LB > 1) {
    const int cus = device_cu_count();
    if (cus > 0 && cus % 8 == 0 && wgs % cus == 0 && wgs / cus >= 2 && wgs <= (long)cus * LB) pass_wgs = cus;
  }
  return launch_kernel(fwd_bf16_kernel<D, BC, NW, LB, CAUSAL, OutT>, dim3(BH * nqb), dim3(64 * NW), st, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (OutT*)o, lse, BH, G, N, nqb, c, pass_wgs);
}

template <int D, bool CAUSAL, typename OutT>
static hipError_t launch_f32(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                             int G, int N, float c, hipStream_t st) {
  const int nqb = (N + 31) / 32;
  return launch_kernel(fwd_f32_kernel<D, CAUSAL, OutT>, dim3(BH * nqb), dim3(256), st, (const float*)q,
                       (const float*)k, (const float*)v, (OutT*)o, lse, BH, G, N, nqb, c);
}

#define FA_DISPATCH(FN, D, causal, OT, ...)                                        \
  ((D) == 64 ? ((causal) ? FN<64, true, OT>(__VA_ARGS__) : FN<64, false, OT>(__VA_ARGS__)) \
             : ((causal) ? FN<128, true, OT>(__VA_ARGS__) : FN<128, false, OT>(__VA_ARGS__)))

int launch_forward(int in_dtype, int o_dtype, const void* q, const void* k, const void* v,
                   const float* descale, void* o, float* lse, int B, int H, int Hkv, int N, int d,
                   float scale, int causal, hipStream_t stream) {
  const int BH = B * H, G = H / Hkv;
  const float c = scale * kLog2e;
  hipError_t err;
  if (in_dtype == FA_BF16) {
    err = (o_dtype == FA_BF16) ? FA_DISPATCH(launch_bf16, d, causal, bf16, q, k, v, o, lse, BH, G, N, c, stream)
                               : FA_DISPATCH(launch_bf16, d, causal, float, q, k, v, o, lse, BH, G, N, c, stream);
  } else if (in_dtype == FA_F32) {
    err = (o_dtype == FA_BF16) ? FA_DISPATCH(launch_f32, d, causal, bf16, q, k, v, o, lse, BH, G, N, c, stream)
                               : FA_DISPATCH(launch_f32, d, causal, float, q, k, v, o, lse, BH, G, N, c, stream);
  } else if ((in_dtype == FA_FP8_E4M3 || in_dtype == FA_FP8_E5M2) && o_dtype == FA_BF16) {
    err = launch_forward_fp8(q, k, v, descale, o, lse, BH, G, N, d, scale, causal, in_dtype == FA_FP8_E5M2, stream);
  } else {
    return FA_ERR_UNSUPPORTED;
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
