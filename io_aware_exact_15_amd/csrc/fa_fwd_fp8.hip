// Forward pass with FP8 operands (the FP8 path of the version table on the
// FlashAttention-family multiple-choice page; E4M3 and E5M2 are named on the
// short-answer page, answer paragraph 2).
//
// Inputs are E4M3 or E5M2 codes (template FMT = 0 / 1, the instruction's
// operand format fields) with per-tensor float32 scales s_q, s_k, s_v (the
// values they stand for are code * s). Both products run on the fp8 matrix
// cores (v_mfma_f32_32x32x64_f8f6f4, float32 accumulation); P is always
// quantised to E4M3:
//   S^T = K Q^T           scaled by scale * s_q * s_k * log2(e) in the exponent
//   O^T += V^T P^T        P quantised to E4M3, O finished as acc * s_v / l
// The online softmax is the one of the bf16 kernel (running max m, running
// denominator l, accumulator rescaled by exp2(m - m_new), lazily: m moves only
// when a block's max exceeds it by more than 3 in log2 units). The
// probabilities are formed as p' = 2^5 * exp2(s c - m) <= 2^8 before
// quantisation, which keeps small probabilities clear of E4M3's subnormal
// range and large ones under its maximum (448); l sums the unrounded float32
// p', so the factor cancels in O = acc / l and lse subtracts 5 in log2 units.
//
// Operand layouts (per wave, K = 64 contraction per instruction): lane l
// holds 32 consecutive contraction bytes of row/column l % 32, half-wave
// l / 32 holding bytes 32..63. For P.V the 64-key step takes its contraction
// order from the score accumulators: accumulator row r of a 32-key tile holds
// key pi(r), where pi swaps bits 2 and 3 of r (K rows are stored to LDS in
// that order). Then lane half h holds keys {16 t + 8 h + 0..7}, t = 0..3, in
// its 32 bytes, and each 8-key group is one transposing LDS read
// (ds_read_b64_tr_b8) of 8 consecutive V rows.
#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

__device__ __forceinline__ int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Packs 4 floats (each in [0, 448]) into 4 E4M3 bytes, round to nearest even.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Swizzle of the 16-byte chunks of an fp8 tile row (D bytes): chunk c of row
// r is stored at c ^ swz8(r). Keeps the K row reads (two ds_read_b128 per
// operand, 16 rows at one chunk) and the V transposing reads (8 consecutive
// rows x 16 bytes) on distinct LDS banks.
template <int D>
__device__ __forceinline__ int swz8(int r) {
  if (D == 128) return (4 * ((r >> 1) & 1)) ^ ((r >> 2) & 3);  // 8 chunks per row
  return (r >> 2) & 3;                                        // 4 chunks per row
}

// The power-of-two scale of P before quantisation (p' = 2^kP8Shift p keeps
// small probabilities out of E4M3's subnormals longer) and the bound on a
// lane's sum of p' over a block, which bounds every p' of it (all are
// non-negative) below E4M3's largest value, 448.
//
// Lazy rescale: the running max m only guards the exponentials (l and the
// accumulator share it, so O and lse do not depend on its value). It is
// formed from the scores on key block 0, which every row sees, so every row's
// max gives p = 1 there and l >= 1 from then on (later probabilities that
// underflow are negligible against it). Later blocks take p with the m
// already held and check the lane's sum of p' against kSumMax8; a block that
// exceeds it (or overflows) is formed again with the max path. For N(0,1)
// data that sum averages ~150, so the retry is rare, and the row max of every
// later block is saved: this kernel is bound by its vector work.
constexpr float kP8Shift = 5.f;
constexpr float kSumMax8 = 384.f;

// 4 waves x 32 query rows (BR = 128), blocks of BC = 64 keys, three
// workgroups per CU (at most 168 registers: three waves per SIMD, whose
// barriers are independent; at d = 128 three values spill outside the key
// loop); K/V tiles HBM -> LDS by DMA into a 2-stage ring of 2 x 16 KB.
// The FP8 products take half the matrix-core time of bf16 ones while the
// softmax costs the same, so the kernel is bound by vector work, and more
// waves per SIMD to overlap it measured 1.5-2 % faster than 8 waves with
// 128-key blocks.
template <int D, bool CAUSAL, int FMT>
__global__ __launch_bounds__(256, 3) void fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                                         const uint8_t* __restrict__ V, bf16* __restrict__ O,
                                                         float* __restrict__ LSE, const float* __restrict__ descale,
                                                         int BH, int G, int N, int nqb, float scale) {
  constexpr int NW = 4, BR = 32 * NW, BC = 64;
  constexpr int ROWB = D, TILEB = BC * ROWB, CPR = D / 16;
  constexpr int NPW = CPR * BC / 64 / NW;  // 1024-byte DMA instructions per wave per tile
  constexpr int NKT = BC / 32, NDT = D / 32, NKS = D / 64, NPV = BC / 64;
  static_assert(NPW >= 1, "tile split");
  // Ring stages [K | V], one object each (see dma_to_lds).
  __shared__ __attribute__((aligned(1024))) char lds0[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * TILEB];

  int bh, qb;
  map_head_block(blockIdx.x, BH, G, nqb, false, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;         // query head
  const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qw = qb * BR + 32 * wave_u;  // wave-uniform: scalar branches below
  const int q = qw + col;
  const float s_v = descale[2];
  const float c = scale * descale[0] * descale[1] * kLog2e;

  const rsrc_t kr = buffer_rsrc(K + kvoff, (unsigned)N * ROWB);
  const rsrc_t vr = buffer_rsrc(V + kvoff, (unsigned)N * ROWB);
  // DMA: instruction n of this wave fills tile chunks 64 (NPW wave + n) + lane,
  // i.e. tile row R = p / CPR, physical chunk p % CPR holding logical chunk
  // (p % CPR) ^ swz8(R). K row R holds key pi(R) (bits 2 and 3 of R swapped);
  // V row R holds key R.
  unsigned koff_g[NPW], voff_g[NPW];
#pragma unroll
  for (int n = 0; n < NPW; ++n) {
    const int p = 64 * (NPW * wave + n) + lane, R = p / CPR, pc = p % CPR;
    const int lc = pc ^ swz8<D>(R);
    koff_g[n] = swap_bits23(R) * ROWB + 16 * lc;
    voff_g[n] = R * ROWB + 16 * lc;
  }
  auto issue_loads = [&](int kb, char* st) {
    const unsigned base = (unsigned)kb * TILEB;
    char* const la = st + 1024 * NPW * wave_u;
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      dma_to_lds<16>(kr, la + 1024 * n, base + koff_g[n]);
      dma_to_lds<16>(vr, la + TILEB + 1024 * n, base + voff_g[n]);
    }
  };
  // K operand reads: row 32 kt + col, bytes 64 kk + 32 hi .. + 31 (chunks 4 kk + 2 hi, + 1).
  int koff[NKS][2];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) koff[kk][h] = col * ROWB + 16 * ((4 * kk + 2 * hi + h) ^ swz8<D>(col));
  // V transposing reads: row 64 u + 16 t + 8 hi + (j >> 1), byte column 32 dt + 16 g + 8 (j & 1).
  int voff[NDT];
  {
    const int j = lane & 15, g = (lane >> 4) & 1;
    const int r = 8 * hi + (j >> 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) voff[dt] = r * ROWB + 16 * ((2 * dt + g) ^ swz8<D>(r)) + 8 * (j & 1);
  }

  i32x8 qf[NKS];
  {
    const i32x4* src = (const i32x4*)(Q + hoff + (size_t)(q < N ? q : 0) * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      i32x4 a = src[4 * ks + 2 * hi], b = src[4 * ks + 2 * hi + 1];
      if (q >= N) a = b = i32x4{};
      qf[ks] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
  }
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int nkb_all = (N + BC - 1) / BC;
  const int q_last = min(N - 1, qb * BR + BR - 1);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;

  enum { kNoMax, kExactMax };
  // FIRST: key block 0 (every row of the wave sees at least key 0 of it).
  auto compute = [&](int kb, const char* st, auto first) {
    constexpr bool FIRST = decltype(first)::value;
    const int k0 = kb * BC;
    if (CAUSAL && !FIRST && k0 > qw + 31) return;
    const char* ks = st;
    const char* vs = st + TILEB;
    auto scores = [&](f32x16 (&s)[NKT]) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        s[kt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const i32x4 a0 = *(const i32x4*)(ks + 32 * kt * ROWB + koff[kk][0]);
          const i32x4 a1 = *(const i32x4*)(ks + 32 * kt * ROWB + koff[kk][1]);
          const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          s[kt] = mfma_f8<FMT, FMT>(a, qf[kk], s[kt]);
        }
      }
      if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw)) {
        // register i of tile kt holds key k0 + 32 kt + (i & 7) + 8 hi + 16 (i >> 3)
        const int lim = min(CAUSAL ? q : N - 1, N - 1) - k0 - 8 * hi;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + (i & 7) + 16 * (i >> 3) > lim) s[kt][i] = kNegInf;
      }
    };
    float rs0, rs1;
    // p' = 2^kP8Shift p replaces the scores in s.
    auto probs = [&](f32x16 (&s)[NKT], auto mode) __attribute__((always_inline)) {
      if constexpr (decltype(mode)::value == kExactMax) {
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
        if (__builtin_amdgcn_ballot_w64(upd)) {
          const float alpha = upd ? fast_exp2(m - mx) : 1.f;  // 0 while m is still -inf (l, acc are 0)
          if (upd) m = mx;
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
        }
      }
      const float shift = kP8Shift - ((m == kNegInf) ? 0.f : m);
      rs0 = 0.f;
      rs1 = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kt][i], c, shift));
          const float p1 = fast_exp2(__builtin_fmaf(s[kt][i + 1], c, shift));
          s[kt][i] = p0;
          s[kt][i + 1] = p1;
          rs0 += p0;
          rs1 += p1;
        }
    };
    using Exact = std::integral_constant<int, kExactMax>;
    f32x16 s[NKT];
    scores(s);
    if constexpr (FIRST) probs(s, Exact{});
    else probs(s, std::integral_constant<int, kNoMax>{});
    if (!FIRST && __builtin_amdgcn_ballot_w64(!(rs0 + rs1 <= kSumMax8))) {  // rare; also catches +inf
      // Formed again with the max path, after which every p' is at most 2^kP8Shift.
      scores(s);
      probs(s, Exact{});
    }
    l += pair_sum(rs0 + rs1);
    // O^T += V^T P^T, 64-key steps; byte j of step u: tile 2u + j / 16, register j % 16.
#pragma unroll
    for (int u = 0; u < NPV; ++u) {
      i32x8 pf;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kt = 2 * u + w / 4, i0 = 4 * (w % 4);
        pf[w] = pack_fp8x4(s[kt][i0], s[kt][i0 + 1], s[kt][i0 + 2], s[kt][i0 + 3]);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        i32x8 a;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const i32x2 r = lds_read_tr8((const uint8_t*)(vs + (64 * u + 16 * t) * ROWB + voff[dt]));
          a[2 * t] = r[0];
          a[2 * t + 1] = r[1];
        }
        acc[dt] = mfma_f8<FMT, 0>(a, pf, acc[dt]);  // V in the input format, P in E4M3
      }
    }
  };

  issue_loads(0, lds0);
  wait_vmem();
  __syncthreads();
  if (1 < nkb) issue_loads(1, lds1);
  compute(0, lds0, std::true_type{});  // key block 0 peeled: it alone forms the max
  for (int kb = 1; kb < nkb; kb += 2) {
    wait_vmem();
    __syncthreads();
    if (kb + 1 < nkb) issue_loads(kb + 1, lds0);
    compute(kb, lds1, std::false_type{});
    if (kb + 1 < nkb) {
      wait_vmem();
      __syncthreads();
      if (kb + 2 < nkb) issue_loads(kb + 2, lds1);
      compute(kb + 1, lds0, std::false_type{});
    }
  }

  if (q < N) {
    const float f = s_v / l;
    bf16* dst = O + hoff + (size_t)q * D + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        bf16x4 v = {(bf16)(acc[dt][4 * gg] * f), (bf16)(acc[dt][4 * gg + 1] * f), (bf16)(acc[dt][4 * gg + 2] * f),
                    (bf16)(acc[dt][4 * gg + 3] * f)};
        *(bf16x4*)(dst + 32 * dt + 8 * gg) = v;
      }
    if (hi == 0) LSE[(size_t)bh * N + q] = (m + __log2f(l) - kP8Shift) * kLn2;
  }
}

template <int D, bool CAUSAL, int FMT>
static hipError_t launch_fp8_d(const void* q, const void* k, const void* v, const float* descale, void* o,
                               float* lse, int BH, int G, int N, float scale, hipStream_t st) {
  const int nqb = (N + 127) / 128;
  return launch_kernel(fwd_fp8_kernel<D, CAUSAL, FMT>, dim3(BH * nqb), dim3(256), st, (const uint8_t*)q,
                       (const uint8_t*)k, (const uint8_t*)v, (bf16*)o, lse, descale, BH, G, N, nqb, scale);
}

template <int FMT>
static hipError_t launch_fp8_fmt(const void* q, const void* k, const void* v, const float* descale, void* o,
                                 float* lse, int BH, int G, int N, int d, float scale, int causal, hipStream_t st) {
  if (d == 64) return causal ? launch_fp8_d<64, true, FMT>(q, k, v, descale, o, lse, BH, G, N, scale, st)
                             : launch_fp8_d<64, false, FMT>(q, k, v, descale, o, lse, BH, G, N, scale, st);
  return causal ? launch_fp8_d<128, true, FMT>(q, k, v, descale, o, lse, BH, G, N, scale, st)
                : launch_fp8_d<128, false, FMT>(q, k, v, descale, o, lse, BH, G, N, scale, st);
}

hipError_t launch_forward_fp8(const void* q, const void* k, const void* v, const float* descale, void* o, float* lse,
                              int BH, int G, int N, int d, float scale, int causal, int e5m2, hipStream_t st) {
  return e5m2 ? launch_fp8_fmt<1>(q, k, v, descale, o, lse, BH, G, N, d, scale, causal, st)
              : launch_fp8_fmt<0>(q, k, v, descale, o, lse, BH, G, N, d, scale, causal, st);
}

}  // namespace fa
