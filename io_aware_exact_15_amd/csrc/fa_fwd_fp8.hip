// Forward pass with FP8 E4M3 operands (the FP8 path of the version table on
// the FlashAttention-family multiple-choice page; E4M3 is named on the
// short-answer page, answer paragraph 2).
//
// Inputs are E4M3 codes with per-tensor float32 scales s_q, s_k, s_v (the
// values they stand for are code * s). Both products run on the fp8 matrix
// cores (v_mfma_f32_32x32x64_f8f6f4, float32 accumulation):
//   S^T = K Q^T           scaled by scale * s_q * s_k * log2(e) in the exponent
//   O^T += V^T P^T        P quantised to E4M3, O finished as acc * s_v / l
// The online softmax is the one of the bf16 kernel (running max m, running
// denominator l, accumulator rescaled by exp2(m - m_new)). The probabilities
// are formed as p' = 2^8 * p in [0, 256] before quantisation, which keeps
// small probabilities clear of E4M3's subnormal range; l sums the unrounded
// float32 p', so the factor cancels in O = acc / l and lse subtracts 8 in
// log2 units.
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

__device__ __forceinline__ void map_block8(int bid, int BH, int nqb, int& bh, int& qb) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, j = bid >> 3, hpx = BH >> 3;
    qb = nqb - 1 - j / hpx;
    bh = xcd + 8 * (j % hpx);
  } else {
    qb = nqb - 1 - bid / BH;
    bh = bid % BH;
  }
}

// Packs 4 floats (each in [0, 448]) into 4 E4M3 bytes, round to nearest even.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D, int QT, int BC, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                                         const uint8_t* __restrict__ V, bf16* __restrict__ O,
                                                         float* __restrict__ LSE, const float* __restrict__ descale,
                                                         int BH, int N, int nqb, float scale) {
  constexpr int BR = 128 * QT;
  constexpr int KS = D + 16, VS = D + 16;  // LDS row strides (bytes)
  constexpr int KT = BC * KS, VT = BC * VS;
  constexpr int NKT = BC / 32, NDT = D / 32, NKS = D / 64, NPV = BC / 64;
  constexpr int CHUNKS = BC * D / 16;
  constexpr int CPT = CHUNKS / 256;
  static_assert(CHUNKS % 256 == 0 && BC % 64 == 0, "tile split");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (KT + VT)];

  int bh, qb;
  map_block8(blockIdx.x, BH, nqb, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;
  const int q0 = qb * BR + wave * 32 * QT;
  const float s_v = descale[2];
  const float c = scale * descale[0] * descale[1] * kLog2e;

  i32x8 qf[QT][NKS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 32 * qt + col;
    const i32x4* src = (const i32x4*)(Q + hoff + (size_t)(q < N ? q : 0) * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      i32x4 a = src[4 * ks + 2 * hi], b = src[4 * ks + 2 * hi + 1];
      if (q >= N) a = b = i32x4{};
      qf[qt][ks] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
  }
  f32x16 acc[QT][NDT];
  float m[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = kNegInf;
    l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] = f32x16{};
  }

  const int nkb_all = (N + BC - 1) / BC;
  const int q_last = min(N - 1, qb * BR + BR - 1);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;

  i32x4 kreg[CPT], vreg[CPT];
  auto load_regs = [&](int kb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 16), c16 = idx % (D / 16);
      const int key = kb * BC + row;
      const size_t off = hoff + (size_t)(key < N ? key : 0) * D + 16 * c16;  // clamped: always in bounds
      const i32x4 a = *(const i32x4*)(K + off), b = *(const i32x4*)(V + off);
      kreg[i] = key < N ? a : i32x4{};
      vreg[i] = key < N ? b : i32x4{};
    }
  };
  auto store_lds = [&](int buf) {
    uint8_t* ks = smem + buf * (KT + VT);
    uint8_t* vs = ks + KT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 16), c16 = idx % (D / 16);
      *(i32x4*)(ks + swap_bits23(row) * KS + 16 * c16) = kreg[i];
      *(i32x4*)(vs + row * VS + 16 * c16) = vreg[i];
    }
  };

  load_regs(0);
  store_lds(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_regs(kb + 1);
    const uint8_t* ks = smem + buf * (KT + VT);
    const uint8_t* vs = ks + KT;
    const int k0 = kb * BC;
    if (!CAUSAL || k0 <= q0 + 32 * QT - 1) {
      f32x16 s[QT][NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[qt][kt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const i32x4* src = (const i32x4*)(ks + (32 * kt + col) * KS + 64 * kk + 32 * hi);
          const i32x4 a0 = src[0], a1 = src[1];
          const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) s[qt][kt] = mfma_fp8(a, qf[qt][kk], s[qt][kt]);
        }
      }
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
      i32x8 pf[QT][NPV];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (need_mask) {
          const int q = q0 + 32 * qt + col;
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              // accumulator row 8 (i/4) + 4 hi + i % 4 holds key pi(row) = (i & 7) + 8 hi + 16 (i >> 3)
              const int key = k0 + 32 * kt + (i & 7) + 8 * hi + 16 * (i >> 3);
              if (key >= N || (CAUSAL && key > q)) s[qt][kt][i] = kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qt][kt][i]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m[qt], mx * c);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m[qt] - m_use);
        const float shift = 8.f - m_use;  // p' = 2^8 p
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(__builtin_fmaf(s[qt][kt][i], c, shift));
            s[qt][kt][i] = p;
            rs += p;
          }
        rs += xor32(rs);
        l[qt] = l[qt] * alpha + rs;
        m[qt] = m_new;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] *= alpha;
        // Byte j of the 64-key step u: tile kt = 2u + j / 16, accumulator register j % 16.
#pragma unroll
        for (int u = 0; u < NPV; ++u)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int kt = 2 * u + w / 4, i0 = 4 * (w % 4);
            pf[qt][u][w] = pack_fp8x4(s[qt][kt][i0], s[qt][kt][i0 + 1], s[qt][kt][i0 + 2], s[qt][kt][i0 + 3]);
          }
      }
      // O^T += V^T P^T. Transposing read t of step u covers V rows 64 u + 16 t + 8 hi + 0..7:
      // lane j of each 16-lane group reads row (j / 2), bytes 8 (j % 2) .. + 7 of its 16 columns.
      const int jl = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int u = 0; u < NPV; ++u) {
          i32x8 a;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint8_t* p = vs + (64 * u + 16 * t + 8 * hi + (jl >> 1)) * VS + 32 * dt + 16 * g + 8 * (jl & 1);
            const i32x2 r = lds_read_tr8(p);
            a[2 * t] = r[0];
            a[2 * t + 1] = r[1];
          }
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) acc[qt][dt] = mfma_fp8(a, pf[qt][u], acc[qt][dt]);
        }
    }
    if (kb + 1 < nkb) store_lds(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 32 * qt + col;
    if (q < N) {
      const float f = s_v / l[qt];
      bf16* dst = O + hoff + (size_t)q * D + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          bf16x4 v = {(bf16)(acc[qt][dt][4 * gg] * f), (bf16)(acc[qt][dt][4 * gg + 1] * f),
                      (bf16)(acc[qt][dt][4 * gg + 2] * f), (bf16)(acc[qt][dt][4 * gg + 3] * f)};
          *(bf16x4*)(dst + 32 * dt + 8 * gg) = v;
        }
      if (hi == 0) LSE[(size_t)bh * N + q] = (m[qt] + __log2f(l[qt]) - 8.f) * kLn2;
    }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fp8_d(const void* q, const void* k, const void* v, const float* descale, void* o,
                               float* lse, int BH, int N, float scale, hipStream_t st) {
  constexpr int QT = 1, BC = 64;
  const int nqb = (N + 128 * QT - 1) / (128 * QT);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, QT, BC, CAUSAL>), dim3(BH * nqb), dim3(256), 0, st, (const uint8_t*)q,
                     (const uint8_t*)k, (const uint8_t*)v, (bf16*)o, lse, descale, BH, N, nqb, scale);
  return hipGetLastError();
}

hipError_t launch_forward_fp8(const void* q, const void* k, const void* v, const float* descale, void* o, float* lse,
                              int BH, int N, int d, float scale, int causal, hipStream_t st) {
  if (d == 64) return causal ? launch_fp8_d<64, true>(q, k, v, descale, o, lse, BH, N, scale, st)
                             : launch_fp8_d<64, false>(q, k, v, descale, o, lse, BH, N, scale, st);
  return causal ? launch_fp8_d<128, true>(q, k, v, descale, o, lse, BH, N, scale, st)
                : launch_fp8_d<128, false>(q, k, v, descale, o, lse, BH, N, scale, st);
}

}  // namespace fa
