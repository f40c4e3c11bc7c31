// Forward pass of exact attention: O = softmax(scale * Q K^T) V and the
// per-row log-sum-exp, one workgroup per (batch*head, block of query rows).
//
// The method: tile Q into row blocks and K, V into column blocks, and for
// each Q block stream the K/V blocks through on-chip memory while keeping a
// running row maximum m, a running denominator l and a rescaled output
// accumulator (the card "FlashAttention Kernel & Online Softmax", definition
// paragraph; the "FlashAttention" explainer by A. Tiwari). When a block
// raises the maximum, l and the accumulator are multiplied by exp(m - m_new);
// one division by l finishes each row. The N x N matrix never leaves
// registers.
//
// gfx950 mapping (per wave of 64 lanes, 32*QT query rows):
//   * Scores are formed transposed, S^T = K Q^T, on the matrix cores: the
//     accumulator layout then gives every lane one query column and 16 keys,
//     so the row max and row sum are in-lane loops plus one exchange with the
//     partner half-wave.
//   * The probabilities P^T, converted in place, are directly the B operand
//     of O^T += V^T P^T; V^T comes from the row-major V tile in LDS through
//     the transposing LDS read, with the contraction (key) order chosen to
//     match the accumulator layout.
//   * Q stays in registers for the whole kernel; K and V tiles are staged
//     HBM -> registers -> LDS one block ahead (double-buffered LDS).
//   * Base-2 exponentials with scale*log2(e) folded into one FMA; the
//     denominator l is summed from the unrounded float32 probabilities.
//   * Causal: key blocks past the diagonal are never visited; only blocks
//     that cross the diagonal (or the ragged tail) are masked element-wise.
//   * Grid order: heaviest causal query blocks first; all query blocks of a
//     head go to the same XCD (workgroups are dealt round-robin to the 8
//     XCDs) so that its K/V stream is shared through one L2.
#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

// Maps the linear workgroup id to (bh, qb): heavy-first query blocks, and
// when BH is a multiple of 8 every query block of head bh runs on XCD bh % 8.
__device__ __forceinline__ void map_block(int bid, int BH, int nqb, int& bh, int& qb) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, j = bid >> 3, hpx = BH >> 3;
    qb = nqb - 1 - j / hpx;
    bh = xcd + 8 * (j % hpx);
  } else {
    qb = nqb - 1 - bid / BH;
    bh = bid % BH;
  }
}

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
// bf16 operands. D: head size; QT: 32-row query tiles per wave; BC: keys per
// block; 4 waves per workgroup (BR = 128 * QT query rows).
template <int D, int QT, int BC, bool CAUSAL, typename OutT, int MINB>
__global__ __launch_bounds__(256, MINB) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqb, float c) {
  constexpr int BR = 128 * QT;
  constexpr int KS = D + 8;    // K tile row stride (elements), 16-byte multiple
  constexpr int VS = D + 16;   // V tile row stride
  constexpr int KT = BC * KS, VT = BC * VS;
  constexpr int NKT = BC / 32;  // 32-key sub-tiles per block
  constexpr int NDT = D / 32;   // 32-dim output tiles
  constexpr int NKS = D / 16;   // k-steps of S^T = K Q^T
  constexpr int CHUNKS = BC * D / 8;  // 16-byte chunks per K (or V) tile
  constexpr int CPT = CHUNKS / 256;
  static_assert(CHUNKS % 256 == 0, "tile must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (KT + VT)];

  int bh, qb;
  map_block(blockIdx.x, BH, nqb, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;
  const int q0 = qb * BR + wave * 32 * QT;  // first query row of this wave

  // Q^T fragments (B operand): lane holds Q[q][16 ks + 8 hi + 0..7].
  bf16x8 qf[QT][NKS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 32 * qt + col;
    const bf16x8* src = (const bf16x8*)(Q + hoff + (size_t)(q < N ? q : 0) * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 x = src[2 * ks + hi];
      if (q >= N) x = bf16x8{};
      qf[qt][ks] = x;
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
      const int idx = tid + 256 * i, row = idx / (D / 8), c8 = idx % (D / 8);
      const int key = kb * BC + row;
      const size_t off = hoff + (size_t)(key < N ? key : 0) * D + c8 * 8;  // clamped: always in bounds
      const i32x4 a = *(const i32x4*)(K + off), b = *(const i32x4*)(V + off);
      kreg[i] = key < N ? a : i32x4{};
      vreg[i] = key < N ? b : i32x4{};
    }
  };
  auto store_lds = [&](int buf) {
    bf16* ks = smem + buf * (KT + VT);
    bf16* vs = ks + KT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 8), c8 = idx % (D / 8);
      *(i32x4*)(ks + row * KS + c8 * 8) = kreg[i];
      *(i32x4*)(vs + row * VS + c8 * 8) = vreg[i];
    }
  };

  load_regs(0);
  store_lds(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_regs(kb + 1);
    const bf16* ks = smem + buf * (KT + VT);
    const bf16* vs = ks + KT;
    const int k0 = kb * BC;
    const bool active = !CAUSAL || k0 <= q0 + 32 * QT - 1;
    if (active) {
      // S^T = K Q^T for BC keys x 32 QT queries.
      f32x16 s[QT][NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[qt][kt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const bf16x8 a = *(const bf16x8*)(ks + (32 * kt + col) * KS + 16 * kk + 8 * hi);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) s[qt][kt] = mfma_bf16(a, qf[qt][kk], s[qt][kt]);
        }
      }
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
      bf16x8 pf[QT][NKT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (need_mask) {
          const int q = q0 + 32 * qt + col;
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = k0 + 32 * kt + 8 * (i / 4) + 4 * hi + (i % 4);
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
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(__builtin_fmaf(s[qt][kt][i], c, -m_use));
            s[qt][kt][i] = p;
            rs += p;
          }
        rs += xor32(rs);
        l[qt] = l[qt] * alpha + rs;
        m[qt] = m_new;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] *= alpha;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            bf16x8 x;
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = (bf16)s[qt][kt][8 * h2 + j];
            pf[qt][kt][h2] = x;
          }
      }
      // O^T += V^T P^T. Contraction slot order per 16-key step (matching the
      // accumulator rows a lane holds): lanes 0-31 keys {0-3, 8-11}, lanes
      // 32-63 keys {4-7, 12-15}.
      const int trow = 4 * hi + ((lane & 15) >> 2);
      const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const bf16* p0 = vs + (32 * kt + 16 * h2 + trow) * VS + 32 * dt + tcol;
            const bf16x8 a = cat4(lds_read_tr16(p0), lds_read_tr16(p0 + 8 * VS));
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) acc[qt][dt] = mfma_bf16(a, pf[qt][kt][h2], acc[qt][dt]);
          }
    }
    if (kb + 1 < nkb) store_lds(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l, lse = (m + log2 l) * ln 2 (m is in log2 units of the scaled scores).
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = q0 + 32 * qt + col;
    if (q < N) {
      const float inv = 1.f / l[qt];
      OutT* dst = O + hoff + (size_t)q * D + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          OutStore<OutT>::store4(dst + 32 * dt + 8 * g, acc[qt][dt][4 * g] * inv, acc[qt][dt][4 * g + 1] * inv,
                                 acc[qt][dt][4 * g + 2] * inv, acc[qt][dt][4 * g + 3] * inv);
      if (hi == 0) LSE[(size_t)bh * N + q] = (m[qt] + __log2f(l[qt])) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// float32 operands (P kept in float32), v_mfma_f32_32x32x2_f32. One 32-row
// query tile per wave, 32 keys per block. K-step i of O^T += V^T P^T pairs
// accumulator register i of both half-waves, so P needs no conversion.
template <int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(256, 2) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqb, float c) {
  constexpr int BR = 128, BC = 32;
  constexpr int KS = D + 4, VS = D + 4;
  constexpr int KT = BC * KS, VT = BC * VS;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) float smem[KT + VT];
  float* ks = smem;
  float* vs = smem + KT;

  int bh, qb;
  map_block(blockIdx.x, BH, nqb, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;
  const int q0 = qb * BR + wave * 32;
  const int q = q0 + col;

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
  const int q_last = min(N - 1, qb * BR + BR - 1);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;

  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * BC;
    __syncthreads();
    for (int idx = tid; idx < BC * D / 4; idx += 256) {
      const int row = idx / (D / 4), c4 = idx % (D / 4), key = k0 + row;
      f32x4 kx = {}, vx = {};
      if (key < N) {
        kx = *(const f32x4*)(K + hoff + (size_t)key * D + 4 * c4);
        vx = *(const f32x4*)(V + hoff + (size_t)key * D + 4 * c4);
      }
      *(f32x4*)(ks + row * KS + 4 * c4) = kx;
      *(f32x4*)(vs + row * VS + 4 * c4) = vx;
    }
    __syncthreads();
    if (CAUSAL && k0 > q0 + 31) continue;
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
// Host-side launch selection.

template <int D, bool CAUSAL, typename OutT>
static hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                              int N, float c, hipStream_t st) {
  constexpr int QT = 1, BC = 64;
  const int nqb = (N + 128 * QT - 1) / (128 * QT);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, BC, CAUSAL, OutT, 2>), dim3(BH * nqb), dim3(256), 0, st,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (OutT*)o, lse, BH, N, nqb, c);
  return hipGetLastError();
}

template <int D, bool CAUSAL, typename OutT>
static hipError_t launch_f32(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                             int N, float c, hipStream_t st) {
  const int nqb = (N + 127) / 128;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, OutT>), dim3(BH * nqb), dim3(256), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, (OutT*)o, lse, BH, N, nqb, c);
  return hipGetLastError();
}

#define FA_DISPATCH(FN, D, causal, OT, ...)                                        \
  ((D) == 64 ? ((causal) ? FN<64, true, OT>(__VA_ARGS__) : FN<64, false, OT>(__VA_ARGS__)) \
             : ((causal) ? FN<128, true, OT>(__VA_ARGS__) : FN<128, false, OT>(__VA_ARGS__)))

int launch_forward(int in_dtype, int o_dtype, const void* q, const void* k, const void* v,
                   const float* descale, void* o, float* lse, int B, int H, int N, int d, float scale,
                   int causal, hipStream_t stream) {
  const int BH = B * H;
  const float c = scale * kLog2e;
  hipError_t err;
  if (in_dtype == FA_BF16) {
    err = (o_dtype == FA_BF16) ? FA_DISPATCH(launch_bf16, d, causal, bf16, q, k, v, o, lse, BH, N, c, stream)
                               : FA_DISPATCH(launch_bf16, d, causal, float, q, k, v, o, lse, BH, N, c, stream);
  } else if (in_dtype == FA_F32) {
    err = (o_dtype == FA_BF16) ? FA_DISPATCH(launch_f32, d, causal, bf16, q, k, v, o, lse, BH, N, c, stream)
                               : FA_DISPATCH(launch_f32, d, causal, float, q, k, v, o, lse, BH, N, c, stream);
  } else if (in_dtype == FA_FP8_E4M3 && o_dtype == FA_BF16) {
    err = launch_forward_fp8(q, k, v, descale, o, lse, BH, N, d, scale, causal, stream);
  } else {
    return FA_ERR_UNSUPPORTED;
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
