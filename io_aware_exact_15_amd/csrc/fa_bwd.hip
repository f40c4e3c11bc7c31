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
//   bwd_pre   D = rowsum(dO * O)                       (bandwidth-bound)
//   bwd_dkdv  one workgroup per block of 128 keys; K, V stay in registers,
//             Q / dO / lse / D stream through LDS; S = Q K^T is formed with
//             keys along the lanes so that P and dS leave the accumulators
//             already in the operand layout of dV += P^T dO and dK += dS^T Q.
//   bwd_dq    one workgroup per block of 128 queries; Q, dO stay in
//             registers, K / V stream through LDS; S^T = K Q^T (queries along
//             lanes) so dS^T feeds dQ^T += K^T dS^T directly.
// No buffer of size N x N exists; the only workspace is D ([B,H,N] float32).
//
// Matrix-core operands are fp16: bf16 inputs convert exactly (their 8-bit
// significand fits fp16's 11 bits inside fp16's exponent range), and P and
// dS, which must be rounded for the products, keep 3 more significant bits
// than bf16 would give them. Accumulation is float32 throughout.
#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 8 bf16 (as raw 16-byte chunk) -> 8 fp16; exact for bf16 values in fp16 range.
__device__ __forceinline__ f16x8 bf16x8_to_f16(i32x4 raw) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned w = (unsigned)raw[j];
    const float lo = __builtin_bit_cast(float, w << 16);
    const float hi = __builtin_bit_cast(float, w & 0xffff0000u);
    r[2 * j] = (f16)lo;
    r[2 * j + 1] = (f16)hi;
  }
  return r;
}

__device__ __forceinline__ f16x8 cat4h(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ s16x4 lds_read_tr16h(const f16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 FA_LDS*)(p));
}

// Same XCD-aware, heavy-first order as the forward pass; `rev` selects
// whether block index 0 (true) or nb-1 (false) is the heaviest.
__device__ __forceinline__ void map_block_b(int bid, int BH, int nb, bool first_is_heavy, int& bh, int& blk) {
  int j;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, hpx = BH >> 3;
    j = bid >> 3;
    bh = xcd + 8 * (j % hpx);
    j = j / hpx;
  } else {
    bh = bid % BH;
    j = bid / BH;
  }
  blk = first_is_heavy ? j : nb - 1 - j;
}

// ---------------------------------------------------------------------------
// D_i = sum_t dO_it * O_it, one group of D/8 lanes per row.
template <int D, typename OT>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ dO, const OT* __restrict__ O,
                                                      float* __restrict__ Dv, long rows) {
  constexpr int L = D / 8;  // lanes per row
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / L;
  const int part = (int)(t % L);
  float acc = 0.f;
  if (row < rows) {
    const i32x4 raw = *(const i32x4*)(dO + row * D + 8 * part);
    const OT* o = O + row * D + 8 * part;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned w = (unsigned)raw[j];
      acc += __builtin_bit_cast(float, w << 16) * (float)o[2 * j];
      acc += __builtin_bit_cast(float, w & 0xffff0000u) * (float)o[2 * j + 1];
    }
  }
#pragma unroll
  for (int s = L / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && part == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV. 4 waves x 32 keys; query blocks of BQ rows streamed through LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int N, int nkb, float c, float scale) {
  constexpr int BKV = 128, BQ = 64;
  constexpr int S = D + 8;  // LDS row stride (elements)
  constexpr int TILE = BQ * S;
  constexpr int NKS = D / 16, NDT = D / 32, NQT = BQ / 32;
  constexpr int CPT = BQ * D / 8 / 256;  // 16-byte chunks per thread per tile
  static_assert((BQ * D / 8) % 256 == 0, "tile split");
  __shared__ __attribute__((aligned(16))) f16 smem[2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float s_lse[2][BQ];
  __shared__ __attribute__((aligned(16))) float s_d[2][BQ];

  int bh, kb;
  map_block_b(blockIdx.x, BH, nkb, CAUSAL, bh, kb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;
  const int k0w = kb * BKV + 32 * wave;  // first key of this wave
  const int key = k0w + col;

  // K and V as B operands: lane holds row `key`, dims 16 ks + 8 hi + 0..7.
  f16x8 kf[NKS], vf[NKS];
  {
    const int kr = key < N ? key : 0;
    const i32x4* ksrc = (const i32x4*)(K + hoff + (size_t)kr * D);
    const i32x4* vsrc = (const i32x4*)(V + hoff + (size_t)kr * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      i32x4 a = ksrc[2 * ks + hi], b = vsrc[2 * ks + hi];
      if (key >= N) a = b = i32x4{};
      kf[ks] = bf16x8_to_f16(a);
      vf[ks] = bf16x8_to_f16(b);
    }
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = f32x16{};

  const int nqb = (N + BQ - 1) / BQ;
  const int qb0 = CAUSAL ? (kb * BKV) / BQ : 0;

  i32x4 qreg[CPT], oreg[CPT];
  float lreg = 0.f, dreg = 0.f;
  auto load_regs = [&](int qb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 8), c8 = idx % (D / 8);
      const int q = qb * BQ + row;
      const size_t off = hoff + (size_t)(q < N ? q : 0) * D + 8 * c8;  // clamped: always in bounds
      const i32x4 a = *(const i32x4*)(Q + off), b = *(const i32x4*)(dO + off);
      qreg[i] = q < N ? a : i32x4{};
      oreg[i] = q < N ? b : i32x4{};
    }
    if (tid < BQ) {
      const int q = qb * BQ + tid;
      // Rows past N get lse = +inf, so their recomputed P is exactly 0.
      lreg = q < N ? LSE[(size_t)bh * N + q] * kLog2e : __builtin_inff();
      dreg = q < N ? Dv[(size_t)bh * N + q] : 0.f;
    }
  };
  auto store_lds = [&](int buf) {
    f16* qs = smem + buf * 2 * TILE;
    f16* os = qs + TILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 8), c8 = idx % (D / 8);
      *(f16x8*)(qs + row * S + 8 * c8) = bf16x8_to_f16(qreg[i]);
      *(f16x8*)(os + row * S + 8 * c8) = bf16x8_to_f16(oreg[i]);
    }
    if (tid < BQ) {
      s_lse[buf][tid] = lreg;
      s_d[buf][tid] = dreg;
    }
  };

  if (qb0 < nqb) {
    load_regs(qb0);
    store_lds(0);
  }
  __syncthreads();

  const int trow = 4 * hi + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  for (int qb = qb0; qb < nqb; ++qb) {
    const int buf = (qb - qb0) & 1;
    if (qb + 1 < nqb) load_regs(qb + 1);
    const f16* qs = smem + buf * 2 * TILE;
    const f16* os = qs + TILE;
    const int qbase = qb * BQ;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int q0 = qbase + 32 * qt;
      // Whole 32x32 tile above the diagonal (every query < every key): nothing to add.
      if (CAUSAL && q0 + 31 < k0w) continue;
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f16x8 aq = *(const f16x8*)(qs + (32 * qt + col) * S + 16 * ks + 8 * hi);
        const f16x8 ao = *(const f16x8*)(os + (32 * qt + col) * S + 16 * ks + 8 * hi);
        s = mfma_f16(aq, kf[ks], s);
        dp = mfma_f16(ao, vf[ks], dp);
      }
      // Rows of this tile held by the lane: query 8 (i/4) + 4 hi + i % 4.
      const bool diag = CAUSAL && (q0 < k0w + 31);
      float pv[16], dsv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)&s_lse[buf][32 * qt + 8 * g + 4 * hi];
        const f32x4 d4 = *(const f32x4*)&s_d[buf][32 * qt + 8 * g + 4 * hi];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[4 * g + r], c, -l4[r]));
          if (diag && key > q0 + 8 * g + 4 * hi + r) p = 0.f;
          pv[4 * g + r] = p;
          dsv[4 * g + r] = p * (dp[4 * g + r] - d4[r]);
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
      // dV += P^T dO and dK += dS^T Q; B operands read transposed from LDS
      // with the query (contraction) order of the accumulator rows.
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const f16* po = os + (32 * qt + 16 * h2 + trow) * S + 32 * dt + tcol;
          const f16* pq = qs + (32 * qt + 16 * h2 + trow) * S + 32 * dt + tcol;
          const f16x8 bo = cat4h(lds_read_tr16h(po), lds_read_tr16h(po + 8 * S));
          const f16x8 bq = cat4h(lds_read_tr16h(pq), lds_read_tr16h(pq + 8 * S));
          dv[dt] = mfma_f16(pf[h2], bo, dv[dt]);
          dk[dt] = mfma_f16(df[h2], bq, dk[dt]);
        }
    }
    if (qb + 1 < nqb) store_lds(buf ^ 1);
    __syncthreads();
  }

  // Accumulator layout: lane holds dim 32 dt + col, keys 8 (i/4) + 4 hi + i % 4.
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = kb * BKV + 32 * wave + 8 * (i / 4) + 4 * hi + (i % 4);
      if (kr < N) {
        dK[hoff + (size_t)kr * D + 32 * dt + col] = dk[dt][i] * scale;
        dV[hoff + (size_t)kr * D + 32 * dt + col] = dv[dt][i];
      }
    }
}

// ---------------------------------------------------------------------------
// dQ. 4 waves x 32 queries; key blocks of BC keys streamed through LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dQ, int BH, int N, int nqb, float c, float scale) {
  constexpr int BR = 128, BC = 64;
  constexpr int S = D + 8;
  constexpr int TILE = BC * S;
  constexpr int NKS = D / 16, NDT = D / 32, NKT = BC / 32;
  constexpr int CPT = BC * D / 8 / 256;
  static_assert((BC * D / 8) % 256 == 0, "tile split");
  __shared__ __attribute__((aligned(16))) f16 smem[2 * 2 * TILE];

  int bh, qb;
  map_block_b(blockIdx.x, BH, nqb, false, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;
  const int q0 = qb * BR + 32 * wave;
  const int q = q0 + col;

  f16x8 qf[NKS], of[NKS];
  {
    const int qr = q < N ? q : 0;
    const i32x4* qsrc = (const i32x4*)(Q + hoff + (size_t)qr * D);
    const i32x4* osrc = (const i32x4*)(dO + hoff + (size_t)qr * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      i32x4 a = qsrc[2 * ks + hi], b = osrc[2 * ks + hi];
      if (q >= N) a = b = i32x4{};
      qf[ks] = bf16x8_to_f16(a);
      of[ks] = bf16x8_to_f16(b);
    }
  }
  const float lq = q < N ? LSE[(size_t)bh * N + q] * kLog2e : 0.f;
  const float dq_d = q < N ? Dv[(size_t)bh * N + q] : 0.f;
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};

  const int nkb_all = (N + BC - 1) / BC;
  const int q_last = min(N - 1, qb * BR + BR - 1);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;

  i32x4 kreg[CPT], vreg[CPT];
  auto load_regs = [&](int kb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 8), c8 = idx % (D / 8);
      const int kr = kb * BC + row;
      const size_t off = hoff + (size_t)(kr < N ? kr : 0) * D + 8 * c8;  // clamped: always in bounds
      const i32x4 a = *(const i32x4*)(K + off), b = *(const i32x4*)(V + off);
      kreg[i] = kr < N ? a : i32x4{};
      vreg[i] = kr < N ? b : i32x4{};
    }
  };
  auto store_lds = [&](int buf) {
    f16* ks = smem + buf * 2 * TILE;
    f16* vs = ks + TILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 8), c8 = idx % (D / 8);
      *(f16x8*)(ks + row * S + 8 * c8) = bf16x8_to_f16(kreg[i]);
      *(f16x8*)(vs + row * S + 8 * c8) = bf16x8_to_f16(vreg[i]);
    }
  };

  load_regs(0);
  store_lds(0);
  __syncthreads();
  const int trow = 4 * hi + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load_regs(kb + 1);
    const f16* ks = smem + buf * 2 * TILE;
    const f16* vs = ks + TILE;
    const int k0 = kb * BC;
    if (!CAUSAL || k0 <= q0 + 31) {
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const f16x8 ak = *(const f16x8*)(ks + (32 * kt + col) * S + 16 * kk + 8 * hi);
          const f16x8 av = *(const f16x8*)(vs + (32 * kt + col) * S + 16 * kk + 8 * hi);
          s = mfma_f16(ak, qf[kk], s);
          dp = mfma_f16(av, of[kk], dp);
        }
        float dsv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(__builtin_fmaf(s[i], c, -lq));
          if (need_mask) {
            const int kr = k0 + 32 * kt + 8 * (i / 4) + 4 * hi + (i % 4);
            if (kr >= N || (CAUSAL && kr > q)) p = 0.f;
          }
          dsv[i] = p * (dp[i] - dq_d);
        }
        f16x8 df[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          df[h2] = f16x8{(f16)dsv[8 * h2], (f16)dsv[8 * h2 + 1], (f16)dsv[8 * h2 + 2], (f16)dsv[8 * h2 + 3],
                         (f16)dsv[8 * h2 + 4], (f16)dsv[8 * h2 + 5], (f16)dsv[8 * h2 + 6], (f16)dsv[8 * h2 + 7]};
        // dQ^T += K^T dS^T: K^T read transposed, key order of the accumulator rows.
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f16* pk = ks + (32 * kt + 16 * h2 + trow) * S + 32 * dt + tcol;
            const f16x8 a = cat4h(lds_read_tr16h(pk), lds_read_tr16h(pk + 8 * S));
            acc[dt] = mfma_f16(a, df[h2], acc[dt]);
          }
      }
    }
    if (kb + 1 < nkb) store_lds(buf ^ 1);
    __syncthreads();
  }
  if (q < N) {
    float* dst = dQ + hoff + (size_t)q * D + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {acc[dt][4 * g] * scale, acc[dt][4 * g + 1] * scale, acc[dt][4 * g + 2] * scale,
                   acc[dt][4 * g + 3] * scale};
        *(f32x4*)(dst + 32 * dt + 8 * g) = v;
      }
  }
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                               const float* lse, float* dq, float* dk, float* dv, float* delta, int BH, int N,
                               float scale, hipStream_t st) {
  const long rows = (long)BH * N;
  const long threads = rows * (D / 8);
  const int pre_blocks = (int)((threads + 255) / 256);
  if (o_dtype == FA_F32)
    hipLaunchKernelGGL((bwd_pre_kernel<D, float>), dim3(pre_blocks), dim3(256), 0, st, (const bf16*)dO,
                       (const float*)o, delta, rows);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<D, bf16>), dim3(pre_blocks), dim3(256), 0, st, (const bf16*)dO,
                       (const bf16*)o, delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c = scale * kLog2e;
  const int nkb = (N + 127) / 128;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(BH * nkb), dim3(256), 0, st, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, (const bf16*)dO, lse, delta, dk, dv, BH, N, nkb, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqb = (N + 127) / 128;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(BH * nqb), dim3(256), 0, st, (const bf16*)q, (const bf16*)k,
                     (const bf16*)v, (const bf16*)dO, lse, delta, dq, BH, N, nqb, c, scale);
  return hipGetLastError();
}

int launch_backward(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dO,
                    const float* lse, float* dq, float* dk, float* dv, float* delta, int B, int H, int N, int d,
                    float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  hipError_t e;
  if (d == 64)
    e = causal ? launch_bwd_d<64, true>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, delta, BH, N, scale, stream)
               : launch_bwd_d<64, false>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, delta, BH, N, scale, stream);
  else
    e = causal ? launch_bwd_d<128, true>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, delta, BH, N, scale, stream)
               : launch_bwd_d<128, false>(q, k, v, o, o_dtype, dO, lse, dq, dk, dv, delta, BH, N, scale, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
