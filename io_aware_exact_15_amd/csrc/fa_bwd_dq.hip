// Backward pass, dQ kernel: dQ = scale * dS K, with S and dP recomputed per
// key block (the backward's design notes are at the top of fa_bwd.hip). A
// source of its own so that it is compiled with the default machine
// scheduler: at 256 registers per lane the iterative ILP strategy, which
// suits the dK/dV kernel, makes this one spill inside its inner loop.
#include <type_traits>

#include "fa_bwd_common.hpp"
#include "fa_internal.h"

namespace fa {

// ---------------------------------------------------------------------------
// dQ. Persistent: one workgroup of 8 waves x 32 queries per CU takes (query
// head, block of 256 queries) items from the work lists; key blocks of 64.
// The exponents of the copies come from the dK/dV launch.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(void* wsb, const float* __restrict__ desc, int fin, int fdo,
                                                        float* __restrict__ dQ, int BH, int G, int N, int nqb,
                                                        float c, float scale) {
  constexpr int NW = 8, BR = 32 * NW, BC = 64;
  constexpr int ROWB = 2 * D, TILEB = BC * ROWB, CPR = D / 8;
  constexpr int NPW = CPR * BC / 64 / NW;
  constexpr int NKS = D / 16, NDT = D / 32, NKT = BC / 32;
  static_assert(NPW >= 1, "tile split");
  // Ring stages [K | V], one object each (see dma_to_lds).
  __shared__ __attribute__((aligned(1024))) char lds0[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * TILEB];
  __shared__ int s_next;

  const unsigned* ctl = (const unsigned*)wsb;  // the workspace starts with the control block
  const float* ef = (const float*)(ctl + kExps);
  const float sq = (fin ? desc[0] : 1.f) * ldexpf(1.f, (int)ef[0]);
  const float sk = (fin ? desc[1] : 1.f) * ldexpf(1.f, (int)ef[1]);
  const float sv = (fin ? desc[2] : 1.f) * ldexpf(1.f, (int)ef[2]);
  const float sdo = (fdo ? desc[3] : 1.f) * ldexpf(1.f, (int)ef[3]);
  // dS in units of sdo * sv (as in the dK/dV kernel); dQ = scale * dS K.
  const float cS = c * sq * sk, fQ = scale * sk * sdo * sv;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nkb_all = (N + BC - 1) / BC;

  const int total = BH * nqb, xcd = xcd_id();
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
    unsigned goff[NPW];
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      const int p = 64 * (NPW * wave + n) + ln, row = p / CPR, pc = p % CPR;
      goff[n] = row * ROWB + 16 * (pc ^ tile_swz<D>(row));
    }
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
    int bh, qb;
    map_head_block(item, BH, G, nqb, false, bh, qb);
    const size_t hoff = (size_t)bh * N * D;         // query head: Q, dO, dQ
    const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head: K, V
    const int qw = qb * BR + 32 * wave_u;           // wave-uniform: the mask test below is a scalar branch
    const int q = qw + col;
    const rsrc_t kr = buffer_rsrc(w.k + kvoff, (unsigned)N * ROWB);
    const rsrc_t vr = buffer_rsrc(w.v + kvoff, (unsigned)N * ROWB);
    auto issue_loads = [&](int kb, char* st) {
      const unsigned base = (unsigned)kb * TILEB;
      char* const la = st + 1024 * NPW * wave_u;
#pragma unroll
      for (int n = 0; n < NPW; ++n) {
        dma_to_lds<16>(kr, la + 1024 * n, base + goff[n]);
        dma_to_lds<16>(vr, la + TILEB + 1024 * n, base + goff[n]);
      }
    };

    // The first K/V block's DMA goes out before the register loads of Q, dO and
    // the row values, so that all of them share one memory round trip.
    issue_loads(0, lds0);
    // Q and dO as B operands: lane holds row q, dims 16 ks + 8 hi + 0..7.
    f16x8 qf[NKS], of[NKS];
    {
      const int qr = q < N ? q : 0;
      const f16x8* qsrc = (const f16x8*)(w.q + hoff + (size_t)qr * D);
      const f16x8* osrc = (const f16x8*)(w.dO + hoff + (size_t)qr * D);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f16x8 a = qsrc[2 * ks + hi], b = osrc[2 * ks + hi];
        qf[ks] = q < N ? a : f16x8{};
        of[ks] = q < N ? b : f16x8{};
      }
    }
    // The workspace's 2^15 on P and 2^-15 on D are for the dK/dV kernel; here P
    // is unscaled. Unconditional loads (rows past N read row N - 1), so that
    // neither waits behind a branch of its own.
    const size_t rrow = (size_t)bh * N + (q < N ? q : N - 1);
    const float nl_raw = w.NL[rrow], d_raw = w.Dv[rrow];
    const float nl = q < N ? nl_raw - kPScale : 0.f;
    const float dq_d = q < N ? d_raw * 32768.f : 0.f;
    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};

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
            dsv[i] = p * (dp[kt][i] - dq_d);
          }
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            df[kt][h2] = f16x8{(f16)dsv[8 * h2], (f16)dsv[8 * h2 + 1], (f16)dsv[8 * h2 + 2], (f16)dsv[8 * h2 + 3],
                               (f16)dsv[8 * h2 + 4], (f16)dsv[8 * h2 + 5], (f16)dsv[8 * h2 + 6],
                               (f16)dsv[8 * h2 + 7]};
        }
      };
      if (need_mask) ds_tiles(std::true_type{});
      else ds_tiles(std::false_type{});
      // dQ^T += K^T dS^T: K^T read transposed, key order of the accumulator
      // rows; 16-key steps outer with the next step's reads issued first.
      constexpr int NST = 2 * NKT;
      auto kread = [&](int stp, int dt) __attribute__((always_inline)) {
        const int rb = 16 * stp * ROWB;
        return cat4h(lds_read_tr16h(ks + rb + toff[dt][0]), lds_read_tr16h(ks + rb + toff[dt][1]));
      };
      f16x8 kf[2][NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) kf[0][dt] = kread(0, dt);
#pragma unroll
      for (int stp = 0; stp < NST; ++stp) {
        if (stp + 1 < NST) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) kf[(stp + 1) & 1][dt] = kread(stp + 1, dt);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] = mfma_f16(kf[stp & 1][dt], df[stp >> 1][stp & 1], acc[dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    for (int kb = 0; kb < nkb; kb += 2) {
      wait_vmem();
      __syncthreads();
      if (kb + 1 < nkb) issue_loads(kb + 1, lds1);
      compute(kb, lds0);
      if (kb + 1 < nkb) {
        wait_vmem();
        __syncthreads();
        if (kb + 2 < nkb) issue_loads(kb + 2, lds0);
        compute(kb + 1, lds1);
      }
    }

    // The next item is taken now: the atomic's latency overlaps the stores.
    int next = -1;
    if (tid == 0) next = pop_item((unsigned*)wsb, 8, total, gridDim.x, xcd);
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
    // The next item's first DMA rewrites stage 0: every wave is past its reads
    // once it is past this barrier (LDS only: this item's stores stay in flight).
    if (tid == 0) s_next = next;
    lds_barrier();
    item = __builtin_amdgcn_readfirstlane(s_next);
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_dq_d(void* workspace, const float* desc, int fin, int fdo, float* dq, int BH, int G, int N,
                              float c, float scale, int grid, hipStream_t st) {
  const int nqb = (N + 255) / 256;
  return launch_kernel(bwd_dq_kernel<D, CAUSAL>, dim3(grid), dim3(512), st, workspace, desc, fin, fdo, dq, BH, G, N,
                       nqb, c, scale);
}

hipError_t launch_bwd_dq(int d, int causal, void* workspace, const float* desc, int fin, int fdo, float* dq, int BH,
                         int G, int N, float c, float scale, int grid, hipStream_t st) {
  if (d == 64)
    return causal ? launch_dq_d<64, true>(workspace, desc, fin, fdo, dq, BH, G, N, c, scale, grid, st)
                  : launch_dq_d<64, false>(workspace, desc, fin, fdo, dq, BH, G, N, c, scale, grid, st);
  return causal ? launch_dq_d<128, true>(workspace, desc, fin, fdo, dq, BH, G, N, c, scale, grid, st)
                : launch_dq_d<128, false>(workspace, desc, fin, fdo, dq, BH, G, N, c, scale, grid, st);
}

}  // namespace fa
