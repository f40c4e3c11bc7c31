// Forward pass of exact attention with a wave-specialised schedule: the
// waves of a workgroup take one of two roles, producer or consumer, instead
// of each running the whole loop.
//
// What is computed is the same as in fa_fwd.hip: per query row, the running
// maximum m, the running denominator l and the rescaled output accumulator
// of the online softmax, with the correction exp(m - m_new) whenever a key
// block raises the maximum, and one division by l at the end (the card
// "FlashAttention Kernel & Online Softmax", definition paragraph; the
// "FlashAttention" explainer by A. Tiwari). The schedule is the
// producer/consumer split that the same card's history paragraph names for
// the Hopper generation (warp specialisation), re-derived for CDNA4:
//
//   * Each SIMD runs one consumer wave and one producer wave (waves w and
//     w + 4 of the workgroup share a SIMD), both for the same 32 query rows.
//   * The consumer runs every matrix-core product: the scores S^T = K Q^T of
//     a key block and O^T += V^T P^T of an earlier one. Q and the output
//     accumulator stay in its registers for the whole kernel.
//   * The producer issues the K/V tile loads (HBM -> LDS by DMA, into 3-stage
//     rings, two ticks ahead of their use) and turns scores into
//     probabilities: row max, lazy rescale decision, exponentials, bf16
//     packing and the running denominator.
//   * Scores go from consumer to producer, and probabilities with the
//     rescale factor back, through LDS, lane for lane: each lane writes its
//     accumulator registers and its partner lane on the other wave reads the
//     same slots, so the softmax runs in the consumer's accumulator layout
//     (one query row per lane, 16 keys per 32-key tile) and the packed
//     probabilities are directly the consumer's B operand.
//
// Tick t (one workgroup barrier per tick, t = 0 .. nkb + 1):
//   consumer: read P(t-2) and its rescale factors from exchange buffer t % 2,
//             form S(t) from K ring stage t % 3 and write it to the same
//             buffer, rescale O, add V(t-2)^T P(t-2)^T (V ring stage
//             (t - 2) % 3);
//   producer: load K(t+2) into K stage (t + 2) % 3 and V(t) into V stage
//             t % 3; read S(t-1) from exchange buffer (t - 1) % 2 and write
//             P(t-1) and the rescale factors there; wait for the loads of
//             tick t - 1.
// Every buffer a tick writes was last read in an earlier tick, so the one
// barrier per tick orders all reuse.
//
// Lazy rescaling as in fa_fwd.hip at d = 128: m moves only when a block's
// max exceeds it by more than kWsTau (log2 units); O and lse do not depend
// on m, which only keeps the exponentials in range.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

namespace {

constexpr float kWsTau = 8.f;
constexpr int kWsPairs = 4;   // consumer/producer pairs per workgroup (one per SIMD)
constexpr int kWsBC = 64;     // keys per block
constexpr int kWsRing = 3;    // stages of the K ring and of the V ring
constexpr int kWsXBytes = 32 * kWsBC * 4;  // exchange slots of one pair: 32 rows x 64 keys float32

template <typename T> struct WsStore;
template <> struct WsStore<bf16> {
  static __device__ __forceinline__ void store4(bf16* dst, float a, float b, float c, float d) {
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *(bf16x4*)dst = v;
  }
};
template <> struct WsStore<float> {
  static __device__ __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
    f32x4 v = {a, b, c, d};
    *(f32x4*)dst = v;
  }
};

// Workgroup barrier for the tick loop: waits for this wave's own LDS reads
// and writes, not for its LDS DMA. (A release fence on LDS would also wait
// for every tile load in flight, which would undo the loads two ticks ahead;
// the producers order their loads with explicit vmcnt waits instead.) The
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void tick_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(64 * 2 * kWsPairs, 1) void fwd_ws_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, int BH, int G, int N, int nqb, float c) {
  constexpr int NP = kWsPairs, BC = kWsBC, RS = kWsRing;
  constexpr int BR = 32 * NP;          // query rows per workgroup
  constexpr int NKT = BC / 32;         // 32-key tiles per block
  constexpr int NST = BC / 16;         // 16-key steps of P.V per block
  constexpr int ROWB = 2 * D;          // bytes per tile row
  constexpr int TILEB = BC * ROWB;     // bytes per K (or V) tile
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int NI = CPR * BC / 64 / NP;  // DMA instructions per producer wave per tile
  constexpr int NDT = D / 32, NKS = D / 16;
  constexpr int XB = NP * kWsXBytes;   // one exchange buffer
  static_assert(NI >= 1 && NI * 64 * NP == CPR * BC, "tile load split");
  static_assert(2 * RS * TILEB + 2 * XB <= 160 * 1024, "LDS");
  static_assert((RS - 1) * TILEB + 16 * (NST - 1) * ROWB + TILEB < 65536, "V reads within the immediate offset");
  // K stages 0..RS-1, then V stages 0..RS-1 (one object: only producers load
  // into it and only consumers read it); the exchange buffers, one object
  // each (see dma_to_lds: the producers' reads of them must not wait for
  // their own tile loads).
  __shared__ __attribute__((aligned(1024))) char kv[2 * RS * TILEB];
  __shared__ __attribute__((aligned(1024))) char xb0[XB];
  __shared__ __attribute__((aligned(1024))) char xb1[XB];

  int bh, qb;
  map_head_block(blockIdx.x, BH, G, nqb, false, bh, qb);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool consumer = wave_u < NP;
  const int pair = consumer ? wave_u : wave_u - NP;
  const int hi = lane >> 5, col = lane & 31;
  const size_t hoff = (size_t)bh * N * D;         // query head
  const size_t kvoff = (size_t)(bh / G) * N * D;  // its key/value head
  const int qw = qb * BR + 32 * pair;             // first query row of the pair
  const int q = qw + col;

  const int nkb_all = (N + BC - 1) / BC;
  const int q_last = min(N - 1, qb * BR + BR - 1);
  const int nkb = CAUSAL ? min(nkb_all, q_last / BC + 1) : nkb_all;
  const int T = nkb + 2;  // ticks
  // Key block j has a key at or before some query row of the pair.
  auto live = [&](int j) { return !CAUSAL || j * BC <= qw + 31; };

  // Exchange slots of this lane, as held LDS addresses (one per buffer; the
  // buffers lie beyond the 16-bit immediate offset of LDS accesses). An
  // access takes the buffer object plus (held address - object address),
  // which the compiler folds back to the held register.
  const int xb_at[2] = {(int)lds_addr(xb0), (int)lds_addr(xb1)};
  int xoff[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    xoff[b] = pair * kWsXBytes + 16 * lane + xb_at[b];
    asm volatile("" : "+v"(xoff[b]));
  }
  auto xbase = [&](auto buf) -> char* {
    constexpr int B = decltype(buf)::value;
    return (B == 0 ? xb0 : xb1) - xb_at[B];
  };

  if (consumer) {
    // ---------------------------------------------------------------- consumer
    const int kv_at = (int)lds_addr(kv);
    int koff[NKS];  // K row 32 kt + col, logical chunk 2 kk + hi (+ stage and tile offsets)
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      koff[kk] = col * ROWB + 16 * ((2 * kk + hi) ^ tile_swz<D>(col)) + kv_at;
      asm volatile("" : "+v"(koff[kk]));
    }
    int voff[NDT][2];  // V row 4 hi + (j >> 2) + 8 sec, byte column 64 dt + 32 g + 8 (j & 3)
    {
      const int j = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int sec = 0; sec < 2; ++sec) {
          const int r = 4 * hi + (j >> 2) + 8 * sec;
          const int bcol = 64 * dt + 32 * g + 8 * (j & 3);
          voff[dt][sec] = RS * TILEB + r * ROWB + 16 * ((bcol >> 4) ^ tile_swz<D>(r)) + (bcol & 15) + kv_at;
          asm volatile("" : "+v"(voff[dt][sec]));
        }
    }
    const char* const kvb = kv - kv_at;

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

    auto tick = [&](int t, auto kstage, auto buf) __attribute__((always_inline)) {
      constexpr int KS = decltype(kstage)::value;   // t % 3: K stage of block t
      constexpr int VS = (KS + 1) % RS;              // (t - 2) % 3: V stage of block t - 2
      constexpr int B = decltype(buf)::value;        // t % 2
      char* const xp = xbase(buf) + xoff[B];
      const bool pv = t >= 2 && live(t - 2);
      bf16x8 pf[NKT][2];
      float alpha = 1.f;
      if (pv) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) pf[kt][h2] = *(const bf16x8*)(xp + (2 * kt + h2) * 1024);
        alpha = *(const float*)(xp + 4096 - 12 * lane);  // slot 4096 + 4 lane
      }
      if (t < nkb && live(t)) {
        const int k0 = t * BC;
        f32x16 s[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};
        bf16x8 a[2][NKT];
        const char* const kb = kvb + KS * TILEB;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) a[0][kt] = *(const bf16x8*)(kb + koff[0] + kt * 32 * ROWB);
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          if (kk + 1 < NKS) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
              a[(kk + 1) & 1][kt] = *(const bf16x8*)(kb + koff[kk + 1] + kt * 32 * ROWB);
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
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(xp + (4 * kt + g) * 1024) = f32x4{s[kt][4 * g], s[kt][4 * g + 1], s[kt][4 * g + 2], s[kt][4 * g + 3]};
      }
      if (pv) {
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
        }
        // O^T += V^T P^T; contraction slots per 16-key step: lanes 0-31 keys
        // {0-3, 8-11}, lanes 32-63 keys {4-7, 12-15} (the accumulator rows).
        const char* const vb = kvb + VS * TILEB;
        auto vread = [&](int st, int dt) __attribute__((always_inline)) {
          const int rb = 16 * st * ROWB;
          return cat4(lds_read_tr16((const bf16*)(vb + voff[dt][0] + rb)),
                      lds_read_tr16((const bf16*)(vb + voff[dt][1] + rb)));
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
      }
      tick_barrier();
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    tick_barrier();  // the producers' prologue loads
    for (int t = 0; t < T; t += 6) {
      tick(t, S0{}, S0{});
      if (t + 1 < T) tick(t + 1, S1{}, S1{});
      if (t + 2 < T) tick(t + 2, S2{}, S0{});
      if (t + 3 < T) tick(t + 3, S0{}, S1{});
      if (t + 4 < T) tick(t + 4, S1{}, S0{});
      if (t + 5 < T) tick(t + 5, S2{}, S1{});
    }
    tick_barrier();  // the producers' 1 / l
    if (q < N) {
      const float inv = *(const float*)(xbase(S0{}) + xoff[0] - 12 * lane);  // slot 4 lane
      OutT* dst = O + hoff + (size_t)q * D + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          WsStore<OutT>::store4(dst + 32 * dt + 8 * g, acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv,
                                acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv);
    }
  } else {
    // ---------------------------------------------------------------- producer
    const rsrc_t kr = buffer_rsrc(K + kvoff, (unsigned)N * ROWB);
    const rsrc_t vr = buffer_rsrc(V + kvoff, (unsigned)N * ROWB);
    // DMA instruction n of this wave fills tile chunks 64 (NI pair + n) + lane,
    // i.e. row p / CPR, physical chunk p % CPR, holding logical chunk
    // (p % CPR) ^ tile_swz(row).
    unsigned goff[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int p = 64 * (NI * pair + n) + lane, row = p / CPR, pc = p % CPR;  // row < BC
      goff[n] = row * ROWB + 16 * (pc ^ tile_swz<D>(row));
    }
    auto load_tile = [&](rsrc_t r, int blk, char* st) __attribute__((always_inline)) {
      const unsigned base = (unsigned)blk * TILEB;
      char* const la = st + 1024 * NI * pair;
#pragma unroll
      for (int n = 0; n < NI; ++n) dma_to_lds<16>(r, la + 1024 * n, base + goff[n]);
    };
    float m = kNegInf, l = 0.f;

    auto tick = [&](int t, auto kstage, auto buf) __attribute__((always_inline)) {
      constexpr int KS = decltype(kstage)::value;  // t % 3
      constexpr int B = decltype(buf)::value;       // t % 2; the producer uses the other buffer
      const bool kload = t + 2 < nkb, vload = t < nkb;
      if (kload) load_tile(kr, t + 2, kv + ((KS + 2) % RS) * TILEB);
      if (vload) load_tile(vr, t, kv + (RS + KS) * TILEB);
      const int j = t - 1;
      if (j >= 0 && j < nkb && live(j)) {
        char* const xp = xbase(std::integral_constant<int, 1 - B>{}) + xoff[1 - B];
        f32x16 s[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 x = *(const f32x4*)(xp + (4 * kt + g) * 1024);
            s[kt][4 * g] = x[0];
            s[kt][4 * g + 1] = x[1];
            s[kt][4 * g + 2] = x[2];
            s[kt][4 * g + 3] = x[3];
          }
        float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          mx0 = fmaxf(fmaxf(mx0, s[0][i]), s[0][i + 1]);
          mx1 = fmaxf(fmaxf(mx1, s[NKT - 1][i]), s[NKT - 1][i + 1]);
        }
        const float mx = pair_max(fmaxf(mx0, mx1)) * c;
        const bool upd = mx > m + kWsTau;
        float alpha = 1.f;
        if (__builtin_amdgcn_ballot_w64(upd)) {  // wave-uniform, rare after the first block
          alpha = upd ? fast_exp2(m - mx) : 1.f;  // 0 while m is still -inf (l and O are 0)
          if (upd) m = mx;
          l *= alpha;
        }
        const float nm = (m == kNegInf) ? 0.f : -m;
        float rs0 = 0.f, rs1 = 0.f;
        bf16x8 pf[NKT][2];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float p[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(s[kt][8 * h2 + i], c, nm));
            rs0 += (p[0] + p[1]) + (p[2] + p[3]);
            rs1 += (p[4] + p[5]) + (p[6] + p[7]);
            pf[kt][h2] = bf16x8{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3],
                                (bf16)p[4], (bf16)p[5], (bf16)p[6], (bf16)p[7]};
          }
        l += pair_sum(rs0 + rs1);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) *(bf16x8*)(xp + (2 * kt + h2) * 1024) = pf[kt][h2];
        *(float*)(xp + 4096 - 12 * lane) = alpha;  // slot 4096 + 4 lane
      }
      // Loads of this tick may stay in flight; those of the tick before feed
      // the next tick.
      if (kload && vload) wait_vmem_n<2 * NI>();
      else if (kload || vload) wait_vmem_n<NI>();
      else wait_vmem();
      tick_barrier();
    };

    // Prologue: K(0) and K(1) into K stages 0 and 1; K(0) before the first tick.
    load_tile(kr, 0, kv);
    if (1 < nkb) {
      load_tile(kr, 1, kv + TILEB);
      wait_vmem_n<NI>();
    } else {
      wait_vmem();
    }
    tick_barrier();
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    for (int t = 0; t < T; t += 6) {
      tick(t, S0{}, S0{});
      if (t + 1 < T) tick(t + 1, S1{}, S1{});
      if (t + 2 < T) tick(t + 2, S2{}, S0{});
      if (t + 3 < T) tick(t + 3, S0{}, S1{});
      if (t + 4 < T) tick(t + 4, S1{}, S0{});
      if (t + 5 < T) tick(t + 5, S2{}, S1{});
    }
    // 1 / l for the consumer (slot 4 lane of buffer 0; every read of the
    // exchange buffers ended with the last tick), and lse.
    *(float*)(xbase(S0{}) + xoff[0] - 12 * lane) = 1.f / l;
    tick_barrier();
    if (q < N && hi == 0) LSE[(size_t)bh * N + q] = (m + __log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL, typename OutT>
static hipError_t launch_ws(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int G,
                            int N, float c, hipStream_t st) {
  constexpr int BR = 32 * kWsPairs;
  const int nqb = (N + BR - 1) / BR;
  return launch_kernel(fwd_ws_kernel<D, CAUSAL, OutT>, dim3(BH * nqb), dim3(64 * 2 * kWsPairs), st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (OutT*)o, lse, BH, G, N, nqb, c);
}

int launch_forward_ws(int o_dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int Hkv, int N, int d, float scale, int causal, hipStream_t stream) {
  const int BH = B * H, G = H / Hkv;
  const float c = scale * kLog2e;
  hipError_t err;
  if (o_dtype == FA_BF16) {
    if (d == 128) err = causal ? launch_ws<128, true, bf16>(q, k, v, o, lse, BH, G, N, c, stream)
                               : launch_ws<128, false, bf16>(q, k, v, o, lse, BH, G, N, c, stream);
    else err = causal ? launch_ws<64, true, bf16>(q, k, v, o, lse, BH, G, N, c, stream)
                      : launch_ws<64, false, bf16>(q, k, v, o, lse, BH, G, N, c, stream);
  } else {
    if (d == 128) err = causal ? launch_ws<128, true, float>(q, k, v, o, lse, BH, G, N, c, stream)
                               : launch_ws<128, false, float>(q, k, v, o, lse, BH, G, N, c, stream);
    else err = causal ? launch_ws<64, true, float>(q, k, v, o, lse, BH, G, N, c, stream)
                      : launch_ws<64, false, float>(q, k, v, o, lse, BH, G, N, c, stream);
  }
  return err == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace fa
