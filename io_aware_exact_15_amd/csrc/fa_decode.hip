// Decode step: a few new query rows against a long key/value cache, as a
// split-K forward.
//
// The card "FlashAttention Kernel & Online Softmax" (prompts) names the
// decode step, where each new token reads the whole cache and the kernel is
// bound by those bytes, not by arithmetic. The Nq query rows are the last Nq
// positions of the sequence, so with the causal mask row i sees keys
// j <= Nk - Nq + i. Query heads share key/value heads in groups of
// G = H / Hkv (grouped-query heads, "FlashAttention" explainer, lineage
// paragraph); the G * Nq rows of one group read the same keys, so they are
// computed together: they are the 32 query columns of one score tile.
//
// Two kernels:
//   decode_split  one workgroup per (batch, key/value head, tile of 32 rows,
//                 split of the keys), 4 waves. 128-key K/V blocks stream
//                 HBM -> LDS by DMA (2-stage ring, XOR-swizzled rows, rows
//                 past Nk read as zeros). Wave w takes keys 32 w .. + 31 of
//                 every block and keeps its own running max m, denominator l
//                 and unnormalised output over them (the online softmax of
//                 the card's definition paragraph); the 4 waves merge through
//                 LDS into one partial result per split.
//   decode_merge  per row, merges the partials with the same combine the
//                 online softmax uses between blocks: m = max m_p,
//                 l = sum l_p 2^(m_p - m), O = sum acc_p 2^(m_p - m) / l.
// Scores are in base 2 (scale * log2 e folded into one multiply).
#include <mutex>
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {

namespace {

constexpr int kDecBC = 128;   // keys per block
constexpr int kDecWaves = 4;  // waves per workgroup (32 keys of each block each)
constexpr float kDecTau = 8.f;


}  // namespace

// Partial results of tile T (of 32 rows) and split s live at index
// p = T * NS + s: acc [p][32 columns][D] float32 (only the tile's valid
// columns are written), then m, l [p][32] float32 (log2 units).
struct DecodeParts {
  float* acc;
  float* ml;
};

static inline size_t dec_align(size_t x) { return (x + 255) & ~(size_t)255; }

static inline void decode_split_shape(int B, int H, int Hkv, int Nq, int Nk, int& nqt, int& ns, int& sb) {
  const int R = (H / Hkv) * Nq;  // rows of one head group
  nqt = (R + 31) / 32;
  const long tiles = (long)B * Hkv * nqt;
  const int nblk = (Nk + kDecBC - 1) / kDecBC;
  // About two workgroups per CU (one fits at a time: 128 KB of LDS), each
  // streaming a long run of blocks: at least 16 (2048 keys), so that a
  // workgroup's ring prologue and merge epilogue stay a small part of it.
  long want = (512 + tiles - 1) / tiles;
  if (want > nblk / 16) want = nblk / 16;
  if (want < 1) want = 1;
  if (want > nblk) want = nblk;
  sb = (nblk + (int)want - 1) / (int)want;  // blocks per split
  ns = (nblk + sb - 1) / sb;
}

size_t decode_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d) {
  int nqt, ns, sb;
  decode_split_shape(B, H, Hkv, Nq, Nk, nqt, ns, sb);
  const size_t parts = (size_t)B * Hkv * nqt * ns;
  return dec_align(parts * 32 * d * sizeof(float)) + dec_align(parts * 64 * sizeof(float));
}

static inline DecodeParts carve_parts(void* ws, size_t parts, int d) {
  DecodeParts p;
  p.acc = (float*)ws;
  p.ml = (float*)((char*)ws + dec_align(parts * 32 * d * sizeof(float)));
  return p;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void decode_split_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                              const bf16* __restrict__ V, DecodeParts parts, int H,
                                                              int Hkv, int Nq, int Nk, int nqt, int ns, int sb,
                                                              float c) {
  constexpr int BC = kDecBC, NW = kDecWaves;
  constexpr int ROWB = 2 * D, TILEB = BC * ROWB, CPR = D / 8;
  constexpr int NI = CPR * BC / 64 / NW;  // 1024-byte DMA instructions per wave per tile
  constexpr int NDT = D / 32, NKS = D / 16;
  static_assert(NI >= 1, "tile split");
  // Ring stages [K | V], one object each (see dma_to_lds).
  __shared__ __attribute__((aligned(1024))) char lds0[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * TILEB];

  const int G = H / Hkv, R = G * Nq;
  const int s = blockIdx.x % ns, T = blockIdx.x / ns;
  const int qt = T % nqt, bk = T / nqt;  // bk = b * Hkv + key/value head
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, col = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // Query column col = row r of the group: query head kvh * G + r / Nq, new
  // token r % Nq at position Nk - Nq + r % Nq.
  const int r = qt * 32 + col;
  const bool rvalid = r < R;
  const int g = rvalid ? r / Nq : 0, ti = rvalid ? r % Nq : 0;
  const int pos = Nk - Nq + ti;
  const size_t kvoff = (size_t)bk * Nk * D;

  const int nblk = (Nk + BC - 1) / BC;
  const int kb0 = s * sb, kb1 = min(nblk, kb0 + sb);

  const rsrc_t kr = buffer_rsrc(K + kvoff, (unsigned)Nk * ROWB);
  const rsrc_t vr = buffer_rsrc(V + kvoff, (unsigned)Nk * ROWB);
  unsigned goff[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int p = 64 * (NI * wave + n) + lane, row = p / CPR, pc = p % CPR;
    goff[n] = row * ROWB + 16 * (pc ^ tile_swz<D>(row));
  }
  auto issue_loads = [&](int kb, char* st) __attribute__((always_inline)) {
    const unsigned base = (unsigned)kb * TILEB;
    char* const la = st + 1024 * NI * wave_u;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      dma_to_lds<16>(kr, la + 1024 * n, base + goff[n]);
      dma_to_lds<16>(vr, la + TILEB + 1024 * n, base + goff[n]);
    }
  };

  // This wave's K rows 32 wave + col (logical chunk 2 kk + hi) and V^T reads
  // (row 4 hi + (j >> 2) + 8 sec, byte column 64 dt + 32 gg + 8 (j & 3)).
  int koff[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    const int row = 32 * wave + col;
    koff[kk] = row * ROWB + 16 * ((2 * kk + hi) ^ tile_swz<D>(row));
  }
  int voff[NDT][2];
  {
    const int j = lane & 15, gg = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int rr = 32 * wave + 4 * hi + (j >> 2) + 8 * sec;
        const int bcol = 64 * dt + 32 * gg + 8 * (j & 3);
        voff[dt][sec] = TILEB + rr * ROWB + 16 * ((bcol >> 4) ^ tile_swz<D>(rr)) + (bcol & 15);
      }
  }

  // Q^T fragments (B operand): lane holds Q[row r][16 ks + 8 hi + 0..7].
  bf16x8 qf[NKS];
  {
    const bf16x8* src = (const bf16x8*)(Q + (((size_t)b * H + (size_t)kvh * G + g) * Nq + ti) * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 x = src[2 * ks + hi];
      qf[ks] = rvalid ? x : bf16x8{};
    }
  }

  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  float m = kNegInf, l = 0.f;

  auto compute = [&](int kb, const char* st) __attribute__((always_inline)) {
    const int k0 = kb * BC + 32 * wave;  // this wave's first key
    f32x16 sc = {};
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) sc = mfma_bf16(*(const bf16x8*)(st + koff[kk]), qf[kk], sc);
    // key of register i: k0 + 8 (i / 4) + 4 hi + i % 4; kept iff < Nk (rows
    // past Nk are zeros) and, with the mask, <= the row's position.
    const int lim = (CAUSAL ? min(pos, Nk - 1) : Nk - 1) - k0 - 4 * hi;
    if (lim < 31 || !rvalid) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!rvalid || 8 * (i / 4) + (i % 4) > lim) sc[i] = kNegInf;
    }
    float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      mx0 = fmaxf(fmaxf(mx0, sc[i]), sc[i + 1]);
      mx1 = fmaxf(fmaxf(mx1, sc[i + 2]), sc[i + 3]);
    }
    const float mx = pair_max(fmaxf(mx0, mx1)) * c;
    const bool upd = mx > m + kDecTau;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float alpha = upd ? fast_exp2(m - mx) : 1.f;
      if (upd) m = mx;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
    }
    const float nm = (m == kNegInf) ? 0.f : -m;
    float rs = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = fast_exp2(__builtin_fmaf(sc[8 * h2 + j], c, nm));
      rs += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pf[h2] = bf16x8{(bf16)p[0], (bf16)p[1], (bf16)p[2], (bf16)p[3], (bf16)p[4], (bf16)p[5], (bf16)p[6], (bf16)p[7]};
    }
    l += pair_sum(rs);
    // O^T += V^T P^T over the wave's 32 keys (two 16-key steps; contraction
    // slots match the accumulator rows of the scores).
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int rb = 16 * h2 * ROWB;
        const bf16x8 a = cat4(lds_read_tr16((const bf16*)(st + voff[dt][0] + rb)),
                              lds_read_tr16((const bf16*)(st + voff[dt][1] + rb)));
        acc[dt] = mfma_bf16(a, pf[h2], acc[dt]);
      }
  };

  if (kb0 < kb1) issue_loads(kb0, lds0);
  for (int kb = kb0; kb < kb1; kb += 2) {
    wait_vmem();
    __syncthreads();
    if (kb + 1 < kb1) issue_loads(kb + 1, lds1);
    compute(kb, lds0);
    if (kb + 1 < kb1) {
      wait_vmem();
      __syncthreads();
      if (kb + 2 < kb1) issue_loads(kb + 2, lds0);
      compute(kb + 1, lds1);
    }
  }

  // The 4 waves' results over their key slices merge through LDS (the ring
  // is free once every wave has passed the barrier) into the split's
  // partial: M = max m_w, acc = sum acc_w 2^(m_w - M), l = sum l_w 2^(m_w - M).
  // A column with no visible key in the split keeps m = -inf, l = 0, acc = 0.
  float* red = (float*)lds0;  // [waves 1..3][NDT][16][64] acc, then [4][64] m, [4][64] l
  float* rm = red + 3 * NDT * 16 * 64;
  float* rl = rm + 4 * 64;
  __syncthreads();
  rm[wave * 64 + lane] = m;
  rl[wave * 64 + lane] = l;
  if (wave > 0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[(((wave - 1) * NDT + dt) * 16 + i) * 64 + lane] = acc[dt][i];
  }
  __syncthreads();
  if (wave == 0) {
    float mw[NW], M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = rm[w * 64 + lane];
      M = fmaxf(M, mw[w]);
    }
    float f[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      f[w] = (mw[w] == kNegInf) ? 0.f : fast_exp2(mw[w] - M);
      L += f[w] * rl[w * 64 + lane];
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float a = f[0] * acc[dt][i];
#pragma unroll
        for (int w = 1; w < NW; ++w) a += f[w] * red[(((w - 1) * NDT + dt) * 16 + i) * 64 + lane];
        acc[dt][i] = a;
      }
    const size_t p = (size_t)T * ns + s;
    if (rvalid) {
      float* dst = parts.acc + (p * 32 + col) * D + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(f32x4*)(dst + 32 * dt + 8 * q4) =
              f32x4{acc[dt][4 * q4], acc[dt][4 * q4 + 1], acc[dt][4 * q4 + 2], acc[dt][4 * q4 + 3]};
      if (hi == 0) {
        parts.ml[p * 64 + col] = M;
        parts.ml[p * 64 + 32 + col] = L;
      }
    }
  }
}

// One wave per output row (b, h, i): merges the ns partials of its tile
// column, 64 at a time: lane j holds partial j's m and weight, every lane
// holds D / 64 consecutive dimensions of the output, and the partials'
// accumulator loads are issued 8 at a time so that they overlap.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParts parts, OutT* __restrict__ O,
                                                           float* __restrict__ LSE, int B, int H, int Hkv, int Nq,
                                                           int nqt, int ns) {
  constexpr int E = D / 64, U = 8;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (long)B * H * Nq) return;
  const int ti = (int)(row % Nq);
  const long bh = row / Nq;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int G = H / Hkv, kvh = h / G, r = (h % G) * Nq + ti;
  const int qt = r / 32, col = r % 32;
  const size_t p0 = (((size_t)b * Hkv + kvh) * nqt + qt) * ns;
  // Global max over the partials.
  float M = kNegInf;
  for (int p = lane; p < ns; p += 64) M = fmaxf(M, parts.ml[(p0 + p) * 64 + col]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float L = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < ns; c0 += 64) {
    // lane j: weight of partial c0 + j (0 past ns or with no visible key in that split)
    const int pj = c0 + lane;
    float w = 0.f;
    if (pj < ns) {
      const float mp = parts.ml[(p0 + pj) * 64 + col];
      w = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
      L += w * parts.ml[(p0 + pj) * 64 + 32 + col];
    }
    const int nc = min(64, ns - c0);
    for (int j0 = 0; j0 < nc; j0 += U) {
      float a[U][E];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u, nc - 1);  // in range; duplicates get weight 0 below
        const float* src = parts.acc + ((p0 + c0 + j) * 32 + col) * D + E * lane;
#pragma unroll
        for (int e = 0; e < E; ++e) a[u][e] = src[e];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = __shfl(w, j0 + u, 64);
        const float wk = (j0 + u < nc) ? wu : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += wk * a[u][e];
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
  const float inv = 1.f / L;
  OutT* dst = O + row * D + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = (OutT)(acc[e] * inv);
  if (lane == 0) LSE[row] = (M + __log2f(L)) * kLn2;
}

template <int D, bool CAUSAL>
static hipError_t launch_decode_d(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
                                  void* workspace, int B, int H, int Hkv, int Nq, int Nk, float scale,
                                  hipStream_t st) {
  int nqt, ns, sb;
  decode_split_shape(B, H, Hkv, Nq, Nk, nqt, ns, sb);
  const size_t parts_n = (size_t)B * Hkv * nqt * ns;
  const DecodeParts parts = carve_parts(workspace, parts_n, D);
  const int grid = B * Hkv * nqt * ns;
  const hipError_t e = launch_kernel(decode_split_kernel<D, CAUSAL>, dim3(grid), dim3(256), st, (const bf16*)q,
                                     (const bf16*)k, (const bf16*)v, parts, H, Hkv, Nq, Nk, nqt, ns, sb, scale * kLog2e);
  if (e != hipSuccess) return e;
  const long rows = (long)B * H * Nq;
  const int mgrid = (int)((rows + 3) / 4);
  if (o_dtype == FA_BF16)
    return launch_kernel(decode_merge_kernel<D, bf16>, dim3(mgrid), dim3(256), st, parts, (bf16*)o, lse, B, H, Hkv, Nq,
                         nqt, ns);
  return launch_kernel(decode_merge_kernel<D, float>, dim3(mgrid), dim3(256), st, parts, (float*)o, lse, B, H, Hkv,
                       Nq, nqt, ns);
}

int launch_decode(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, void* workspace,
                  int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream) {
  hipError_t e;
  if (d == 64)
    e = causal ? launch_decode_d<64, true>(q, k, v, o, o_dtype, lse, workspace, B, H, Hkv, Nq, Nk, scale, stream)
               : launch_decode_d<64, false>(q, k, v, o, o_dtype, lse, workspace, B, H, Hkv, Nq, Nk, scale, stream);
  else
    e = causal ? launch_decode_d<128, true>(q, k, v, o, o_dtype, lse, workspace, B, H, Hkv, Nq, Nk, scale, stream)
               : launch_decode_d<128, false>(q, k, v, o, o_dtype, lse, workspace, B, H, Hkv, Nq, Nk, scale, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate. The
// partial results live in `scratch`, a file-scope device array of fixed size
// that the library owns: each GPU the library runs on holds its own copy
// until the process ends. On the host the array's name only stands for the
// symbol; its device address is looked up once per device (with that device
// current) and cached, and only that address is handed to kernels. The
// partials need no clearing (every one of them that the merge reads is
// written by its split workgroup earlier in the same call), and calls that
// overlap on one GPU share the array and race.
static __device__ __align__(256) char scratch[FA_DECODE_NOALLOC_MAX_WORKSPACE];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

// Device address of the current GPU's scratch array.
static hipError_t scratch_address(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

int launch_decode_noalloc(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, int B, int H,
                          int Hkv, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream) {
  if (decode_workspace_bytes(B, H, Hkv, Nq, Nk, d) > sizeof(scratch)) return FA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess || ws == nullptr) return FA_ERR_LAUNCH;
  return launch_decode(q, k, v, o, o_dtype, lse, ws, B, H, Hkv, Nq, Nk, d, scale, causal, stream);
}

}  // namespace fa
