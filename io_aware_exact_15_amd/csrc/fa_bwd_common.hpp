// Pieces shared by the backward kernels (fa_bwd.hip: prep, dK/dV, group sum;
// fa_bwd_dq.hip: dQ): fp16 matrix-core helpers, the workspace layout, the
// per-tensor exponents of the fp16 copies, and the work lists of the
// persistent kernels. The design notes are at the top of fa_bwd.hip.
#pragma once

#include <stdint.h>

#include "fa_device.hpp"

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


constexpr float kPScale = 15.f;            // P is scaled by 2^kPScale for the dV product
constexpr float kPScaleInv = 1.f / 32768.f;  // 2^-kPScale
constexpr int kPrepWgs = 1024;             // bwd_prep's largest grid (one magnitude record each)
// Control block (u32 indices): the work-list counters, each in a 128-byte
// line of its own (list y of the dK/dV lists at kCtr + 32 y, of the dQ lists
// at kCtr + 32 (8 + y)), the grid barrier, the exponents chosen (floats).
constexpr int kCtlWords = 1024, kBarrier = 32 * 16, kExps = 32 * 17;

// Element formats of the backward inputs: 0 = bf16, 1 = FP8 E4M3, 2 = FP8 E5M2.
// Default exponent of a format's fp16 copy: E4M3 codes reach 448, E5M2 codes
// 57344; 2^-6 and 2^-13 bring both below 8.
__host__ __device__ constexpr int default_exp(int fmt) { return fmt == 1 ? 6 : fmt == 2 ? 13 : 0; }

// Workspace layout (all offsets 256-byte aligned):
//   ctl [kCtlWords] u32: the control block (work-list counters, grid
//       barrier, and the exponents chosen for Q, K, V, dO, written by
//       bwd_dkdv for bwd_dq);
//   amax [kPrepWgs][4] f32: largest |value| of Q, K, V, dO per prep workgroup;
//   D [q_rows] f32 (dO . O in units of the dO and V copies, times 2^-15);
//   NL [q_rows] f32 = kPScale - lse*log2(e);
//   Q [q_rows, d], K and V [kv_rows, d], dO [q_rows, d] fp16 copies;
//   when q_rows > kv_rows (grouped heads) per-query-head dK and dV
//   [q_rows, d] f32. q_rows = B*H*N, kv_rows = B*Hkv*N.
struct BwdWs {
  unsigned* ctl;
  float* amax;
  float* Dv;
  float* NL;
  f16 *q, *k, *v, *dO;
  float *dKp, *dVp;
};
__host__ __device__ inline size_t ws_align(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline BwdWs carve_ws(void* base, size_t q_rows, size_t kv_rows, int d) {
  char* p = (char*)base;
  BwdWs w;
  const size_t cbytes = kCtlWords * 4, abytes = ws_align(kPrepWgs * 4 * sizeof(float));
  const size_t fbytes = ws_align(q_rows * sizeof(float));
  const size_t qbytes = ws_align(q_rows * (size_t)d * sizeof(f16));
  const size_t kvbytes = ws_align(kv_rows * (size_t)d * sizeof(f16));
  const size_t pbytes = ws_align(q_rows * (size_t)d * sizeof(float));
  w.ctl = (unsigned*)p;
  p += cbytes;
  w.amax = (float*)p;
  p += abytes;
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

// The inputs as the caller gave them (for rewriting a copy at a new exponent).
struct BwdIn {
  const void *q, *k, *v, *dO;
  const float* desc;  // FP8: {s_q, s_k, s_v, s_dO}; bf16: unused
  int fin, fdo;       // formats of Q, K, V and of dO
  long rows, kv_rows;
};

// ---------------------------------------------------------------------------
// Values of 8 consecutive elements (bf16 values, or FP8 code values; every
// E4M3 and E5M2 value is exact in float32 and in fp16).
template <bool E5M2, int SEL>
__device__ __forceinline__ float fp8_byte(int w) {
  return E5M2 ? __builtin_amdgcn_cvt_f32_bf8(w, SEL) : __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}
template <int FMT>
__device__ __forceinline__ void load8(const void* base, size_t elem, float* f) {
  if (FMT == 0) {
    const i32x4 raw = *(const i32x4*)((const bf16*)base + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned w = (unsigned)raw[j];
      f[2 * j] = __builtin_bit_cast(float, w << 16);
      f[2 * j + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
    }
  } else {
    const i32x2 raw = *(const i32x2*)((const uint8_t*)base + elem);
    f[0] = fp8_byte<FMT == 2, 0>(raw[0]);
    f[1] = fp8_byte<FMT == 2, 1>(raw[0]);
    f[2] = fp8_byte<FMT == 2, 2>(raw[0]);
    f[3] = fp8_byte<FMT == 2, 3>(raw[0]);
    f[4] = fp8_byte<FMT == 2, 0>(raw[1]);
    f[5] = fp8_byte<FMT == 2, 1>(raw[1]);
    f[6] = fp8_byte<FMT == 2, 2>(raw[1]);
    f[7] = fp8_byte<FMT == 2, 3>(raw[1]);
  }
}
__device__ __forceinline__ void load8_fmt(int fmt, const void* base, size_t elem, float* f) {
  if (fmt == 0) load8<0>(base, elem, f);
  else if (fmt == 1) load8<1>(base, elem, f);
  else load8<2>(base, elem, f);
}
// fp16 copy of 8 values times mul (a power of two: exact unless it leaves fp16's range).
__device__ __forceinline__ f16x8 pack_f16(const float* f, float mul) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (f16)(f[j] * mul);
  return r;
}
__device__ __forceinline__ float amax8(const float* f) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  return m;
}

// Exponent that puts a tensor's largest magnitude amax into [4, 8).
__device__ __forceinline__ int exp_for(float amax) {
  int E;
  frexpf(amax, &E);  // amax = m 2^E, m in [0.5, 1)
  return min(120, max(-120, E - 3));
}

// Exponents e (copy = value * 2^-e) of Q, K, V, dO from the largest
// magnitudes of their values. A tensor keeps its format's default unless its
// default copy leaves the range where the fp16 products are safe: Q and K
// copies peak within [2^-6, 2^13]; V and dO copies too, and their peaks
// multiply to [1, 2^7], which keeps |dS| in copy units (at most 2 d times
// that product, d <= 128) below 2^15 while leaving it far above fp16's
// subnormals. Such a tensor takes exp_for(amax) instead (V and dO together).
// Zero and non-finite maxima keep the default.
__device__ __forceinline__ void choose_exps(const float* amax, int fin, int fdo, int* e) {
  const int ed[4] = {default_exp(fin), default_exp(fin), default_exp(fin), default_exp(fdo)};
  float a[4];
  bool odd[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    a[x] = ldexpf(amax[x], -ed[x]);
    odd[x] = !(amax[x] > 0.f) || !(amax[x] <= 3.0e38f);
  }
  auto fits = [](float v) { return v >= 0x1p-6f && v <= 0x1p13f; };
#pragma unroll
  for (int x = 0; x < 2; ++x) e[x] = (odd[x] || fits(a[x])) ? ed[x] : exp_for(amax[x]);
  const bool vd_ok = odd[2] || odd[3] || (fits(a[2]) && fits(a[3]) && a[2] * a[3] >= 1.f && a[2] * a[3] <= 128.f);
  e[2] = (vd_ok || odd[2]) ? ed[2] : exp_for(amax[2]);
  e[3] = (vd_ok || odd[3]) ? ed[3] : exp_for(amax[3]);
}

// The XCD this wave runs on.
__device__ __forceinline__ int xcd_id() {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return (int)(x & 7u);
}

// Next item of the work lists (see the top of this file), -1 when all are
// empty. List y holds items 8 t + y (t = 0, 1, ...) of the `total`. Each of
// the `grid` workgroups of a launch starts with item blockIdx.x (workgroups
// are dealt round-robin to the XCDs, so that is an item of its own XCD's
// list); the counter of list y (in line `set` + y of the control block,
// zero at launch) counts the items taken from it after those.
__device__ __forceinline__ int pop_item(unsigned* ctl, int set, int total, int grid, int x) {
  for (int s = 0; s < 8; ++s) {
    const int y = (x + s) & 7;
    const int ny = (total - y + 7) / 8, gy = (grid - y + 7) / 8;  // items of list y, taken at the start
    if (ny <= gy) continue;
    const int t = gy + (int)atomicAdd(ctl + 32 * (set + y), 1u);
    if (t < ny) return 8 * t + y;
  }
  return -1;
}

// Grid-wide barrier over the n workgroups of a persistent launch (all of
// them resident, one per CU), on a counter that is zero at launch. Memory
// written before it by any workgroup is visible after it. The wait is
// bounded (far beyond any real skew) so that it always ends.
__device__ __forceinline__ void grid_barrier(unsigned* ctr, unsigned n) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicAdd(ctr, 1u);
    for (int spin = 0; spin < (1 << 20); ++spin) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) break;
      __builtin_amdgcn_s_sleep(4);
    }
    __threadfence();
  }
  __syncthreads();
}

}  // namespace fa
