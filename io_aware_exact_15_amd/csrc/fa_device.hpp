// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand (32 x 16): lane l holds A[l % 32][8 * (l / 32) + 0..7]
//   B operand (16 x 32): lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   C/D (32 x 32, 16 floats): lane l, register i holds
//       C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32]
// The contraction index only has to be assigned consistently between A and
// B, which the kernels exploit to feed accumulator registers straight back
// into the next product without moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// E4M3 x E4M3, K = 64: lane l holds 32 codes of row/column l % 32; the two
// half-waves hold the two halves of the contraction.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Same product with the operand formats chosen per operand: 0 = E4M3,
// 1 = E5M2 (the instruction's A / B format fields).
template <int FMT_A, int FMT_B>
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT_A, FMT_B, 0, 0, 0, 0);
}

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16). Within each
// group of 16 lanes, lane j supplies the address of 4 consecutive elements
// (row j / 4, columns 4 * (j % 4) .. + 3 of a 4 x 16 block); lane n then
// receives column n of that block, one element per row.
__device__ __forceinline__ s16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 FA_LDS*)(p));
}

// Transposing LDS read of 8-bit data (ds_read_b64_tr_b8): within each group
// of 16 lanes, lane j supplies the address of 8 consecutive bytes (row
// j / 2, columns 8 * (j % 2) .. + 7 of an 8 x 16 block); lane n receives
// column n, one byte per row.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 FA_LDS*)(p));
}

__device__ __forceinline__ bf16x8 cat4(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Value held by the partner lane in the other half-wave (lane ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of x over the lane pair (l, l ^ 32) with one v_permlane32_swap:
// the swap returns {lower half of x in both halves, upper half of x in both
// halves}, so combining the two results gives the pair value in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup -> (head bh, block blk). Workgroups are dealt round-robin to the
// 8 XCDs; every query head of a head group (G consecutive query heads that
// share one key/value head) and all their blocks land on the same XCD, so a
// key/value head's tiles are read through one L2. heavy_first selects the
// order of the blocks: j-th wave of workgroups takes block j, or nb - 1 - j.
__device__ __forceinline__ void map_head_block(int bid, int BH, int G, int nb, bool heavy_first, int& bh, int& blk) {
  int j;
  if (((BH / G) & 7) == 0) {
    const int xcd = bid & 7, hpx = BH >> 3;  // query heads per XCD
    j = bid >> 3;
    const int r = j % hpx;
    bh = (xcd + 8 * (r / G)) * G + r % G;
    j /= hpx;
  } else if ((BH & 7) == 0) {
    const int xcd = bid & 7, hpx = BH >> 3;
    j = bid >> 3;
    bh = xcd + 8 * (j % hpx);
    j /= hpx;
  } else {
    bh = bid % BH;
    j = bid / BH;
  }
  blk = heavy_first ? j : nb - 1 - j;
}

// LDS address (byte offset inside the workgroup's LDS) of a __shared__ pointer.
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(size_t)(const FA_LDS void*)p; }

// Buffer resource (V#) for the LDS DMA below: 48-bit base, stride 0,
// num_records = bytes, default format word; buffer loads at offsets past
// `bytes` return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// BYTES (4 or 16) per lane from buffer byte offset `voff` straight into LDS
// (LDS DMA): lane l's data lands at dst + BYTES * l; dst must be wave-uniform.
// The compiler tracks which __shared__ object the load writes: a later read
// of that object by this wave waits for it, a read of another object does
// not, so the kernels give each stage of a load ring an object of its own.
// Other waves' loads into the same stage are ordered by the kernel itself
// (wait_vmem() by every loading wave, then a workgroup barrier).
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(rsrc_t r, const void* dst, unsigned voff) {
  static_assert(BYTES == 4 || BYTES == 16, "LDS DMA width");
  if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)dst, 16, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)dst, 4, voff, 0, 0, 0);
}

// Tile layout in LDS shared by the bf16/fp16 kernels: rows of D 2-byte
// elements (D / 8 chunks of 16 bytes), chunk c of row r stored at chunk
// c ^ tile_swz<D>(r). Reads of 16 rows at one chunk (ds_read_b128) and the
// transposing reads of 4 rows x 64 bytes (ds_read_b64_tr_b16) then hit
// distinct LDS banks.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if (D == 128) return (4 * (r & 3)) ^ ((r >> 2) & 3);  // 16 chunks per row
  return (4 * ((r >> 1) & 1)) ^ ((r >> 2) & 3);        // 8 chunks per row
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for this wave's global stores to complete.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace fa
