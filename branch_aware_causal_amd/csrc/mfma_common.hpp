// Shared pieces of the bf16 MFMA attention kernels (gfx950, wave64).
//
// MFMA used: v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, C/D 32x32 fp32).
// Lane l (n = l % 32, hi = l / 32) supplies row n of A and column n of B,
// each as 8 k-elements; accumulator register r of lane l holds
// D[8*(r/4) + 4*hi + (r%4)][n].
//
// Operand conventions used by every kernel here:
//   * "row operand": a lane reads 16 contiguous bytes of one tile row
//     (row n, k-elements 16*ks + 8*hi + 0..7) with ds_read_b128.
//   * "transposed operand": the MFMA rows are tile COLUMNS col0 + n and the
//     k-elements are tile rows kbase + 8*(j/4) + 4*hi + (j%4), j = 0..7.  Two
//     ds_read_b64_tr_b16 produce it from a row-major tile: inside each 16-lane
//     group, lanes pointing 4-per-row at 4 consecutive rows (16 columns) get
//     that 4x16 block transposed, one column per lane.
//   * "accumulator operand": registers r = 8*s + j (j = 0..7) of a 32x32
//     accumulator, rounded to bf16, are the B operand of k-step s.  Their
//     k-elements are accumulator rows 16*s + 8*(j/4) + 4*hi + (j%4), the same
//     order as a transposed operand with kbase = 16*s.
//
// LDS tiles are row-major bf16 with the 16-byte chunks of each row XOR-swizzled
// by the row index, so that both access patterns (16 consecutive rows at one
// chunk, and 4 consecutive rows x 4 chunks) touch distinct banks.
#pragma once

#include "device_common.hpp"

namespace bac {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(0.f);
  return r;
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(p[j]);
  return r;
}

// Swizzled position of 16-byte chunk c of row r in a tile with D columns.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) return c ^ ((4 * (r & 3)) | ((r >> 2) & 3));
  else return c ^ ((4 * ((r >> 1) & 1)) | ((r >> 2) & 3));
}

// Element offset of (row, col) in a swizzled tile; col % 4 == 0 keeps 8-byte alignment.
template <int D>
__device__ __forceinline__ int toff(int r, int col) {
  return r * D + 8 * swz<D>(r, col >> 3) + (col & 7);
}

// Per-lane operand addressing.  The swizzle depends only on row & 15, so for
// tile rows that differ by multiples of 16 a lane's offsets differ by the
// plain row stride: each lane precomputes its offsets once, and the kernels
// add compile-time row offsets (which fold into the LDS instruction's
// immediate offset).
template <int D>
struct LaneOffsets {
  static constexpr int KS = D / 16;
  static constexpr int MB = D / 32;
  int row[KS];       // row operand: tile row n, columns 16*ks + 8*hi .. +7
  int tr[MB][2];     // transposed operand: column block mb, first / second read
  __device__ __forceinline__ explicit LaneOffsets(int lane) {
    const int n = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) row[ks] = toff<D>(n, 16 * ks + 8 * hi);
    const int g = lane >> 4, i = lane & 15;
    const int r0 = 4 * (g >> 1) + (i >> 2);
    const int c0 = 16 * (g & 1) + 4 * (i & 3);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      tr[mb][0] = toff<D>(r0, 32 * mb + c0);
      tr[mb][1] = toff<D>(r0 + 8, 32 * mb + c0);
    }
  }
};

// Row operand: tile row (row16 + n) where row16 % 16 == 0, k-step ks.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* tile, const LaneOffsets<D>& lo,
                                              int row16, int ks) {
  return *reinterpret_cast<const bf16x8*>(tile + row16 * D + lo.row[ks]);
}

// Transposed operand: MFMA rows = tile columns 32*mb + n, k-elements = tile
// rows kbase + 8*(j/4) + 4*hi + (j%4), kbase % 16 == 0.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, const LaneOffsets<D>& lo,
                                             int kbase, int mb) {
  // generic -> LDS address space (the tile lives in __shared__ memory)
  lds_bf16x4* p0 = (lds_bf16x4*)(tile + kbase * D + lo.tr[mb][0]);
  lds_bf16x4* p1 = (lds_bf16x4*)(tile + kbase * D + lo.tr[mb][1]);
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p0);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p1);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Transposed operand from precomputed lane offsets (LaneOffsets::tr[mb]).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand_at(const uint16_t* tile, int kbase, int off0, int off1) {
  lds_bf16x4* p0 = (lds_bf16x4*)(tile + kbase * D + off0);
  lds_bf16x4* p1 = (lds_bf16x4*)(tile + kbase * D + off1);
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p0);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p1);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Accumulator row of register r for lane half hi.
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// XCD-aware block order: hardware dispatches block b to XCD b % 8.  Give
// every XCD a contiguous range of logical blocks so that blocks sharing K/V
// (same kv-head, neighbouring rows) share one L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int xcd = b & 7, idx = b >> 3;
  const int full = nb >> 3, rem = nb & 7;
  return xcd < rem ? xcd * (full + 1) + idx : rem * (full + 1) + (xcd - rem) * full + idx;
}

// m = max(m, x[0..15]) as eight chained v_max3_f32.  fmaxf would first
// quiet each operand (IEEE mode), one extra instruction per element, and
// separate asm statements would each be followed by a hazard nop; the
// values fed here are finite or -inf.
__device__ __forceinline__ float max16_raw(float m, const f32x16& x) {
  asm("v_max3_f32 %0, %0, %1, %2\n\t"
      "v_max3_f32 %0, %0, %3, %4\n\t"
      "v_max3_f32 %0, %0, %5, %6\n\t"
      "v_max3_f32 %0, %0, %7, %8\n\t"
      "v_max3_f32 %0, %0, %9, %10\n\t"
      "v_max3_f32 %0, %0, %11, %12\n\t"
      "v_max3_f32 %0, %0, %13, %14\n\t"
      "v_max3_f32 %0, %0, %15, %16"
      : "+v"(m)
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]),
        "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]),
        "v"(x[15]));
  return m;
}

// max(v, v of lane l ^ 32) without going through LDS.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Marks v as computed at this point.  Barriers order memory accesses only,
// so without this the compiler may sink register arithmetic past them.
__device__ __forceinline__ void keep(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void keep(bf16x8 v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void keep(f32x16 v) { asm volatile("" ::"v"(v)); }

// Compile-time flag as a value, to pick lambda variants.
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14])
constexpr int kWaitAll = 0;
constexpr int kWaitLgkm = 0xC07F;   // lgkmcnt(0), vmcnt and expcnt not waited on
constexpr int kWaitNone = 0xCF7F;   // nothing waited on

template <int kWait>
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWait);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)p));
}

// Scalar-register copy of a wave-uniform pointer.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Direct global->LDS loads: lane l reads global address base + voff (base
// wave-uniform, in scalar registers; voff a per-lane 32-bit byte offset) and
// writes LDS[lds + l*bytes].  Issued as inline assembly so that the compiler
// does not guard later LDS reads with waits on these loads: the kernel waits
// for them itself (vmcnt) before the barrier that publishes a ring stage.
// `lds` must be wave-uniform.  The s_nop covers the M0 write -> LDS-DMA
// hazard.
__device__ __forceinline__ void dma_b128(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(uniform_ptr(base)), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
// Same with a full 64-bit per-lane address (no scalar base).
__device__ __forceinline__ void dma_b32_at(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(addr), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

}  // namespace bac
