// Shared pieces of the bf16 MFMA attention kernels (gfx950, wave64).
//
// MFMA used: v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, C/D 32x32 fp32).
// Lane l (n = l % 32, hi = l / 32) supplies row n of A and column n of B,
// each as 8 consecutive k-elements of the half hi; accumulator register r of
// lane l holds D[8*(r/4) + 4*hi + (r%4)][n].
//
// Row permutation rho: if A-operand lane n carries logical row rho(n), the
// accumulator registers r = 0..15 of lane (n, hi) hold logical rows
// 16*hi + r, i.e. each half-wave owns 16 consecutive rows.  Tiles are stored
// in LDS with logical row t at LDS row rho_inv(t), so lane n always reads LDS
// row n (consecutive rows, conflict-free with the row padding below).
#pragma once

#include "device_common.hpp"

namespace bac {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// rho(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3); rho_inv(t) = 8*((t>>2)&3) + 4*(t>>4) + (t&3).
__host__ __device__ constexpr int rho(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
__host__ __device__ constexpr int rho_inv(int t) { return 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3); }

// Position of logical row t inside a tile made of 32-row blocks.
__device__ __forceinline__ int perm_row(int t) { return (t & ~31) | rho_inv(t & 31); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(p[j]);
  return r;
}

__device__ __forceinline__ bf16x8 lds_read8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(0.f);
  return r;
}

// XCD-aware block order: hardware dispatches block b to XCD b % 8.  Give
// every XCD a contiguous range of logical blocks so that blocks sharing K/V
// (same kv-head, neighbouring rows) share one L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int xcd = b & 7, idx = b >> 3;
  const int full = nb >> 3, rem = nb & 7;
  return xcd < rem ? xcd * (full + 1) + idx : rem * (full + 1) + (xcd - rem) * full + idx;
}

}  // namespace bac
