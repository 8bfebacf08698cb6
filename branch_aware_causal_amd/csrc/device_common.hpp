// Device helpers shared by the gfx950 kernels of libbac.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bac {

constexpr float kLog2e = 1.4426950408889634f;   // log2(e)
constexpr float kLn2 = 0.6931471805599453f;     // ln(2)
constexpr float kNegInf = -__builtin_huge_valf();

// v_exp_f32 / v_log_f32 are base-2; callers work in log2 units and convert
// with the mathematical constants above.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN); gfx950 has a native
// instruction for the pair form, used through the __bf16 conversion.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(float_to_bf16_bits(lo)) |
         (static_cast<uint32_t>(float_to_bf16_bits(hi)) << 16);
}

// Element loads for the two supported element types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {   // bf16 stored as raw bits
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf16_bits_to_float(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float x) {
    p[i] = float_to_bf16_bits(x);
  }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Merge of two partials in log2 units: (oa, la) <- merge((oa, la), (ob, lb)).
// Returns the weights (wa, wb) with wa + wb = 1 (or 0, 0 when both empty) and
// writes the merged log2-sum-exp.  [G] 技术贡献: l = ln(e^la + e^lb),
// O = e^(la-l) Oa + e^(lb-l) Ob.
__device__ __forceinline__ void merge_weights_log2(float la2, float lb2, float& wa, float& wb,
                                                   float& l2) {
  float m = fmaxf(la2, lb2);
  if (m == kNegInf) {
    wa = 0.f;
    wb = 0.f;
    l2 = kNegInf;
    return;
  }
  float ea = exp2_fast(la2 - m);   // exp2(-inf) = 0
  float eb = exp2_fast(lb2 - m);
  float s = ea + eb;
  float inv = 1.f / s;
  wa = ea * inv;
  wb = eb * inv;
  l2 = m + log2_fast(s);
}

// Lexicographic (seq, pos) comparisons used by the range searches.
__device__ __forceinline__ bool lex_less(int s0, int p0, int s1, int p1) {
  return s0 < s1 || (s0 == s1 && p0 < p1);
}

// First index j in [0, n) with (seq[j], pos[j]) >= (s, p); n if none.
__device__ __forceinline__ int lower_bound_sp(const int32_t* seq, const int32_t* pos, int n,
                                              int s, int p) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (lex_less(seq[mid], pos[mid], s, p)) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// First index j in [0, n) with (seq[j], pos[j]) > (s, p); n if none.
__device__ __forceinline__ int upper_bound_sp(const int32_t* seq, const int32_t* pos, int n,
                                              int s, int p) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (!lex_less(s, p, seq[mid], pos[mid])) lo = mid + 1; else hi = mid;
  }
  return lo;
}

}  // namespace bac
