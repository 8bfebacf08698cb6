// HBM-bound kernels: the online-softmax merge, the backward's Delta and the
// device-side index check.  gfx950, wave64.
//
// Merge: [G] 技术贡献 / 方法详解 · CP计算 (l = ln(e^la + e^lb),
// O = e^(la-l) Oa + e^(lb-l) Ob).  Each thread owns 4 consecutive elements of
// one (row, head) vector, so loads and stores are 16-byte and coalesced.

#include "device_common.hpp"
#include "launch.hpp"

namespace bac {

template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(float* __restrict__ o_acc,
                                                        float* __restrict__ lse_acc,
                                                        const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part, int n,
                                                        int hq, int out_dt, void* o_out) {
  constexpr int TPR = D / 4;   // threads per (row, head)
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t rh = tid / TPR;
  const int c = static_cast<int>(tid % TPR);
  if (rh >= static_cast<int64_t>(n) * hq) return;
  const int i = static_cast<int>(rh / hq);
  const int h = static_cast<int>(rh % hq);
  const size_t li = static_cast<size_t>(h) * n + i;
  float wa, wb, l2;
  merge_weights_log2(lse_acc[li] * kLog2e, lse_part[li] * kLog2e, wa, wb, l2);
  const size_t off = static_cast<size_t>(rh) * D + 4 * c;
  float4 a = *reinterpret_cast<const float4*>(o_acc + off);
  float4 b = *reinterpret_cast<const float4*>(o_part + off);
  float4 r;
  r.x = wa * a.x + wb * b.x;
  r.y = wa * a.y + wb * b.y;
  r.z = wa * a.z + wb * b.z;
  r.w = wa * a.w + wb * b.w;
  *reinterpret_cast<float4*>(o_acc + off) = r;
  if (o_out) {
    if (out_dt == kBF16) {
      uint2 pk;
      pk.x = pack_bf16x2(r.x, r.y);
      pk.y = pack_bf16x2(r.z, r.w);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o_out) + off) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(o_out) + off) = r;
    }
  }
  if (c == 0) lse_acc[li] = (l2 == kNegInf) ? kNegInf : l2 * kLn2;
}

hipError_t launch_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                            int n, int hq, int d, int out_dt, void* o_out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t threads = static_cast<int64_t>(n) * hq * (d / 4);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (d == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(256), 0, s, o_acc, lse_acc, o_part,
                       lse_part, n, hq, out_dt, o_out);
  else
    hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(256), 0, s, o_acc, lse_acc, o_part,
                       lse_part, n, hq, out_dt, o_out);
  return hipGetLastError();
}

// Delta[h, i] = <dout[i, h, :], o[i, h, :]>, fp32.  D/4 threads per (row, head)
// (a half or a quarter of a wave), reduced with xor shuffles inside the group.
template <int D, typename TO, typename TD>
__global__ __launch_bounds__(256) void delta_kernel(const TO* __restrict__ o,
                                                    const TD* __restrict__ dout, int n, int hq,
                                                    float* __restrict__ delta) {
  constexpr int TPR = D / 4;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t rh = tid / TPR;
  const int c = static_cast<int>(tid % TPR);
  const bool live = rh < static_cast<int64_t>(n) * hq;
  float acc = 0.f;
  if (live) {
    const size_t off = static_cast<size_t>(rh) * D + 4 * c;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += Elem<TO>::load(o, off + e) * Elem<TD>::load(dout, off + e);
  }
#pragma unroll
  for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
  if (live && c == 0) {
    const int i = static_cast<int>(rh / hq);
    const int h = static_cast<int>(rh % hq);
    delta[static_cast<size_t>(h) * n + i] = acc;
  }
}

template <int D>
static void launch_delta_d(const void* o, int o_dt, const void* dout, int dt, int n, int hq,
                           float* delta, hipStream_t s) {
  const int64_t threads = static_cast<int64_t>(n) * hq * (D / 4);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (o_dt == kF32 && dt == kF32)
    hipLaunchKernelGGL((delta_kernel<D, float, float>), grid, dim3(256), 0, s,
                       static_cast<const float*>(o), static_cast<const float*>(dout), n, hq, delta);
  else if (o_dt == kF32 && dt == kBF16)
    hipLaunchKernelGGL((delta_kernel<D, float, uint16_t>), grid, dim3(256), 0, s,
                       static_cast<const float*>(o), static_cast<const uint16_t*>(dout), n, hq,
                       delta);
  else if (o_dt == kBF16 && dt == kBF16)
    hipLaunchKernelGGL((delta_kernel<D, uint16_t, uint16_t>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), n, hq,
                       delta);
  else
    hipLaunchKernelGGL((delta_kernel<D, uint16_t, float>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(o), static_cast<const float*>(dout), n, hq,
                       delta);
}

hipError_t launch_delta(const void* o, int o_dt, const void* dout, int dt, int n, int hq, int d,
                        float* delta, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (d == 128) launch_delta_d<128>(o, o_dt, dout, dt, n, hq, delta, s);
  else launch_delta_d<64>(o, o_dt, dout, dt, n, hq, delta, s);
  return hipGetLastError();
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

__global__ __launch_bounds__(256) void check_index_kernel(const int32_t* __restrict__ seq,
                                                          const int32_t* __restrict__ pos, int n,
                                                          int strict, int32_t* bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  bool ok = pos[i] >= 0;
  if (i > 0) {
    const int s0 = seq[i - 1], p0 = pos[i - 1], s1 = seq[i], p1 = pos[i];
    const bool less = lex_less(s1, p1, s0, p0);
    const bool equal = (s0 == s1) && (p0 == p1);
    ok = ok && !less && !(strict && equal);
  }
  if (!ok) atomicAdd(bad, 1);
}

hipError_t launch_check_index(const int32_t* seq, const int32_t* pos, int n, int strict,
                              int32_t* bad, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, bad);
  if (n > 0)
    hipLaunchKernelGGL(check_index_kernel, dim3((n + 255) / 256), dim3(256), 0, s, seq, pos, n,
                       strict, bad);
  return hipGetLastError();
}

}  // namespace bac
