// TapChannel-style one-way feature hand-off through preallocated device
// slots with sequence stamps ([G] 技术贡献 and 方法详解 · PP传输: producer
// stages write target features into the consumer's preallocated slots and
// bump a sequence stamp; the consumer reads by stamp, off the pipeline
// schedule).  This is the single-GPU part: producer and consumer are two
// streams of one device.
//
// Ordering: tap_send is two launches on the producer's stream -- the payload
// copy, then a one-lane kernel that stores the stamp with release semantics
// at device scope -- so the stamp is written only after every byte of the
// payload has landed.  tap_recv polls the stamp with acquire loads (device
// scope) and copies the slot only once the stamp equals the expected
// sequence number.  Every wait is bounded by the caller's spin limit; a
// consumer that gives up reports it in its status word and copies nothing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace bac {

namespace tap {
constexpr int kThreads = 256;
constexpr int kBlocks = 1024;      // grid-stride copy
}  // namespace tap

// dst[i] = src[i] for 16-byte words (both 16-byte aligned), grid-stride.
__global__ __launch_bounds__(256) void tap_copy_kernel(uint4* __restrict__ dst,
                                                       const uint4* __restrict__ src, int64_t n16,
                                                       const uint8_t* __restrict__ src_tail,
                                                       uint8_t* __restrict__ dst_tail, int tail) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
  if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

// *status = 0 (a kernel rather than a memset, so the call can be captured).
__global__ void tap_status_init_kernel(int32_t* status) {
  if (threadIdx.x == 0) *status = 0;
}

// stamps[slot] = seq, released at device scope after everything the stream
// wrote before it.
__global__ void tap_stamp_kernel(uint64_t* stamps, int slot, uint64_t seq) {
  if (threadIdx.x == 0)
    __hip_atomic_store(stamps + slot, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Each block's first lane polls the stamp (acquire) until it is at least
// seq or spin_limit polls have passed; the block then copies its share of
// the slot if the stamp equals seq.  status: 0 received, 1 gave up,
// 2 the slot already holds a newer sequence (set by any block that sees it).
__global__ __launch_bounds__(256) void tap_recv_kernel(const uint64_t* stamps, int slot,
                                                       uint64_t seq, int64_t spin_limit,
                                                       uint4* __restrict__ dst,
                                                       const uint4* src, int64_t n16,
                                                       const uint8_t* src_tail,
                                                       uint8_t* __restrict__ dst_tail, int tail,
                                                       int32_t* status) {
  __shared__ int verdict;
  if (threadIdx.x == 0) {
    uint64_t s = 0;
    int64_t it = 0;
    for (;;) {
      s = __hip_atomic_load(stamps + slot, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      if (s >= seq || ++it >= spin_limit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    // 0 equal, 1 older, 2 newer, as the sum of two comparisons: this
    // compiler turned the equivalent nested conditional into two scalar
    // selects on one stale condition code (equal gave 1, newer gave 0)
    const int v = static_cast<int>(s != seq) + static_cast<int>(s > seq);
    verdict = v;
    if (v != 0) *status = v;   // vector store; every writer writes a nonzero code
  }
  __syncthreads();
  if (verdict != 0) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // every lane reads after the stamp
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
  if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

static int blocks_for(int64_t n16) {
  const int64_t b = (n16 + tap::kThreads - 1) / tap::kThreads;
  return static_cast<int>(b < 1 ? 1 : (b > tap::kBlocks ? tap::kBlocks : b));
}

hipError_t launch_tap_send(void* slot_ptr, uint64_t* stamps, int slot, const void* payload,
                           int64_t nbytes, uint64_t seq, hipStream_t s) {
  const int64_t n16 = nbytes / 16;
  const int tail = static_cast<int>(nbytes % 16);
  if (nbytes > 0)
    hipLaunchKernelGGL(tap_copy_kernel, dim3(blocks_for(n16)), dim3(tap::kThreads), 0, s,
                       static_cast<uint4*>(slot_ptr), static_cast<const uint4*>(payload), n16,
                       static_cast<const uint8_t*>(payload) + n16 * 16,
                       static_cast<uint8_t*>(slot_ptr) + n16 * 16, tail);
  hipLaunchKernelGGL(tap_stamp_kernel, dim3(1), dim3(64), 0, s, stamps, slot, seq);
  return hipGetLastError();
}

hipError_t launch_tap_recv(const void* slot_ptr, const uint64_t* stamps, int slot, uint64_t seq,
                           int64_t spin_limit, void* out, int64_t nbytes, int32_t* status,
                           hipStream_t s) {
  const int64_t n16 = nbytes / 16;
  const int tail = static_cast<int>(nbytes % 16);
  hipLaunchKernelGGL(tap_status_init_kernel, dim3(1), dim3(64), 0, s, status);
  hipLaunchKernelGGL(tap_recv_kernel, dim3(blocks_for(n16)), dim3(tap::kThreads), 0, s, stamps,
                     slot, seq, spin_limit, static_cast<uint4*>(out),
                     static_cast<const uint4*>(slot_ptr), n16,
                     static_cast<const uint8_t*>(slot_ptr) + n16 * 16,
                     static_cast<uint8_t*>(out) + n16 * 16, tail, status);
  return hipGetLastError();
}

}  // namespace bac
