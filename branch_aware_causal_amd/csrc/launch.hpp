// Internal launcher interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bac {

enum DType : int { kF32 = 0, kBF16 = 1 };

// One main-attention call: query rows against one K/V shard.
struct MainArgs {
  const void* q;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int nq;
  const void* k;
  const void* v;
  const int32_t* k_seq;
  const int32_t* k_pos;
  int nk;
  int hq, hkv, d;
  int dt;
  float scale;
  // forward
  float* o_acc;
  float* lse_acc;
  int mode;            // 0 write, 1 merge
  void* o_out;
  // backward
  const void* dout;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  hipStream_t stream;
};

// One branch-attention call over rank-local branches.
struct BranchArgs {
  const void* qb;
  const void* kb;
  const void* vb;
  int nb;
  const int32_t* branch_cu;
  int num_branches;
  int max_len;
  int bidir;                   // kind of every branch when kinds is null
  const int32_t* kinds;        // per-branch kind (device) or null
  int hq, hkv, d;
  int dt;
  float scale;
  float* o_acc;
  float* lse_acc;
  int mode;
  void* o_out;
  const void* dout;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  hipStream_t stream;
};

hipError_t launch_main_fwd_valu(const MainArgs& a);
hipError_t launch_main_bwd_valu(const MainArgs& a, int part = 0);
hipError_t launch_main_fwd_mfma(const MainArgs& a);
// part: 0 = dq and dk/dv, 1 = dq only, 2 = dk/dv only
hipError_t launch_main_bwd_mfma(const MainArgs& a, int part = 0);
hipError_t launch_branch_fwd(const BranchArgs& a);
hipError_t launch_branch_bwd(const BranchArgs& a);
hipError_t launch_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                            int n, int hq, int d, int out_dt, void* o_out, hipStream_t s);
hipError_t launch_delta(const void* o, int o_dt, const void* dout, int dt, int n, int hq, int d,
                        float* delta, hipStream_t s);
hipError_t launch_tap_send(void* slot_ptr, uint64_t* stamps, int slot, const void* payload,
                           int64_t nbytes, uint64_t seq, hipStream_t s);
hipError_t launch_tap_recv(const void* slot_ptr, const uint64_t* stamps, int slot, uint64_t seq,
                           int64_t spin_limit, void* out, int64_t nbytes, int32_t* status,
                           hipStream_t s);
hipError_t launch_check_index(const int32_t* seq, const int32_t* pos, int n, int strict,
                              int32_t* bad, hipStream_t s);

}  // namespace bac
