// Vector-ALU attention kernels (gfx950, wave64):
//   * rank-local branch attention, forward and backward ([G] 技术贡献: the
//     local branch part of a branch query; branch K/V stays on its rank);
//   * the fp32 main-attention path (one wave per (row, head); fp32 has no
//     MFMA product worth the packing at the sizes it serves).
// Branch work is a few keys per row and HBM-bound, so one wave handles one
// (branch, kv-head), each row spread over D/8 lanes with several q-heads of
// the group side by side; dot products are DPP sums inside a row's lanes.
// All index reads are range-clamped.

#include <climits>

#include "device_common.hpp"
#include "launch.hpp"

namespace bac {

template <typename T, int EPL>
__device__ __forceinline__ void load_lane(const T* base, size_t off, int lane, float (&x)[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = Elem<T>::load(base, off + lane * EPL + e);
}

// Normalise a row's running (o, m2, l), optionally merge it into the
// accumulators, and store.  m2 is the running max in log2 units, l the
// running sum of exp2(x - m2).
template <typename T, int EPL>
__device__ __forceinline__ void finish_row(const float (&o)[EPL], float m2, float l, size_t voff,
                                           size_t lidx, int mode, float* o_acc, float* lse_acc,
                                           T* o_out, int lane) {
  float lse2, inv;
  if (l > 0.f) {
    lse2 = m2 + log2_fast(l);
    inv = 1.f / l;
  } else {
    lse2 = kNegInf;
    inv = 0.f;
  }
  float res[EPL];
  float lnew = lse2;
  if (mode == 1) {
    float wa, wb;
    merge_weights_log2(lse_acc[lidx] * kLog2e, lse2, wa, wb, lnew);
#pragma unroll
    for (int e = 0; e < EPL; ++e) res[e] = wa * o_acc[voff + lane * EPL + e] + wb * (o[e] * inv);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) res[e] = o[e] * inv;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    o_acc[voff + lane * EPL + e] = res[e];
    if (o_out) Elem<T>::store(o_out, voff + lane * EPL + e, res[e]);
  }
  if (lane == 0) lse_acc[lidx] = (lnew == kNegInf) ? kNegInf : lnew * kLn2;
}

// Compensated (Kahan) accumulation: the fp32 gradients sum up to thousands
// of terms per element, and plain sequential fp32 sums lose ~sqrt(n) ulps.
__device__ __forceinline__ void kahan_add(float& sum, float& comp, float x) {
  const float y = x - comp;
  const float t = sum + y;
  comp = (t - sum) - y;
  sum = t;
}

// Online-softmax update with one key's score x (log2 units) and value v.
template <int EPL>
__device__ __forceinline__ void online_update(float x, const float (&v)[EPL], float& m2, float& l,
                                              float (&o)[EPL]) {
  const float mn = fmaxf(m2, x);
  const float corr = exp2_fast(m2 - mn);   // m2 = -inf -> 0
  const float p = exp2_fast(x - mn);
  l = l * corr + p;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = o[e] * corr + p * v[e];
  m2 = mn;
}

// Eight consecutive elements of a row as fp32 (16-byte loads for bf16, two
// for fp32); the offset is a multiple of 8 elements.
template <typename T>
__device__ __forceinline__ void load8(const T* base, size_t off, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 w = *reinterpret_cast<const uint4*>(base + off);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(base + off);
    const float4 b = *reinterpret_cast<const float4*>(base + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* base, size_t off, const float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    uint4 w;
    w.x = pack_bf16x2(x[0], x[1]);
    w.y = pack_bf16x2(x[2], x[3]);
    w.z = pack_bf16x2(x[4], x[5]);
    w.w = pack_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(base + off) = w;
  } else {
    *reinterpret_cast<float4*>(base + off) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(base + off + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// Sum over each aligned group of N lanes (N = 8 or 16), every lane of the
// group receiving it, with DPP moves inside the 16-lane rows: swap within
// pairs, then within quads, then mirror the half-rows, then the rows.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "DPP row moves stay inside 16-lane rows");
  auto mov = [](float v, int ctrl) -> float {
    switch (ctrl) {
      case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
      case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
      case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
      default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
    }
  };
  x += mov(x, 0);   // quad_perm [1,0,3,2]: lane ^ 1
  x += mov(x, 1);   // quad_perm [2,3,0,1]: lane ^ 2
  x += mov(x, 2);   // row_half_mirror: lane i <-> 7 - i within each 8
  if constexpr (N == 16) x += mov(x, 3);   // row_mirror: lane i <-> 15 - i
  return x;
}

// ---------------------------------------------------------------------------
// Branch forward: wave w of block b handles branch a = 4b + w, kv-head
// blockIdx.y, i.e. rows (t, h) for every token t of the branch and every
// q-head h of the group, TB tokens at a time.  A row occupies D/8 lanes (eight elements each, so
// every access is 16 or 32 contiguous bytes per lane) and a pass covers
// 64/(D/8) q-heads of the group at once; dot products are DPP sums inside
// each row's lanes.  No LDS; tokens past max_len are left untouched.
// ---------------------------------------------------------------------------
template <typename T, int D, int TB>
__global__ __launch_bounds__(256) void branch_fwd_kernel(const T* __restrict__ qb,
                                                         const T* __restrict__ kb,
                                                         const T* __restrict__ vb, int nb,
                                                         const int32_t* __restrict__ bcu, int A,
                                                         int max_len, int bidir_all,
                                                         const int32_t* __restrict__ kinds,
                                                         int hq, int hkv,
                                                         float scale_log2, float* o_acc,
                                                         float* lse_acc, int mode, T* o_out) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPW = 64 / LPR;    // q-heads per pass
  const int lane = threadIdx.x & 63;
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (a >= A) return;
  const bool bidir = kinds ? kinds[a] == 1 : bidir_all != 0;   // 1 = BAC_BRANCH_BIDIR
  const int g = blockIdx.y;
  const int G = hq / hkv;
  const int r = lane / LPR, col = 8 * (lane % LPR);
  const int t0 = max(0, min(bcu[a], nb));
  const int t1 = max(t0, min(bcu[a + 1], nb));
  const int len = min(t1 - t0, max_len);   // tokens past the bound are left untouched
  // TB tokens per step: each K/V row loaded serves TB rows (the per-row
  // online-softmax updates run in the same key order as one token at a time)
  for (int c0 = 0; c0 < G; c0 += RPW) {
    // lanes past the group's last q-head repeat its first and store nothing
    const bool row_ok = c0 + r < G;
    const int h = g * G + (row_ok ? c0 + r : 0);
    for (int tb = 0; tb < len; tb += TB) {
      const int nt = min(TB, len - tb);
      float q[TB][8], o[TB][8], m2[TB], l[TB];
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        // slots past the last token repeat it; their results are dropped
        const int t = tb + min(j, nt - 1);
        load8<T>(qb, (static_cast<size_t>(t0 + t) * hq + h) * D + col, q[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
        m2[j] = kNegInf;
        l[j] = 0.f;
      }
      const int kend = bidir ? len : tb + nt;   // keys some token of the step sees
      for (int u = 0; u < kend; ++u) {
        const size_t koff = (static_cast<size_t>(t0 + u) * hkv + g) * D + col;
        float kk[8], vv[8];
        load8<T>(kb, koff, kk);
        load8<T>(vb, koff, vv);
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          if (j < nt && (bidir || u <= tb + j)) {   // wave-uniform
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(q[j][e], kk[e], dot);
            dot = group_sum<LPR>(dot);
            online_update<8>(dot * scale_log2, vv, m2[j], l[j], o[j]);
          }
        }
      }
      if (!row_ok) continue;
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if (j >= nt) break;
        const int t = tb + j;
        const size_t qoff = (static_cast<size_t>(t0 + t) * hq + h) * D + col;
        // normalise, merge into the accumulators if asked, store
        float lse2, inv;
        if (l[j] > 0.f) {
          lse2 = m2[j] + log2_fast(l[j]);
          inv = 1.f / l[j];
        } else {
          lse2 = kNegInf;
          inv = 0.f;
        }
        const size_t lidx = static_cast<size_t>(h) * nb + t0 + t;
        float res[8];
        float lnew = lse2;
        if (mode == 1) {
          float wa, wb, prev[8];
          merge_weights_log2(lse_acc[lidx] * kLog2e, lse2, wa, wb, lnew);
          load8<float>(o_acc, qoff, prev);
#pragma unroll
          for (int e = 0; e < 8; ++e) res[e] = wa * prev[e] + wb * (o[j][e] * inv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) res[e] = o[j][e] * inv;
        }
        store8<float>(o_acc, qoff, res);
        if (o_out) store8<T>(o_out, qoff, res);
        if (col == 0) lse_acc[lidx] = (lnew == kNegInf) ? kNegInf : lnew * kLn2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Branch backward: one wave per (branch, kv-head), rows laid out as in the
// forward (D/8 lanes per row, 64/(D/8) q-heads per pass).  For a row (t, h)
// and a visible key u: s = <q, k_u>, P = exp2(s*c - lse2), dP = <dO, v_u>,
// dS = P (dP - Delta).  Two passes, both recomputing s and dP:
//   1. token-outer, TB tokens per step: dq_row += dS k_u in registers, one
//      += per row;
//   2. key-outer, KB keys per step: dk_u += dS q_row, dv_u += P dO_row in
//      registers over every row that sees u, then summed over the pass's
//      q-heads (shuffles across the row groups) and added once per key.
// Each K/V row loaded in pass 1 serves TB rows and each Q/dO row loaded in
// pass 2 serves KB keys; every row and key still sums its terms in the same
// order as one at a time.
// The wave owns every row and key it touches, so += on the global
// accumulators is race-free and no LDS is needed.
// ---------------------------------------------------------------------------
template <typename T, int D, int TB, int KB>
__global__ __launch_bounds__(256) void branch_bwd_kernel(
    const T* __restrict__ qb, const T* __restrict__ kb, const T* __restrict__ vb, int nb,
    const int32_t* __restrict__ bcu, int A, int max_len, int bidir_all,
    const int32_t* __restrict__ kinds, int hq, int hkv, float scale,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* dq, float* dk, float* dv) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPW = 64 / LPR;    // q-heads per pass
  const int lane = threadIdx.x & 63;
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (a >= A) return;
  const bool bidir = kinds ? kinds[a] == 1 : bidir_all != 0;   // 1 = BAC_BRANCH_BIDIR
  const int g = blockIdx.y;
  const int G = hq / hkv;
  const int r = lane / LPR, col = 8 * (lane % LPR);
  const float scale_log2 = scale * kLog2e;
  const int t0 = max(0, min(bcu[a], nb));
  const int t1 = max(t0, min(bcu[a + 1], nb));
  const int len = min(t1 - t0, max_len);   // tokens past the bound are left untouched
  // P and dS of row (t, h) and key u, given the row's q, dO, lse2, Delta
  auto p_ds = [&](const float (&q)[8], const float (&d_o)[8], float lse2, float dl,
                  const float (&kk)[8], const float (&vv)[8], float& p, float& ds) {
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s = fmaf(q[e], kk[e], s);
      dp = fmaf(d_o[e], vv[e], dp);
    }
    s = group_sum<LPR>(s);
    dp = group_sum<LPR>(dp);
    p = (lse2 == kNegInf) ? 0.f : exp2_fast(s * scale_log2 - lse2);
    ds = p * (dp - dl);
  };
  // pass 1: dQ, TB tokens per step (each K/V row loaded serves TB rows; every
  // row sums its keys in the same order as one token at a time)
  for (int c0 = 0; c0 < G; c0 += RPW) {
    const bool row_ok = c0 + r < G;
    const int h = g * G + (row_ok ? c0 + r : 0);
    for (int tb = 0; tb < len; tb += TB) {
      const int nt = min(TB, len - tb);
      float q[TB][8], d_o[TB][8], dqr[TB][8], lse2[TB], dl[TB];
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        // slots past the last token repeat it; their results are dropped
        const int t = tb + min(j, nt - 1);
        const size_t qoff = (static_cast<size_t>(t0 + t) * hq + h) * D + col;
        const size_t li = static_cast<size_t>(h) * nb + t0 + t;
        load8<T>(qb, qoff, q[j]);
        load8<T>(dout, qoff, d_o[j]);
        lse2[j] = lse[li] * kLog2e;
        dl[j] = delta[li];
#pragma unroll
        for (int e = 0; e < 8; ++e) dqr[j][e] = 0.f;
      }
      const int kend = bidir ? len : tb + nt;   // keys some token of the step sees
      for (int u = 0; u < kend; ++u) {
        const size_t koff = (static_cast<size_t>(t0 + u) * hkv + g) * D + col;
        float kk[8], vv[8];
        load8<T>(kb, koff, kk);
        load8<T>(vb, koff, vv);
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          if (j < nt && (bidir || u <= tb + j)) {   // wave-uniform
            float p, ds;
            p_ds(q[j], d_o[j], lse2[j], dl[j], kk, vv, p, ds);
#pragma unroll
            for (int e = 0; e < 8; ++e) dqr[j][e] = fmaf(ds, kk[e], dqr[j][e]);
          }
        }
      }
      if (!row_ok) continue;
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if (j >= nt) break;
        const size_t qoff = (static_cast<size_t>(t0 + tb + j) * hq + h) * D + col;
        float cur[8];
        load8<float>(dq, qoff, cur);
#pragma unroll
        for (int e = 0; e < 8; ++e) cur[e] = fmaf(scale, dqr[j][e], cur[e]);
        store8<float>(dq, qoff, cur);
      }
    }
  }
  // pass 2: dK, dV, KB keys per step (each Q/dO row loaded serves KB keys;
  // every key sums its rows in the same order as one key at a time)
  for (int ub = 0; ub < len; ub += KB) {
    const int nk = min(KB, len - ub);
    float kk[KB][8], vv[KB][8], dka[KB][8], dva[KB][8];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const size_t koff = (static_cast<size_t>(t0 + ub + min(i, nk - 1)) * hkv + g) * D + col;
      load8<T>(kb, koff, kk[i]);
      load8<T>(vb, koff, vv[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dka[i][e] = 0.f;
        dva[i][e] = 0.f;
      }
    }
    for (int c0 = 0; c0 < G; c0 += RPW) {
      const bool row_ok = c0 + r < G;
      const int h = g * G + (row_ok ? c0 + r : 0);
      for (int t = bidir ? 0 : ub; t < len; ++t) {   // rows some key of the step is seen by
        const size_t qoff = (static_cast<size_t>(t0 + t) * hq + h) * D + col;
        const size_t li = static_cast<size_t>(h) * nb + t0 + t;
        float q[8], d_o[8];
        load8<T>(qb, qoff, q);
        load8<T>(dout, qoff, d_o);
        const float lse2 = lse[li] * kLog2e, dl = delta[li];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          if (i < nk && (bidir || t >= ub + i)) {   // wave-uniform
            float p, ds;
            p_ds(q, d_o, lse2, dl, kk[i], vv[i], p, ds);
            if (row_ok) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                dka[i][e] = fmaf(ds, q[e], dka[i][e]);
                dva[i][e] = fmaf(p, d_o[e], dva[i][e]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (i >= nk) break;
      // sum over the row groups (lanes that differ by multiples of LPR)
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dka[i][e] += __shfl_xor(dka[i][e], off);
          dva[i][e] += __shfl_xor(dva[i][e], off);
        }
      if (r != 0) continue;
      const size_t koff = (static_cast<size_t>(t0 + ub + i) * hkv + g) * D + col;
      float ck[8], cv[8];
      load8<float>(dk, koff, ck);
      load8<float>(dv, koff, cv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ck[e] = fmaf(scale, dka[i][e], ck[e]);
        cv[e] += dva[i][e];
      }
      store8<float>(dk, koff, ck);
      store8<float>(dv, koff, cv);
    }
  }
}

// Branch backward for branches of at most MAXL tokens (used with MAXL = 4): one
// token-outer pass in the same row layout, with dK/dV of every key of the
// branch in registers (dQ accumulates per row as in the two-pass kernel), so
// each row's Q and dO are read once.  The keys' sums over the group's
// q-heads are taken at the end.
template <typename T, int D, int MAXL>
__global__ __launch_bounds__(256) void branch_bwd_short_kernel(
    const T* __restrict__ qb, const T* __restrict__ kb, const T* __restrict__ vb, int nb,
    const int32_t* __restrict__ bcu, int A, int max_len, int bidir_all,
    const int32_t* __restrict__ kinds, int hq, int hkv, float scale,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* dq, float* dk, float* dv) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPW = 64 / LPR;    // q-heads per pass
  const int lane = threadIdx.x & 63;
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (a >= A) return;
  const bool bidir = kinds ? kinds[a] == 1 : bidir_all != 0;   // 1 = BAC_BRANCH_BIDIR
  const int g = blockIdx.y;
  const int G = hq / hkv;
  const int r = lane / LPR, col = 8 * (lane % LPR);
  const float scale_log2 = scale * kLog2e;
  const int t0 = max(0, min(bcu[a], nb));
  const int t1 = max(t0, min(bcu[a + 1], nb));
  const int len = min(min(t1 - t0, max_len), MAXL);   // tokens past the bound are left untouched
  float dka[MAXL][8], dva[MAXL][8];
#pragma unroll
  for (int u = 0; u < MAXL; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dka[u][e] = 0.f;
      dva[u][e] = 0.f;
    }
  for (int c0 = 0; c0 < G; c0 += RPW) {
    const bool row_ok = c0 + r < G;
    const int h = g * G + (row_ok ? c0 + r : 0);
    const float keep_row = row_ok ? 1.f : 0.f;
#pragma unroll
    for (int t = 0; t < MAXL; ++t) {
      if (t >= len) break;
      const int kend = bidir ? len : t + 1;
      const size_t qoff = (static_cast<size_t>(t0 + t) * hq + h) * D + col;
      const size_t li = static_cast<size_t>(h) * nb + t0 + t;
      float q[8], d_o[8], dqr[8];
      load8<T>(qb, qoff, q);
      load8<T>(dout, qoff, d_o);
      const float lse2 = lse[li] * kLog2e, dl = delta[li];
#pragma unroll
      for (int e = 0; e < 8; ++e) dqr[e] = 0.f;
#pragma unroll
      for (int u = 0; u < MAXL; ++u) {
        if (u >= kend) break;
        const size_t koff = (static_cast<size_t>(t0 + u) * hkv + g) * D + col;
        float kk[8], vv[8];
        load8<T>(kb, koff, kk);
        load8<T>(vb, koff, vv);
        float sc = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sc = fmaf(q[e], kk[e], sc);
          dp = fmaf(d_o[e], vv[e], dp);
        }
        sc = group_sum<LPR>(sc);
        dp = group_sum<LPR>(dp);
        const float p = (lse2 == kNegInf) ? 0.f : exp2_fast(sc * scale_log2 - lse2);
        const float ds = p * (dp - dl);
        const float dsk = ds * keep_row, pk = p * keep_row;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dqr[e] = fmaf(ds, kk[e], dqr[e]);
          dka[u][e] = fmaf(dsk, q[e], dka[u][e]);
          dva[u][e] = fmaf(pk, d_o[e], dva[u][e]);
        }
      }
      if (!row_ok) continue;
      float cur[8];
      load8<float>(dq, qoff, cur);
#pragma unroll
      for (int e = 0; e < 8; ++e) cur[e] = fmaf(scale, dqr[e], cur[e]);
      store8<float>(dq, qoff, cur);
    }
  }
  // dK/dV: sum over the row groups (lanes that differ by multiples of LPR)
#pragma unroll
  for (int u = 0; u < MAXL; ++u) {
    if (u >= len) break;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dka[u][e] += __shfl_xor(dka[u][e], off);
        dva[u][e] += __shfl_xor(dva[u][e], off);
      }
    if (r != 0) continue;
    const size_t koff = (static_cast<size_t>(t0 + u) * hkv + g) * D + col;
    float ck[8], cv[8];
    load8<float>(dk, koff, ck);
    load8<float>(dv, koff, cv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ck[e] = fmaf(scale, dka[u][e], ck[e]);
      cv[e] += dva[u][e];
    }
    store8<float>(dk, koff, ck);
    store8<float>(dv, koff, cv);
  }
}

template <typename T, int D>
static void branch_fwd_d(const BranchArgs& a) {
  const dim3 grid((a.num_branches + 3) / 4, a.hkv);
  // branches of at most 4 tokens one token per step (more registers would
  // cost occupancy for little reuse), longer ones four (measured on 16-token
  // DFlash blocks: 4 beat 2 and 8)
  auto kern = a.max_len <= 4 ? branch_fwd_kernel<T, D, 1> : branch_fwd_kernel<T, D, 4>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, a.stream,
                     static_cast<const T*>(a.qb), static_cast<const T*>(a.kb),
                     static_cast<const T*>(a.vb), a.nb, a.branch_cu, a.num_branches, a.max_len,
                     a.bidir, a.kinds, a.hq, a.hkv, a.scale * kLog2e, a.o_acc, a.lse_acc, a.mode,
                     static_cast<T*>(a.o_out));
}

hipError_t launch_branch_fwd(const BranchArgs& a) {
  if (a.num_branches == 0) return hipSuccess;
  if (a.dt == kF32) {
    if (a.d == 128) branch_fwd_d<float, 128>(a); else branch_fwd_d<float, 64>(a);
  } else {
    if (a.d == 128) branch_fwd_d<uint16_t, 128>(a); else branch_fwd_d<uint16_t, 64>(a);
  }
  return hipGetLastError();
}

template <typename T, int D>
static void branch_bwd_d(const BranchArgs& a) {
  const dim3 grid((a.num_branches + 3) / 4, a.hkv);
  if (a.max_len <= 4) {
    // every key's dK/dV in registers: one pass.  (For 8-token branches the
    // registers this takes cut occupancy below what the second pass costs.)
    hipLaunchKernelGGL((branch_bwd_short_kernel<T, D, 4>), grid, dim3(256), 0, a.stream,
                       static_cast<const T*>(a.qb), static_cast<const T*>(a.kb),
                       static_cast<const T*>(a.vb), a.nb, a.branch_cu, a.num_branches, a.max_len,
                       a.bidir, a.kinds, a.hq, a.hkv, a.scale, static_cast<const T*>(a.dout), a.lse,
                       a.delta, a.dq, a.dk, a.dv);
    return;
  }
  // two tokens per step in the dQ pass and two keys per step in the dK/dV
  // pass (measured on 8- and 16-token blocks: 4 keys cost more occupancy
  // than they save)
  hipLaunchKernelGGL((branch_bwd_kernel<T, D, 2, 2>), grid, dim3(256), 0, a.stream,
                     static_cast<const T*>(a.qb), static_cast<const T*>(a.kb),
                     static_cast<const T*>(a.vb), a.nb, a.branch_cu, a.num_branches, a.max_len,
                     a.bidir, a.kinds, a.hq, a.hkv, a.scale, static_cast<const T*>(a.dout), a.lse,
                     a.delta,
                     a.dq, a.dk, a.dv);
}

hipError_t launch_branch_bwd(const BranchArgs& a) {
  if (a.num_branches == 0) return hipSuccess;
  if (a.dt == kF32) {
    if (a.d == 128) branch_bwd_d<float, 128>(a); else branch_bwd_d<float, 64>(a);
  } else {
    if (a.d == 128) branch_bwd_d<uint16_t, 128>(a); else branch_bwd_d<uint16_t, 64>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Main attention on vector ALUs: one wave per (query row, q-head).  Keys of
// the row's sequence with pos <= the row's pos form one contiguous range of
// the (seq, pos)-sorted shard, found by binary search.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void main_fwd_valu_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    int nq, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ k_seq,
    const int32_t* __restrict__ k_pos, int nk, int hq, int hkv, float scale_log2, float* o_acc,
    float* lse_acc, int mode, T* o_out) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= static_cast<int64_t>(nq) * hq) return;
  const int i = static_cast<int>(w / hq);
  const int h = static_cast<int>(w % hq);
  const int g = h / (hq / hkv);
  const int s = q_seq[i], p = q_pos[i];
  const int lo = lower_bound_sp(k_seq, k_pos, nk, s, INT_MIN);
  const int hi = upper_bound_sp(k_seq, k_pos, nk, s, p);
  const size_t qoff = (static_cast<size_t>(i) * hq + h) * D;
  float qq[EPL], o[EPL];
  load_lane<T, EPL>(q, qoff, lane, qq);
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  float m2 = kNegInf, l = 0.f;
  for (int j = lo; j < hi; ++j) {
    if (k_seq[j] != s || k_pos[j] > p) continue;
    const size_t koff = (static_cast<size_t>(j) * hkv + g) * D;
    float kk[EPL], vv[EPL];
    load_lane<T, EPL>(k, koff, lane, kk);
    load_lane<T, EPL>(v, koff, lane, vv);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dot += qq[e] * kk[e];
    dot = wave_sum(dot);
    online_update<EPL>(dot * scale_log2, vv, m2, l, o);
  }
  finish_row<T, EPL>(o, m2, l, qoff, static_cast<size_t>(h) * nq + i, mode, o_acc, lse_acc, o_out,
                     lane);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void main_bwd_dq_valu_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    int nq, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ k_seq,
    const int32_t* __restrict__ k_pos, int nk, int hq, int hkv, float scale,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* dq) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= static_cast<int64_t>(nq) * hq) return;
  const int i = static_cast<int>(w / hq);
  const int h = static_cast<int>(w % hq);
  const int g = h / (hq / hkv);
  const int s = q_seq[i], p = q_pos[i];
  const int lo = lower_bound_sp(k_seq, k_pos, nk, s, INT_MIN);
  const int hi = upper_bound_sp(k_seq, k_pos, nk, s, p);
  const size_t qoff = (static_cast<size_t>(i) * hq + h) * D;
  const size_t li = static_cast<size_t>(h) * nq + i;
  const float lse2 = lse[li] * kLog2e;
  const float dl = delta[li];
  const float scale_log2 = scale * kLog2e;
  float qq[EPL], d_o[EPL], acc[EPL], accc[EPL];
  load_lane<T, EPL>(q, qoff, lane, qq);
  load_lane<T, EPL>(dout, qoff, lane, d_o);
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = accc[e] = 0.f;
  if (lse2 != kNegInf) {
    for (int j = lo; j < hi; ++j) {
      if (k_seq[j] != s || k_pos[j] > p) continue;
      const size_t koff = (static_cast<size_t>(j) * hkv + g) * D;
      float kk[EPL], vv[EPL];
      load_lane<T, EPL>(k, koff, lane, kk);
      load_lane<T, EPL>(v, koff, lane, vv);
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        sc += qq[e] * kk[e];
        dp += d_o[e] * vv[e];
      }
      sc = wave_sum(sc);
      dp = wave_sum(dp);
      const float pr = exp2_fast(sc * scale_log2 - lse2);
      const float ds = pr * (dp - dl);
#pragma unroll
      for (int e = 0; e < EPL; ++e) kahan_add(acc[e], accc[e], ds * kk[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) dq[qoff + lane * EPL + e] += scale * (acc[e] - accc[e]);
}

// One wave per (key, kv-head): rows of the key's sequence with pos >= the
// key's pos form one contiguous range of the sorted query rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void main_bwd_dkdv_valu_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos,
    int nq, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ k_seq,
    const int32_t* __restrict__ k_pos, int nk, int hq, int hkv, float scale,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* dk, float* dv) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= static_cast<int64_t>(nk) * hkv) return;
  const int j = static_cast<int>(w / hkv);
  const int g = static_cast<int>(w % hkv);
  const int G = hq / hkv;
  const int s = k_seq[j], p = k_pos[j];
  const int lo = lower_bound_sp(q_seq, q_pos, nq, s, p);
  const int hi = upper_bound_sp(q_seq, q_pos, nq, s, INT_MAX);
  const size_t koff = (static_cast<size_t>(j) * hkv + g) * D;
  const float scale_log2 = scale * kLog2e;
  float kk[EPL], vv[EPL], dka[EPL], dva[EPL], dkc[EPL], dvc[EPL];
  load_lane<T, EPL>(k, koff, lane, kk);
  load_lane<T, EPL>(v, koff, lane, vv);
#pragma unroll
  for (int e = 0; e < EPL; ++e) dka[e] = dva[e] = dkc[e] = dvc[e] = 0.f;
  for (int i = lo; i < hi; ++i) {
    if (q_seq[i] != s || q_pos[i] < p) continue;
    for (int hl = 0; hl < G; ++hl) {
      const int h = g * G + hl;
      const size_t qoff = (static_cast<size_t>(i) * hq + h) * D;
      const size_t li = static_cast<size_t>(h) * nq + i;
      const float lse2 = lse[li] * kLog2e;
      if (lse2 == kNegInf) continue;
      float qq[EPL], d_o[EPL];
      load_lane<T, EPL>(q, qoff, lane, qq);
      load_lane<T, EPL>(dout, qoff, lane, d_o);
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        sc += qq[e] * kk[e];
        dp += d_o[e] * vv[e];
      }
      sc = wave_sum(sc);
      dp = wave_sum(dp);
      const float pr = exp2_fast(sc * scale_log2 - lse2);
      const float ds = pr * (dp - delta[li]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kahan_add(dka[e], dkc[e], ds * qq[e]);
        kahan_add(dva[e], dvc[e], pr * d_o[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    dk[koff + lane * EPL + e] += scale * (dka[e] - dkc[e]);
    dv[koff + lane * EPL + e] += dva[e] - dvc[e];
  }
}

template <typename T, int D>
static void main_fwd_valu_d(const MainArgs& a) {
  const int64_t waves = static_cast<int64_t>(a.nq) * a.hq;
  hipLaunchKernelGGL((main_fwd_valu_kernel<T, D>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                     dim3(256), 0, a.stream, static_cast<const T*>(a.q), a.q_seq, a.q_pos, a.nq,
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.k_seq, a.k_pos, a.nk,
                     a.hq, a.hkv, a.scale * kLog2e, a.o_acc, a.lse_acc, a.mode,
                     static_cast<T*>(a.o_out));
}

hipError_t launch_main_fwd_valu(const MainArgs& a) {
  if (a.nq == 0) return hipSuccess;
  if (a.dt == kF32) {
    if (a.d == 128) main_fwd_valu_d<float, 128>(a); else main_fwd_valu_d<float, 64>(a);
  } else {
    if (a.d == 128) main_fwd_valu_d<uint16_t, 128>(a); else main_fwd_valu_d<uint16_t, 64>(a);
  }
  return hipGetLastError();
}

template <typename T, int D>
static void main_bwd_valu_d(const MainArgs& a, int part) {
  const int64_t qw = static_cast<int64_t>(a.nq) * a.hq;
  if (qw > 0 && part != 2)
    hipLaunchKernelGGL((main_bwd_dq_valu_kernel<T, D>), dim3(static_cast<unsigned>((qw + 3) / 4)),
                       dim3(256), 0, a.stream, static_cast<const T*>(a.q), a.q_seq, a.q_pos, a.nq,
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.k_seq, a.k_pos,
                       a.nk, a.hq, a.hkv, a.scale, static_cast<const T*>(a.dout), a.lse, a.delta,
                       a.dq);
  const int64_t kw = static_cast<int64_t>(a.nk) * a.hkv;
  if (kw > 0 && part != 1)
    hipLaunchKernelGGL((main_bwd_dkdv_valu_kernel<T, D>),
                       dim3(static_cast<unsigned>((kw + 3) / 4)), dim3(256), 0, a.stream,
                       static_cast<const T*>(a.q), a.q_seq, a.q_pos, a.nq,
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.k_seq, a.k_pos,
                       a.nk, a.hq, a.hkv, a.scale, static_cast<const T*>(a.dout), a.lse, a.delta,
                       a.dk, a.dv);
}

hipError_t launch_main_bwd_valu(const MainArgs& a, int part) {
  if (a.nq == 0 || a.nk == 0) return hipSuccess;
  if (a.dt == kF32) {
    if (a.d == 128) main_bwd_valu_d<float, 128>(a, part); else main_bwd_valu_d<float, 64>(a, part);
  } else {
    if (a.d == 128) main_bwd_valu_d<uint16_t, 128>(a, part);
    else main_bwd_valu_d<uint16_t, 64>(a, part);
  }
  return hipGetLastError();
}

}  // namespace bac
