// attn_main_fwd, bf16 on MFMA (gfx950).
//
// One ring step of the main part ([G] 方法详解 · CP计算): query rows (main
// tokens at their own position, branch tokens at their anchor's position)
// against one main K/V shard, with the causal rule k_seq == q_seq and
// k_pos <= q_pos, followed by the online-softmax merge into the accumulators
// ([G] 技术贡献).
//
// Work decomposition
//   * A workgroup has 8 waves and owns TPB = 8 * 32/G consecutive query tokens
//     of one kv-head group: 256 (token, q-head) rows that all read the same
//     K/V tiles.  Wave w owns 32 rows: tokens tok0 + w*32/G + n/G, heads
//     g*G + n%G for n = 0..31 (the GQA heads of a token are adjacent rows).
//   * Keys stream through LDS in row-major tiles of 64, double buffered, one
//     barrier per tile.  The key range of a workgroup is [first key of its
//     first row's sequence, last key visible to its last row], found by binary
//     search on the (seq, pos)-sorted shard.
//   * Scores are computed transposed, S^T = K Q^T (keys x rows), so each lane
//     holds 32 scores of ONE query row: the row max is in-lane plus one
//     exchange with lane n+32, and the row sums stay per lane until the end.
//   * O^T += V^T P^T: P^T comes straight from the score registers (bf16),
//     V^T from transposing LDS reads of the row-major V tile.
//   * Lazy rescale: the running max only moves when a tile's max exceeds it by
//     more than 8 (log2 units), so P stays below 2^8 and most tiles skip the
//     rescale of O.  Normalisation by the row sum makes this exact.
//   * Tiles wholly visible to a wave skip the mask; tiles wholly beyond a
//     wave's rows skip the compute.
//   * Blocks are ordered heavy-first (later tokens see more keys) and remapped
//     so that each XCD works on one kv-head's K/V.

#include <climits>

#include "launch.hpp"
#include "mfma_common.hpp"

namespace bac {

namespace fwd {
constexpr int BN = 64;          // keys per tile
constexpr int NW = 8;           // waves per workgroup
constexpr float kRescale = 8.f; // lazy-rescale threshold (log2 units)
}  // namespace fwd

template <int D, int G>
__global__ __launch_bounds__(512, 1) void main_fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int nq, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ k_seq,
    const int32_t* __restrict__ k_pos, int nk, int hq, int hkv, float scale_log2,
    float* __restrict__ o_acc, float* __restrict__ lse_acc, int mode, uint16_t* __restrict__ o_out) {
  using namespace fwd;
  constexpr int TPW = 32 / G;           // tokens per wave
  constexpr int TPB = NW * TPW;         // tokens per workgroup
  constexpr int KS = D / 16;            // k-steps of QK^T
  constexpr int MB = D / 32;            // 32-row blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int LOADS = BN * CPR / 512; // 16-byte chunks per thread per tile

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * D];
  __shared__ __attribute__((aligned(16))) int kseq_s[2][BN];
  __shared__ __attribute__((aligned(16))) int kpos_s[2][BN];

  const int nblk_tok = (nq + TPB - 1) / TPB;
  const int L = xcd_remap(blockIdx.x, nblk_tok * hkv);
  const int g = L / nblk_tok;
  const int tb = nblk_tok - 1 - (L % nblk_tok);   // heavy (late) token blocks first
  const int tok0 = tb * TPB;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hi = lane >> 5;
  const LaneOffsets<D> lo_off(lane);

  // ---- this lane's query row -------------------------------------------
  const int wtok0 = tok0 + wave * TPW;
  const int my_tok = wtok0 + n / G;
  const int my_head = g * G + n % G;
  const bool row_valid = my_tok < nq;
  const int my_seq = row_valid ? q_seq[my_tok] : 0;
  const int my_pos = row_valid ? q_pos[my_tok] : 0;

  // wave-level row summary (rows are sorted by (seq, pos))
  const int wlast = min(nq, wtok0 + TPW) - 1;
  const bool wave_valid = wtok0 < nq;
  const bool wave_complete = wtok0 + TPW <= nq;
  const int wf_seq = wave_valid ? q_seq[wtok0] : 0, wf_pos = wave_valid ? q_pos[wtok0] : 0;
  const int wl_seq = wave_valid ? q_seq[wlast] : 0, wl_pos = wave_valid ? q_pos[wlast] : 0;

  // ---- key range of the workgroup ----------------------------------------
  const int blast = min(nq, tok0 + TPB) - 1;
  const int lo = lower_bound_sp(k_seq, k_pos, nk, q_seq[tok0], INT_MIN);
  const int hi_k = upper_bound_sp(k_seq, k_pos, nk, q_seq[blast], q_pos[blast]);
  const int ntiles = hi_k > lo ? (hi_k - lo + BN - 1) / BN : 0;

  // ---- Q operands (B of S^T = K Q^T): row n, d = 16*ks + 8*hi + 0..7 -------
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = q + (static_cast<size_t>(my_tok) * hq + my_head) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = row_valid ? *reinterpret_cast<const bf16x8*>(qp + 16 * ks) : zero8();
  }

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = zero16();
  float m_run = kNegInf;   // reference max (log2 units), same in lanes n and n+32
  float l_run = 0.f;       // this lane's part of the running sum

  // ---- tile staging: global -> registers -> LDS ---------------------------
  uint4 kreg[LOADS], vreg[LOADS];
  int sreg = 0, preg = 0;
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int c = tid + 512 * it;
      const int key = c / CPR, col = (c % CPR) * 8;
      const int j = j0 + key;
      if (j < nk) {
        const size_t off = (static_cast<size_t>(j) * hkv + g) * D + col;
        kreg[it] = *reinterpret_cast<const uint4*>(k + off);
        vreg[it] = *reinterpret_cast<const uint4*>(v + off);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        vreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BN) {
      const int j = j0 + tid;
      const bool ok = j < hi_k;
      sreg = ok ? k_seq[j] : INT_MIN;
      preg = ok ? k_pos[j] : INT_MAX;
    }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int c = tid + 512 * it;
      const int key = c / CPR, col = (c % CPR) * 8;
      *reinterpret_cast<uint4*>(&Ks[b][toff<D>(key, col)]) = kreg[it];
      *reinterpret_cast<uint4*>(&Vs[b][toff<D>(key, col)]) = vreg[it];
    }
    if (tid < BN) {
      kseq_s[b][tid] = sreg;
      kpos_s[b][tid] = preg;
    }
  };

  if (ntiles > 0) {
    load_tile(lo);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    const int j0 = lo + t * BN;
    if (t + 1 < ntiles) load_tile(j0 + BN);

    // classify the tile for this wave
    const int jl = min(hi_k, j0 + BN) - 1 - j0;      // last in-range key of the tile
    const int kf_seq = kseq_s[b][0], kf_pos = kpos_s[b][0];
    const int kl_seq = kseq_s[b][jl], kl_pos = kpos_s[b][jl];
    const bool wave_any = wave_valid && !lex_less(wl_seq, wl_pos, kf_seq, kf_pos) &&
                          !lex_less(kl_seq, kl_pos, wf_seq, INT_MIN);
    const bool wave_full = wave_complete && jl == BN - 1 && kf_seq == kl_seq &&
                           kf_seq == wf_seq && wf_seq == wl_seq && kl_pos <= wf_pos;

    if (wave_any) {
      // S^T = K Q^T over two 32-key blocks: lane (n, hi) register r of block kb
      // holds key kb*32 + acc_row(r, hi) of query row n.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sacc[kb] = mfma32(row_operand<D>(Ks[b], lo_off, kb * 32, ks), qreg[ks], sacc[kb]);
      }
      // raw scores; masked entries become -inf (scale > 0 keeps the max in place)
      float x[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[kb][r] = sacc[kb][r];
      if (!wave_full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int t0 = kb * 32 + 8 * r4 + 4 * hi;
            const int4 ss = *reinterpret_cast<const int4*>(&kseq_s[b][t0]);
            const int4 pp = *reinterpret_cast<const int4*>(&kpos_s[b][t0]);
            const int sv[4] = {ss.x, ss.y, ss.z, ss.w};
            const int pv[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool vis = row_valid & (sv[e] == my_seq) & (pv[e] <= my_pos);
              x[kb][4 * r4 + e] = vis ? x[kb][4 * r4 + e] : kNegInf;
            }
          }
      }
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(x[kb][r], x[kb][r + 1]));
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
      // lazy rescale: move the reference only when the tile max clears it by kRescale
      if (__any(mt > m_run + kRescale)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == kNegInf) ? 0.f : exp2_fast(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x[kb][r] = exp2_fast(fmaf(x[kb][r], scale_log2, -m_use));
          l_run += x[kb][r];
        }
      // O^T += V^T P^T, four k-steps of 16 keys
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8 pb = pack8(&x[kb][8 * s2]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            oacc[mb] = mfma32(tr_operand<D>(Vs[b], lo_off, kb * 32 + 16 * s2, mb), pb, oacc[mb]);
        }
    }

    if (t + 1 < ntiles) store_tile(b ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, merge, store ---------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_valid) return;
  const float lse2 = l_tot > 0.f ? m_run + log2_fast(l_tot) : kNegInf;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const size_t li = static_cast<size_t>(my_head) * nq + my_tok;
  float wa = 0.f, wb = 1.f, lnew = lse2;
  if (mode == 1) merge_weights_log2(lse_acc[li] * kLog2e, lse2, wa, wb, lnew);
  const size_t obase = (static_cast<size_t>(my_tok) * hq + my_head) * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const size_t off = obase + mb * 32 + 8 * gq + 4 * hi;
      float4 r;
      r.x = oacc[mb][4 * gq + 0] * inv;
      r.y = oacc[mb][4 * gq + 1] * inv;
      r.z = oacc[mb][4 * gq + 2] * inv;
      r.w = oacc[mb][4 * gq + 3] * inv;
      if (mode == 1) {
        const float4 a = *reinterpret_cast<const float4*>(o_acc + off);
        r.x = wa * a.x + wb * r.x;
        r.y = wa * a.y + wb * r.y;
        r.z = wa * a.z + wb * r.z;
        r.w = wa * a.w + wb * r.w;
      }
      *reinterpret_cast<float4*>(o_acc + off) = r;
      if (o_out) {
        uint2 pk;
        pk.x = pack_bf16x2(r.x, r.y);
        pk.y = pack_bf16x2(r.z, r.w);
        *reinterpret_cast<uint2*>(o_out + off) = pk;
      }
    }
  if (hi == 0) lse_acc[li] = (lnew == kNegInf) ? kNegInf : lnew * kLn2;
}

template <int D, int G>
static void main_fwd_mfma_dg(const MainArgs& a) {
  constexpr int TPB = fwd::NW * (32 / G);
  const int nblk_tok = (a.nq + TPB - 1) / TPB;
  const int nb = nblk_tok * a.hkv;
  hipLaunchKernelGGL((main_fwd_mfma_kernel<D, G>), dim3(nb), dim3(512), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), a.q_seq, a.q_pos, a.nq,
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.k_seq,
                     a.k_pos, a.nk, a.hq, a.hkv, a.scale * kLog2e, a.o_acc, a.lse_acc, a.mode,
                     static_cast<uint16_t*>(a.o_out));
}

template <int D>
static void main_fwd_mfma_d(const MainArgs& a) {
  switch (a.hq / a.hkv) {
    case 1: main_fwd_mfma_dg<D, 1>(a); break;
    case 2: main_fwd_mfma_dg<D, 2>(a); break;
    case 4: main_fwd_mfma_dg<D, 4>(a); break;
    case 8: main_fwd_mfma_dg<D, 8>(a); break;
    case 16: main_fwd_mfma_dg<D, 16>(a); break;
    default: main_fwd_mfma_dg<D, 32>(a); break;
  }
}

hipError_t launch_main_fwd_mfma(const MainArgs& a) {
  if (a.nq == 0) return hipSuccess;
  if (a.d == 128) main_fwd_mfma_d<128>(a); else main_fwd_mfma_d<64>(a);
  return hipGetLastError();
}

}  // namespace bac
