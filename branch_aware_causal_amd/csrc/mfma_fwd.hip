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
//   * Keys stream through LDS in row-major tiles of 128, double buffered,
//     copied straight from global memory into LDS (no register staging).  The
//     key range of a workgroup is [first key of its first row's sequence, last
//     key visible to its last row], found by binary search on the (seq,
//     pos)-sorted shard.  Within it the keys a row sees form one index
//     interval, also found by binary search, so masks are index compares.
//   * Ping-pong: waves w and w+4 share a SIMD; in each tile period one runs
//     its MFMA stream and then its softmax, the other its softmax and then
//     its MFMA stream, so that while one issues the tile's MFMAs the other
//     runs its softmax on the vector ALUs.  One barrier per tile period.  The
//     MFMA stream runs at raised wave priority, so the partner's vector work
//     yields to it.
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
constexpr int BN = 128;         // keys per tile
constexpr int NKB = BN / 32;    // 32-key blocks per tile
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

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * D];

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

  // ---- tile loads: direct global -> LDS, issued by team 0 --------------
  // Lane l of round `it` of team-0 wave w fills 16-byte slot (it*4 + w)*64 + l
  // of a K (V) tile, i.e. physical chunk p of key row r; it fetches logical
  // chunk swz(r, p) (the swizzle is an involution).  Keys past the end re-read
  // the last key; they and keys past hi_k are masked by index.  Addresses are
  // a wave-uniform base plus a per-lane 32-bit byte offset from the tile's
  // first key.
  constexpr int ROUNDS = BN * CPR / 256;
  uint32_t lane_row[ROUNDS], lane_col[ROUNDS];
#pragma unroll
  for (int it = 0; it < ROUNDS; ++it) {
    const int slot = (it * 4 + (wave & 3)) * 64 + lane;
    const int r = slot / CPR, pc = slot % CPR;
    lane_row[it] = r;
    lane_col[it] = 2u * (g * D + 8 * swz<D>(r, pc));
  }
  const uint32_t krow_bytes = static_cast<uint32_t>(hkv * D * 2);
  // round `it` of the load of the tile at j0 from src into the LDS tile dst
  auto issue_round = [&](const uint16_t* src, const uint16_t* dst_tile, int j0, int it) {
    const char* base = reinterpret_cast<const char*>(src) + static_cast<size_t>(j0) * krow_bytes;
    const int rmax = nk - 1 - j0;     // last valid key row of the tile
    const uint32_t off =
        static_cast<uint32_t>(min(static_cast<int>(lane_row[it]), rmax)) * krow_bytes + lane_col[it];
    dma_b128(base, off, lds_addr(dst_tile) + (it * 4 + (wave & 3)) * 64 * 16);
  };
  auto issue_rows = [&](const uint16_t* src, const uint16_t* dst_tile, int j0) {
#pragma unroll
    for (int it = 0; it < ROUNDS; ++it) issue_round(src, dst_tile, j0, it);
  };

  // ---- visible keys of each row ------------------------------------------
  // The shard is sorted by (seq, pos), so the keys a row sees (same sequence,
  // pos <= its pos) are one index interval [r_lo, r_hi) of [lo, hi_k).  Rows
  // past nq see nothing.  A wave classifies a tile from the extremes of its
  // rows' intervals: some row may see it, or every row sees all of it.
  int r_lo = 0, r_hi = 0;
  if (row_valid) {
    r_lo = lo + lower_bound_sp(k_seq + lo, k_pos + lo, hi_k - lo, my_seq, INT_MIN);
    r_hi = lo + upper_bound_sp(k_seq + lo, k_pos + lo, hi_k - lo, my_seq, my_pos);
  }
  int lo_min = row_valid ? r_lo : INT_MAX, hi_max = row_valid ? r_hi : INT_MIN;
  int lo_max = row_valid ? r_lo : INT_MIN, hi_min = row_valid ? r_hi : INT_MAX;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo_min = min(lo_min, __shfl_xor(lo_min, o));
    hi_max = max(hi_max, __shfl_xor(hi_max, o));
    lo_max = max(lo_max, __shfl_xor(lo_max, o));
    hi_min = min(hi_min, __shfl_xor(hi_min, o));
  }
  lo_min = __builtin_amdgcn_readfirstlane(lo_min);
  hi_max = __builtin_amdgcn_readfirstlane(hi_max);
  lo_max = __builtin_amdgcn_readfirstlane(lo_max);
  hi_min = __builtin_amdgcn_readfirstlane(hi_min);
  auto tile_any = [&](int j0) { return lo_min < min(j0 + BN, hi_k) && hi_max > j0; };
  auto tile_full = [&](int j0) { return wave_complete && lo_max <= j0 && j0 + BN <= hi_min; };

  // ---- ping-pong schedule ------------------------------------------------
  // Waves w and w+4 share a SIMD.  Team 0 (waves 0-3) and team 1 (waves 4-7)
  // run one tile period between workgroup barriers, in opposite orders, so
  // that on every SIMD one wave feeds the matrix core while the other runs
  // the softmax:
  //   period t: team 0  MFMA(t) = PV(t-1), S(t), then softmax(t)
  //             team 1  softmax(t-1), then MFMA(t)
  // K(t) and V(t-1) are read in period t.  Team 0 issues K(t+1) and V(t)
  // during its MFMA stream of period t and waits for them at the barrier that
  // ends it, so both are double buffered.  (A barrier between the MFMA and
  // softmax halves of a period cost 2.3% more time at 256K.)
  const int team = wave >> 2;
  if (team == 0 && ntiles > 0) issue_rows(k, &Ks[0][0], lo);
  wg_barrier<kWaitAll>();

  f32x16 sacc[NKB];
  bf16x8 pb[2 * NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    sacc[kb] = zero16();
    pb[2 * kb] = zero8();
    pb[2 * kb + 1] = zero8();
  }

  // One MFMA stream of a period: O^T += V^T P^T for tile t-1
  // (2*NKB*MB MFMAs, transposed V operands), then S^T = K Q^T for tile t
  // (NKB*KS MFMAs, the NKB 32-key blocks interleaved).  LDS operands are read
  // kPre MFMAs ahead.  (Tiles of 128 keys rather than 64 halve the barriers
  // per key: 3.6% less forward time at 256K.)
  constexpr int kPre = 4;
  // With loads (team 0), the rounds of K(kj0) -> kdst and V(vj0) -> vdst are
  // spread over the stream, one every N / (2*ROUNDS) MFMAs, so that no burst
  // of them stalls the wave.
  auto mfma_stream = [&](auto pv_c, auto s_c, auto dma_c, const uint16_t* vt, const uint16_t* kt,
                         const uint16_t* kdst, int kj0, const uint16_t* vdst, int vj0) {
    constexpr bool kPV = decltype(pv_c)::value, kS = decltype(s_c)::value;
    constexpr bool kDMA = decltype(dma_c)::value;
    constexpr int NP = kPV ? 2 * NKB * MB : 0, N = NP + (kS ? NKB * KS : 0);
    __builtin_amdgcn_s_setprio(1);
    constexpr int kGap = N / (2 * ROUNDS);
    static_assert(!kDMA || kGap >= 1, "load rounds fit in the stream");
    auto load = [&](int j) {
      if (j < NP) {
        const int kb = j / (2 * MB), s2 = (j / MB) % 2, mb = j % MB;
        return tr_operand<D>(vt, lo_off, kb * 32 + 16 * s2, mb);
      }
      const int kb = (j - NP) % NKB, ks = (j - NP) / NKB;
      return row_operand<D>(kt, lo_off, kb * 32, ks);
    };
    bf16x8 opnd[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) opnd[j] = load(j);
    if (kS) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = zero16();
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (j < NP) {
        const int kb = j / (2 * MB), s2 = (j / MB) % 2, mb = j % MB;
        oacc[mb] = mfma32(opnd[j % kPre], pb[2 * kb + s2], oacc[mb]);
      } else {
        const int kb = (j - NP) % NKB, ks = (j - NP) / NKB;
        sacc[kb] = mfma32(opnd[j % kPre], qreg[ks], sacc[kb]);
      }
      if (j + kPre < N) opnd[j % kPre] = load(j + kPre);
      if (kDMA && j % kGap == 0 && j / kGap < 2 * ROUNDS) {
        const int r = j / kGap;
        if (r & 1)
          issue_round(v, vdst, vj0, r / 2);
        else
          issue_round(k, kdst, kj0, r / 2);
      }
    }
    // pin the order: kPre operands, then one MFMA and the next operand
    // (a transposed operand is two LDS reads, a row operand one)
    static_assert(NP == 0 || NP >= kPre, "prefetch covers one operand kind");
    if constexpr (NP > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);
    else
      __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j + kPre < NP)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (j + kPre < N)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // the stream stays before the softmax of the period
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) keep(oacc[mb]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) keep(sacc[kb]);
    __builtin_amdgcn_s_setprio(0);
  };

  // softmax of the tile at j0: scores -> P (bf16) in pb; a tile this wave
  // skips leaves zeros, so the next MFMA stream may run its PV
  // regardless
  auto softmax = [&](int j0, bool do_s) {
    if (!do_s) {
#pragma unroll
      for (int i = 0; i < 2 * NKB; ++i) pb[i] = zero8();
      return;
    }
    // masked entries become -inf (scale > 0 keeps the max in place); the
    // softmax works in place on the score registers
    if (!tile_full(j0)) {
      const int a = r_lo - j0 - 4 * hi, e_end = r_hi - j0 - 4 * hi;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r / 4) + (r % 4);
          sacc[kb][r] = (c >= a && c < e_end) ? sacc[kb][r] : kNegInf;
        }
    }
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) mt = max16_raw(mt, sacc[kb]);
    mt = max_xor32(mt) * scale_log2;
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
    for (int kb = 0; kb < NKB; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2_fast(fmaf(sacc[kb][r], scale_log2, -m_use));
        l_run += p[r];
      }
      pb[2 * kb] = pack8(&p[0]);
      pb[2 * kb + 1] = pack8(&p[8]);
    }
#pragma unroll
    for (int i = 0; i < 2 * NKB; ++i) keep(pb[i]);
    keep(l_run);
  };

  // One barrier per period t: team 0 runs MFMA(t) then softmax(t), team 1
  // softmax(t-1) then MFMA(t), so on every SIMD one wave's MFMA stream meets
  // the other's softmax without a barrier between them.  Team 0 loads K(t+1)
  // and V(t) during period t and waits for them at the barrier that ends it;
  // past the last tile K repeats the last tile into the buffer of K(t-1),
  // which no later period reads.
  bool any_prev = false;   // the previous tile was visible to the wave
  // (the first and last periods are peeled: inside the loop the register
  // allocator then keeps each team's live set to what its order needs)
  if (ntiles > 0) {
    // period 0: S(0)
    const bool do_s = tile_any(lo);
    if (team == 0) {
      if (ntiles > 1) issue_rows(k, &Ks[1][0], lo + BN);
      issue_rows(v, &Vs[0][0], lo);
    }
    if (do_s)
      mfma_stream(BoolC<false>(), BoolC<true>(), BoolC<false>(), &Vs[1][0], &Ks[0][0], nullptr, 0, nullptr,
                  0);
    if (team == 0) softmax(lo, do_s);
    any_prev = do_s;
    wg_barrier<kWaitAll>();
  }
  for (int t = 1; t < ntiles; ++t) {
    const int j0 = lo + t * BN;
    const int kj0 = min(j0 + BN, lo + (ntiles - 1) * BN);
    const uint16_t* kdst = &Ks[(t + 1) & 1][0];
    const uint16_t* vdst = &Vs[t & 1][0];
    const bool do_s = tile_any(j0);
    const uint16_t* vt = &Vs[(t - 1) & 1][0];
    const uint16_t* kt = &Ks[t & 1][0];
    if (team == 0) {
      if (any_prev || do_s) {
        mfma_stream(BoolC<true>(), BoolC<true>(), BoolC<true>(), vt, kt, kdst, kj0, vdst, j0);
      } else {
        issue_rows(k, kdst, kj0);
        issue_rows(v, vdst, j0);
      }
      softmax(j0, do_s);
    } else {
      softmax(j0 - BN, any_prev);
      if (any_prev || do_s)
        mfma_stream(BoolC<true>(), BoolC<true>(), BoolC<false>(), vt, kt, kdst, kj0, vdst, j0);
    }
    any_prev = do_s;
    wg_barrier<kWaitAll>();
  }
  // period ntiles: PV(ntiles-1) (team 1 first finishes softmax(ntiles-1))
  if (ntiles > 0) {
    if (team == 1) softmax(lo + (ntiles - 1) * BN, any_prev);
    if (any_prev)
      mfma_stream(BoolC<true>(), BoolC<false>(), BoolC<false>(), &Vs[(ntiles - 1) & 1][0], &Ks[0][0],
                  nullptr, 0, nullptr, 0);
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
