// attn_main_bwd, bf16 on MFMA (gfx950).
//
// Gradients of one ring step's main part, recomputed from the merged lse of
// each row (P = exp2(s*c - lse2)); the pages leave the backward open, so this
// is the vector-Jacobian product of the forward for upstream dO:
//   dS = P (dP - Delta),  dP = dO V^T,
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO  (dK/dV summed over the
//   q-heads of a GQA group).
//
// Two kernels, no atomics (deterministic):
//   * dq kernel, query-outer like the forward: 8 waves x 32 (token, head)
//     rows stream the visible K/V tiles; S^T = K Q^T and dP^T = V dO^T keep one
//     query row per lane, dQ^T += K^T dS^T reads a transposed K tile.
//   * dkdv kernel, key-outer: 4 waves x 32 keys hold K and V as MFMA operands
//     in registers and stream the query rows that can see them in tiles of 32
//     rows; S = Q K^T and dP = dO V^T keep one key per lane, dV^T += dO^T P and
//     dK^T += Q^T dS read transposed Q / dO tiles.
// Every workgroup owns its output rows, so the += into the fp32 accumulators
// is race-free within a launch and ordered across launches on one stream.

#include <climits>

#include "launch.hpp"
#include "mfma_common.hpp"

namespace bac {

namespace bwdq {
constexpr int BN = 64;
constexpr int NW = 8;
}  // namespace bwdq

// dq kernel layout:
//   * A workgroup has 8 waves and owns TPB = 8 * 32/G consecutive query
//     tokens of one kv-head group; wave w owns 32 (token, head) rows, one per
//     lane pair (n, n+32).  Q stays in registers, the wave's dO rows in LDS.
//   * Keys stream through LDS in tiles of 64, copied straight from global
//     memory (K in a ring of three, V in a ring of two).  The keys a row sees
//     are one index interval of the (seq, pos)-sorted shard, found by binary
//     search, so masks are index compares.
//   * Ping-pong: waves w and w+4 share a SIMD; team 0 (waves 0-3) and team 1
//     (waves 4-7) run the same half-steps one apart with a barrier between
//     half-steps:
//       half-step 2t   : team 0 MFMA(t)             team 1 GRAD(t-1)
//       half-step 2t+1 : team 0 GRAD(t)             team 1 MFMA(t)
//     MFMA(t) = dQ^T += K^T dS^T for tile t-1, then S^T = K Q^T and
//     dP^T = V dO^T for tile t, as one stream of 48 MFMAs with LDS operands
//     read ahead; GRAD(t) = dS = P (dP - Delta) on the vector ALUs.  K(t) is
//     read in half-steps 2t .. 2t+3, V(t) in 2t and 2t+1.  Team 0 loads
//     K(t+1) and V(t+1) at the start of half-step 2t and waits for them
//     before the barrier that ends half-step 2t+1.
template <int D, int G>
__global__ __launch_bounds__(512, 1) void main_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int nq, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ k_seq,
    const int32_t* __restrict__ k_pos, int nk, int hq, int hkv, float scale,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq) {
  using namespace bwdq;
  constexpr int TPW = 32 / G;
  constexpr int TPB = NW * TPW;
  constexpr int KS = D / 16;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 8;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[3][BN * D];   // keys x d, swizzled
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[NW][32 * D];  // each wave's dO rows

  const float scale_log2 = scale * kLog2e;
  const int nblk_tok = (nq + TPB - 1) / TPB;
  const int L = xcd_remap(blockIdx.x, nblk_tok * hkv);
  const int g = L / nblk_tok;
  const int tb = nblk_tok - 1 - (L % nblk_tok);
  const int tok0 = tb * TPB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int n = lane & 31, hi = lane >> 5;
  const LaneOffsets<D> lo_off(lane);

  const int wtok0 = tok0 + wave * TPW;
  const int my_tok = wtok0 + n / G;
  const int my_head = g * G + n % G;
  const bool row_valid = my_tok < nq;
  const int my_seq = row_valid ? q_seq[my_tok] : 0;
  const int my_pos = row_valid ? q_pos[my_tok] : 0;
  const size_t li = static_cast<size_t>(my_head) * nq + my_tok;
  const float my_lse2 = row_valid ? lse[li] * kLog2e : kNegInf;
  const float my_delta = row_valid ? delta[li] : 0.f;
  // a row with lse = -inf sees no key anywhere, so it is masked everywhere
  const float lse_use = my_lse2 != kNegInf ? my_lse2 : 0.f;
  const bool wave_complete = wtok0 + TPW <= nq;

  const int blast = min(nq, tok0 + TPB) - 1;
  const int lo = lower_bound_sp(k_seq, k_pos, nk, q_seq[tok0], INT_MIN);
  const int hi_k = upper_bound_sp(k_seq, k_pos, nk, q_seq[blast], q_pos[blast]);
  const int ntiles = hi_k > lo ? (hi_k - lo + BN - 1) / BN : 0;

  // Q operands stay in registers; the wave's dO rows go to LDS (read back as
  // the B operand of dP^T = V dO^T) to keep the wave within 256 registers.
  bf16x8 qreg[KS];
  uint16_t* my_do = dOs[wave];
  {
    const size_t off = (static_cast<size_t>(my_tok) * hq + my_head) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = row_valid ? *reinterpret_cast<const bf16x8*>(q + off + 16 * ks) : zero8();
      const bf16x8 dv = row_valid ? *reinterpret_cast<const bf16x8*>(dout + off + 16 * ks) : zero8();
      *reinterpret_cast<bf16x8*>(my_do + lo_off.row[ks]) = dv;
    }
  }
  f32x16 dqacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dqacc[mb] = zero16();

  // ---- tile loads: direct global -> LDS by team 0 -------------------------
  // Lane l of round `it` of team-0 wave w fills 16-byte slot (it*4 + w)*64 + l
  // of a tile, i.e. physical chunk p of key row r; it fetches logical chunk
  // swz(r, p) (the swizzle is an involution).  Keys past the end re-read the
  // last key; they and keys past hi_k are masked by index.
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
  auto issue_rows = [&](const uint16_t* src, const uint16_t* dst_tile, int j0) {
    const char* base = reinterpret_cast<const char*>(src) + static_cast<size_t>(j0) * krow_bytes;
    const int rmax = nk - 1 - j0;     // last valid key row of the tile
#pragma unroll
    for (int it = 0; it < ROUNDS; ++it) {
      const uint32_t off =
          static_cast<uint32_t>(min(static_cast<int>(lane_row[it]), rmax)) * krow_bytes + lane_col[it];
      dma_b128(base, off, lds_addr(dst_tile) + (it * 4 + (wave & 3)) * 64 * 16);
    }
  };

  // ---- visible keys of each row (see the forward kernel) -----------------
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

  const int team = wave >> 2;
  if (team == 0 && ntiles > 0) {
    issue_rows(k, &Ks[0][0], lo);
    issue_rows(v, &Vs[0][0], lo);
  }
  wg_barrier<kWaitAll>();     // also publishes the dO rows
  if (team == 1) wg_barrier<kWaitNone>();

  f32x16 sacc[2] = {zero16(), zero16()}, dpacc[2] = {zero16(), zero16()};
  bf16x8 db[4] = {zero8(), zero8(), zero8(), zero8()};

  // One MFMA half-step as a single stream: dQ^T += K^T dS^T for the previous
  // tile (4*MB MFMAs, transposed K operands), then S^T = K Q^T and
  // dP^T = V dO^T for this tile (4*KS MFMAs, alternating).  LDS operands are
  // read kPre MFMAs ahead.
  constexpr int kPre = 4;
  auto mfma_stream = [&](auto dq_c, auto s_c, const uint16_t* kprev, const uint16_t* kt,
                         const uint16_t* vt) {
    constexpr bool kDQ = decltype(dq_c)::value, kS = decltype(s_c)::value;
    constexpr int NP = kDQ ? 4 * MB : 0, N = NP + (kS ? 4 * KS : 0);
    // step j >= NP: i = j - NP; S (even i) / dP (odd i) of block kb, k-step ks
    auto load_a = [&](int j) {
      if (j < NP) {
        const int kb = j / (2 * MB), s2 = (j / MB) % 2, mb = j % MB;
        return tr_operand<D>(kprev, lo_off, kb * 32 + 16 * s2, mb);
      }
      const int i = j - NP, kb = (i / 2) % 2, ks = i / 4;
      return row_operand<D>((i & 1) ? vt : kt, lo_off, kb * 32, ks);
    };
    auto load_b = [&](int j) {   // dO operand of a dP step
      const int ks = (j - NP) / 4;
      return row_operand<D>(my_do, lo_off, 0, ks);
    };
    auto is_dp = [&](int j) { return j >= NP && ((j - NP) & 1); };
    bf16x8 opa[kPre], opb[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      opa[j] = load_a(j);
      if (is_dp(j)) opb[j] = load_b(j);
    }
    if (kS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
        dpacc[kb] = zero16();
      }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (j < NP) {
        const int kb = j / (2 * MB), s2 = (j / MB) % 2, mb = j % MB;
        dqacc[mb] = mfma32(opa[j % kPre], db[2 * kb + s2], dqacc[mb]);
      } else {
        const int i = j - NP, kb = (i / 2) % 2, ks = i / 4;
        if (i & 1)
          dpacc[kb] = mfma32(opa[j % kPre], opb[j % kPre], dpacc[kb]);
        else
          sacc[kb] = mfma32(opa[j % kPre], qreg[ks], sacc[kb]);
      }
      if (j + kPre < N) {
        opa[j % kPre] = load_a(j + kPre);
        if (is_dp(j + kPre)) opb[j % kPre] = load_b(j + kPre);
      }
    }
    // pin the order: the first kPre steps' operands, then one MFMA and the
    // operands of the step kPre ahead (2 LDS reads for dQ and dP steps, 1 for S)
    static_assert(NP == 0 || NP >= kPre, "prefetch covers one operand kind");
    static_assert(kPre % 2 == 0, "S / dP alternate");
    if constexpr (NP > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);
    else
      __builtin_amdgcn_sched_group_barrier(0x100, 3 * kPre / 2, 0);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j + kPre < NP || (j + kPre < N && is_dp(j + kPre)))
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (j + kPre < N)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // the stream stays in its half-step
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) keep(dqacc[mb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      keep(sacc[kb]);
      keep(dpacc[kb]);
    }
  };

  // GRAD half-step of the tile at j0: dS (bf16) into db; a tile this wave
  // skips leaves zeros, so the next MFMA half-step may run its dQ regardless
  auto grad = [&](int j0, bool do_s) {
    if (!do_s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) db[i] = zero8();
      return;
    }
    const bool full = tile_full(j0);
    const int a = r_lo - j0 - 4 * hi, e_end = r_hi - j0 - 4 * hi;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(sacc[kb][r], scale_log2, -lse_use));
        ds[r] = p * (dpacc[kb][r] - my_delta);
      }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 8 * (r / 4) + (r % 4);
          ds[r] = (c >= a && c < e_end) ? ds[r] : 0.f;
        }
      }
      db[2 * kb] = pack8(&ds[0]);
      db[2 * kb + 1] = pack8(&ds[8]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) keep(db[i]);
  };

  // t = 0: S(0), dP(0) only
  bool any_prev = false;
  if (ntiles > 0) {
    if (team == 0) {
      if (ntiles > 1) {
        issue_rows(k, &Ks[1][0], lo + BN);
        issue_rows(v, &Vs[1][0], lo + BN);
      }
    }
    const bool do_s = tile_any(lo);
    if (do_s) mfma_stream(BoolC<false>(), BoolC<true>(), &Ks[2][0], &Ks[0][0], &Vs[0][0]);
    wg_barrier<kWaitNone>();
    grad(lo, do_s);
    any_prev = do_s;
    wg_barrier<kWaitAll>();     // team 0's loads of this tile pair have landed
  }
  // 0 < t < ntiles: dQ(t-1), S(t), dP(t) as one stream; c = t % 3
  int c = 1;
  for (int t = 1; t < ntiles; ++t) {
    const int j0 = lo + t * BN;
    const int cn = c == 2 ? 0 : c + 1, cp = c == 0 ? 2 : c - 1;
    if (team == 0 && t + 1 < ntiles) {
      issue_rows(k, &Ks[cn][0], j0 + BN);
      issue_rows(v, &Vs[(t + 1) & 1][0], j0 + BN);
    }
    const bool do_s = tile_any(j0);
    if (any_prev || do_s)
      mfma_stream(BoolC<true>(), BoolC<true>(), &Ks[cp][0], &Ks[c][0], &Vs[t & 1][0]);
    wg_barrier<kWaitNone>();
    grad(j0, do_s);
    any_prev = do_s;
    wg_barrier<kWaitAll>();
    c = cn;
  }
  // t = ntiles: dQ(ntiles-1) only
  if (any_prev)
    mfma_stream(BoolC<true>(), BoolC<false>(), &Ks[(ntiles - 1) % 3][0], &Ks[0][0], &Vs[0][0]);
  wg_barrier<kWaitNone>();
  if (team == 0) wg_barrier<kWaitNone>();

  if (!row_valid) return;
  const size_t obase = (static_cast<size_t>(my_tok) * hq + my_head) * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      float4* p = reinterpret_cast<float4*>(dq + obase + mb * 32 + 8 * gq + 4 * hi);
      float4 a = *p;
      a.x += scale * dqacc[mb][4 * gq + 0];
      a.y += scale * dqacc[mb][4 * gq + 1];
      a.z += scale * dqacc[mb][4 * gq + 2];
      a.w += scale * dqacc[mb][4 * gq + 3];
      *p = a;
    }
}

// ---------------------------------------------------------------------------
// dK / dV: key-outer.  The workgroup owns 128 keys of one kv-head; the query
// rows that can see them stream through in tiles of 64 rows.
//
// Eight waves, two per SIMD.  Wave w = (kw, rh) = (w % 4, w / 4):
//   * for tile rows 32*rh .. +31 and key group kw (32 keys; K and V held in
//     registers) it computes S, dP, P and dS;
//   * the wave with rh = 0 accumulates dV^T = dO^T P and the one with rh = 1
//     dK^T = Q^T dS for the key group, each over the tile's 64 rows and the
//     full head dimension.  The partner's half of P (or dS) arrives through
//     LDS as packed bf16 MFMA operands.
//
// Two teams of four waves (key groups 0-1 and 2-3), placed so that the two
// waves sharing a SIMD belong to different teams.  Each tile takes three
// steps per wave: GRAD (dV / dK MFMAs of the previous tile, partner packs
// read from LDS), SDP (S / dP MFMAs of the tile) and SOFT (softmax gradient,
// writes the packs).  Every wave runs the same loop, one iteration per tile:
//   barrier, GRAD(i-1) + SDP(i), barrier, SOFT(i)
// but team 1 runs one barrier behind team 0 (an extra barrier at its start,
// one at team 0's end), so between any two barriers one wave of each SIMD
// feeds the matrix core while the other works on the vector ALUs.  A team
// writes its exchange in one window and reads it in the next, so one
// exchange buffer suffices.  Team 0 alone loads the Q / dO tiles, by direct
// global->LDS loads into a three-stage ring: tile i+1 is loaded while team 0
// works on GRAD(i-1) + SDP(i) (its load rounds spread over the SDP MFMAs, so
// that no burst of them stalls the wave) into the stage of tile i-2, whose
// last reader, team 1's GRAD(i-2), finished before that window; team 0 waits
// for it before the barrier that opens its next MFMA window, which team 1
// passes before it reads the tile.
//
// Query tiles are visited from the END of the visible range backwards: every
// key block of a sequence sees the same trailing rows, so the workgroups that
// an XCD runs together read the same tiles at nearly the same time and share
// them through L2.
// ---------------------------------------------------------------------------
namespace bwdkv {
constexpr int NW = 8;          // waves per workgroup
constexpr int KB = 128;        // keys per workgroup (4 key groups of 32)
constexpr int TR = 64;         // query rows per tile (2 halves of 32)
constexpr float kSplitP = 1.f / 256.f;
}  // namespace bwdkv

template <int D, int G>
__global__ __launch_bounds__(512, 1) void main_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int nq, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ k_seq,
    const int32_t* __restrict__ k_pos, int nk, int hq, int hkv, float scale,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv) {
  using namespace bwdkv;
  constexpr int TPT = TR / G;               // tokens per tile
  constexpr int KS = D / 16;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int TS = TR * D;                // elements of one tensor tile
  constexpr int QROUNDS = TR * CPR / 512;   // 16-byte DMA rounds per thread per tensor per tile
  constexpr int XN = NW * 2 * 64;           // packs per exchange buffer

  // three-stage ring; a stage holds Q | dO (rows x d, swizzled) and
  // meta = lse | delta | seq | pos of its 64 rows
  __shared__ __attribute__((aligned(16))) uint16_t R[3][2 * TS];
  __shared__ __attribute__((aligned(16))) uint32_t Mr[3][4 * TR];
  // partner-bound packs, MFMA B-operand layout: [wave][k-step][lane] x 8 bf16
  __shared__ __attribute__((aligned(16))) bf16x8 Xh[XN], Xl[XN];
  __shared__ int Xf[NW];    // 0: nothing visible, 1: hi only, 2: hi + lo

  const float scale_log2 = scale * kLog2e;
  const int nblk = (nk + KB - 1) / KB;
  const int L = xcd_remap(blockIdx.x, nblk * hkv);
  const int g = L / nblk;
  const int kblk = L % nblk;             // early keys are seen by the most rows: heavy first
  const int key0 = kblk * KB;
  const int tid = threadIdx.x;
  // wave w: team w / 4, key group 2*team + (w / 2) % 2, row half / role w % 2
  // (0: dV, 1: dK); waves w and w + 4 share a SIMD under the usual
  // round-robin placement, and belong to different teams
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int team = wave >> 2;
  const int kw = 2 * team + ((wave >> 1) & 1), rh = wave & 1;
  const int partner = wave ^ 1;
  const int n = lane & 31, hi = lane >> 5;
  const LaneOffsets<D> lo_off(lane);

  // this lane's key (column n of the wave's 32-key group)
  const int my_key = key0 + kw * 32 + n;
  const bool key_valid = my_key < nk;
  const int kseq = key_valid ? k_seq[my_key] : INT_MIN;
  const int kpos = key_valid ? k_pos[my_key] : INT_MAX;
  const int wk0 = key0 + kw * 32;
  const bool wave_valid = wk0 < nk;
  const int wkl = min(nk, wk0 + 32) - 1;
  const bool wave_complete = wk0 + 32 <= nk;
  const int wf_seq = __builtin_amdgcn_readfirstlane(wave_valid ? k_seq[wk0] : 0);
  const int wf_pos = __builtin_amdgcn_readfirstlane(wave_valid ? k_pos[wk0] : 0);
  const int wl_seq = __builtin_amdgcn_readfirstlane(wave_valid ? k_seq[wkl] : 0);
  const int wl_pos = __builtin_amdgcn_readfirstlane(wave_valid ? k_pos[wkl] : 0);

  // K and V rows of the lane's key as MFMA B operands (k-elements 16*ks + 8*hi ..)
  bf16x8 kreg[KS], vreg[KS];
  {
    const size_t kb = (static_cast<size_t>(key_valid ? my_key : 0) * hkv + g) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = key_valid ? *reinterpret_cast<const bf16x8*>(k + kb + 16 * ks) : zero8();
      vreg[ks] = key_valid ? *reinterpret_cast<const bf16x8*>(v + kb + 16 * ks) : zero8();
    }
  }

  // query tokens that can see any key of the block; tile i covers tokens
  // [qhi - (i+1)*TPT, qhi - i*TPT) clipped at qlo
  const int klast = min(nk, key0 + KB) - 1;
  const int qlo = __builtin_amdgcn_readfirstlane(
      lower_bound_sp(q_seq, q_pos, nq, k_seq[key0], k_pos[key0]));
  const int qhi = __builtin_amdgcn_readfirstlane(
      upper_bound_sp(q_seq, q_pos, nq, k_seq[klast], INT_MAX));
  const int ntiles = qhi > qlo ? (qhi - qlo + TPT - 1) / TPT : 0;

  f32x16 acc[MB];   // dV^T (rh = 0) or dK^T (rh = 1): rows = head-dim columns, cols = keys
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
  // this wave's own packs (P for rh = 0, dS for rh = 1) of the previous tile.
  // Every pack is defined on every path (zero where unused): the lo MFMAs are
  // conditional, and undefined operands on the untaken side have let the
  // compiler produce wrong accumulators.
  bf16x8 own_h[2] = {zero8(), zero8()}, own_l[2] = {zero8(), zero8()};
  int own_f = 0;

  auto tile_t0 = [&](int i) { return max(qlo, qhi - (i + 1) * TPT); };

  // Loads of tile i into ring stage st, issued by the four waves of team 0.
  // Lane l of round `it` of wave w fills 16-byte slot (it*4 + w)*64 + l of
  // the tile, i.e. physical chunk p of row r; it fetches logical chunk
  // swz(r, p) (the swizzle is an involution).  Rows past the tile's end (only
  // in the tile at the start of the range) re-read its last row; they are
  // masked by index.  Addresses are a wave-uniform 64-bit base for the tile
  // plus a per-lane 32-bit byte offset relative to the tile's first token.
  constexpr int LROUNDS = 2 * QROUNDS;
  uint32_t lane_off[LROUNDS];   // bytes
#pragma unroll
  for (int it = 0; it < LROUNDS; ++it) {
    const int slot = (it * 4 + (wave & 3)) * 64 + lane;
    const int r = slot / CPR, p = slot % CPR;
    lane_off[it] = 2u * (((r / G) * hq + g * G + r % G) * D + 8 * swz<D>(r, p));
  }
  // meta: row = lane; lse / delta at [head][token], seq / pos at [token].
  // Recomputed per tile from an opaque copy of the lane id, so that it is not
  // kept live (and spilled) across the loop.
  const bool meta_by_head = (wave & 3) < 2;
  auto meta_off_of = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return 4u * (meta_by_head ? (g * G + l % G) * nq + l / G : l / G);
  };
  const char* const meta_src = reinterpret_cast<const char*>(
      (wave & 3) == 0 ? static_cast<const void*>(lse)
    : (wave & 3) == 1 ? static_cast<const void*>(delta)
    : (wave & 3) == 2 ? static_cast<const void*>(q_seq)
                      : static_cast<const void*>(q_pos));
  // One round of the loads of tile i into stage st: 16 bytes of Q and of dO
  // per lane.  Rows past the tile's end (only in the tile at the start of
  // the range) re-read its last row; they are masked by index.
  auto issue_round = [&](int st, int i, int it) {
    const int t0 = tile_t0(i);
    const int t1 = qhi - i * TPT;
    const char* qt = reinterpret_cast<const char*>(q) + static_cast<size_t>(t0) * hq * D * 2;
    const char* ot = reinterpret_cast<const char*>(dout) + static_cast<size_t>(t0) * hq * D * 2;
    const int r = ((it * 4 + (wave & 3)) * 64 + lane) / CPR;
    const int dt = min(r / G, t1 - 1 - t0) - r / G;
    const uint32_t base = lds_addr(&R[st][(it * 4 + (wave & 3)) * 64 * 8]);
    const uint32_t off = lane_off[it] + static_cast<uint32_t>(dt * hq * D * 2);
    dma_b128(qt, off, base);
    dma_b128(ot, off, base + TS * 2);
  };
  auto issue_meta = [&](int st, int i) {
    const int t0 = tile_t0(i);
    const int t1 = qhi - i * TPT;
    const char* mt = meta_src + static_cast<size_t>(t0) * 4;
    const int dtok = min(lane / G, t1 - 1 - t0) - lane / G;
    dma_b32(mt, meta_off_of() + 4 * dtok, lds_addr(&Mr[st][(wave & 3) * TR]));
  };

  // ---- GRAD: dV^T += dO^T P (rh = 0) or dK^T += Q^T dS (rh = 1) over the
  // 64 rows of the previous tile, held in ring stage `st`.  Rows
  // 32*h + 16*s2 + 8*(j/4) + 4*hi + (j%4) are k-element j of k-step (h, s2):
  // the register order of the packs.
  auto grad = [&](const uint16_t* tile) {
    const uint16_t* At = tile + (rh ? 0 : TS);
    const int par_f = __builtin_amdgcn_readfirstlane(Xf[partner]);
    if (own_f == 1 && par_f == 1) {
      // common case, both halves visible and no split: 4*MB MFMAs, own
      // rows first, transposed operands loaded kPre MFMAs ahead
      constexpr int kPre = 4;
      constexpr int NSTEP = 4 * MB;
      const uint16_t* Aown = At + 32 * rh * D;
      const uint16_t* Apar = At + 32 * (1 - rh) * D;
      const bf16x8 pb0 = Xh[(partner * 2 + 0) * 64 + lane];
      const bf16x8 pb1 = Xh[(partner * 2 + 1) * 64 + lane];
      auto load = [&](int j) {
        const int hh = j / (2 * MB), s2 = (j / MB) % 2, mb = j % MB;
        return tr_operand<D>(hh == 0 ? Aown : Apar, lo_off, 16 * s2, mb);
      };
      bf16x8 opnd[kPre];
#pragma unroll
      for (int j = 0; j < kPre; ++j) opnd[j] = load(j);
#pragma unroll
      for (int j = 0; j < NSTEP; ++j) {
        const int hh = j / (2 * MB), s2 = (j / MB) % 2, mb = j % MB;
        const bf16x8 b = hh == 0 ? own_h[s2] : (s2 == 0 ? pb0 : pb1);
        acc[mb] = mfma32(opnd[j % kPre], b, acc[mb]);
        if (j + kPre < NSTEP) opnd[j % kPre] = load(j + kPre);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + 2 * kPre, 0);
#pragma unroll
      for (int j = 0; j < NSTEP - kPre; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
      return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool mine = h == rh;
      const int f = mine ? own_f : par_f;
      if (f == 0) continue;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int xi = (partner * 2 + s2) * 64 + lane;
        const bf16x8 bh = mine ? own_h[s2] : Xh[xi];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8 a = tr_operand<D>(At, lo_off, 32 * h + 16 * s2, mb);
          acc[mb] = mfma32(a, bh, acc[mb]);
        }
        if (f == 2) {
          const bf16x8 bl = mine ? own_l[s2] : Xl[xi];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const bf16x8 a = tr_operand<D>(At, lo_off, 32 * h + 16 * s2, mb);
            acc[mb] = mfma32(a, bl, acc[mb]);
          }
        }
      }
    }
  };

  // ---- SDP: S = Q K^T, dP = dO V^T of tile i (ring stage st): lane (n = key,
  // hi) register r holds row r0 + acc_row(r, hi).  The state below carries
  // the tile to its SOFT step.
  const int r0 = 32 * rh;
  bool active = false, wave_full = false;
  int nrows = 0, soft_st = 0;
  f32x16 sacc = zero16(), dpacc = zero16();
  // Visibility of tile i for this wave's key group and row half, from the
  // sequence / position of the row half's first and last rows in the tile's
  // meta: LDS reads issued right after the barrier that publishes the tile
  // (vis_load) and evaluated after the dV / dK MFMAs (vis_eval), so that
  // their latency stays hidden.
  bool nx_active = false, nx_full = false;
  int nx_nrows = 0;
  int v_nr = 0, v_rl = 0, v_fs = 0, v_fp = 0, v_ls = 0, v_lp = 0;
  bool v_some = false;
  auto vis_load = [&](int i, int st) {
    v_some = false;
    v_nr = 0;
    if (i >= ntiles) return;
    const int t0 = tile_t0(i);
    v_nr = (qhi - i * TPT - t0) * G;
    if (r0 >= v_nr) return;
    v_some = true;
    v_rl = min(v_nr, r0 + 32) - 1;
    const int* rseq_s = reinterpret_cast<const int*>(&Mr[st][2 * TR]);
    const int* rpos_s = reinterpret_cast<const int*>(&Mr[st][3 * TR]);
    v_fs = rseq_s[r0];
    v_fp = rpos_s[r0];
    v_ls = rseq_s[v_rl];
    v_lp = rpos_s[v_rl];
  };
  auto vis_eval = [&]() {
    nx_nrows = v_nr;
    nx_active = __builtin_amdgcn_readfirstlane(
        v_some && wave_valid && !lex_less(v_ls, v_lp, wf_seq, wf_pos) &&
        !lex_less(wl_seq, INT_MAX, v_fs, v_fp));
    nx_full = __builtin_amdgcn_readfirstlane(
        v_some && wave_complete && v_rl == r0 + 31 && v_fs == v_ls && v_fs == wf_seq &&
        wf_seq == wl_seq && v_fp >= wl_pos);
  };

  auto sdp = [&](int i, int st, auto dma_c, int dst, int di) {
    constexpr bool kDMA = decltype(dma_c)::value;
    static_assert(2 * LROUNDS + 1 < 2 * KS, "load rounds fit in the stream");
    active = nx_active;
    wave_full = nx_full;
    nrows = nx_nrows;
    soft_st = st;
    if (i >= ntiles) {
      sacc = zero16();
      dpacc = zero16();
      if (kDMA) {
#pragma unroll
        for (int it = 0; it < LROUNDS; ++it) issue_round(dst, di, it);
        issue_meta(dst, di);
      }
      return;
    }
    // 2*KS MFMAs (S then dP), operands loaded kPre steps ahead; computed for
    // every wave so that the accumulators are redefined on every path (rows
    // past the tile's end hold copies of its last row), used only if active
    // S and dP MFMAs alternate (j even: S k-step j/2, j odd: dP), so that
    // consecutive MFMAs are independent and the two accumulation chains
    // cover each other's result latency.  Team 0 spreads the loads of the
    // next tile over the stream (one round every other MFMA), so that no
    // burst of them stalls the wave.
    const uint16_t* cur = R[st];
    constexpr int kPre = 8;
    bf16x8 opnd[kPre];
    auto load = [&](int j) {
      return row_operand<D>(cur + (j & 1) * TS, lo_off, r0, j >> 1);
    };
#pragma unroll
    for (int j = 0; j < kPre; ++j) opnd[j] = load(j);
#pragma unroll
    for (int j = 0; j < 2 * KS; ++j) {
      const int ks = j >> 1;
      if (j == 0) sacc = mfma32(opnd[0], kreg[0], zero16());
      else if (j == 1) dpacc = mfma32(opnd[1], vreg[0], zero16());
      else if ((j & 1) == 0) sacc = mfma32(opnd[j % kPre], kreg[ks], sacc);
      else dpacc = mfma32(opnd[j % kPre], vreg[ks], dpacc);
      if (j + kPre < 2 * KS) opnd[j % kPre] = load(j + kPre);
      if (kDMA && (j & 1) && j / 2 < LROUNDS) issue_round(dst, di, j / 2);
      if (kDMA && j == 2 * LROUNDS + 1) issue_meta(dst, di);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int j = 0; j < 2 * KS - kPre; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
  };

  // ---- SOFT: softmax gradient of the tile last passed to SDP: P, dS; own
  // packs replace the previous tile's (already used by GRAD), partner-bound
  // packs go to the exchange.
  auto soft = [&]() {
    own_f = 0;
    if (active) {
      const uint32_t* M = Mr[soft_st];
      const float* lse_s = reinterpret_cast<const float*>(M);
      const float* dl_s = reinterpret_cast<const float*>(M + TR);
      const int* rseq_s = reinterpret_cast<const int*>(M + 2 * TR);
      const int* rpos_s = reinterpret_cast<const int*>(M + 3 * TR);
      float p[16], ds[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rb = r0 + 8 * r4 + 4 * hi;
        const float4 l4 = *reinterpret_cast<const float4*>(&lse_s[rb]);
        const float4 d4 = *reinterpret_cast<const float4*>(&dl_s[rb]);
        const float lv[4] = {l4.x * kLog2e, l4.y * kLog2e, l4.z * kLog2e, l4.w * kLog2e};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        if (wave_full) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            p[r] = exp2_fast(fmaf(sacc[r], scale_log2, -lv[e]));
            ds[r] = p[r] * (dpacc[r] - dv4[e]);
          }
        } else {
          const int4 ss = *reinterpret_cast<const int4*>(&rseq_s[rb]);
          const int4 pp = *reinterpret_cast<const int4*>(&rpos_s[rb]);
          const int sv[4] = {ss.x, ss.y, ss.z, ss.w};
          const int pv[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            const bool vis = key_valid & (rb + e < nrows) & (lv[e] != kNegInf) &
                             (sv[e] == kseq) & (pv[e] >= kpos);
            const float pr = vis ? exp2_fast(fmaf(sacc[r], scale_log2, -lv[e])) : 0.f;
            p[r] = pr;
            ds[r] = pr * (dpacc[r] - dv4[e]);
          }
        }
      }
      // P and dS enter the gradient MFMAs as bf16.  Where some P of the
      // block reaches kSplitP they enter as hi + lo bf16 pairs (lo = x - hi,
      // a second MFMA on the same A operand): rows that give a key a large
      // weight would otherwise carry bf16's 2^-9 relative rounding into the
      // key's gradient with a large coefficient.  Below the threshold the
      // dropped lo terms are at most kSplitP * 2^-9 each.
      // own: P (rh = 0) or dS (rh = 1); partner-bound: the other one.  The
      // partner-bound hi packs are written first, so that their LDS latency
      // overlaps the rest of the step.
      auto emit = [&](const float (&mine)[16], const float (&theirs)[16]) {
        bf16x8 th[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          th[s2] = pack8(&theirs[8 * s2]);
          Xh[(wave * 2 + s2) * 64 + lane] = th[s2];
        }
        f32x16 pv;
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = p[r];
        const bool split = __any(max16_raw(0.f, pv) >= kSplitP);
        own_f = split ? 2 : 1;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) own_h[s2] = pack8(&mine[8 * s2]);
        if (split) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            float ol[8], tl[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              ol[j] = mine[8 * s2 + j] - static_cast<float>(own_h[s2][j]);
              tl[j] = theirs[8 * s2 + j] - static_cast<float>(th[s2][j]);
            }
            own_l[s2] = pack8(ol);
            Xl[(wave * 2 + s2) * 64 + lane] = pack8(tl);
          }
        }
      };
      if (rh) emit(ds, p);
      else emit(p, ds);
    }
    if (lane == 0) Xf[wave] = own_f;
  };

  // Iterations run 0 .. ntiles; tile i sits in stage i % 3.  The last
  // iteration only finishes tile ntiles-1.
  if (team == 0 && ntiles > 0) {
#pragma unroll
    for (int it = 0; it < LROUNDS; ++it) issue_round(0, 0, it);
    issue_meta(0, 0);
  }
  if (team == 1) wg_barrier<kWaitLgkm>();
  int sc = 0;
  for (int i = 0; i <= ntiles; ++i) {
    const int sn = sc == 2 ? 0 : sc + 1;
    const int sp = sc == 0 ? 2 : sc - 1;
    // MFMA window: tile i landed (team 0 waited for its loads); stage sn
    // (tile i-2) is free
    wg_barrier<kWaitAll>();
    vis_load(i, sc);
    if (i >= 1) grad(R[sp]);
    vis_eval();
    if (team == 0 && i + 1 < ntiles)
      sdp(i, sc, BoolC<true>(), sn, i + 1);
    else
      sdp(i, sc, BoolC<false>(), 0, 0);
    // VALU window
    wg_barrier<kWaitLgkm>();
    soft();
    sc = sn;
  }
  if (team == 0) wg_barrier<kWaitLgkm>();

  if (!key_valid) return;
  const size_t obase = (static_cast<size_t>(my_key) * hkv + g) * D;
  float* const out = rh ? dk : dv;
  const float sc_out = rh ? scale : 1.f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      float4* po = reinterpret_cast<float4*>(out + obase + mb * 32 + 8 * gq + 4 * hi);
      float4 a = *po;
      a.x += sc_out * acc[mb][4 * gq + 0];
      a.y += sc_out * acc[mb][4 * gq + 1];
      a.z += sc_out * acc[mb][4 * gq + 2];
      a.w += sc_out * acc[mb][4 * gq + 3];
      *po = a;
    }
}

template <int D, int G>
static void main_bwd_mfma_dg(const MainArgs& a, int part) {
  if (part != 2) {
    constexpr int TPB = bwdq::NW * (32 / G);
    const int nblk_tok = (a.nq + TPB - 1) / TPB;
    hipLaunchKernelGGL((main_bwd_dq_kernel<D, G>), dim3(nblk_tok * a.hkv), dim3(512), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), a.q_seq, a.q_pos, a.nq,
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       a.k_seq, a.k_pos, a.nk, a.hq, a.hkv, a.scale,
                       static_cast<const uint16_t*>(a.dout), a.lse, a.delta, a.dq);
  }
  if (part != 1) {
    const int nblk = (a.nk + bwdkv::KB - 1) / bwdkv::KB;
    hipLaunchKernelGGL((main_bwd_dkdv_kernel<D, G>), dim3(nblk * a.hkv), dim3(512), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), a.q_seq, a.q_pos, a.nq,
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       a.k_seq, a.k_pos, a.nk, a.hq, a.hkv, a.scale,
                       static_cast<const uint16_t*>(a.dout), a.lse, a.delta, a.dk, a.dv);
  }
}

template <int D>
static void main_bwd_mfma_d(const MainArgs& a, int part) {
  switch (a.hq / a.hkv) {
    case 1: main_bwd_mfma_dg<D, 1>(a, part); break;
    case 2: main_bwd_mfma_dg<D, 2>(a, part); break;
    case 4: main_bwd_mfma_dg<D, 4>(a, part); break;
    case 8: main_bwd_mfma_dg<D, 8>(a, part); break;
    case 16: main_bwd_mfma_dg<D, 16>(a, part); break;
    default: main_bwd_mfma_dg<D, 32>(a, part); break;
  }
}

hipError_t launch_main_bwd_mfma(const MainArgs& a, int part) {
  if (a.nq == 0 || a.nk == 0) return hipSuccess;
  if (a.d == 128) main_bwd_mfma_d<128>(a, part); else main_bwd_mfma_d<64>(a, part);
  return hipGetLastError();
}

}  // namespace bac
