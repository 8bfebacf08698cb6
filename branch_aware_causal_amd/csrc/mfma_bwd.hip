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
//     lane pair (n, n+32).  Q and dO stay in registers (B operands of S^T
//     and dP^T), so every MFMA of the stream reads one operand from LDS.
//   * Keys stream through LDS in tiles of 64, copied straight from global
//     memory (K in a ring of three, V in a ring of two).  The keys a row sees
//     are one index interval of the (seq, pos)-sorted shard, found by binary
//     search, so masks are index compares.
//   * Ping-pong: waves w and w+4 share a SIMD; team 0 (waves 0-3) and team 1
//     (waves 4-7) run the same iteration -- MFMA(t), then GRAD(t) -- with
//     one workgroup barrier per tile period, which team 0 passes after
//     GRAD(t) and team 1 after MFMA(t).  So between two barriers
//       team 0: MFMA(t) then GRAD(t)      team 1: GRAD(t-1) then MFMA(t)
//     and on every SIMD one wave's MFMAs meet the other's vector work.
//     (A barrier between the MFMA and GRAD halves cost 1.6% more time at
//     256K; both teams run the same code, so the register allocator sees
//     one live set.)  MFMA(t) = dQ^T += K^T dS^T for tile t-1, then
//     S^T = K Q^T and dP^T = V dO^T for tile t, as one stream of 48 MFMAs
//     with LDS operands read ahead; GRAD(t) = dS = P (dP - Delta) on the
//     vector ALUs.  K(t) is read in periods t and t+1, V(t) in period t.
//     Team 0 loads K(t+1) and V(t+1) at the start of its iteration t and
//     waits for them at its barrier.
//   * A wave reads the first K^T operands of its next MFMA stream at the end
//     of its GRAD step (it has slack there), and runs its MFMA streams at
//     raised issue priority so that the partner's vector work yields to them
//     on the shared SIMD.
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

  // Q and dO rows in registers: the B operands of S^T = K Q^T and dP^T = V dO^T.
  bf16x8 qreg[KS], doreg[KS];
  {
    const size_t off = (static_cast<size_t>(my_tok) * hq + my_head) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = row_valid ? *reinterpret_cast<const bf16x8*>(q + off + 16 * ks) : zero8();
      doreg[ks] = row_valid ? *reinterpret_cast<const bf16x8*>(dout + off + 16 * ks) : zero8();
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
  // Round `it` covers key rows RPR*it + r0 (r0 = slot's row in round 0);
  // the swizzle depends on the row modulo 16 only, so one column offset
  // serves every round.
  constexpr int ROUNDS = BN * CPR / 256;
  constexpr int RPR = 256 / CPR;     // key rows per round
  static_assert(RPR % 16 == 0, "rounds keep the row's swizzle");
  const int lane_r0 = ((wave & 3) * 64 + lane) / CPR;
  const uint32_t lane_col = 2u * (g * D + 8 * swz<D>(lane_r0, ((wave & 3) * 64 + lane) % CPR));
  const uint32_t krow_bytes = static_cast<uint32_t>(hkv * D * 2);
  auto issue_rows = [&](const uint16_t* src, const uint16_t* dst_tile, int j0) {
    const char* base = reinterpret_cast<const char*>(src) + static_cast<size_t>(j0) * krow_bytes;
    const int rmax = nk - 1 - j0;     // last valid key row of the tile
#pragma unroll
    for (int it = 0; it < ROUNDS; ++it) {
      const uint32_t off =
          static_cast<uint32_t>(min(lane_r0 + RPR * it, rmax)) * krow_bytes + lane_col;
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

  f32x16 sacc[2] = {zero16(), zero16()}, dpacc[2] = {zero16(), zero16()};
  bf16x8 db[4] = {zero8(), zero8(), zero8(), zero8()};

  // One MFMA step as a single stream: dQ^T += K^T dS^T for the previous
  // tile (4*MB MFMAs, transposed K operands), then S^T = K Q^T and
  // dP^T = V dO^T for this tile (4*KS MFMAs, alternating).  LDS operands are
  // read kPre MFMAs ahead.
  constexpr int kPre = 2;
  // the first kPre operands of a stream that starts with dQ are read at the
  // end of the wave's previous GRAD step (pre_dq), off the MFMA path
  bf16x8 opa[kPre];
  auto pre_dq = [&](const uint16_t* kprev) {
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int kb = j / (2 * MB), s2 = (j / MB) % 2, mb = j % MB;
      opa[j] = tr_operand<D>(kprev, lo_off, kb * 32 + 16 * s2, mb);
    }
  };
  auto mfma_stream = [&](auto dq_c, auto s_c, const uint16_t* kprev, const uint16_t* kt,
                         const uint16_t* vt) {
    constexpr bool kDQ = decltype(dq_c)::value, kS = decltype(s_c)::value;
    __builtin_amdgcn_s_setprio(1);
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
    if constexpr (!kDQ) {
#pragma unroll
      for (int j = 0; j < kPre; ++j) opa[j] = load_a(j);
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
          dpacc[kb] = mfma32(opa[j % kPre], doreg[ks], dpacc[kb]);
        else
          sacc[kb] = mfma32(opa[j % kPre], qreg[ks], sacc[kb]);
      }
      if (j + kPre < N) {
        opa[j % kPre] = load_a(j + kPre);
      }
    }
    // pin the order: (without dQ) the first kPre operands, then one MFMA and
    // the operand of the step kPre ahead (2 LDS reads for a dQ step, 1 for S / dP)
    static_assert(NP == 0 || NP >= kPre, "prefetch covers one operand kind");
    static_assert(kPre % 2 == 0, "S / dP alternate");
    if constexpr (NP == 0) __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (j + kPre < NP)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (j + kPre < N)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // the stream stays before the GRAD step
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) keep(dqacc[mb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      keep(sacc[kb]);
      keep(dpacc[kb]);
    }    __builtin_amdgcn_s_setprio(0);
  };

  // GRAD step of the tile at j0: dS (bf16) into db; a tile this wave skips
  // leaves zeros, so the next MFMA step may run its dQ regardless
  auto grad = [&](int j0, bool do_s) {
    if (!do_s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) db[i] = zero8();
      return;
    }
    const bool full = tile_full(j0);
    const int a = r_lo - j0 - 4 * hi, e_end = r_hi - j0 - 4 * hi;
    // in place and in three phases, as in the dK/dV kernel: exponent
    // arguments, exponentials beside the dP - Delta subtractions, products
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = fmaf(sacc[kb][r], scale_log2, -lse_use);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[kb][r] = exp2_fast(sacc[kb][r]);
        dpacc[kb][r] -= my_delta;
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = sacc[kb][r] * dpacc[kb][r];
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

  // One barrier per tile period, at a different place in each team's
  // iteration: team 0 passes it after GRAD(t), team 1 after MFMA(t), so that
  // between two barriers team 0 runs MFMA(t) then GRAD(t) while team 1 runs
  // GRAD(t-1) then MFMA(t).  Team 0 loads K(t+1) and V(t+1) at the start of
  // its iteration t and waits for them at its barrier.
  bool any_prev = false;
  if (ntiles > 0) {
    // t = 0: S(0), dP(0) only
    if (team == 0 && ntiles > 1) {
      issue_rows(k, &Ks[1][0], lo + BN);
      issue_rows(v, &Vs[1][0], lo + BN);
    }
    const bool do_s = tile_any(lo);
    if (do_s) mfma_stream(BoolC<false>(), BoolC<true>(), &Ks[2][0], &Ks[0][0], &Vs[0][0]);
    if (team == 1) wg_barrier<kWaitLgkm>();
    grad(lo, do_s);
    pre_dq(&Ks[0][0]);
    any_prev = do_s;
    if (team == 0) wg_barrier<kWaitAll>();     // team 0's loads of tile 1 have landed
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
    if (team == 1) wg_barrier<kWaitLgkm>();
    grad(j0, do_s);
    pre_dq(&Ks[c][0]);
    any_prev = do_s;
    if (team == 0) wg_barrier<kWaitAll>();
    c = cn;
  }
  // t = ntiles: dQ(ntiles-1) only
  if (any_prev)
    mfma_stream(BoolC<true>(), BoolC<false>(), &Ks[(ntiles - 1) % 3][0], &Ks[0][0], &Vs[0][0]);

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
// dK / dV: key-outer.  The workgroup owns 128 keys of one kv-head (four key
// groups of 32); the query rows that can see them stream through in tiles of
// 32 rows, visited from the END of the visible range backwards (every key
// block of a sequence sees the same trailing rows, so the workgroups an XCD
// runs together read the same tiles at nearly the same time, through L2).
//
// Eight waves in two teams; waves w and w+4 share a SIMD:
//   * producer w (waves 0-3) serves key group w: K and V of the group's 32 keys in registers as
//     MFMA A operands; per tile, S^T = K Q^T and dP^T = V dO^T (one query row
//     per lane), then P = exp2(s*c - lse2) and dS = P (dP - Delta); P and dS
//     go to LDS as bf16 [row][key] tiles (hi + lo pairs where some P of the
//     tile reaches kSplitP, see below), with a flag per group;
//   * consumer (waves 4-7): dV^T += dO^T P and dK^T += Q^T dS over the
//     tile's rows, both operands by transposing LDS reads, the accumulators
//     in registers for the whole block.  Consumer c covers key groups
//     2*(c/2) and 2*(c/2)+1 for half of d (d-blocks 2*(c%2) ..): each
//     transposed Q / dO operand then feeds two MFMAs, 32 transposing reads
//     per tile instead of 40 with one group over all of d (0.6-1.5% less
//     dK/dV time at 256K).
// One barrier per tile.  In iteration i the producer runs the S / dP MFMAs
// of tile i and then its softmax gradient (vector ALUs), writing the P / dS
// tiles of tile i into exchange buffer i % 2; the consumer issues the loads
// of tile i+2, reads the P / dS tiles of tile i-1 from the other buffer and
// runs its dV / dK MFMAs of tile i-1.  The two waves of a SIMD interleave
// freely between barriers.  (Two barriers per tile, splitting the iteration
// into an MFMA half-step and a softmax half-step, cost 6% more time at 256K:
// the second barrier's wait outweighed the pairing it enforced.)  Q / dO
// tiles and their rows' lse, Delta, seq, pos come by direct global->LDS
// loads, issued by the consumer waves, into a four-stage ring: tile i+2 is
// loaded in iteration i into the stage of tile i-2 (whose last readers, the
// producer in iteration i-2 and the consumer in iteration i-1, finished
// before the barrier that opened iteration i), and each consumer waits for
// its loads of tile i+1 at the barrier that opens iteration i+1, keeping
// only its newest batch in flight.  Past the last tile the loads repeat the
// last tile into a stage no later iteration reads.  The producer reads a
// tile's row meta before its MFMAs and decides afterwards whether the group
// sees the tile.
//
// Exchange-tile columns are keys in the producer's register order: column
// 16*hi + r holds key 8*(r/4) + 4*hi + (r%4), so a producer lane writes its
// 16 values of one row as 32 contiguous bytes and the consumer's output
// column c belongs to key kmap(c).  Rows have a stride of 40 elements, which
// keeps the producer's 16-lane write phases free of bank conflicts and lets
// two sets of exchange tiles fit beside the ring.
// ---------------------------------------------------------------------------
namespace bwdkv {
constexpr int NW = 8;          // waves per workgroup
constexpr int KB = 128;        // keys per workgroup (4 key groups of 32)
constexpr int TR = 32;         // query rows per tile
constexpr int NST = 4;         // ring stages
constexpr int XS = 40;         // row stride (elements) of an exchange tile
constexpr int MS = 64;         // stride (entries) of one meta array in a stage
constexpr float kSplitP = 1.f / 256.f;
__device__ __forceinline__ int kmap(int c) { return 8 * ((c & 15) >> 2) + 4 * (c >> 4) + (c & 3); }
}  // namespace bwdkv

// s_waitcnt immediate: vmcnt(n) (n <= 15) and lgkmcnt(0)
template <int n>
constexpr int wait_vm_lgkm() {
  static_assert(n >= 0 && n <= 15, "vmcnt immediate");
  return 0x0070 | n;
}

template <int D, int G>
__global__ __launch_bounds__(512, 1) void main_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int nq, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ k_seq,
    const int32_t* __restrict__ k_pos, int nk, int hq, int hkv, float scale,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv) {
  using namespace bwdkv;
  constexpr int TPT = TR / G;                  // tokens per tile
  constexpr int KS = D / 16;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int TS = TR * D;                   // elements of one tensor tile
  constexpr int CROUNDS = 2 * TR * CPR / 256;  // 16-byte load rounds per consumer wave per tile (Q and dO)
  constexpr int XT = TR * XS;                  // elements of one exchange tile
  static_assert(TPT >= 1, "at most 32 q-heads per kv-head");

  __shared__ __attribute__((aligned(16))) uint16_t R[NST][2 * TS];   // Q | dO, rows x d, swizzled
  __shared__ __attribute__((aligned(16))) uint32_t Mr[NST][4 * MS];  // lse | delta | seq | pos
  __shared__ __attribute__((aligned(16))) uint16_t X[2][4][4][XT];  // [tile parity][group][P, dS, P lo, dS lo]
  __shared__ __attribute__((aligned(16))) int kseq_s[KB];
  __shared__ __attribute__((aligned(16))) int kpos_s[KB];
  __shared__ int Xf[2][4];   // per tile parity and group: 0 nothing visible, 1 hi only, 2 hi + lo

  const float scale_log2 = scale * kLog2e;
  const int nblk = (nk + KB - 1) / KB;
  const int L = xcd_remap(blockIdx.x, nblk * hkv);
  const int g = L / nblk;
  const int kblk = L % nblk;             // early keys are seen by the most rows: heavy first
  const int key0 = kblk * KB;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int team = wave >> 2, kg = wave & 3;
  const int n = lane & 31, hi = lane >> 5;
  const LaneOffsets<D> lo_off(lane);
  const int wk0 = key0 + 32 * kg;        // first key of the group

  if (tid < KB) {
    const bool ok = key0 + tid < nk;
    kseq_s[tid] = ok ? k_seq[key0 + tid] : INT_MIN;
    kpos_s[tid] = ok ? k_pos[key0 + tid] : INT_MAX;
  }

  // query tokens that can see any key of the block; tile i covers tokens
  // [qhi - (i+1)*TPT, qhi - i*TPT) clipped at qlo
  const int klast = min(nk, key0 + KB) - 1;
  const int qlo = __builtin_amdgcn_readfirstlane(
      lower_bound_sp(q_seq, q_pos, nq, k_seq[key0], k_pos[key0]));
  const int qhi = __builtin_amdgcn_readfirstlane(
      upper_bound_sp(q_seq, q_pos, nq, k_seq[klast], INT_MAX));
  const int ntiles = qhi > qlo ? (qhi - qlo + TPT - 1) / TPT : 0;
  auto tile_t0 = [&](int i) { return max(qlo, qhi - (i + 1) * TPT); };

  // ---- loads of tile i into stage st, by the consumer waves --------------
  // Lane l of round `it` of consumer wave w (w = wave % 4) fills 16-byte slot
  // (it*4 + w)*64 + l of the stage (Q then dO), i.e. physical chunk p of row r
  // of one tensor; it fetches logical chunk swz(r, p) (the swizzle is an
  // involution).  Rows past the tile's end (only in the tile at the start of
  // the range) re-read its last row; they are masked by index.  Each consumer
  // wave also loads one meta array (lse, Delta, seq, pos; lanes 32-63 fill
  // padding).  CROUNDS + 1 loads per wave and tile.
  uint32_t lane_off[CROUNDS];   // bytes from the tile's first token, row 0 head 0
  int lane_tok[CROUNDS];        // token offset of the lane's row
#pragma unroll
  for (int it = 0; it < CROUNDS; ++it) {
    const int slot = (it * 4 + kg) * 64 + lane;
    const int s2 = slot % (TR * CPR);
    const int r = s2 / CPR, p = s2 % CPR;
    lane_tok[it] = r / G;
    lane_off[it] = 2u * static_cast<uint32_t>(((r / G) * hq + g * G + r % G) * D + 8 * swz<D>(r, p));
  }
  const char* const meta_src = reinterpret_cast<const char*>(
      kg == 0 ? static_cast<const void*>(lse)
    : kg == 1 ? static_cast<const void*>(delta)
    : kg == 2 ? static_cast<const void*>(q_seq)
              : static_cast<const void*>(q_pos));
  // load number j (0 .. CROUNDS) of tile i into stage st
  auto issue_one = [&](int st, int i, int j) {
    const int t0 = tile_t0(i);
    const int tmax = qhi - i * TPT - 1 - t0;   // last token offset of the tile
    if (j < CROUNDS) {
      const int tensor = ((j * 4 + kg) * 64) / (TR * CPR);   // wave-uniform
      const char* src = reinterpret_cast<const char*>(tensor == 0 ? q : dout) +
                        static_cast<size_t>(t0) * hq * D * 2;
      const int dt = min(lane_tok[j], tmax) - lane_tok[j];
      const uint32_t off = lane_off[j] + static_cast<uint32_t>(dt * hq * D * 2);
      dma_b128(src, off, lds_addr(&R[st][(j * 4 + kg) * 64 * 8]));
    } else {
      const int r = min(lane, TR - 1);
      const int tok = min(r / G, tmax);
      // lse / Delta are [hq, nq]: a 64-bit element index, since (head * nq)
      // exceeds 32 bits of bytes once hq * nq reaches 2^30
      const size_t idx = static_cast<size_t>(t0 + tok) +
                         (kg < 2 ? static_cast<size_t>(g * G + r % G) * nq : 0);
      dma_b32_at(meta_src + 4 * idx, lds_addr(&Mr[st][kg * MS]));
    }
  };
  auto issue = [&](int st, int i) {
#pragma unroll
    for (int j = 0; j <= CROUNDS; ++j) issue_one(st, i, j);
  };

  if (ntiles > 0 && team == 1) {
    issue(0, 0);
    issue(1, min(1, ntiles - 1));
  }
  wg_barrier<kWaitAll>();   // also publishes the key meta

  if (team == 0) {
    // ======================= producer: S, dP, P, dS =========================
    const int wkl = min(nk, wk0 + 32) - 1;
    const bool wave_valid = wk0 < nk;
    const bool wave_complete = wk0 + 32 <= nk;
    const int kf_seq = __builtin_amdgcn_readfirstlane(wave_valid ? kseq_s[32 * kg] : 0);
    const int kf_pos = __builtin_amdgcn_readfirstlane(wave_valid ? kpos_s[32 * kg] : 0);
    const int kl_seq = __builtin_amdgcn_readfirstlane(wave_valid ? kseq_s[wkl - key0] : 0);
    const int kl_pos = __builtin_amdgcn_readfirstlane(wave_valid ? kpos_s[wkl - key0] : 0);
    // K and V rows of the lane's key as MFMA A operands (k-elements 16*ks + 8*hi ..)
    bf16x8 kreg[KS], vreg[KS];
    {
      const bool key_valid = wk0 + n < nk;
      const size_t kb = (static_cast<size_t>(key_valid ? wk0 + n : 0) * hkv + g) * D + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kreg[ks] = key_valid ? *reinterpret_cast<const bf16x8*>(k + kb + 16 * ks) : zero8();
        vreg[ks] = key_valid ? *reinterpret_cast<const bf16x8*>(v + kb + 16 * ks) : zero8();
      }
    }
    f32x16 sacc = zero16(), dpacc = zero16();
    for (int i = 0; i < ntiles; ++i) {
      // tile i landed (the consumers waited for their loads of it)
      if (i > 0) wg_barrier<kWaitLgkm>();
      const int st = i % NST;
      int nrows = 0, fs = 0, fp = 0, ls = 0, lp = 0;
      float lse_n = 0.f, dl = 0.f;
      int rseq = 0, rpos = 0;
      if (i < ntiles) {
        // this tile's row meta: read now, used after the MFMAs
        const int t0 = tile_t0(i);
        nrows = (qhi - i * TPT - t0) * G;
        const int* rseq_s = reinterpret_cast<const int*>(&Mr[st][2 * MS]);
        const int* rpos_s = reinterpret_cast<const int*>(&Mr[st][3 * MS]);
        lse_n = reinterpret_cast<const float*>(&Mr[st][0])[n];
        dl = reinterpret_cast<const float*>(&Mr[st][MS])[n];
        rseq = rseq_s[n];
        rpos = rpos_s[n];
        // S^T = K Q^T and dP^T = V dO^T, alternating, B operands (one query
        // row per lane) loaded kPre MFMAs ahead: lane (n, hi) register r
        // holds key 8*(r/4) + 4*hi + (r%4) of row n.  Computed for every
        // tile; used only if the group sees some of its rows.
        const uint16_t* cur = R[st];
        constexpr int kPre = 6;   // operands read ahead (6 and 8 measured alike, 12 slower)
        bf16x8 opnd[kPre];
        auto load = [&](int j) { return row_operand<D>(cur + (j & 1) * TS, lo_off, 0, j >> 1); };
#pragma unroll
        for (int j = 0; j < kPre; ++j) opnd[j] = load(j);
#pragma unroll
        for (int j = 0; j < 2 * KS; ++j) {
          const int ks = j >> 1;
          if (j == 0) sacc = mfma32(kreg[0], opnd[0], zero16());
          else if (j == 1) dpacc = mfma32(vreg[0], opnd[1], zero16());
          else if ((j & 1) == 0) sacc = mfma32(kreg[ks], opnd[j % kPre], sacc);
          else dpacc = mfma32(vreg[ks], opnd[j % kPre], dpacc);
          if (j + kPre < 2 * KS) opnd[j % kPre] = load(j + kPre);
        }
        // pin the order: the 4 meta reads and the first kPre operands, then
        // one MFMA and the next operand
        __builtin_amdgcn_sched_group_barrier(0x100, 4 + kPre, 0);
#pragma unroll
        for (int j = 0; j < 2 * KS - kPre; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kPre, 0);
        keep(sacc);
        keep(dpacc);
      }
      // the tile's first and last rows, from the lanes that hold them
      if (i < ntiles) {
        fs = __builtin_amdgcn_readlane(rseq, 0);
        fp = __builtin_amdgcn_readlane(rpos, 0);
        ls = __builtin_amdgcn_readlane(rseq, nrows - 1);
        lp = __builtin_amdgcn_readlane(rpos, nrows - 1);
      }
      const bool active = i < ntiles && wave_valid && !lex_less(ls, lp, kf_seq, kf_pos) &&
                          !lex_less(kl_seq, INT_MAX, fs, fp);
      const bool full = wave_complete && nrows == TR && fs == ls && fs == kf_seq && kf_seq == kl_seq &&
                        fp >= kl_pos;
      // softmax gradient of tile i -> exchange tiles of the group (parity i)
      int flag = 0;
      if (active) {
        const float lse2 = lse_n * kLog2e;
        float p[16], ds[16];
        if (full) {
          // three phases, kept apart: the exponent arguments, then the
          // exponentials beside the dP - Delta subtractions (the
          // transcendental unit runs beside the other vector instructions),
          // then the products (1-2.5% less dK/dV time at 256K than one loop
          // per element)
          float x[16], dd[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = fmaf(sacc[r], scale_log2, -lse2);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = exp2_fast(x[r]);
            dd[r] = dpacc[r] - dl;
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < 16; ++r) ds[r] = p[r] * dd[r];
        } else {
          const bool row_ok = n < nrows && lse2 != kNegInf;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int kk = 32 * kg + 8 * r4 + 4 * hi;
            const int4 ss = *reinterpret_cast<const int4*>(&kseq_s[kk]);
            const int4 pp = *reinterpret_cast<const int4*>(&kpos_s[kk]);
            const int sv[4] = {ss.x, ss.y, ss.z, ss.w};
            const int pv[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * r4 + e;
              const bool vis = row_ok & (sv[e] == rseq) & (pv[e] <= rpos);
              const float pr = vis ? exp2_fast(fmaf(sacc[r], scale_log2, -lse2)) : 0.f;
              p[r] = pr;
              ds[r] = pr * (dpacc[r] - dl);
            }
          }
        }
        // P and dS enter the gradient MFMAs as bf16.  Where some P of the
        // tile reaches kSplitP they enter as hi + lo bf16 pairs (lo = x - hi,
        // a second MFMA on the same A operand): rows that give a key a large
        // weight would otherwise carry bf16's 2^-9 relative rounding into the
        // key's gradient with a large coefficient.  Below the threshold the
        // dropped lo terms are at most kSplitP * 2^-9 each.
        uint16_t* xrow = &X[i & 1][kg][0][n * XS + 16 * hi];
        bf16x8 ph[2], dh[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          ph[s2] = pack8(&p[8 * s2]);
          dh[s2] = pack8(&ds[8 * s2]);
          *reinterpret_cast<bf16x8*>(xrow + 8 * s2) = ph[s2];
          *reinterpret_cast<bf16x8*>(xrow + XT + 8 * s2) = dh[s2];
        }
        f32x16 pv;
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = p[r];
        const bool split = __any(max16_raw(0.f, pv) >= kSplitP);
        flag = split ? 2 : 1;
        if (split) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            float pl[8], dl8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              pl[j] = p[8 * s2 + j] - static_cast<float>(ph[s2][j]);
              dl8[j] = ds[8 * s2 + j] - static_cast<float>(dh[s2][j]);
            }
            *reinterpret_cast<bf16x8*>(xrow + 2 * XT + 8 * s2) = pack8(pl);
            *reinterpret_cast<bf16x8*>(xrow + 3 * XT + 8 * s2) = pack8(dl8);
          }
        }
      }
      if (lane == 0) Xf[i & 1][kg] = flag;
    }
    // the consumers read the last tile's exchange tiles after this barrier
    if (ntiles > 0) wg_barrier<kWaitLgkm>();
    // every load of this workgroup has landed before its LDS is released
    wg_barrier<kWaitAll>();
  } else {
    // ======================= consumer: dV, dK ===============================
    // Consumer c serves key groups cg0 and cg0+1 over the d-blocks mb0 ..
    // mb0+MH-1, so that each transposed Q / dO operand it reads feeds two
    // MFMAs (one per key group).
    constexpr int MH = MB / 2;              // d-blocks per consumer
    const int cg0 = 2 * (kg >> 1);          // first key group
    const int mb0 = MH * (kg & 1);          // first d-block
    // transposed-read offsets of this consumer's d-blocks (selected, not
    // indexed, so that they stay in registers)
    int tro[MH][2];
#pragma unroll
    for (int mh = 0; mh < MH; ++mh)
#pragma unroll
      for (int e = 0; e < 2; ++e) tro[mh][e] = (kg & 1) ? lo_off.tr[MH + mh][e] : lo_off.tr[mh][e];
    f32x16 acc_v[2][MH], acc_k[2][MH];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int mb = 0; mb < MH; ++mb) {
        acc_v[gg][mb] = zero16();
        acc_k[gg][mb] = zero16();
      }
    // transposing reads of an exchange tile (one 32-column block)
    const int xg = lane >> 4, xi = lane & 15;
    const int xr0 = 4 * (xg >> 1) + (xi >> 2), xc0 = 16 * (xg & 1) + 4 * (xi & 3);
    const int xo0 = xr0 * XS + xc0, xo1 = (xr0 + 8) * XS + xc0;
    for (int i = 0; i <= ntiles; ++i) {
      // tile i landed: only this wave's newest batch (tile i+1) may be in flight
      if (i > 0) wg_barrier<wait_vm_lgkm<CROUNDS + 1>()>();
      // this iteration's loads, tile i+2
      if (i < ntiles) issue((i + 2) % NST, min(i + 2, ntiles - 1));
      // and the exchange tiles of tile i-1 into registers; a group that
      // skips the tile contributes zeros
      int fl[2] = {0, 0};
      bf16x8 pop[2][2], dop[2][2];
      if (i > 0) {
        const int xp = (i - 1) & 1;   // exchange tiles of tile i-1
        fl[0] = __builtin_amdgcn_readfirstlane(Xf[xp][cg0]);
        fl[1] = __builtin_amdgcn_readfirstlane(Xf[xp][cg0 + 1]);
        if (fl[0] + fl[1] > 0) {
#pragma unroll
          for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              pop[gg][s2] = tr_operand_at<XS>(&X[xp][cg0 + gg][0][0], 16 * s2, xo0, xo1);
              dop[gg][s2] = tr_operand_at<XS>(&X[xp][cg0 + gg][1][0], 16 * s2, xo0, xo1);
            }
#pragma unroll
          for (int gg = 0; gg < 2; ++gg)
            if (fl[gg] == 0) {
#pragma unroll
              for (int s2 = 0; s2 < 2; ++s2) {
                pop[gg][s2] = zero8();
                dop[gg][s2] = zero8();
              }
            }
        }
      }
      if (fl[0] + fl[1] == 0) continue;
      // dV^T += dO^T P, dK^T += Q^T dS over the 32 rows of tile i-1 for
      // both groups; A operands (transposed Q / dO, indexed (tensor,
      // k-step, d-block)) loaded kPre operands ahead
      const int xp = (i - 1) & 1;
      const uint16_t* prev = R[(i - 1) % NST];
      constexpr int NA = 4 * MH;   // A operands per tile
      constexpr int kPre = NA < 4 ? NA : 4;
      auto load = [&](int j) {
        const int tsr = j / (2 * MH), s2 = (j / MH) % 2, mh = j % MH;
        return tr_operand_at<D>(prev + (tsr == 0 ? TS : 0), 16 * s2, tro[mh][0], tro[mh][1]);
      };
      bf16x8 opnd[kPre];
#pragma unroll
      for (int j = 0; j < kPre; ++j) opnd[j] = load(j);
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        const int tsr = j / (2 * MH), s2 = (j / MH) % 2, mh = j % MH;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          if (tsr == 0) acc_v[gg][mh] = mfma32(opnd[j % kPre], pop[gg][s2], acc_v[gg][mh]);
          else acc_k[gg][mh] = mfma32(opnd[j % kPre], dop[gg][s2], acc_k[gg][mh]);
        }
        if (j + kPre < NA) opnd[j % kPre] = load(j + kPre);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);
#pragma unroll
      for (int j = 0; j < NA - kPre; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kPre, 0);
      // lo pass of the groups whose P reaches kSplitP somewhere in the tile
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        if (fl[gg] == 2) {
          bf16x8 plo[2], dlo[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            plo[s2] = tr_operand_at<XS>(&X[xp][cg0 + gg][2][0], 16 * s2, xo0, xo1);
            dlo[s2] = tr_operand_at<XS>(&X[xp][cg0 + gg][3][0], 16 * s2, xo0, xo1);
          }
#pragma unroll
          for (int j = 0; j < NA; ++j) {
            const int tsr = j / (2 * MH), s2 = (j / MH) % 2, mh = j % MH;
            const bf16x8 a = load(j);
            if (tsr == 0) acc_v[gg][mh] = mfma32(a, plo[s2], acc_v[gg][mh]);
            else acc_k[gg][mh] = mfma32(a, dlo[s2], acc_k[gg][mh]);
          }
        }
      }
      // the MFMAs stay before the next barrier
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int mh = 0; mh < MH; ++mh) {
          keep(acc_v[gg][mh]);
          keep(acc_k[gg][mh]);
        }
    }
    wg_barrier<kWaitAll>();
    // ---- store: output column n holds key kmap(n) of the group -----------
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int my_key = key0 + 32 * (cg0 + gg) + kmap(n);
      if (my_key < nk) {
        const size_t obase = (static_cast<size_t>(my_key) * hkv + g) * D;
#pragma unroll
        for (int mh = 0; mh < MH; ++mh)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = (mb0 + mh) * 32 + 8 * gq + 4 * hi;
            float4* pv = reinterpret_cast<float4*>(dv + obase + col);
            float4* pk = reinterpret_cast<float4*>(dk + obase + col);
            float4 a = *pv, b = *pk;
            a.x += acc_v[gg][mh][4 * gq + 0];
            a.y += acc_v[gg][mh][4 * gq + 1];
            a.z += acc_v[gg][mh][4 * gq + 2];
            a.w += acc_v[gg][mh][4 * gq + 3];
            b.x += scale * acc_k[gg][mh][4 * gq + 0];
            b.y += scale * acc_k[gg][mh][4 * gq + 1];
            b.z += scale * acc_k[gg][mh][4 * gq + 2];
            b.w += scale * acc_k[gg][mh][4 * gq + 3];
            *pv = a;
            *pk = b;
          }
      }
    }
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
