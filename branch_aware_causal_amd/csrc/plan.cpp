// zigzag_shard_plan: rank r's share of a packed batch under a zigzag ring.
//
// [G] 新颖性 / 核心创新: packed, load-balanced zigzag ring attention; the main
// K/V circulates while branch K/V stays on the anchor's rank.  [R] "两条路，
// 绕开并行训练的堵点": packing and interleaved chunk assignment avoid padding
// and imbalance.  Readings where the pages are silent: chunk bounds
// floor(k*L/(2C)), chunk k -> rank k (k < C) or 2C-1-k, ring step s reads the
// shard of rank (r - s) mod C.

#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../include/bac.h"
#include "abi_internal.hpp"

namespace {

inline int64_t bound(int64_t k, int64_t L, int64_t C) { return (k * L) / (2 * C); }

// Chunk index k in [0, 2C) with bound(k) <= p < bound(k+1), for 0 <= p < L.
inline int64_t chunk_of(int64_t p, int64_t L, int64_t C) {
  int64_t k = (p * 2 * C) / L;
  if (k > 2 * C - 1) k = 2 * C - 1;
  while (k + 1 <= 2 * C - 1 && bound(k + 1, L, C) <= p) ++k;
  while (k > 0 && bound(k, L, C) > p) --k;
  return k;
}

}  // namespace

extern "C" bac_status zigzag_shard_plan(const int32_t* cu_seqlens, int32_t num_seqs,
                                        const int32_t* branch_cu, const int32_t* branch_anchor,
                                        int32_t num_branches, int32_t cp_size, int32_t rank,
                                        bac_plan_sizes* sizes, bac_plan_out* out) {
  bac::clear_error();
  if (!cu_seqlens || !sizes) return bac::fail(BAC_EINVAL, "zigzag_shard_plan: null cu_seqlens or sizes");
  if (num_seqs < 0 || num_branches < 0)
    return bac::fail(BAC_EINVAL, "zigzag_shard_plan: negative num_seqs or num_branches");
  if (num_branches > 0 && (!branch_cu || !branch_anchor))
    return bac::fail(BAC_EINVAL, "zigzag_shard_plan: null branch_cu or branch_anchor");
  if (cp_size < 1 || cp_size > (1 << 20))
    return bac::fail(BAC_EINVAL, "zigzag_shard_plan: cp_size %d outside [1, 2^20]", cp_size);
  if (rank < 0 || rank >= cp_size)
    return bac::fail(BAC_EINVAL, "zigzag_shard_plan: rank %d outside [0, %d)", rank, cp_size);
  if (cu_seqlens[0] != 0) return bac::fail(BAC_EINVAL, "zigzag_shard_plan: cu_seqlens[0] != 0");
  for (int32_t s = 0; s < num_seqs; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s])
      return bac::fail(BAC_EINVAL, "zigzag_shard_plan: cu_seqlens decreases at %d", s);
  const int64_t N = cu_seqlens[num_seqs];
  if (num_branches > 0) {
    if (branch_cu[0] != 0) return bac::fail(BAC_EINVAL, "zigzag_shard_plan: branch_cu[0] != 0");
    for (int32_t a = 0; a < num_branches; ++a) {
      if (branch_cu[a + 1] < branch_cu[a])
        return bac::fail(BAC_EINVAL, "zigzag_shard_plan: branch_cu decreases at %d", a);
      if (branch_anchor[a] < 0 || branch_anchor[a] >= N)
        return bac::fail(BAC_EINVAL, "zigzag_shard_plan: anchor %d of branch %d outside [0, %lld)",
                         branch_anchor[a], a, static_cast<long long>(N));
      if (a > 0 && branch_anchor[a] < branch_anchor[a - 1])
        return bac::fail(BAC_EINVAL, "zigzag_shard_plan: anchors not sorted at branch %d", a);
    }
  }
  const int64_t C = cp_size;
  const int64_t k_lo = rank, k_hi = 2 * C - 1 - rank;   // k_lo < k_hi since rank < C

  // Main tokens.
  int64_t n_main = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = cu_seqlens[s + 1] - cu_seqlens[s];
    n_main += bound(k_lo + 1, L, C) - bound(k_lo, L, C);
    n_main += bound(k_hi + 1, L, C) - bound(k_hi, L, C);
  }
  // Branches owned: the anchor's chunk belongs to this rank.
  std::vector<int32_t> owned;
  int64_t n_btok = 0;
  for (int32_t a = 0; a < num_branches; ++a) {
    const int32_t ag = branch_anchor[a];
    const int32_t* it = std::upper_bound(cu_seqlens, cu_seqlens + num_seqs + 1, ag);
    const int64_t s = (it - cu_seqlens) - 1;
    const int64_t L = cu_seqlens[s + 1] - cu_seqlens[s];
    const int64_t p = ag - cu_seqlens[s];
    const int64_t k = chunk_of(p, L, C);
    const int64_t owner = k < C ? k : 2 * C - 1 - k;
    if (owner == rank) {
      owned.push_back(a);
      n_btok += branch_cu[a + 1] - branch_cu[a];
    }
  }
  if (n_main > INT32_MAX || n_btok > INT32_MAX)
    return bac::fail(BAC_ESIZE, "zigzag_shard_plan: share exceeds int32");
  sizes->n_main = static_cast<int32_t>(n_main);
  sizes->n_branch_tok = static_cast<int32_t>(n_btok);
  sizes->n_branches = static_cast<int32_t>(owned.size());
  if (!out) return BAC_OK;
  if (!out->kv_src || !out->local_branch_cu ||
      (n_main > 0 && (!out->main_index || !out->main_seq || !out->main_pos)) ||
      (!owned.empty() && !out->branch_ids) ||
      (n_btok > 0 && (!out->branch_index || !out->branch_seq || !out->branch_pos || !out->branch_t)))
    return bac::fail(BAC_EINVAL, "zigzag_shard_plan: null output array");

  int64_t w = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = cu_seqlens[s + 1] - cu_seqlens[s];
    for (int64_t kk : {k_lo, k_hi}) {
      for (int64_t p = bound(kk, L, C); p < bound(kk + 1, L, C); ++p, ++w) {
        out->main_index[w] = static_cast<int32_t>(cu_seqlens[s] + p);
        out->main_seq[w] = s;
        out->main_pos[w] = static_cast<int32_t>(p);
      }
    }
  }
  int64_t bt = 0;
  out->local_branch_cu[0] = 0;
  for (size_t i = 0; i < owned.size(); ++i) {
    const int32_t a = owned[i];
    const int32_t ag = branch_anchor[a];
    const int32_t* it = std::upper_bound(cu_seqlens, cu_seqlens + num_seqs + 1, ag);
    const int32_t s = static_cast<int32_t>((it - cu_seqlens) - 1);
    const int32_t p = ag - cu_seqlens[s];
    out->branch_ids[i] = a;
    for (int32_t tok = branch_cu[a]; tok < branch_cu[a + 1]; ++tok, ++bt) {
      out->branch_index[bt] = tok;
      out->branch_seq[bt] = s;
      out->branch_pos[bt] = p;
      out->branch_t[bt] = tok - branch_cu[a];
    }
    out->local_branch_cu[i + 1] = static_cast<int32_t>(bt);
  }
  for (int32_t s = 0; s < cp_size; ++s)
    out->kv_src[s] = static_cast<int32_t>(((rank - s) % cp_size + cp_size) % cp_size);
  return BAC_OK;
}
