// C ABI of libbac: argument validation, error state and kernel dispatch.
// Every entry point validates host-visible arguments before enqueuing any
// device work and reports problems through a status code plus a thread-local
// message; nothing here throws or aborts.

#include <initializer_list>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/bac.h"
#include "abi_internal.hpp"
#include "launch.hpp"

namespace bac {

static thread_local std::string g_error;

void clear_error() { g_error.clear(); }

bac_status fail(bac_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

static bac_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return BAC_OK;
  return fail(BAC_EHIP, "%s: HIP error %d (%s)", where, static_cast<int>(e), hipGetErrorString(e));
}

// fp32 main attention runs on the vector-ALU kernels, bf16 on MFMA.
static bool main_uses_valu(int dt) { return dt == kF32; }

static bac_status check_heads(const char* fn, int32_t hq, int32_t hkv, int32_t d, int32_t dt) {
  if (hq < 1 || hkv < 1) return fail(BAC_EINVAL, "%s: hq=%d hkv=%d must be >= 1", fn, hq, hkv);
  if (hq % hkv != 0) return fail(BAC_EINVAL, "%s: hq=%d is not a multiple of hkv=%d", fn, hq, hkv);
  if (32 % (hq / hkv) != 0)
    return fail(BAC_EUNSUPPORTED, "%s: GQA ratio hq/hkv=%d must divide 32", fn, hq / hkv);
  if (d != 64 && d != 128) return fail(BAC_EUNSUPPORTED, "%s: head dim %d not in {64, 128}", fn, d);
  if (dt != BAC_F32 && dt != BAC_BF16) return fail(BAC_EINVAL, "%s: unknown dtype %d", fn, dt);
  return BAC_OK;
}

static bac_status check_count(const char* fn, const char* what, int32_t n, int32_t heads) {
  if (n < 0) return fail(BAC_EINVAL, "%s: %s=%d is negative", fn, what, n);
  if (static_cast<int64_t>(n) * heads > INT32_MAX)
    return fail(BAC_ESIZE, "%s: %s*heads exceeds 2^31", fn, what);
  return BAC_OK;
}

// Tensors are read and written with 16-byte vector accesses.
static bac_status check_aligned(const char* fn, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15u))
      return fail(BAC_EINVAL, "%s: tensor pointer %p is not 16-byte aligned", fn, p);
  return BAC_OK;
}

// The softmax scale must be finite and positive: the MFMA forward masks a
// score to -inf before scaling and takes the row maximum of unscaled scores.
static bac_status check_scale(const char* fn, float scale) {
  if (!std::isfinite(scale)) return fail(BAC_EINVAL, "%s: scale is not finite", fn);
  if (!(scale > 0.f)) return fail(BAC_EUNSUPPORTED, "%s: scale %g is not positive", fn, scale);
  return BAC_OK;
}

#define BAC_TRY(expr)              \
  do {                             \
    bac_status _st = (expr);       \
    if (_st != BAC_OK) return _st; \
  } while (0)

static bac_status check_main(const char* fn, const void* q, const int32_t* q_seq,
                             const int32_t* q_pos, int32_t nq, const void* k, const void* v,
                             const int32_t* k_seq, const int32_t* k_pos, int32_t nk, int32_t hq,
                             int32_t hkv, int32_t d, int32_t dt, float scale) {
  BAC_TRY(check_heads(fn, hq, hkv, d, dt));
  BAC_TRY(check_count(fn, "nq", nq, hq));
  BAC_TRY(check_count(fn, "nk", nk, hq));
  if (nq > 0 && (!q || !q_seq || !q_pos)) return fail(BAC_EINVAL, "%s: null query array", fn);
  if (nk > 0 && (!k || !v || !k_seq || !k_pos)) return fail(BAC_EINVAL, "%s: null key array", fn);
  BAC_TRY(check_scale(fn, scale));
  return BAC_OK;
}

// Longest branch the branch kernels accept (one wave walks a branch's tokens).
constexpr int32_t kMaxBranchLen = 256;

static bac_status check_branch(const char* fn, const void* qb, const void* kb, const void* vb,
                               int32_t nb, const int32_t* branch_cu, int32_t num_branches,
                               int32_t max_len, int32_t kind, int32_t hq, int32_t hkv, int32_t d,
                               int32_t dt, float scale) {
  BAC_TRY(check_heads(fn, hq, hkv, d, dt));
  BAC_TRY(check_count(fn, "nb", nb, hq));
  if (num_branches < 0) return fail(BAC_EINVAL, "%s: num_branches=%d is negative", fn, num_branches);
  if (num_branches > 0 && !branch_cu) return fail(BAC_EINVAL, "%s: null branch_cu", fn);
  if (nb > 0 && (!qb || !kb || !vb)) return fail(BAC_EINVAL, "%s: null branch tensor", fn);
  if (kind != BAC_BRANCH_CAUSAL && kind != BAC_BRANCH_BIDIR)
    return fail(BAC_EINVAL, "%s: unknown branch kind %d", fn, kind);
  if (max_len < 1 || max_len > kMaxBranchLen)
    return fail(BAC_EUNSUPPORTED, "%s: max_branch_len=%d outside [1, %d]", fn, max_len,
                kMaxBranchLen);
  BAC_TRY(check_scale(fn, scale));
  return BAC_OK;
}

}  // namespace bac

using namespace bac;

extern "C" {

const char* bac_last_error(void) { return g_error.c_str(); }

int32_t bac_version(void) { return 200; }   // 0.2.0: per-branch kinds, tap_send / tap_recv

bac_status attn_main_fwd(const void* q, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                         const void* k, const void* v, const int32_t* k_seq, const int32_t* k_pos,
                         int32_t nk, int32_t hq, int32_t hkv, int32_t d, bac_dtype dt, float scale,
                         float* o_acc, float* lse, bac_acc_mode mode, void* o_out, void* stream) {
  clear_error();
  const char* fn = "attn_main_fwd";
  BAC_TRY(check_main(fn, q, q_seq, q_pos, nq, k, v, k_seq, k_pos, nk, hq, hkv, d, dt, scale));
  if (mode != BAC_WRITE && mode != BAC_MERGE) return fail(BAC_EINVAL, "%s: unknown mode %d", fn, mode);
  if (nq > 0 && (!o_acc || !lse)) return fail(BAC_EINVAL, "%s: null o_acc or lse", fn);
  if (nq == 0) return BAC_OK;
  BAC_TRY(check_aligned(fn, {q, k, v, o_acc, o_out}));
  MainArgs a{};
  a.q = q; a.q_seq = q_seq; a.q_pos = q_pos; a.nq = nq;
  a.k = k; a.v = v; a.k_seq = k_seq; a.k_pos = k_pos; a.nk = nk;
  a.hq = hq; a.hkv = hkv; a.d = d; a.dt = dt; a.scale = scale;
  a.o_acc = o_acc; a.lse_acc = lse; a.mode = mode; a.o_out = o_out;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = main_uses_valu(dt) ? launch_main_fwd_valu(a) : launch_main_fwd_mfma(a);
  return hip_status(e, fn);
}

bac_status attn_branch_fwd(const void* qb, const void* kb, const void* vb, int32_t nb,
                           const int32_t* branch_cu, int32_t num_branches, int32_t max_branch_len,
                           bac_branch_kind kind, const int32_t* branch_kinds, int32_t hq,
                           int32_t hkv, int32_t d, bac_dtype dt, float scale, float* o_acc,
                           float* lse, bac_acc_mode mode, void* o_out, void* stream) {
  clear_error();
  const char* fn = "attn_branch_fwd";
  BAC_TRY(check_branch(fn, qb, kb, vb, nb, branch_cu, num_branches, max_branch_len, kind, hq, hkv,
                       d, dt, scale));
  if (mode != BAC_WRITE && mode != BAC_MERGE) return fail(BAC_EINVAL, "%s: unknown mode %d", fn, mode);
  if (nb > 0 && (!o_acc || !lse)) return fail(BAC_EINVAL, "%s: null o_acc or lse", fn);
  if (nb == 0 || num_branches == 0) return BAC_OK;
  BAC_TRY(check_aligned(fn, {qb, kb, vb, o_acc, o_out}));
  BranchArgs a{};
  a.qb = qb; a.kb = kb; a.vb = vb; a.nb = nb;
  a.branch_cu = branch_cu; a.num_branches = num_branches; a.max_len = max_branch_len;
  a.bidir = kind == BAC_BRANCH_BIDIR;
  a.kinds = branch_kinds;
  a.hq = hq; a.hkv = hkv; a.d = d; a.dt = dt; a.scale = scale;
  a.o_acc = o_acc; a.lse_acc = lse; a.mode = mode; a.o_out = o_out;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_branch_fwd(a), fn);
}

bac_status lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                     int32_t n, int32_t hq, int32_t d, bac_dtype out_dt, void* o_out,
                     void* stream) {
  clear_error();
  const char* fn = "lse_merge";
  if (hq < 1) return fail(BAC_EINVAL, "%s: hq=%d must be >= 1", fn, hq);
  if (d != 64 && d != 128) return fail(BAC_EUNSUPPORTED, "%s: head dim %d not in {64, 128}", fn, d);
  BAC_TRY(check_count(fn, "n", n, hq));
  if (out_dt != BAC_F32 && out_dt != BAC_BF16) return fail(BAC_EINVAL, "%s: unknown dtype", fn);
  if (n > 0 && (!o_acc || !lse_acc || !o_part || !lse_part))
    return fail(BAC_EINVAL, "%s: null accumulator or part", fn);
  if (n > 0 && o_acc == o_part) return fail(BAC_EINVAL, "%s: o_part aliases o_acc", fn);
  if (n == 0) return BAC_OK;
  BAC_TRY(check_aligned(fn, {o_acc, o_part, o_out}));
  return hip_status(launch_lse_merge(o_acc, lse_acc, o_part, lse_part, n, hq, d, out_dt, o_out,
                                     static_cast<hipStream_t>(stream)),
                    fn);
}

bac_status attn_bwd_delta(const void* o, bac_dtype o_dt, const void* dout, bac_dtype dt, int32_t n,
                          int32_t hq, int32_t d, float* delta, void* stream) {
  clear_error();
  const char* fn = "attn_bwd_delta";
  if (hq < 1) return fail(BAC_EINVAL, "%s: hq=%d must be >= 1", fn, hq);
  if (d != 64 && d != 128) return fail(BAC_EUNSUPPORTED, "%s: head dim %d not in {64, 128}", fn, d);
  BAC_TRY(check_count(fn, "n", n, hq));
  if ((o_dt != BAC_F32 && o_dt != BAC_BF16) || (dt != BAC_F32 && dt != BAC_BF16))
    return fail(BAC_EINVAL, "%s: unknown dtype", fn);
  if (n > 0 && (!o || !dout || !delta)) return fail(BAC_EINVAL, "%s: null pointer", fn);
  if (n == 0) return BAC_OK;
  BAC_TRY(check_aligned(fn, {o, dout}));
  return hip_status(launch_delta(o, o_dt, dout, dt, n, hq, d, delta, static_cast<hipStream_t>(stream)),
                    fn);
}

// part: 0 = whole backward, 1 = dq only, 2 = dk/dv only.
static bac_status main_bwd_impl(const char* fn, int part, const void* q, const int32_t* q_seq,
                                const int32_t* q_pos, int32_t nq, const void* k, const void* v,
                                const int32_t* k_seq, const int32_t* k_pos, int32_t nk, int32_t hq,
                                int32_t hkv, int32_t d, int32_t dt, float scale, const void* dout,
                                const float* lse, const float* delta, float* dq_acc, float* dk_acc,
                                float* dv_acc, void* stream) {
  BAC_TRY(check_main(fn, q, q_seq, q_pos, nq, k, v, k_seq, k_pos, nk, hq, hkv, d, dt, scale));
  if (nq > 0 && (!dout || !lse || !delta))
    return fail(BAC_EINVAL, "%s: null dout, lse or delta", fn);
  if (nq > 0 && part != 2 && !dq_acc) return fail(BAC_EINVAL, "%s: null dq_acc", fn);
  if (nk > 0 && part != 1 && (!dk_acc || !dv_acc))
    return fail(BAC_EINVAL, "%s: null dk_acc or dv_acc", fn);
  if (nq == 0 || nk == 0) return BAC_OK;
  BAC_TRY(check_aligned(fn, {q, k, v, dout, dq_acc, dk_acc, dv_acc}));
  MainArgs a{};
  a.q = q; a.q_seq = q_seq; a.q_pos = q_pos; a.nq = nq;
  a.k = k; a.v = v; a.k_seq = k_seq; a.k_pos = k_pos; a.nk = nk;
  a.hq = hq; a.hkv = hkv; a.d = d; a.dt = dt; a.scale = scale;
  a.dout = dout; a.lse = lse; a.delta = delta; a.dq = dq_acc; a.dk = dk_acc; a.dv = dv_acc;
  a.stream = static_cast<hipStream_t>(stream);
  hipError_t e = main_uses_valu(dt) ? launch_main_bwd_valu(a, part) : launch_main_bwd_mfma(a, part);
  return hip_status(e, fn);
}

bac_status attn_main_bwd(const void* q, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                         const void* k, const void* v, const int32_t* k_seq, const int32_t* k_pos,
                         int32_t nk, int32_t hq, int32_t hkv, int32_t d, bac_dtype dt, float scale,
                         const void* dout, const float* lse, const float* delta, float* dq_acc,
                         float* dk_acc, float* dv_acc, void* stream) {
  clear_error();
  return main_bwd_impl("attn_main_bwd", 0, q, q_seq, q_pos, nq, k, v, k_seq, k_pos, nk, hq, hkv,
                       d, dt, scale, dout, lse, delta, dq_acc, dk_acc, dv_acc, stream);
}

bac_status attn_main_bwd_dq(const void* q, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                            const void* k, const void* v, const int32_t* k_seq,
                            const int32_t* k_pos, int32_t nk, int32_t hq, int32_t hkv, int32_t d,
                            bac_dtype dt, float scale, const void* dout, const float* lse,
                            const float* delta, float* dq_acc, void* stream) {
  clear_error();
  return main_bwd_impl("attn_main_bwd_dq", 1, q, q_seq, q_pos, nq, k, v, k_seq, k_pos, nk, hq,
                       hkv, d, dt, scale, dout, lse, delta, dq_acc, nullptr, nullptr, stream);
}

bac_status attn_main_bwd_dkdv(const void* q, const int32_t* q_seq, const int32_t* q_pos,
                              int32_t nq, const void* k, const void* v, const int32_t* k_seq,
                              const int32_t* k_pos, int32_t nk, int32_t hq, int32_t hkv, int32_t d,
                              bac_dtype dt, float scale, const void* dout, const float* lse,
                              const float* delta, float* dk_acc, float* dv_acc, void* stream) {
  clear_error();
  return main_bwd_impl("attn_main_bwd_dkdv", 2, q, q_seq, q_pos, nq, k, v, k_seq, k_pos, nk, hq,
                       hkv, d, dt, scale, dout, lse, delta, nullptr, dk_acc, dv_acc, stream);
}

bac_status attn_branch_bwd(const void* qb, const void* kb, const void* vb, int32_t nb,
                           const int32_t* branch_cu, int32_t num_branches, int32_t max_branch_len,
                           bac_branch_kind kind, const int32_t* branch_kinds, int32_t hq,
                           int32_t hkv, int32_t d, bac_dtype dt, float scale, const void* doutb,
                           const float* lseb, const float* deltab, float* dqb_acc,
                           float* dkb_acc, float* dvb_acc, void* stream) {
  clear_error();
  const char* fn = "attn_branch_bwd";
  BAC_TRY(check_branch(fn, qb, kb, vb, nb, branch_cu, num_branches, max_branch_len, kind, hq, hkv,
                       d, dt, scale));
  if (nb > 0 && (!doutb || !lseb || !deltab || !dqb_acc || !dkb_acc || !dvb_acc))
    return fail(BAC_EINVAL, "%s: null gradient argument", fn);
  if (nb == 0 || num_branches == 0) return BAC_OK;
  BAC_TRY(check_aligned(fn, {qb, kb, vb, doutb, dqb_acc, dkb_acc, dvb_acc}));
  BranchArgs a{};
  a.qb = qb; a.kb = kb; a.vb = vb; a.nb = nb;
  a.branch_cu = branch_cu; a.num_branches = num_branches; a.max_len = max_branch_len;
  a.bidir = kind == BAC_BRANCH_BIDIR;
  a.kinds = branch_kinds;
  a.hq = hq; a.hkv = hkv; a.d = d; a.dt = dt; a.scale = scale;
  a.dout = doutb; a.lse = lseb; a.delta = deltab; a.dq = dqb_acc; a.dk = dkb_acc; a.dv = dvb_acc;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_branch_bwd(a), fn);
}

bac_status attn_check_index(const int32_t* seq, const int32_t* pos, int32_t n, int32_t strict,
                            int32_t* bad_count, void* stream) {
  clear_error();
  const char* fn = "attn_check_index";
  if (n < 0) return fail(BAC_EINVAL, "%s: n=%d is negative", fn, n);
  if (!bad_count || (n > 0 && (!seq || !pos))) return fail(BAC_EINVAL, "%s: null pointer", fn);
  return hip_status(launch_check_index(seq, pos, n, strict ? 1 : 0, bad_count,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

static bac_status check_mailbox(const char* fn, const void* slots, const void* stamps,
                                int32_t nslots, int64_t slot_bytes, int32_t slot, int64_t nbytes,
                                uint64_t seq, const void* buf) {
  if (!slots || !stamps || (nbytes > 0 && !buf))
    return fail(BAC_EINVAL, "%s: null slots, stamps or buffer", fn);
  if (nslots < 1 || slot < 0 || slot >= nslots)
    return fail(BAC_EINVAL, "%s: slot %d outside [0, %d)", fn, slot, nslots);
  if (slot_bytes < 16 || slot_bytes % 16 != 0)
    return fail(BAC_EINVAL, "%s: slot_bytes %lld is not a positive multiple of 16", fn,
                static_cast<long long>(slot_bytes));
  if (nbytes < 0 || nbytes > slot_bytes)
    return fail(BAC_EINVAL, "%s: nbytes %lld outside [0, slot_bytes]", fn,
                static_cast<long long>(nbytes));
  if (seq == 0) return fail(BAC_EINVAL, "%s: sequence numbers start at 1", fn);
  BAC_TRY(check_aligned(fn, {slots, buf}));
  if (reinterpret_cast<uintptr_t>(stamps) & 7u)
    return fail(BAC_EINVAL, "%s: stamps are not 8-byte aligned", fn);
  return BAC_OK;
}

bac_status tap_send(void* slots, uint64_t* stamps, int32_t nslots, int64_t slot_bytes,
                    int32_t slot, const void* payload, int64_t nbytes, uint64_t seq,
                    void* stream) {
  clear_error();
  const char* fn = "tap_send";
  BAC_TRY(check_mailbox(fn, slots, stamps, nslots, slot_bytes, slot, nbytes, seq, payload));
  char* dst = static_cast<char*>(slots) + static_cast<int64_t>(slot) * slot_bytes;
  return hip_status(launch_tap_send(dst, stamps, slot, payload, nbytes, seq,
                                    static_cast<hipStream_t>(stream)),
                    fn);
}

bac_status tap_recv(const void* slots, const uint64_t* stamps, int32_t nslots,
                    int64_t slot_bytes, int32_t slot, uint64_t seq, int64_t spin_limit,
                    void* out, int64_t nbytes, int32_t* status, void* stream) {
  clear_error();
  const char* fn = "tap_recv";
  BAC_TRY(check_mailbox(fn, slots, stamps, nslots, slot_bytes, slot, nbytes, seq, out));
  if (!status) return fail(BAC_EINVAL, "%s: null status", fn);
  if (spin_limit < 1) return fail(BAC_EINVAL, "%s: spin_limit %lld < 1", fn,
                                  static_cast<long long>(spin_limit));
  const char* src = static_cast<const char*>(slots) + static_cast<int64_t>(slot) * slot_bytes;
  return hip_status(launch_tap_recv(src, stamps, slot, seq, spin_limit, out, nbytes, status,
                                    static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
