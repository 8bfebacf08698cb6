/*
 * bac.h -- C ABI of libbac, branch-aware causal attention for gfx950.
 *
 * The method (page keys: [G] gptget.net summary of report 2609.07108,
 * [R] rebasdaily.com article on it): a draft model's branch query attends to
 * the causal main sequence up to its anchor and to its own rank-local branch
 * keys; the two parts are computed separately and combined with the
 * online-softmax merge  l = ln(e^lm + e^lb),  O = e^(lm-l) Om + e^(lb-l) Ob
 * ([G] 技术贡献; 方法详解 · CP计算).  Under context parallelism the main K/V
 * makes C ring steps over a packed, load-balanced zigzag sharding while the
 * branch queries and branch K/V stay on the anchor's rank ([G] 核心创新;
 * [R] "两条路，绕开并行训练的堵点").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Status:    every call returns bac_status; 0 is success, a negative value an
 *            error.  No call throws, aborts or prints.  bac_last_error()
 *            returns a message for the last failing call on the calling
 *            thread (valid until that thread's next bac_* call).
 * Ownership: every buffer belongs to the caller; the library allocates
 *            nothing and keeps no pointer after returning.
 * Memory:    "device" pointers are HIP device memory; "host" pointers are
 *            ordinary host memory.  Index arrays are int32.  Tensor pointers
 *            (q, k, v, dout, o_out and the fp32 o / dq / dk / dv buffers)
 *            must be 16-byte aligned (BAC_EINVAL otherwise); index and lse
 *            arrays need only their element alignment.
 * Streams:   `stream` is a hipStream_t (NULL = the null stream).  Device work
 *            is enqueued on it and the call returns without synchronising.
 * Layouts:   packed token-major ("THD"): queries [n, hq, d], keys/values
 *            [n, hkv, d], outputs o [n, hq, d]; log-sum-exp values are fp32
 *            head-major [hq, n] in natural-log units.  Q-head h uses kv-head
 *            h / (hq / hkv).
 * Types:     bac_dtype selects the element type of q, k, v, dout and o_out
 *            (fp32 or bf16).  Accumulators (o_acc, lse, dq/dk/dv) are fp32.
 * Limits:    d in {64, 128}; hq % hkv == 0 and hq / hkv divides 32;
 *            n * hq < 2^31 for every row count n (BAC_ESIZE otherwise).
 * Scale:     the softmax scale of the attention calls is finite and
 *            positive; 0 or a negative scale is BAC_EUNSUPPORTED, a
 *            non-finite one BAC_EINVAL.
 * Checks:    host-side arguments are validated before anything is enqueued
 *            (BAC_EINVAL / BAC_EUNSUPPORTED, nothing launched).  The contents
 *            of device index arrays are preconditions; attn_check_index()
 *            validates them on the device.  Kernels stay in bounds whatever
 *            those arrays hold.
 */
#ifndef BAC_H
#define BAC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bac_status;
#define BAC_OK 0
#define BAC_EINVAL (-1)        /* invalid argument (null pointer, bad size, bad enum)   */
#define BAC_EUNSUPPORTED (-2)  /* valid but not implemented (head dim, GQA ratio, ...)  */
#define BAC_ESIZE (-3)         /* caller buffer too small / size overflow               */
#define BAC_EHIP (-4)          /* HIP runtime error; message holds hipGetErrorString   */

typedef enum { BAC_F32 = 0, BAC_BF16 = 1 } bac_dtype;

/* Branch pattern inside a branch ([G] 深度分析 · 研究背景):
 * CAUSAL: token t sees branch tokens 0..t (EAGLE-3 test-time-training chains,
 *         DSpark Markov-head blocks);
 * BIDIR:  every token sees the whole branch (DFlash block diffusion). */
typedef enum { BAC_BRANCH_CAUSAL = 0, BAC_BRANCH_BIDIR = 1 } bac_branch_kind;

/* WRITE overwrites (o_acc, lse) with this call's partial result;
 * MERGE combines it into the existing (o_acc, lse) with the online-softmax
 * merge.  An empty partial is (O = 0, lse = -inf), the merge's identity. */
typedef enum { BAC_WRITE = 0, BAC_MERGE = 1 } bac_acc_mode;

const char* bac_last_error(void);
int32_t bac_version(void);             /* major*10000 + minor*100 + patch */

/* ------------------------------------------------------------------------
 * zigzag_shard_plan -- rank r's share of a packed batch under a zigzag ring
 * of C ranks ([G] 新颖性, 核心创新; [R] "两条路，绕开并行训练的堵点").
 * Host function, integer only, deterministic.
 *
 * Sequence s of length L (from cu_seqlens) is cut into 2C chunks at
 * floor(k*L/(2C)), k = 0..2C (no padding); chunk k belongs to rank k when
 * k < C and to rank 2C-1-k otherwise.  A branch belongs to the rank owning its
 * anchor position.  Ring step s on rank r uses the main K/V shard of rank
 * (r - s) mod C.
 *
 * Inputs (host): cu_seqlens [num_seqs+1] (cu[0] = 0, non-decreasing);
 *   branch_cu [num_branches+1] (branch token offsets, non-decreasing,
 *   branch_cu[0] = 0); branch_anchor [num_branches] (global main index of each
 *   anchor, branches sorted by anchor).
 * Two-phase: with out == NULL only *sizes is filled.  Otherwise every pointer
 * of *out must hold at least the sizes reported (kv_src: cp_size entries;
 * local_branch_cu: n_branches+1).
 * Outputs (host, caller-owned):
 *   main_index/main_seq/main_pos [n_main]: owned main tokens, (seq, pos) order;
 *   branch_ids [n_branches]: owned branches, global order;
 *   branch_index [n_branch_tok]: their tokens (global branch-token index);
 *   branch_seq / branch_pos [n_branch_tok]: the anchor's sequence and position
 *     (the position a branch row takes in the main attention);
 *   branch_t [n_branch_tok]: index of the token inside its branch;
 *   local_branch_cu [n_branches+1]: offsets into the rank-local branch tokens;
 *   kv_src [cp_size].
 * Errors: BAC_EINVAL for null inputs, cp_size < 1, rank outside [0, C),
 *   malformed offsets, anchors out of range or not sorted.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_main;
  int32_t n_branch_tok;
  int32_t n_branches;
} bac_plan_sizes;

typedef struct {
  int32_t* main_index;
  int32_t* main_seq;
  int32_t* main_pos;
  int32_t* branch_ids;
  int32_t* branch_index;
  int32_t* branch_seq;
  int32_t* branch_pos;
  int32_t* branch_t;
  int32_t* local_branch_cu;
  int32_t* kv_src;
} bac_plan_out;

bac_status zigzag_shard_plan(const int32_t* cu_seqlens, int32_t num_seqs,
                             const int32_t* branch_cu, const int32_t* branch_anchor,
                             int32_t num_branches, int32_t cp_size, int32_t rank,
                             bac_plan_sizes* sizes, bac_plan_out* out);

/* ------------------------------------------------------------------------
 * attn_main_fwd -- causal attention of query rows over one main K/V shard
 * ([G] 方法详解 · CP计算: one ring step of the main part).
 *
 * Query row i (sequence q_seq[i], position q_pos[i]) sees key j iff
 * k_seq[j] == q_seq[i] and k_pos[j] <= q_pos[i].  Main rows carry their own
 * position; branch rows carry their anchor's position (they see the main
 * prefix up to and including the anchor).  Scores are scale * <q, k>.
 *
 * q [nq, hq, d], k/v [nk, hkv, d]: device, dtype dt.
 * q_seq/q_pos [nq], k_seq/k_pos [nk]: device int32.  Preconditions: rows
 *   sorted by (seq, pos) non-decreasing; keys sorted by (seq, pos) strictly
 *   increasing (any zigzag shard of packed sequences is).
 * o_acc [nq, hq, d], lse [hq, nq]: device fp32, per `mode` (WRITE / MERGE).
 * o_out: NULL, or device [nq, hq, d] of dtype dt that receives the merged O
 *   rounded to dt (bf16: round-to-nearest-even).
 * bf16 runs on MFMA (bf16 products, fp32 accumulation, P rounded to bf16 for
 * the PV product); fp32 runs on fp32 vector ALUs.
 * ---------------------------------------------------------------------- */
bac_status attn_main_fwd(const void* q, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                         const void* k, const void* v, const int32_t* k_seq, const int32_t* k_pos,
                         int32_t nk, int32_t hq, int32_t hkv, int32_t d, bac_dtype dt, float scale,
                         float* o_acc, float* lse, bac_acc_mode mode, void* o_out, void* stream);

/* ------------------------------------------------------------------------
 * attn_branch_fwd -- rank-local branch attention ([G] 技术贡献: the local
 * branch part of a branch query; branch K/V never leaves the anchor's rank).
 *
 * Branch a owns tokens [branch_cu[a], branch_cu[a+1]) of qb/kb/vb; token t of
 * the branch sees tokens 0..t of the same branch (CAUSAL) or all of them
 * (BIDIR).  No branch sees another.  Each branch may have its own kind, so
 * one call serves a pack that mixes EAGLE-3 chains, DFlash blocks and DSpark
 * blocks ([G] 技术贡献: one design serves all three drafts).
 *
 * qb [nb, hq, d], kb/vb [nb, hkv, d]: device, dtype dt.
 * branch_cu [num_branches+1]: device int32, branch_cu[0] = 0,
 *   branch_cu[num_branches] = nb, non-decreasing.
 * max_branch_len: host bound on every branch's length, 1..256.  A longer
 *   branch is a precondition violation: its rows past the bound are left
 *   untouched.
 * kind: the kind of every branch when branch_kinds is NULL.
 * branch_kinds: NULL, or device int32 [num_branches]: branch a is
 *   bidirectional when branch_kinds[a] == BAC_BRANCH_BIDIR and causal for any
 *   other value (kind is then ignored).
 * o_acc/lse/mode/o_out: as attn_main_fwd, rows = branch tokens.
 * ---------------------------------------------------------------------- */
bac_status attn_branch_fwd(const void* qb, const void* kb, const void* vb, int32_t nb,
                           const int32_t* branch_cu, int32_t num_branches, int32_t max_branch_len,
                           bac_branch_kind kind, const int32_t* branch_kinds, int32_t hq,
                           int32_t hkv, int32_t d, bac_dtype dt, float scale, float* o_acc,
                           float* lse, bac_acc_mode mode, void* o_out, void* stream);

/* ------------------------------------------------------------------------
 * lse_merge -- the online-softmax merge of [G] 技术贡献:
 *   l = ln(e^la + e^lb),  O = e^(la-l) Oa + e^(lb-l) Ob,
 * evaluated as m = max(la, lb), l = m + ln(e^(la-m) + e^(lb-m)); if both
 * parts are empty the result is (0, -inf).
 * o_acc [n, hq, d], lse_acc [hq, n]: device fp32, updated in place (part a).
 * o_part, lse_part: device fp32, same shapes (part b); may not alias o_acc.
 * o_out: NULL or device [n, hq, d] of dtype out_dt receiving the merged O.
 * ---------------------------------------------------------------------- */
bac_status lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                     int32_t n, int32_t hq, int32_t d, bac_dtype out_dt, void* o_out,
                     void* stream);

/* ------------------------------------------------------------------------
 * attn_bwd_delta -- Delta[h, i] = sum_d dout[i, h, d] * o[i, h, d] in fp32,
 * computed once per row for the backward pass (which the pages leave open;
 * this is the vector-Jacobian product of the softmax for upstream dout).
 * o: device [n, hq, d] of dtype o_dt (fp32 accumulator or final output);
 * dout: device [n, hq, d] of dtype dt; delta: device fp32 [hq, n].
 * ---------------------------------------------------------------------- */
bac_status attn_bwd_delta(const void* o, bac_dtype o_dt, const void* dout, bac_dtype dt,
                          int32_t n, int32_t hq, int32_t d, float* delta, void* stream);

/* ------------------------------------------------------------------------
 * attn_main_bwd -- gradients of attn_main_fwd's rows over one K/V shard,
 * recomputed from the merged lse (P = exp(s - lse)):
 *   dS = P * (<dout, v> - delta),  dq += scale * dS k,
 *   dk += scale * dS^T q,  dv += P^T dout  (dk/dv summed over each GQA group).
 * Arguments as attn_main_fwd, plus dout [nq, hq, d] (dtype dt), lse and delta
 * [hq, nq] fp32 (merged over every part of the row), and fp32 accumulators
 * dq_acc [nq, hq, d], dk_acc / dv_acc [nk, hkv, d], which are added to (the
 * caller zeroes them once).  Calls on one stream accumulate in order.
 * ---------------------------------------------------------------------- */
bac_status attn_main_bwd(const void* q, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                         const void* k, const void* v, const int32_t* k_seq, const int32_t* k_pos,
                         int32_t nk, int32_t hq, int32_t hkv, int32_t d, bac_dtype dt, float scale,
                         const void* dout, const float* lse, const float* delta,
                         float* dq_acc, float* dk_acc, float* dv_acc, void* stream);

/* attn_main_bwd_dq / attn_main_bwd_dkdv -- the two halves of attn_main_bwd,
 * each a single kernel launch: the first adds to dq_acc only, the second to
 * dk_acc / dv_acc only.  Same arguments and preconditions as attn_main_bwd
 * (unused accumulator pointers may be NULL).  For callers that overlap the
 * dK/dV return of a ring step with the dQ work, or time the two apart. */
bac_status attn_main_bwd_dq(const void* q, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                            const void* k, const void* v, const int32_t* k_seq,
                            const int32_t* k_pos, int32_t nk, int32_t hq, int32_t hkv, int32_t d,
                            bac_dtype dt, float scale, const void* dout, const float* lse,
                            const float* delta, float* dq_acc, void* stream);
bac_status attn_main_bwd_dkdv(const void* q, const int32_t* q_seq, const int32_t* q_pos,
                              int32_t nq, const void* k, const void* v, const int32_t* k_seq,
                              const int32_t* k_pos, int32_t nk, int32_t hq, int32_t hkv, int32_t d,
                              bac_dtype dt, float scale, const void* dout, const float* lse,
                              const float* delta, float* dk_acc, float* dv_acc, void* stream);

/* ------------------------------------------------------------------------
 * attn_branch_bwd -- gradients of attn_branch_fwd's rows over their own
 * branch keys, from the merged lse/delta of those rows.  Arguments as
 * attn_branch_fwd (kind / branch_kinds included) plus doutb [nb, hq, d],
 * lseb / deltab [hq, nb] and fp32 accumulators dqb_acc [nb, hq, d],
 * dkb_acc / dvb_acc [nb, hkv, d] (added to).
 * ---------------------------------------------------------------------- */
bac_status attn_branch_bwd(const void* qb, const void* kb, const void* vb, int32_t nb,
                           const int32_t* branch_cu, int32_t num_branches, int32_t max_branch_len,
                           bac_branch_kind kind, const int32_t* branch_kinds, int32_t hq,
                           int32_t hkv, int32_t d, bac_dtype dt, float scale, const void* doutb,
                           const float* lseb, const float* deltab, float* dqb_acc,
                           float* dkb_acc, float* dvb_acc, void* stream);

/* ------------------------------------------------------------------------
 * attn_check_index -- device-side validation of the index preconditions.
 * Checks that (seq[i], pos[i]) is non-decreasing (strict = 0) or strictly
 * increasing (strict = 1) in lexicographic order and that pos[i] >= 0.
 * Writes the number of violating positions i to *bad_count (device int32,
 * overwritten).  Enqueued on `stream`; the caller synchronises to read it.
 * ---------------------------------------------------------------------- */
bac_status attn_check_index(const int32_t* seq, const int32_t* pos, int32_t n, int32_t strict,
                            int32_t* bad_count, void* stream);

/* ------------------------------------------------------------------------
 * tap_send / tap_recv -- one-way hand-off of a feature buffer through
 * preallocated device slots with sequence stamps, off any pipeline schedule
 * ([G] 技术贡献 and 方法详解 · PP传输: producers write target features into
 * the consumer's preallocated slots and bump a sequence stamp; the consumer
 * reads by stamp).  Single-device form: producer and consumer are streams
 * of one GPU.
 *
 * Mailbox (device, caller-owned): slots = nslots slots of slot_bytes bytes
 * each (slot_bytes a multiple of 16; slots 16-byte aligned); stamps =
 * nslots uint64 sequence stamps, zeroed by the caller before first use
 * (0 = nothing sent yet).  Sequence numbers are >= 1.
 *
 * tap_send: copies nbytes (<= slot_bytes) of payload (device, 16-byte
 *   aligned) into slot `slot`, then stores stamps[slot] = seq with release
 *   semantics: a consumer that sees the stamp sees the whole payload.  Both
 *   steps are enqueued on `stream`.  The caller does not reuse a slot while
 *   a consumer of its previous contents may still be reading it.
 * tap_recv: enqueued on `stream`; waits until stamps[slot] >= seq, polling
 *   at most spin_limit (>= 1) times per workgroup with a short sleep between
 *   polls, then copies nbytes of the slot to out (device, 16-byte aligned)
 *   if the stamp equals seq.  *status (device int32, overwritten):
 *   0 = received; 1 = gave up (the stamp stayed below seq for spin_limit
 *   polls; out is not fully written); 2 = the slot already holds a newer
 *   sequence.  The wait never outlasts its spin limit.
 * Errors: BAC_EINVAL for null pointers, slot outside [0, nslots), nbytes
 *   outside [0, slot_bytes], slot_bytes not a multiple of 16, misaligned
 *   buffers, seq == 0 or spin_limit < 1.
 * ---------------------------------------------------------------------- */
bac_status tap_send(void* slots, uint64_t* stamps, int32_t nslots, int64_t slot_bytes,
                    int32_t slot, const void* payload, int64_t nbytes, uint64_t seq,
                    void* stream);
bac_status tap_recv(const void* slots, const uint64_t* stamps, int32_t nslots,
                    int64_t slot_bytes, int32_t slot, uint64_t seq, int64_t spin_limit,
                    void* out, int64_t nbytes, int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BAC_H */
