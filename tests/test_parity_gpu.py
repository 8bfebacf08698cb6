"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Small and medium problems, compared element by element with the full oracle
(definition mode): several 64-key tiles, ragged tails, every branch kind,
every GQA ratio 1..32, head dims 64 and 128, fp32 and bf16, zigzag rings.
Tolerances (max abs): bf16 2e-2 on O and gradients (fp32 accumulators),
fp32 1e-5, lse 1e-3; masks and indices bit-exact.
"""

import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_util import TOL, check_rne, compare_full, host64, inputs, maxdiff, run_path, say  # noqa: E402
import oracle  # noqa: E402
from workloads import WORKLOADS, specs  # noqa: E402
from workloads.gen import make_structure_custom, make_tensors  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import branch_aware_causal_amd  # noqa: F401  (fails loudly if libbac.so is missing)


SMALL = {
    "eagle3_ragged_bf16": specs.small("e", (300, 129, 1, 77), hq=8, hkv=2, d=128, dtype="bf16",
                                      branch="eagle3", branch_len=3, seed_base=1000),
    "dflash_bf16": specs.small("f", (256, 100), hq=8, hkv=2, d=128, dtype="bf16", branch="dflash",
                               branch_len=16, anchor_stride=16, seed_base=1100),
    "dspark_d64_bf16": specs.small("s", (200, 64, 3), hq=4, hkv=1, d=64, dtype="bf16",
                                   branch="dspark", branch_len=8, anchor_stride=8, seed_base=1200),
    "eagle3_gqa1_bf16": specs.small("g1", (150,), hq=4, hkv=4, d=128, dtype="bf16",
                                    branch="eagle3", branch_len=2, seed_base=1300),
    "eagle3_gqa8_d64_bf16": specs.small("g8", (97, 40), hq=16, hkv=2, d=64, dtype="bf16",
                                        branch="eagle3", branch_len=4, seed_base=1400),
    "eagle3_f32": specs.small("f32", (70, 33), hq=8, hkv=2, d=128, dtype="f32", branch="eagle3",
                              branch_len=3, seed_base=1500),
    "dflash_d64_f32": specs.small("f32b", (64, 20), hq=4, hkv=2, d=64, dtype="f32",
                                  branch="dflash", branch_len=8, anchor_stride=8, seed_base=1600),
    # Long rows with scores of std 0.25: about 95% of the 32x32 (row, key)
    # blocks of the dK/dV kernel have every P below 2^-8, so they take the
    # path without the hi+lo split of P and dS (the short cases above almost
    # always split).
    "eagle3_long_rows_bf16": specs.small("long", (2600, 300), hq=4, hkv=1, d=128, dtype="bf16",
                                         branch="eagle3", branch_len=2, value_scale=0.5,
                                         seed_base=1700),
    # every GQA ratio the MFMA kernels are built for (hq / hkv = 2, 16, 32),
    # each at both head dims, with ragged lengths
    "eagle3_gqa2_d64_bf16": specs.small("q2a", (130, 67, 5), hq=4, hkv=2, d=64, dtype="bf16",
                                        branch="eagle3", branch_len=3, seed_base=1800),
    "dspark_gqa2_d128_bf16": specs.small("q2b", (200, 33), hq=4, hkv=2, d=128, dtype="bf16",
                                         branch="dspark", branch_len=8, anchor_stride=8,
                                         seed_base=1900),
    "eagle3_gqa16_d128_bf16": specs.small("q16a", (90, 41), hq=32, hkv=2, d=128, dtype="bf16",
                                          branch="eagle3", branch_len=2, seed_base=2000),
    "dflash_gqa16_d64_bf16": specs.small("q16b", (96, 40), hq=32, hkv=2, d=64, dtype="bf16",
                                         branch="dflash", branch_len=16, anchor_stride=16,
                                         seed_base=2100),
    "eagle3_gqa32_d64_bf16": specs.small("q32a", (77, 100, 3), hq=32, hkv=1, d=64, dtype="bf16",
                                         branch="eagle3", branch_len=3, seed_base=2200),
    "eagle3_gqa32_d128_bf16": specs.small("q32b", (150, 9), hq=32, hkv=1, d=128, dtype="bf16",
                                          branch="eagle3", branch_len=2, seed_base=2300),
    # empty sequences inside a pack (their ids own no token) and a sequence
    # shorter than one DSpark block
    "dspark_empty_seqs_bf16": specs.small("e0", (120, 0, 64, 0, 7), hq=8, hkv=2, d=128,
                                          dtype="bf16", branch="dspark", branch_len=8,
                                          anchor_stride=8, seed_base=2800),
    # one pack mixing the three families, each branch with its own kind
    "mixed_kinds_bf16": specs.small("mix", (150, 96, 40), hq=8, hkv=2, d=128, dtype="bf16",
                                    branch="mixed", seed_base=2400,
                                    mix=(("eagle3", 3, 1), ("dflash", 16, 16), ("dspark", 8, 8))),
    "mixed_kinds_f32": specs.small("mixf", (40, 33, 17), hq=4, hkv=2, d=64, dtype="f32",
                                   branch="mixed", seed_base=2500,
                                   mix=(("dspark", 4, 2), ("eagle3", 2, 1), ("dflash", 8, 8))),
    # branches longer than 32 tokens (bidirectional blocks of 64, causal of 48)
    "dflash_b64_bf16": specs.small("b64", (256, 130), hq=8, hkv=2, d=64, dtype="bf16",
                                   branch="dflash", branch_len=64, anchor_stride=64,
                                   seed_base=2600),
    "dspark_b48_bf16": specs.small("b48", (200, 97), hq=8, hkv=2, d=128, dtype="bf16",
                                   branch="dspark", branch_len=48, anchor_stride=32,
                                   seed_base=2700),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_problem_matches_oracle(name):
    w = SMALL[name]
    say(f"case {name}: seqs={w.seqlens} hq={w.hq} hkv={w.hkv} d={w.d} {w.dtype} {w.branch}")
    st, t = inputs(w)
    gpu = run_path(st, t)
    compare_full(st, t, gpu, TOL[w.dtype], name)
    check_rne(gpu)


def test_tiny_eagle3_fp32_workload():
    """Two packed sequences of 96 and 160 tokens, EAGLE-3 TTT depth 3,
    Hq=4, Hkv=2, d=64, fp32: the whole problem, fp32 tolerance."""
    w = WORKLOADS["eagle3_tiny_fp32"]
    st, t = inputs(w)
    gpu = run_path(st, t)
    compare_full(st, t, gpu, TOL["f32"], w.name)
    check_rne(gpu)


@pytest.mark.parametrize("cp", [2, 3, 4])
def test_zigzag_ring_small_matches_oracle(cp):
    w = SMALL["eagle3_ragged_bf16"]
    st, t = inputs(w)
    gpu = run_path(st, t, cp=cp)
    compare_full(st, t, gpu, TOL["bf16"], f"ring C={cp}")


@pytest.mark.parametrize("cp", [3, 4])
def test_zigzag_ring_mixed_kinds_matches_oracle(cp):
    w = SMALL["mixed_kinds_bf16"]
    st, t = inputs(w)
    gpu = run_path(st, t, cp=cp)
    compare_full(st, t, gpu, TOL["bf16"], f"mixed ring C={cp}")


@pytest.mark.parametrize("cp", [2, 3])
def test_zigzag_ring_with_empty_sequences_matches_oracle(cp):
    w = SMALL["dspark_empty_seqs_bf16"]
    st, t = inputs(w)
    gpu = run_path(st, t, cp=cp)
    compare_full(st, t, gpu, TOL["bf16"], f"empty-sequence ring C={cp}")


def test_ring_dflash_matches_unsharded():
    w = SMALL["dflash_bf16"]
    st, t = inputs(w)
    a = run_path(st, t, cp=1)
    b = run_path(st, t, cp=4)
    for key in a:
        tol = 1e-3 if key.startswith("lse") else 2e-2
        assert maxdiff(host64(b[key]), host64(a[key])) <= tol, key


@pytest.mark.parametrize("impl", ["bf16", "f32"])
def test_mask_is_bit_exact_with_one_hot_values(impl):
    """Q = 0 and V = one-hot(key id): every visible score is equal, so
    O = (1/|V(q)|) on exactly the visible keys and 0 elsewhere, and
    lse = ln |V(q)|.  Checked on the hand-written mask fixtures' structures."""
    import os
    from test_oracle import GOLDEN_FILES, load_golden
    for fname in GOLDEN_FILES:
        spec, mat = load_golden(fname)
        seqlens = [int(x) for x in spec["seqlens"]]
        anchors = [int(x) for x in spec["anchors"]]
        blens = [int(x) for x in spec["branch_lens"]]
        cu = np.concatenate([[0], np.cumsum(seqlens)])
        per_seq = [[a - cu[s] for a in anchors if cu[s] <= a < cu[s + 1]] for s in range(len(seqlens))]
        kind = spec["kinds"] if "kinds" in spec else spec["kind"][0]
        st = make_structure_custom(seqlens, per_seq, blens, kind)
        d = 64
        dt = torch.bfloat16 if impl == "bf16" else torch.float32
        n = mat.shape[0]
        N, Nb = st.n_main, st.n_branch_tok
        eye = torch.eye(n, d, dtype=dt, device="cuda")
        t = dict(q=torch.zeros(N, 2, d, dtype=dt, device="cuda"),
                 qb=torch.zeros(Nb, 2, d, dtype=dt, device="cuda"),
                 k=torch.randn(N, 1, d, device="cuda").to(dt),
                 kb=torch.randn(Nb, 1, d, device="cuda").to(dt),
                 v=eye[:N, None, :].contiguous(), vb=eye[N:, None, :].contiguous(),
                 do=torch.zeros(N, 2, d, dtype=dt, device="cuda"),
                 dob=torch.zeros(Nb, 2, d, dtype=dt, device="cuda"))
        gpu = run_path(st, t)
        O = torch.cat([gpu["o_main_acc"], gpu["o_br_acc"]])[:, 0, :n].cpu().numpy()
        lse = torch.cat([gpu["lse_main"], gpu["lse_br"]], dim=1)[0].cpu().numpy()
        assert np.array_equal(O > 0, mat), fname
        counts = mat.sum(axis=1)
        assert np.all(np.abs(lse - np.log(counts)) < 1.0 / (2 * counts)), fname
        assert np.allclose(O[mat], np.repeat(1.0 / counts, counts), rtol=1e-2), fname


def test_lse_merge_kernel_matches_oracle_merge():
    from branch_aware_causal_amd import lse_merge
    g = torch.Generator(device="cuda").manual_seed(5)
    n, hq, d = 333, 4, 128
    oa = torch.randn(n, hq, d, generator=g, device="cuda")
    ob = torch.randn(n, hq, d, generator=g, device="cuda")
    la = torch.randn(hq, n, generator=g, device="cuda") * 4
    lb = torch.randn(hq, n, generator=g, device="cuda") * 4
    la[0, :50] = -math.inf
    lb[1, 25:75] = -math.inf
    la[2, 10:20] = -math.inf
    lb[2, 10:20] = -math.inf
    oa[la.T == -math.inf] = 0
    ob[lb.T == -math.inf] = 0
    ref_o, ref_l = oracle.lse_merge(host64(oa), host64(la).T, host64(ob), host64(lb).T)
    o_out = torch.empty(n, hq, d, dtype=torch.bfloat16, device="cuda")
    lse_merge(oa, la, ob, lb, o_out=o_out)
    torch.cuda.synchronize()
    assert maxdiff(host64(oa), ref_o) < 1e-5
    assert maxdiff(host64(la).T, ref_l) < 1e-5
    assert torch.equal(oa.to(torch.bfloat16), o_out)


def test_delta_kernel():
    from branch_aware_causal_amd import attn_bwd_delta
    g = torch.Generator(device="cuda").manual_seed(6)
    n, hq, d = 129, 8, 64
    o = torch.randn(n, hq, d, generator=g, device="cuda")
    do = torch.randn(n, hq, d, generator=g, device="cuda").to(torch.bfloat16)
    delta = torch.empty(hq, n, device="cuda")
    attn_bwd_delta(o, do, delta)
    ref = oracle.delta(host64(o), host64(do)).T
    assert maxdiff(host64(delta), ref) < 1e-4


def test_empty_and_fully_masked_shards():
    """WRITE over an empty key set or a shard wholly after the rows gives
    (O = 0, lse = -inf); MERGE of it leaves the accumulators unchanged."""
    from branch_aware_causal_amd import attn_main_fwd
    dev = "cuda"
    nq, hq, hkv, d = 70, 8, 2, 128
    q = torch.randn(nq, hq, d, device=dev).to(torch.bfloat16)
    qs = torch.zeros(nq, dtype=torch.int32, device=dev)
    qp = torch.arange(nq, dtype=torch.int32, device=dev)
    k = torch.randn(100, hkv, d, device=dev).to(torch.bfloat16)
    ks = torch.zeros(100, dtype=torch.int32, device=dev)
    kp = torch.arange(1000, 1100, dtype=torch.int32, device=dev)    # all after the rows
    o = torch.full((nq, hq, d), 7.0, device=dev)
    l = torch.full((hq, nq), 3.0, device=dev)
    attn_main_fwd(q, qs, qp, k, k, ks, kp, o, l, "merge")
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(l == 3.0)
    attn_main_fwd(q, qs, qp, k, k, ks, kp, o, l, "write")
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(l == -math.inf)
    e = torch.empty(0, hkv, d, dtype=torch.bfloat16, device=dev)
    ei = torch.empty(0, dtype=torch.int32, device=dev)
    o.fill_(1.0)
    attn_main_fwd(q, qs, qp, e, e, ei, ei, o, l, "write")
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(l == -math.inf)


def test_check_index_counts_violations():
    from branch_aware_causal_amd import attn_check_index
    seq = torch.tensor([0, 0, 0, 1, 1, 0], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0, 1, 1, 0, -3, 5], dtype=torch.int32, device="cuda")
    assert attn_check_index(seq, pos, strict=False) == 2   # (1,-3): pos<0 and order; (0,5)<(1,-3)
    assert attn_check_index(seq, pos, strict=True) == 3    # plus the repeated (0,1)


@pytest.mark.parametrize("kind,d", [("causal", 128), ("bidir", 64)])
def test_branch_tokens_past_max_len_are_left_untouched(kind, d):
    """Branches of 6 tokens called with max_branch_len = 4 (a precondition
    violation the header defines): tokens 4 and 5 keep the buffers' previous
    contents, and tokens 0..3 get exactly what a call on the branches cut to
    their first 4 tokens gives (same kernel arithmetic, so bit-exact)."""
    from branch_aware_causal_amd import api
    say(f"case branch max_len clamp: kind={kind} d={d}")
    dev = torch.device("cuda:0")
    A, L, B, hq, hkv = 37, 6, 4, 8, 2
    nb = A * L
    gen = torch.Generator(device=dev).manual_seed(2024 + d)
    rnd = lambda *s: torch.randn(*s, generator=gen, device=dev).to(torch.bfloat16)
    qb, dob = rnd(nb, hq, d), rnd(nb, hq, d)
    kb, vb = rnd(nb, hkv, d), rnd(nb, hkv, d)
    cu = torch.arange(0, nb + 1, L, dtype=torch.int32, device=dev)
    idx = torch.tensor([a * L + t for a in range(A) for t in range(B)], device=dev)
    rest = torch.tensor([a * L + t for a in range(A) for t in range(B, L)], device=dev)
    cu_c = torch.arange(0, A * B + 1, B, dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    # forward
    o = torch.full((nb, hq, d), 7.0, **f32)
    lse = torch.full((hq, nb), 7.0, **f32)
    api.attn_branch_fwd(qb, kb, vb, cu, B, kind, o, lse, "write")
    o_c, lse_c = torch.empty(A * B, hq, d, **f32), torch.empty(hq, A * B, **f32)
    api.attn_branch_fwd(qb[idx].contiguous(), kb[idx].contiguous(), vb[idx].contiguous(), cu_c, B,
                        kind, o_c, lse_c, "write")
    torch.cuda.synchronize()
    assert torch.equal(o[idx], o_c) and torch.equal(lse[:, idx], lse_c)
    assert bool((o[rest] == 7.0).all()) and bool((lse[:, rest] == 7.0).all())
    # backward
    delta = torch.randn(hq, nb, generator=gen, device=dev)
    lse_in = lse.clone()
    lse_in[:, rest] = 0.0
    grads = [torch.zeros(nb, hq, d, **f32), torch.zeros(nb, hkv, d, **f32), torch.zeros(nb, hkv, d, **f32)]
    api.attn_branch_bwd(qb, kb, vb, cu, B, kind, dob, lse_in, delta, *grads)
    grads_c = [torch.zeros(A * B, hq, d, **f32), torch.zeros(A * B, hkv, d, **f32),
               torch.zeros(A * B, hkv, d, **f32)]
    api.attn_branch_bwd(qb[idx].contiguous(), kb[idx].contiguous(), vb[idx].contiguous(), cu_c, B,
                        kind, dob[idx].contiguous(), lse_c, delta[:, idx].contiguous(), *grads_c)
    torch.cuda.synchronize()
    for full, comp in zip(grads, grads_c):
        assert torch.equal(full[idx], comp)
        assert bool((full[rest] == 0.0).all())
        assert bool(torch.isfinite(comp).all()) and float(comp.abs().max()) > 0
