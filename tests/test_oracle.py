"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin is independent of the oracle's own vectorised code path: hand-written
mask fixtures (tests/golden/), pure-Python brute force, closed forms, torch's
SDPA on the purely causal case, finite differences, torch autograd, exact
invariants and metamorphic shifts.
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute, zigzag
from oracle.problem import Problem
from workloads import splitmix64, varlen_lengths
from workloads.gen import make_structure_custom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seqlens, anchors_per_seq, branch_lens, kind, hq=4, hkv=2, d=8, seed=0,
                 scale_vals=1.0):
    st = make_structure_custom(seqlens, anchors_per_seq, branch_lens, kind)
    rng = np.random.default_rng(seed)
    N, Nb = st.n_main, st.n_branch_tok
    t = lambda n, h: rng.standard_normal((n, h, d)) * scale_vals
    return Problem(st.cu_seqlens, st.branch_cu, st.branch_anchor, kind, hq, hkv, d,
                   t(N, hq), t(N, hkv), t(N, hkv), t(Nb, hq), t(Nb, hkv), t(Nb, hkv))


def every(seqlens, stride):
    return [list(range(0, L, stride)) for L in seqlens]


def eagle(seqlens, D, **kw):
    an = every(seqlens, 1)
    return rand_problem(seqlens, an, [D] * sum(len(a) for a in an), "causal", **kw)


def dflash(seqlens, B, stride, **kw):
    an = every(seqlens, stride)
    return rand_problem(seqlens, an, [B] * sum(len(a) for a in an), "bidir", **kw)


def dspark(seqlens, B, stride, **kw):
    an = every(seqlens, stride)
    return rand_problem(seqlens, an, [B] * sum(len(a) for a in an), "causal", **kw)


def kind_of(prob, a):
    """Kind of branch a as given to the problem (one for all, or per branch)."""
    return prob.kind if isinstance(prob.kind, str) else prob.kind[a]


# one packed batch of the three families: an EAGLE-3 depth-2 chain at every
# position of a 6-token sequence, DFlash blocks of 4 every 4 positions of an
# 8-token sequence, DSpark blocks of 3 every 2 positions of a 5-token one
MIXED = dict(seqlens=(6, 8, 5), anchors=[list(range(6)), [0, 4], [0, 2, 4]],
             lens=[2] * 6 + [4, 4] + [3, 3, 3],
             kinds=["causal"] * 6 + ["bidir"] * 2 + ["causal"] * 3)


SMALL_CASES = {
    "eagle_d3": lambda **kw: eagle((5, 7), 3, **kw),
    "dflash_b4": lambda **kw: dflash((8, 6), 4, 4, **kw),
    "dspark_b3": lambda **kw: dspark((9, 4), 3, 2, **kw),
    "ragged": lambda **kw: rand_problem((1, 6, 3), [[0], [0, 2, 5], [1]], [2, 1, 4, 3, 2],
                                        "causal", **kw),
    "ragged_bidir": lambda **kw: rand_problem((4, 5), [[3], [0, 4]], [3, 1, 5], "bidir", **kw),
    "mixed_kinds": lambda **kw: rand_problem(MIXED["seqlens"], MIXED["anchors"], MIXED["lens"],
                                             MIXED["kinds"], **kw),
}


# ---------------------------------------------------------------------------
# Mask: hand-written fixtures, brute force, closed forms
# ---------------------------------------------------------------------------

def load_golden(name):
    spec, mat = {}, []
    in_mat = False
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line == "matrix":
                in_mat = True
                continue
            if in_mat:
                mat.append([int(c) for c in line])
            else:
                key, *vals = line.split()
                spec[key] = vals
    return spec, np.array(mat, dtype=bool)


GOLDEN_FILES = sorted(f for f in os.listdir(GOLDEN) if f.startswith("mask_"))


def golden_problem(spec, d=4):
    seqlens = [int(x) for x in spec["seqlens"]]
    anchors = [int(x) for x in spec["anchors"]]
    blens = [int(x) for x in spec["branch_lens"]]
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    per_seq = [[a - cu[s] for a in anchors if cu[s] <= a < cu[s + 1]] for s in range(len(seqlens))]
    kind = spec["kinds"] if "kinds" in spec else spec["kind"][0]
    return rand_problem(seqlens, per_seq, blens, kind, hq=2, hkv=1, d=d)


@pytest.mark.parametrize("fname", GOLDEN_FILES)
def test_visibility_matches_hand_written_fixture(fname):
    spec, mat = load_golden(fname)
    prob = golden_problem(spec)
    ids = np.arange(prob.N + prob.Nb)
    assert mat.shape == (ids.size, ids.size)
    assert np.array_equal(prob.visibility(ids, ids), mat)


@pytest.mark.parametrize("fname", GOLDEN_FILES)
def test_brute_keys_match_hand_written_fixture(fname):
    spec, mat = load_golden(fname)
    prob = golden_problem(spec)
    N = prob.N
    rows = [("m", i) for i in range(N)] + [("b", i) for i in range(prob.Nb)]
    for r_i, row in enumerate(rows):
        keys = brute._row_keys(list(prob.cu), list(prob.bcu), list(prob.anchor), prob.kind, row)
        got = np.zeros(mat.shape[1], bool)
        for kind, idx in keys:
            got[idx if kind == "m" else N + idx] = True
        assert np.array_equal(got, mat[r_i]), (fname, row)


@pytest.mark.parametrize("case", sorted(SMALL_CASES))
def test_definition_matches_brute_force(case):
    prob = SMALL_CASES[case](hq=4, hkv=2, d=6, seed=3)
    O, lse = oracle.forward(prob, block_pos=4)
    ref = brute.forward(prob.cu, prob.bcu, prob.anchor, prob.kind, prob.hq, prob.hkv, prob.d,
                        prob.q, prob.k, prob.v, prob.qb, prob.kb, prob.vb)
    for (kind, i), (Os, lses) in ref.items():
        row = i if kind == "m" else prob.N + i
        assert np.max(np.abs(np.array(Os) - O[row])) < 1e-12
        assert np.max(np.abs(np.array(lses) - lse[row])) < 1e-12


def closed_form_count(prob, row):
    """|V(row)| from the pattern's closed form: p+1 for a main row; anchor+1
    plus t+1 (causal) or the branch length (bidir) for a branch row."""
    if row < prob.N:
        s = np.searchsorted(prob.cu, row, side="right") - 1
        return int(row - prob.cu[s] + 1)
    bt = row - prob.N
    a = np.searchsorted(prob.bcu, bt, side="right") - 1
    ag = prob.anchor[a]
    s = np.searchsorted(prob.cu, ag, side="right") - 1
    j = int(ag - prob.cu[s])
    blen = int(prob.bcu[a + 1] - prob.bcu[a])
    t = int(bt - prob.bcu[a])
    return j + 1 + (t + 1 if kind_of(prob, a) == "causal" else blen)


@pytest.mark.parametrize("case", sorted(SMALL_CASES))
def test_q_zero_closed_form(case):
    """With Q = 0 every visible score is 0: lse = ln|V(q)| and O is the mean
    of the visible V rows."""
    prob = SMALL_CASES[case](hq=4, hkv=2, d=5, seed=7)
    prob.q = np.zeros_like(prob.q)
    prob.qb = np.zeros_like(prob.qb)
    O, lse = oracle.forward(prob, block_pos=3)
    for row in range(prob.N + prob.Nb):
        n = closed_form_count(prob, row)
        assert np.allclose(lse[row], math.log(n), atol=1e-13, rtol=0)
        # explicit visible set: main prefix range plus branch token range
        if row < prob.N:
            s = np.searchsorted(prob.cu, row, side="right") - 1
            vrows = prob.v[prob.cu[s]:row + 1]
        else:
            bt = row - prob.N
            a = np.searchsorted(prob.bcu, bt, side="right") - 1
            ag = prob.anchor[a]
            s = np.searchsorted(prob.cu, ag, side="right") - 1
            last = bt + 1 if kind_of(prob, a) == "causal" else prob.bcu[a + 1]
            vrows = np.concatenate([prob.v[prob.cu[s]:ag + 1], prob.vb[prob.bcu[a]:last]])
        assert vrows.shape[0] == n
        mean = vrows.mean(axis=0)                       # [Hkv, d]
        for h in range(prob.hq):
            assert np.allclose(O[row, h], mean[h * prob.hkv // prob.hq], atol=1e-13)


@pytest.mark.parametrize("fname", GOLDEN_FILES)
def test_one_hot_v_reconstructs_mask(fname):
    """Q = 0 and V = one-hot(key id): O * |V(q)| is exactly the mask row."""
    spec, mat = load_golden(fname)
    n = mat.shape[0]
    prob = golden_problem(spec, d=n)
    prob.q = np.zeros_like(prob.q)
    prob.qb = np.zeros_like(prob.qb)
    eye = np.eye(n)
    prob.v = np.repeat(eye[:prob.N, None, :], prob.hkv, axis=1)
    prob.vb = np.repeat(eye[prob.N:, None, :], prob.hkv, axis=1)
    O, lse = oracle.forward(prob)
    counts = mat.sum(axis=1)
    rec = O[:, 0, :] * counts[:, None]
    assert np.allclose(rec, mat.astype(float), atol=1e-12)


def closed_form_pairs(seqlens, stride, blen, kind):
    """Closed-form pair counts per q-head: causal main L(L+1)/2; branch rows
    see anchor+1 main keys each; inside a branch B(B+1)/2 (causal) or B^2."""
    main = sum(L * (L + 1) // 2 for L in seqlens)
    br_main = sum(blen * (p + 1) for L in seqlens for p in range(0, L, stride))
    n_anchor = sum(len(range(0, L, stride)) for L in seqlens)
    local = n_anchor * (blen * (blen + 1) // 2 if kind == "causal" else blen * blen)
    return main, br_main, local


@pytest.mark.parametrize("seqlens,stride,blen,kind", [
    ((5, 7), 1, 3, "causal"), ((16,), 4, 4, "bidir"), ((8, 8), 2, 2, "causal"),
    ((9, 1, 4), 3, 5, "bidir")])
def test_pair_counts_closed_form(seqlens, stride, blen, kind):
    an = every(seqlens, stride)
    prob = rand_problem(seqlens, an, [blen] * sum(len(a) for a in an), kind, hq=2, hkv=1, d=2)
    total = sum(closed_form_pairs(seqlens, stride, blen, kind))
    assert prob.count_visible() == total
    assert brute.count_pairs(prob.cu, prob.bcu, prob.anchor, kind) == total


def test_pair_counts_of_the_named_workloads():
    """Closed-form counts at the full workload sizes (used for FLOP accounting)."""
    assert closed_form_pairs((32768,), 16, 16, "bidir") == (536887296, 536641536, 524288)
    assert closed_form_pairs((16384,) * 4, 8, 8, "causal") == (536903680, 536674304, 294912)
    assert closed_form_pairs((262144,), 1, 3, "causal") == (34359869440, 103079608320, 1572864)
    assert closed_form_pairs((96, 160), 1, 3, "causal") == (17536, 52608, 1536)
    m, bm, lo = closed_form_pairs(varlen_lengths(20480, 512, 8192, 0), 1, 4, "causal")
    assert (m, bm, lo) == (50874399, 203497596, 204800)


# ---------------------------------------------------------------------------
# Library routine on the purely causal case
# ---------------------------------------------------------------------------

def test_no_branch_equals_torch_sdpa_causal():
    torch = pytest.importorskip("torch")
    seqlens = (7, 1, 12)
    prob = rand_problem(seqlens, [[] for _ in seqlens], [], "causal", hq=4, hkv=2, d=16, seed=5)
    O, lse = oracle.forward(prob, block_pos=5)
    for s, L in enumerate(seqlens):
        a, b = int(prob.cu[s]), int(prob.cu[s + 1])
        q = torch.from_numpy(prob.q[a:b]).permute(1, 0, 2)[None]           # [1,Hq,L,d]
        k = torch.from_numpy(prob.k[a:b]).permute(1, 0, 2)[None]
        v = torch.from_numpy(prob.v[a:b]).permute(1, 0, 2)[None]
        k = k.repeat_interleave(prob.hq // prob.hkv, dim=1)
        v = v.repeat_interleave(prob.hq // prob.hkv, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        got = O[a:b].transpose(1, 0, 2)[None]
        assert np.max(np.abs(ref.numpy() - got)) < 1e-12
        # lse: log-sum-exp of the causal scores
        sc = (q @ k.transpose(-1, -2)) / math.sqrt(prob.d)
        sc = sc.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), -math.inf)
        ref_lse = torch.logsumexp(sc, dim=-1)[0].T.numpy()
        assert np.max(np.abs(ref_lse - lse[a:b])) < 1e-12


# ---------------------------------------------------------------------------
# Merge identity, decomposition and zigzag
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", sorted(SMALL_CASES))
def test_decomposed_merge_equals_definition(case):
    prob = SMALL_CASES[case](seed=11)
    O, lse = oracle.forward(prob)
    Om, lm = oracle.forward_decomposed(prob)
    assert np.max(np.abs(O - Om)) < 1e-12
    assert np.max(np.abs(lse - lm)) < 1e-12


def test_merge_empty_is_identity_and_order_free():
    rng = np.random.default_rng(0)
    o = [rng.standard_normal((6, 3, 4)) for _ in range(3)]
    l = [rng.standard_normal((6, 3)) * 3 for _ in range(3)]
    empty_o, empty_l = np.zeros((6, 3, 4)), np.full((6, 3), -np.inf)
    mo, ml = oracle.lse_merge(o[0], l[0], empty_o, empty_l)
    assert np.array_equal(ml, l[0]) and np.max(np.abs(mo - o[0])) == 0
    mo, ml = oracle.lse_merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(ml == -np.inf) and np.all(mo == 0)
    a = oracle.lse_merge(*oracle.lse_merge(o[0], l[0], o[1], l[1]), o[2], l[2])
    b = oracle.lse_merge(o[2], l[2], *oracle.lse_merge(o[1], l[1], o[0], l[0]))
    assert np.max(np.abs(a[0] - b[0])) < 1e-12 and np.max(np.abs(a[1] - b[1])) < 1e-12
    # closed form for two parts: lse = log(e^a + e^b)
    assert np.allclose(oracle.lse_merge(o[0], l[0], o[1], l[1])[1],
                       np.log(np.exp(l[0]) + np.exp(l[1])), atol=1e-13)


ZZ_CASES = [
    ("eagle", lambda: eagle((9, 16, 3), 2, hq=4, hkv=2, d=4, seed=2)),
    ("dflash", lambda: dflash((16, 11), 4, 4, hq=2, hkv=1, d=4, seed=3)),
    ("dspark", lambda: dspark((7, 13), 3, 2, hq=4, hkv=1, d=4, seed=4)),
    ("mixed", lambda: SMALL_CASES["mixed_kinds"](hq=4, hkv=2, d=4, seed=5)),
]


@pytest.mark.parametrize("C", [1, 2, 3, 4])
@pytest.mark.parametrize("name,mk", ZZ_CASES)
def test_zigzag_ring_equals_definition(name, mk, C):
    prob = mk()
    O, lse = oracle.forward(prob)
    Oz, lz = zigzag.ring_forward(prob, C)
    assert np.max(np.abs(O - Oz)) < 1e-12
    assert np.max(np.abs(lse - lz)) < 1e-12
    rng = np.random.default_rng(C)
    dO = rng.standard_normal(O.shape)
    g = oracle.backward(prob, dO, fwd=(O, lse))
    gz = zigzag.ring_backward(prob, C, dO, fwd=(Oz, lz))
    for a, b in zip(g, gz):
        assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("C", [1, 2, 3, 4, 8])
def test_zigzag_plan_partitions_tokens(C):
    seqlens = (9, 16, 3, 40)
    an = every(seqlens, 2)
    st = make_structure_custom(seqlens, an, [2] * sum(len(a) for a in an), "causal")
    plans = [zigzag.plan(st.cu_seqlens, st.branch_cu, st.branch_anchor, C, r) for r in range(C)]
    mains = np.concatenate([p["main_index"] for p in plans])
    assert np.array_equal(np.sort(mains), np.arange(st.n_main))
    brs = np.concatenate([p["branch_ids"] for p in plans])
    assert np.array_equal(np.sort(brs), np.arange(st.n_branches))
    toks = np.concatenate([p["branch_index"] for p in plans])
    assert np.array_equal(np.sort(toks), np.arange(st.n_branch_tok))
    for r, p in enumerate(plans):
        assert np.array_equal(p["kv_src"], [(r - s) % C for s in range(C)])
        # (seq, pos) order inside the rank
        key = p["main_seq"] * 10**6 + p["main_pos"]
        assert np.all(np.diff(key) > 0)
        # a branch lives where its anchor lives
        owned = set(p["main_index"].tolist())
        assert all(int(st.branch_anchor[a]) in owned for a in p["branch_ids"])


@pytest.mark.parametrize("C", [2, 4, 8])
def test_zigzag_balances_pairs_when_chunks_divide(C):
    L = 16 * C
    prob = eagle((L, 2 * L), 2, hq=2, hkv=1, d=2)
    counts = []
    for r in range(C):
        p = zigzag.plan(prob.cu, prob.bcu, prob.anchor, C, r)
        rows = np.concatenate([p["main_index"], prob.N + p["branch_index"]])
        counts.append(int(prob.visibility(rows, np.arange(prob.N + prob.Nb)).sum()))
    assert len(set(counts)) == 1


@pytest.mark.parametrize("C", [2, 4, 8])
def test_ring_bytes_match_volume_formula(C):
    """[G] 方法详解 · 通信: each rank receives 2(C-1)(N/C) d_kv b bytes of main
    K/V per forward (d_kv = Hkv*d, b = bytes per element)."""
    N, hkv, d, b = 64 * C, 8, 128, 2
    st = make_structure_custom((N,), [[0]], [1], "causal")
    for r in range(C):
        got = zigzag.ring_bytes_received(st.cu_seqlens, st.branch_cu, st.branch_anchor,
                                         C, r, hkv, d, b)
        assert got == 2 * (C - 1) * (N // C) * hkv * d * b


# ---------------------------------------------------------------------------
# Backward: finite differences, autograd, invariants, metamorphic shifts
# ---------------------------------------------------------------------------

def _loss(prob, dO):
    O, _ = oracle.forward(prob, block_pos=4)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("case", ["eagle_d3", "dflash_b4", "ragged"])
def test_backward_matches_finite_differences(case):
    prob = SMALL_CASES[case](hq=2, hkv=1, d=3, seed=13)
    rng = np.random.default_rng(1)
    n = prob.N + prob.Nb
    dO = rng.standard_normal((n, prob.hq, prob.d))
    dQ, dK, dV = oracle.backward(prob, dO, block_pos=4)
    eps = 1e-6
    for name, grad, off in [("q", dQ, 0), ("qb", dQ, prob.N), ("k", dK, 0), ("kb", dK, prob.N),
                            ("v", dV, 0), ("vb", dV, prob.N)]:
        arr = getattr(prob, name)
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(prob, dO)
            arr[idx] = old - eps
            lm = _loss(prob, dO)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        an = grad[off:off + arr.shape[0]]
        err = np.max(np.abs(fd - an)) / max(1.0, np.max(np.abs(an)))
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("case", sorted(SMALL_CASES))
def test_backward_matches_torch_autograd(case):
    torch = pytest.importorskip("torch")
    prob = SMALL_CASES[case](hq=4, hkv=2, d=8, seed=17)
    n = prob.N + prob.Nb
    ids = np.arange(n)
    mask = torch.from_numpy(prob.visibility(ids, ids))
    Q = torch.from_numpy(np.concatenate([prob.q, prob.qb])).requires_grad_()
    K = torch.from_numpy(np.concatenate([prob.k, prob.kb])).requires_grad_()
    V = torch.from_numpy(np.concatenate([prob.v, prob.vb])).requires_grad_()
    rep = prob.hq // prob.hkv
    Kh, Vh = K.repeat_interleave(rep, dim=1), V.repeat_interleave(rep, dim=1)
    S = torch.einsum("qhd,khd->hqk", Q, Kh) * prob.scale
    S = S.masked_fill(~mask[None], -math.inf)
    P = torch.softmax(S, dim=-1)
    O = torch.einsum("hqk,khd->qhd", P, Vh)
    dO = torch.from_numpy(np.random.default_rng(2).standard_normal((n, prob.hq, prob.d)))
    (O * dO).sum().backward()
    dQ, dK, dV = oracle.backward(prob, dO.numpy(), block_pos=3)
    assert np.max(np.abs(dQ - Q.grad.numpy())) < 1e-11
    assert np.max(np.abs(dK - K.grad.numpy())) < 1e-11
    assert np.max(np.abs(dV - V.grad.numpy())) < 1e-11


@pytest.mark.parametrize("case", sorted(SMALL_CASES))
def test_gradient_invariants(case):
    """sum_k dV_{k,g} = sum_{h in g} sum_q dO_{q,h} (each P row sums to 1) and
    sum_k dK_{k,g} = 0 (each dS row sums to 0)."""
    prob = SMALL_CASES[case](hq=4, hkv=2, d=6, seed=19)
    n = prob.N + prob.Nb
    dO = np.random.default_rng(4).standard_normal((n, prob.hq, prob.d))
    dQ, dK, dV = oracle.backward(prob, dO)
    for g in range(prob.hkv):
        heads = [h for h in range(prob.hq) if h * prob.hkv // prob.hq == g]
        assert np.allclose(dV[:, g].sum(0), dO[:, heads].sum((0, 1)), atol=1e-11)
        assert np.allclose(dK[:, g].sum(0), 0.0, atol=1e-11)


@pytest.mark.parametrize("case", sorted(SMALL_CASES))
def test_metamorphic_shifts(case):
    """K += u leaves O and the gradients unchanged and shifts lse by
    scale*<q,u>; V += w shifts O by w."""
    prob = SMALL_CASES[case](hq=4, hkv=2, d=6, seed=23)
    n = prob.N + prob.Nb
    dO = np.random.default_rng(5).standard_normal((n, prob.hq, prob.d))
    O, lse = oracle.forward(prob)
    g0 = oracle.backward(prob, dO, fwd=(O, lse))
    u = np.random.default_rng(6).standard_normal((prob.hkv, prob.d))
    w = np.random.default_rng(7).standard_normal((prob.hkv, prob.d))
    prob.k = prob.k + u[None]
    prob.kb = prob.kb + u[None]
    O2, lse2 = oracle.forward(prob)
    assert np.max(np.abs(O2 - O)) < 1e-11
    Qall = np.concatenate([prob.q, prob.qb])
    shift = prob.scale * np.einsum("rhd,hd->rh", Qall, u[prob.group])
    assert np.max(np.abs(lse2 - lse - shift)) < 1e-11
    g1 = oracle.backward(prob, dO, fwd=(O2, lse2))
    for a, b in zip(g0, g1):
        assert np.max(np.abs(a - b)) < 1e-10
    prob.v = prob.v + w[None]
    prob.vb = prob.vb + w[None]
    O3, _ = oracle.forward(prob)
    assert np.max(np.abs(O3 - O2 - w[prob.group][None])) < 1e-11


# ---------------------------------------------------------------------------
# Sampled evaluation agrees with the full definition
# ---------------------------------------------------------------------------

def test_sampled_rows_and_keys_agree_with_full():
    prob = eagle((13, 21), 3, hq=4, hkv=2, d=8, seed=29)
    n = prob.N + prob.Nb
    dO = np.random.default_rng(8).standard_normal((n, prob.hq, prob.d))
    O, lse = oracle.forward(prob)
    dQ, dK, dV = oracle.backward(prob, dO, fwd=(O, lse))
    rows = np.array([0, 5, prob.N - 1, prob.N, prob.N + 7, n - 1])
    o, l = oracle.forward_rows(prob, rows)
    assert np.max(np.abs(o - O[rows])) < 1e-12 and np.max(np.abs(l - lse[rows])) < 1e-12
    dq, _, _ = oracle.backward_rows(prob, rows, dO[rows])
    assert np.max(np.abs(dq - dQ[rows])) < 1e-12
    keys = np.array([prob.N - 3, prob.N - 1, 2, prob.N + 4, n - 1])
    dk, dv = oracle.key_grads(prob, keys, dO, row_chunk=5)
    assert np.max(np.abs(dk - dK[keys])) < 1e-12 and np.max(np.abs(dv - dV[keys])) < 1e-12
    # restricted to one kv group's heads
    dk1, dv1 = oracle.key_grads(prob, keys, dO, heads=[0, 1])
    dO1 = dO.copy()
    dO1[:, 2:] = 0
    _, dK1, dV1 = oracle.backward(prob, dO1, fwd=(O, lse))
    assert np.max(np.abs(dk1 - dK1[keys])) < 1e-12 and np.max(np.abs(dv1 - dV1[keys])) < 1e-12
    # restricted to one zigzag rank's rows: equal to the definition with the
    # other rows' dO set to zero (their dS and P dO vanish), and the ranks'
    # shares sum to the whole
    C = 3
    tot_k, tot_v = np.zeros_like(dk), np.zeros_like(dv)
    for r in range(C):
        pl = zigzag.plan(prob.cu, prob.bcu, prob.anchor, C, r)
        mine = np.concatenate([pl["main_index"], prob.N + pl["branch_index"]])
        dkr, dvr = oracle.key_grads(prob, keys, dO, row_chunk=7, rows=mine)
        dOr = np.zeros_like(dO)
        dOr[mine] = dO[mine]
        _, dKr, dVr = oracle.backward(prob, dOr, fwd=(O, lse))
        assert np.max(np.abs(dkr - dKr[keys])) < 1e-12 and np.max(np.abs(dvr - dVr[keys])) < 1e-12
        tot_k += dkr
        tot_v += dvr
    assert np.max(np.abs(tot_k - dK[keys])) < 1e-12 and np.max(np.abs(tot_v - dV[keys])) < 1e-12


# ---------------------------------------------------------------------------
# Input generator
# ---------------------------------------------------------------------------

def test_splitmix64_published_sequence():
    g = splitmix64(0)
    assert [next(g) for _ in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                           0x06C45D188009454F]


def test_varlen_lengths_seed0():
    lens = varlen_lengths(20480, 512, 8192, 0)
    assert sum(lens) == 20480 and all(512 <= L <= 8192 for L in lens[:-1])
    assert lens == (4573, 1522, 1382, 1818, 7909, 3276)


# ---------------------------------------------------------------------------
# Zigzag plan against hand-computed fixtures (chunk split, ownership, ring
# order and received bytes where 2C does not divide the length)
# ---------------------------------------------------------------------------

PLAN_FILES = sorted(f for f in os.listdir(GOLDEN) if f.startswith("plan_"))
PLAN_KEYS = ("main_index", "main_seq", "main_pos", "branch_ids", "branch_index", "branch_seq",
             "branch_pos", "branch_t", "local_branch_cu", "kv_src")


def load_plan_golden(name):
    """Returns (cu_seqlens, branch_cu, anchors, C, bytes_params, {rank: {key: array}})."""
    head, ranks, cur = {}, {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            vals = [int(v) for v in vals]
            if key == "rank":
                cur = ranks.setdefault(vals[0], {})
            elif cur is None:
                head[key] = vals
            else:
                cur[key] = np.asarray(vals, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(head["seqlens"])]).astype(np.int64)
    bcu = np.concatenate([[0], np.cumsum(head["branch_lens"])]).astype(np.int64)
    return cu, bcu, np.asarray(head["anchors"], np.int64), head["C"][0], head["bytes_params"], ranks


@pytest.mark.parametrize("fname", PLAN_FILES)
def test_zigzag_plan_matches_hand_computed_fixture(fname):
    cu, bcu, anchors, C, (hkv, d, eb), ranks = load_plan_golden(fname)
    assert sorted(ranks) == list(range(C))
    for r, want in ranks.items():
        got = zigzag.plan(cu, bcu, anchors, C, r)
        for key in PLAN_KEYS:
            assert np.array_equal(got[key], want[key]), (fname, r, key, got[key], want[key])
        assert zigzag.ring_bytes_received(cu, bcu, anchors, C, r, hkv, d, eb) == want["ring_bytes"][0]


# ---------------------------------------------------------------------------
# Mixed kinds: a packed batch equals its sequences run one by one, each with
# its single kind (packed sequences never see each other)
# ---------------------------------------------------------------------------

def test_mixed_pack_equals_sequences_alone():
    pack = SMALL_CASES["mixed_kinds"](hq=4, hkv=2, d=6, seed=11)
    O, lse = oracle.forward(pack, block_pos=3)
    dO = np.random.default_rng(5).standard_normal(O.shape)
    dQ, dK, dV = oracle.backward(pack, dO, fwd=(O, lse), block_pos=3)
    b0 = 0
    for s, L in enumerate(MIXED["seqlens"]):
        nA = len(MIXED["anchors"][s])
        lens = MIXED["lens"][b0:b0 + nA]
        kinds = set(MIXED["kinds"][b0:b0 + nA])
        assert len(kinds) == 1
        m = slice(int(pack.cu[s]), int(pack.cu[s + 1]))
        br = slice(int(pack.bcu[b0]), int(pack.bcu[b0 + nA]))
        alone = Problem([0, L], np.concatenate([[0], np.cumsum(lens)]), MIXED["anchors"][s],
                        kinds.pop(), pack.hq, pack.hkv, pack.d, pack.q[m], pack.k[m], pack.v[m],
                        pack.qb[br], pack.kb[br], pack.vb[br])
        rows = np.concatenate([np.arange(m.start, m.stop), pack.N + np.arange(br.start, br.stop)])
        o1, l1 = oracle.forward(alone, block_pos=3)
        g1 = oracle.backward(alone, dO[rows], fwd=(o1, l1), block_pos=3)
        assert np.allclose(O[rows], o1, atol=1e-13) and np.allclose(lse[rows], l1, atol=1e-13)
        for full, one in zip((dQ, dK, dV), g1):
            assert np.allclose(full[rows], one, atol=1e-12)
        b0 += nA


def test_mixed_pack_pair_count():
    """Per-branch closed forms: main L(L+1)/2; a branch row sees its anchor's
    position + 1 main keys; inside a branch B(B+1)/2 (causal) or B^2 (bidir)."""
    pack = SMALL_CASES["mixed_kinds"](hq=2, hkv=1, d=2)
    main = sum(L * (L + 1) // 2 for L in MIXED["seqlens"])
    pos = [p for ps in MIXED["anchors"] for p in ps]
    br_main = sum(B * (p + 1) for B, p in zip(MIXED["lens"], pos))
    local = sum(B * (B + 1) // 2 if k == "causal" else B * B
                for B, k in zip(MIXED["lens"], MIXED["kinds"]))
    assert pack.count_visible() == main + br_main + local
    assert brute.count_pairs(pack.cu, pack.bcu, pack.anchor, MIXED["kinds"]) == main + br_main + local
