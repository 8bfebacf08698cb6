"""Host-side tests of libbac: exports, argument validation, and the C++ zigzag
plan against the oracle's independent Python plan (bit-exact).  No GPU work
is launched: every call here either is host-only or fails validation before
anything is enqueued."""

import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import zigzag as ozz
from workloads import WORKLOADS, make_structure
from workloads.gen import make_structure_custom

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from branch_aware_causal_amd import _lib
    return _lib.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "bac.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:bac_status|const char\*|int32_t)\s+(\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol(lib):
    names = header_functions()
    assert {"zigzag_shard_plan", "attn_main_fwd", "attn_main_bwd", "attn_branch_fwd",
            "attn_branch_bwd", "lse_merge", "attn_bwd_delta", "attn_check_index",
            "bac_last_error", "bac_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_matches_the_header_generation(lib):
    # 0.2.0 added the per-branch kind array of the branch calls and the
    # feature hand-off pair
    assert lib.bac_version() == 200
    assert {"tap_send", "tap_recv"} <= set(header_functions())


def test_binding_rejects_mixed_kind_without_per_branch_kinds():
    from branch_aware_causal_amd import api
    with pytest.raises(ValueError, match="mixed"):
        api._branch_kinds("mixed", None, 3)
    assert api._branch_kinds("causal", None, 3).value is None


def test_binding_has_the_same_names():
    import branch_aware_causal_amd as bac
    for n in header_functions():
        if n.startswith("bac_"):
            continue
        assert callable(getattr(bac, n)), n


def _call_main_fwd(lib, **over):
    a = dict(q=1, q_seq=1, q_pos=1, nq=4, k=1, v=1, k_seq=1, k_pos=1, nk=4, hq=8, hkv=2, d=128,
             dt=1, scale=0.1, o_acc=1, lse=1, mode=0, o_out=None, stream=None)
    a.update(over)
    vpp = lambda x: C.c_void_p(x)
    return lib.attn_main_fwd(vpp(a["q"]), vpp(a["q_seq"]), vpp(a["q_pos"]), a["nq"], vpp(a["k"]),
                             vpp(a["v"]), vpp(a["k_seq"]), vpp(a["k_pos"]), a["nk"], a["hq"],
                             a["hkv"], a["d"], a["dt"], a["scale"], vpp(a["o_acc"]),
                             vpp(a["lse"]), a["mode"], vpp(a["o_out"]), vpp(a["stream"]))


@pytest.mark.parametrize("over,code,needle", [
    (dict(q=None), -1, "null query"),
    (dict(k_seq=None), -1, "null key"),
    (dict(hq=6, hkv=4), -1, "multiple"),
    (dict(hq=12, hkv=4), -2, "divide 32"),
    (dict(d=96), -2, "head dim"),
    (dict(dt=7), -1, "dtype"),
    (dict(mode=3), -1, "mode"),
    (dict(nq=-1), -1, "negative"),
    (dict(o_acc=None), -1, "o_acc"),
    (dict(scale=float("inf")), -1, "scale"),
    (dict(scale=0.0), -2, "not positive"),
    (dict(scale=-0.1), -2, "not positive"),
    (dict(nq=2**29, hq=8), -3, "2^31"),
    (dict(nq=2**28, hq=8), -3, "2^31"),      # n * hq = 2^31 exactly
    (dict(nk=2**26, hq=32), -3, "2^31"),
])
def test_main_fwd_rejects_bad_arguments(lib, over, code, needle):
    from branch_aware_causal_amd import _lib
    assert _call_main_fwd(lib, **over) == code
    assert needle in _lib.last_error()


def test_misaligned_tensors_are_rejected_before_launch(lib):
    # every other argument valid; tensor pointers off a 16-byte boundary
    from branch_aware_causal_amd import _lib
    assert _call_main_fwd(lib, q=24, k=32, v=48, o_acc=64) == -1
    assert "16-byte aligned" in _lib.last_error()
    vp = C.c_void_p
    st = lib.attn_branch_fwd(vp(16), vp(40), vp(48), 8, vp(4), 2, 3, 0, vp(None), 8, 2, 128, 1,
                             0.1, vp(64), vp(4), 0, vp(None), vp(None))
    assert st == -1 and "16-byte aligned" in _lib.last_error()
    st = lib.lse_merge(vp(16), vp(4), vp(36), vp(4), 4, 8, 128, 1, vp(None), vp(None))
    assert st == -1 and "16-byte aligned" in _lib.last_error()


def test_empty_calls_are_noops(lib):
    # nothing to do -> success without touching any pointer or device
    assert _call_main_fwd(lib, nq=0, q=None, q_seq=None, q_pos=None, o_acc=None, lse=None) == 0
    vp = C.c_void_p
    assert lib.lse_merge(vp(None), vp(None), vp(None), vp(None), 0, 8, 128, 1, vp(None), vp(None)) == 0
    assert lib.attn_bwd_delta(vp(None), 0, vp(None), 1, 0, 8, 128, vp(None), vp(None)) == 0


def test_branch_and_merge_validation(lib):
    from branch_aware_causal_amd import _lib
    vp = C.c_void_p
    # max_branch_len beyond the supported bound
    st = lib.attn_branch_fwd(vp(1), vp(1), vp(1), 8, vp(1), 2, 257, 0, vp(None), 8, 2, 128, 1,
                             0.1, vp(1), vp(1), 0, vp(None), vp(None))
    assert st == -2 and "max_branch_len" in _lib.last_error()
    st = lib.attn_branch_bwd(vp(1), vp(1), vp(1), 8, vp(1), 2, 4, 5, vp(None), 8, 2, 128, 1, 0.1,
                             vp(1), vp(1), vp(1), vp(1), vp(1), vp(1), vp(None))
    assert st == -1 and "kind" in _lib.last_error()
    for bad in (0.0, -1.0):
        st = lib.attn_branch_fwd(vp(16), vp(16), vp(16), 8, vp(4), 2, 4, 0, vp(None), 8, 2, 128,
                                 1, bad, vp(16), vp(4), 0, vp(None), vp(None))
        assert st == -2 and "not positive" in _lib.last_error()
        st = lib.attn_main_bwd(vp(16), vp(4), vp(4), 4, vp(16), vp(16), vp(4), vp(4), 4, 8, 2, 128,
                               1, bad, vp(16), vp(4), vp(4), vp(16), vp(16), vp(16), vp(None))
        assert st == -2 and "not positive" in _lib.last_error()
    st = lib.lse_merge(vp(1), vp(1), vp(1), vp(1), 4, 8, 128, 1, vp(None), vp(None))
    assert st == -1 and "alias" in _lib.last_error()
    st = lib.attn_main_bwd(vp(1), vp(1), vp(1), 4, vp(1), vp(1), vp(1), vp(1), 4, 8, 2, 128, 1,
                           0.1, vp(None), vp(1), vp(1), vp(1), vp(1), vp(1), vp(None))
    assert st == -1 and "dout" in _lib.last_error()


def _plan_c(st, C_, r):
    from branch_aware_causal_amd import zigzag_shard_plan
    return zigzag_shard_plan(st.cu_seqlens, st.branch_cu, st.branch_anchor, C_, r)


STRUCTS = {
    "eagle_varlen": lambda: make_structure_custom((9, 16, 3, 40, 1), [list(range(L)) for L in (9, 16, 3, 40, 1)],
                                                  [3] * 69, "causal"),
    "dflash": lambda: make_structure_custom((64, 33), [list(range(0, 64, 16)), list(range(0, 33, 16))],
                                            [16] * 7, "bidir"),
    "ragged": lambda: make_structure_custom((5, 0, 7, 2), [[0, 4], [], [1, 2, 6], [1]],
                                            [2, 1, 4, 3, 2, 5], "causal"),
    "varlen_20k": lambda: make_structure(WORKLOADS["eagle3_varlen_20k"]),
}


@pytest.mark.parametrize("C_", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("name", sorted(STRUCTS))
def test_plan_matches_oracle_plan_bit_exactly(name, C_):
    st = STRUCTS[name]()
    for r in range(C_):
        got = _plan_c(st, C_, r)
        ref = ozz.plan(st.cu_seqlens, st.branch_cu, st.branch_anchor, C_, r)
        for key in ref:
            assert np.array_equal(got[key], ref[key].astype(np.int32)), (name, C_, r, key)


def test_plan_of_256k_rank0_of_8():
    st = make_structure(WORKLOADS["eagle3_256k_rank0_of_8"])
    got = _plan_c(st, 8, 0)
    assert got["main_index"].size == 32768
    assert np.array_equal(got["main_index"][:16384], np.arange(16384))
    assert np.array_equal(got["main_index"][16384:], np.arange(15 * 16384, 16 * 16384))
    assert np.array_equal(got["kv_src"], [0, 7, 6, 5, 4, 3, 2, 1])
    assert got["branch_index"].size == 3 * 32768


@pytest.mark.parametrize("args,needle", [
    (dict(cp=0), "cp_size"),
    (dict(rank=4), "rank"),
    (dict(cu=[1, 4]), "cu_seqlens[0]"),
    (dict(cu=[0, 5, 3]), "decreases"),
    (dict(anchor=[1, 0]), "not sorted"),
    (dict(anchor=[0, 99]), "outside"),
])
def test_plan_rejects_malformed_inputs(args, needle):
    from branch_aware_causal_amd import BacError, zigzag_shard_plan
    cu = args.get("cu", [0, 5, 9])
    anchor = args.get("anchor", [0, 6])
    bcu = [0, 2, 4]
    with pytest.raises(BacError) as ei:
        zigzag_shard_plan(cu, bcu, anchor, args.get("cp", 2), args.get("rank", 0))
    assert ei.value.status == -1 and needle in ei.value.message


def test_plan_matches_hand_computed_fixtures():
    """The C++ plan against the hand-computed fixtures of tests/golden
    (floor chunk split where 2C does not divide the length, an empty
    sequence, branch ownership, ring order)."""
    from test_oracle import PLAN_FILES, PLAN_KEYS, load_plan_golden
    from branch_aware_causal_amd import zigzag_shard_plan
    for fname in PLAN_FILES:
        cu, bcu, anchors, C_, _, ranks = load_plan_golden(fname)
        for r, want in ranks.items():
            got = zigzag_shard_plan(cu, bcu, anchors, C_, r)
            for key in PLAN_KEYS:
                assert np.array_equal(got[key], want[key].astype(np.int32)), (fname, r, key)


@pytest.mark.parametrize("over,needle", [
    (dict(slots=None), "null"),
    (dict(slot=2), "outside"),
    (dict(slot=-1), "outside"),
    (dict(nbytes=4097), "outside [0, slot_bytes]"),
    (dict(slot_bytes=100), "multiple of 16"),
    (dict(seq=0), "start at 1"),
    (dict(buf=8), "16-byte aligned"),
    (dict(stamps=12), "8-byte aligned"),
])
def test_mailbox_calls_reject_bad_arguments(lib, over, needle):
    from branch_aware_causal_amd import _lib
    a = dict(slots=256, stamps=16, nslots=2, slot_bytes=4096, slot=1, buf=512, nbytes=4096, seq=3)
    a.update(over)
    vp = C.c_void_p
    st = lib.tap_send(vp(a["slots"]), vp(a["stamps"]), a["nslots"], a["slot_bytes"], a["slot"],
                      vp(a["buf"]), a["nbytes"], a["seq"], vp(None))
    assert st == -1 and needle in _lib.last_error(), _lib.last_error()
    st = lib.tap_recv(vp(a["slots"]), vp(a["stamps"]), a["nslots"], a["slot_bytes"], a["slot"],
                      a["seq"], 100, vp(a["buf"]), a["nbytes"], vp(64), vp(None))
    assert st == -1 and needle in _lib.last_error(), _lib.last_error()


def test_mailbox_recv_rejects_bad_wait_arguments(lib):
    from branch_aware_causal_amd import _lib
    vp = C.c_void_p
    st = lib.tap_recv(vp(256), vp(16), 2, 4096, 1, 3, 0, vp(512), 4096, vp(64), vp(None))
    assert st == -1 and "spin_limit" in _lib.last_error()
    st = lib.tap_recv(vp(256), vp(16), 2, 4096, 1, 3, 10, vp(512), 4096, vp(None), vp(None))
    assert st == -1 and "status" in _lib.last_error()
