"""ctypes loader for libbac.so (the C ABI declared in include/bac.h).

The library is loaded after torch so that both share one HIP runtime (they
resolve the same libamdhip64 soname).  A missing library is an error: there
is no fallback implementation.
"""

from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbac.so")

i32 = C.c_int32
f32 = C.c_float
vp = C.c_void_p
pi32 = C.POINTER(C.c_int32)


class PlanSizes(C.Structure):
    _fields_ = [("n_main", i32), ("n_branch_tok", i32), ("n_branches", i32)]


class PlanOut(C.Structure):
    _fields_ = [(name, pi32) for name in (
        "main_index", "main_seq", "main_pos", "branch_ids", "branch_index", "branch_seq",
        "branch_pos", "branch_t", "local_branch_cu", "kv_src")]


# name -> argtypes (restype is always int32 status unless noted)
SIGNATURES = {
    "zigzag_shard_plan": [pi32, i32, pi32, pi32, i32, i32, i32, C.POINTER(PlanSizes),
                          C.POINTER(PlanOut)],
    "attn_main_fwd": [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                      vp, vp, i32, vp, vp],
    "attn_branch_fwd": [vp, vp, vp, i32, vp, i32, i32, i32, vp, i32, i32, i32, i32, f32,
                        vp, vp, i32, vp, vp],
    "lse_merge": [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp],
    "attn_bwd_delta": [vp, i32, vp, i32, i32, i32, i32, vp, vp],
    "attn_main_bwd": [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                      vp, vp, vp, vp, vp, vp, vp],
    "attn_main_bwd_dq": [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                         vp, vp, vp, vp, vp],
    "attn_main_bwd_dkdv": [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                           vp, vp, vp, vp, vp, vp],
    "attn_branch_bwd": [vp, vp, vp, i32, vp, i32, i32, i32, vp, i32, i32, i32, i32, f32,
                        vp, vp, vp, vp, vp, vp, vp],
    "attn_check_index": [vp, vp, i32, i32, vp, vp],
    "tap_send": [vp, vp, i32, C.c_int64, i32, vp, C.c_int64, C.c_uint64, vp],
    "tap_recv": [vp, vp, i32, C.c_int64, i32, C.c_uint64, C.c_int64, vp, C.c_int64, vp, vp],
    "bac_version": [],
}

_lib = None


def load(path: str | None = None):
    """Load libbac.so once and declare its entry points."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    # BAC_LIB names another build of the same ABI (e.g. a sanitizer build)
    p = path or os.environ.get("BAC_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build it with `python -m branch_aware_causal_amd.build` "
            "(hipcc, gfx950); there is no fallback implementation")
    try:
        import torch  # noqa: F401  -- share torch's HIP runtime
    except ImportError:
        pass
    lib = C.CDLL(p)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = i32
    lib.bac_last_error.argtypes = []
    lib.bac_last_error.restype = C.c_char_p
    if path is None:
        _lib = lib
    return lib


def last_error() -> str:
    msg = load().bac_last_error()
    return msg.decode() if msg else ""
