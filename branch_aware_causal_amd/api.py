"""Python binding of libbac: the C ABI's entry points, same names, torch
tensors in, argument marshalling only.  Every computation runs in the HIP
library; a failing call raises BacError with the library's message.
"""

from __future__ import annotations

import ctypes as C
import math

import numpy as np

from . import _lib

BAC_OK, BAC_EINVAL, BAC_EUNSUPPORTED, BAC_ESIZE, BAC_EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
WRITE, MERGE = 0, 1
CAUSAL, BIDIR = 0, 1

_MODES = {"write": WRITE, "merge": MERGE, WRITE: WRITE, MERGE: MERGE}
# "mixed": per-branch kinds come in branch_kinds; the default kind is unused
_KINDS = {"causal": CAUSAL, "bidir": BIDIR, "mixed": CAUSAL, CAUSAL: CAUSAL, BIDIR: BIDIR}


class BacError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libbac status {status}: {message}")
        self.status = status
        self.message = message


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t):
    return C.c_void_p(None) if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, shape=None, device=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check(status: int):
    if status != BAC_OK:
        raise BacError(status, _lib.last_error())


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def zigzag_shard_plan(cu_seqlens, branch_cu, branch_anchor, cp_size: int, rank: int):
    """Host plan of rank `rank` under a zigzag ring of `cp_size` ranks.
    Returns a dict of int32 numpy arrays (see include/bac.h)."""
    lib = _lib.load()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    bcu = np.ascontiguousarray(np.asarray(branch_cu, dtype=np.int32))
    anc = np.ascontiguousarray(np.asarray(branch_anchor, dtype=np.int32))
    A = int(anc.shape[0])
    P = lambda a: a.ctypes.data_as(_lib.pi32)
    sizes = _lib.PlanSizes()
    st = lib.zigzag_shard_plan(P(cu), int(cu.shape[0]) - 1, P(bcu), P(anc), A, int(cp_size),
                               int(rank), C.byref(sizes), None)
    _check(st)
    nm, nbt, nbr = sizes.n_main, sizes.n_branch_tok, sizes.n_branches
    arrs = {
        "main_index": nm, "main_seq": nm, "main_pos": nm, "branch_ids": nbr,
        "branch_index": nbt, "branch_seq": nbt, "branch_pos": nbt, "branch_t": nbt,
        "local_branch_cu": nbr + 1, "kv_src": int(cp_size),
    }
    out_np = {k: np.zeros(max(v, 1), dtype=np.int32) for k, v in arrs.items()}
    out = _lib.PlanOut(**{k: P(a) for k, a in out_np.items()})
    st = lib.zigzag_shard_plan(P(cu), int(cu.shape[0]) - 1, P(bcu), P(anc), A, int(cp_size),
                               int(rank), C.byref(sizes), C.byref(out))
    _check(st)
    return {k: out_np[k][:arrs[k]].copy() for k in arrs}


def attn_main_fwd(q, q_seq, q_pos, k, v, k_seq, k_pos, o_acc, lse, mode="write", o_out=None,
                  scale=None, stream=None):
    nq, hq, d = q.shape
    nk, hkv = k.shape[0], k.shape[1]
    torch = _torch()
    _need(q, "q")
    dt = _dt(q)
    _need(k, "k", q.dtype, (nk, hkv, d))
    _need(v, "v", q.dtype, (nk, hkv, d))
    for t, nm, n in ((q_seq, "q_seq", nq), (q_pos, "q_pos", nq), (k_seq, "k_seq", nk),
                     (k_pos, "k_pos", nk)):
        _need(t, nm, torch.int32, (n,))
    _need(o_acc, "o_acc", torch.float32, (nq, hq, d))
    _need(lse, "lse", torch.float32, (hq, nq))
    if o_out is not None:
        _need(o_out, "o_out", q.dtype, (nq, hq, d))
    st = _lib.load().attn_main_fwd(_ptr(q), _ptr(q_seq), _ptr(q_pos), nq, _ptr(k), _ptr(v),
                                   _ptr(k_seq), _ptr(k_pos), nk, hq, hkv, d, dt, _scale(scale, d),
                                   _ptr(o_acc), _ptr(lse), _MODES[mode], _ptr(o_out),
                                   _stream(stream))
    _check(st)


def _branch_kinds(kind, branch_kinds, A):
    """Per-branch kinds (device int32 [A], or None for one kind for all);
    kind "mixed" requires them."""
    if kind == "mixed" and branch_kinds is None:
        raise ValueError('kind "mixed" needs branch_kinds (int32, one per branch)')
    if branch_kinds is not None:
        _need(branch_kinds, "branch_kinds", _torch().int32, (A,))
    return _ptr(branch_kinds)


def attn_branch_fwd(qb, kb, vb, branch_cu, max_branch_len, kind, o_acc, lse, mode="write",
                    o_out=None, scale=None, stream=None, branch_kinds=None):
    nb, hq, d = qb.shape
    hkv = kb.shape[1]
    torch = _torch()
    _need(qb, "qb")
    dt = _dt(qb)
    _need(kb, "kb", qb.dtype, (nb, hkv, d))
    _need(vb, "vb", qb.dtype, (nb, hkv, d))
    _need(branch_cu, "branch_cu", torch.int32)
    A = branch_cu.shape[0] - 1
    kinds = _branch_kinds(kind, branch_kinds, A)
    _need(o_acc, "o_acc", torch.float32, (nb, hq, d))
    _need(lse, "lse", torch.float32, (hq, nb))
    if o_out is not None:
        _need(o_out, "o_out", qb.dtype, (nb, hq, d))
    st = _lib.load().attn_branch_fwd(_ptr(qb), _ptr(kb), _ptr(vb), nb, _ptr(branch_cu), A,
                                     int(max_branch_len), _KINDS[kind], kinds, hq, hkv, d, dt,
                                     _scale(scale, d), _ptr(o_acc), _ptr(lse), _MODES[mode],
                                     _ptr(o_out), _stream(stream))
    _check(st)


def lse_merge(o_acc, lse_acc, o_part, lse_part, o_out=None, stream=None):
    n, hq, d = o_acc.shape
    torch = _torch()
    _need(o_acc, "o_acc", torch.float32)
    _need(lse_acc, "lse_acc", torch.float32, (hq, n))
    _need(o_part, "o_part", torch.float32, (n, hq, d))
    _need(lse_part, "lse_part", torch.float32, (hq, n))
    out_dt = F32
    if o_out is not None:
        _need(o_out, "o_out", None, (n, hq, d))
        out_dt = _dt(o_out)
    st = _lib.load().lse_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), n, hq, d,
                               out_dt, _ptr(o_out), _stream(stream))
    _check(st)


def attn_bwd_delta(o, dout, delta, stream=None):
    n, hq, d = dout.shape
    torch = _torch()
    _need(o, "o", None, (n, hq, d))
    _need(dout, "dout")
    _need(delta, "delta", torch.float32, (hq, n))
    st = _lib.load().attn_bwd_delta(_ptr(o), _dt(o), _ptr(dout), _dt(dout), n, hq, d, _ptr(delta),
                                    _stream(stream))
    _check(st)


def _main_bwd_args(q, q_seq, q_pos, k, v, k_seq, k_pos, dout, lse, delta, dq, dk, dv):
    nq, hq, d = q.shape
    nk, hkv = k.shape[0], k.shape[1]
    torch = _torch()
    _need(q, "q")
    _need(k, "k", q.dtype, (nk, hkv, d))
    _need(v, "v", q.dtype, (nk, hkv, d))
    for t, nm, n in ((q_seq, "q_seq", nq), (q_pos, "q_pos", nq), (k_seq, "k_seq", nk),
                     (k_pos, "k_pos", nk)):
        _need(t, nm, torch.int32, (n,))
    _need(dout, "dout", q.dtype, (nq, hq, d))
    _need(lse, "lse", torch.float32, (hq, nq))
    _need(delta, "delta", torch.float32, (hq, nq))
    if dq is not None:
        _need(dq, "dq", torch.float32, (nq, hq, d))
    if dk is not None:
        _need(dk, "dk", torch.float32, (nk, hkv, d))
        _need(dv, "dv", torch.float32, (nk, hkv, d))
    return nq, hq, d, nk, hkv, _dt(q)


def attn_main_bwd(q, q_seq, q_pos, k, v, k_seq, k_pos, dout, lse, delta, dq, dk, dv, scale=None,
                  stream=None):
    nq, hq, d, nk, hkv, dt = _main_bwd_args(q, q_seq, q_pos, k, v, k_seq, k_pos, dout, lse, delta,
                                            dq, dk, dv)
    st = _lib.load().attn_main_bwd(_ptr(q), _ptr(q_seq), _ptr(q_pos), nq, _ptr(k), _ptr(v),
                                   _ptr(k_seq), _ptr(k_pos), nk, hq, hkv, d, dt, _scale(scale, d),
                                   _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _stream(stream))
    _check(st)


def attn_main_bwd_dq(q, q_seq, q_pos, k, v, k_seq, k_pos, dout, lse, delta, dq, scale=None,
                     stream=None):
    nq, hq, d, nk, hkv, dt = _main_bwd_args(q, q_seq, q_pos, k, v, k_seq, k_pos, dout, lse, delta,
                                            dq, None, None)
    st = _lib.load().attn_main_bwd_dq(_ptr(q), _ptr(q_seq), _ptr(q_pos), nq, _ptr(k), _ptr(v),
                                      _ptr(k_seq), _ptr(k_pos), nk, hq, hkv, d, dt,
                                      _scale(scale, d), _ptr(dout), _ptr(lse), _ptr(delta),
                                      _ptr(dq), _stream(stream))
    _check(st)


def attn_main_bwd_dkdv(q, q_seq, q_pos, k, v, k_seq, k_pos, dout, lse, delta, dk, dv, scale=None,
                       stream=None):
    nq, hq, d, nk, hkv, dt = _main_bwd_args(q, q_seq, q_pos, k, v, k_seq, k_pos, dout, lse, delta,
                                            None, dk, dv)
    st = _lib.load().attn_main_bwd_dkdv(_ptr(q), _ptr(q_seq), _ptr(q_pos), nq, _ptr(k), _ptr(v),
                                        _ptr(k_seq), _ptr(k_pos), nk, hq, hkv, d, dt,
                                        _scale(scale, d), _ptr(dout), _ptr(lse), _ptr(delta),
                                        _ptr(dk), _ptr(dv), _stream(stream))
    _check(st)


def attn_branch_bwd(qb, kb, vb, branch_cu, max_branch_len, kind, doutb, lseb, deltab, dqb, dkb,
                    dvb, scale=None, stream=None, branch_kinds=None):
    nb, hq, d = qb.shape
    hkv = kb.shape[1]
    torch = _torch()
    _need(qb, "qb")
    dt = _dt(qb)
    _need(kb, "kb", qb.dtype, (nb, hkv, d))
    _need(vb, "vb", qb.dtype, (nb, hkv, d))
    _need(branch_cu, "branch_cu", torch.int32)
    A = branch_cu.shape[0] - 1
    _need(doutb, "doutb", qb.dtype, (nb, hq, d))
    _need(lseb, "lseb", torch.float32, (hq, nb))
    _need(deltab, "deltab", torch.float32, (hq, nb))
    _need(dqb, "dqb", torch.float32, (nb, hq, d))
    _need(dkb, "dkb", torch.float32, (nb, hkv, d))
    _need(dvb, "dvb", torch.float32, (nb, hkv, d))
    kinds = _branch_kinds(kind, branch_kinds, A)
    st = _lib.load().attn_branch_bwd(_ptr(qb), _ptr(kb), _ptr(vb), nb, _ptr(branch_cu), A,
                                     int(max_branch_len), _KINDS[kind], kinds, hq, hkv, d, dt,
                                     _scale(scale, d), _ptr(doutb), _ptr(lseb), _ptr(deltab),
                                     _ptr(dqb), _ptr(dkb), _ptr(dvb), _stream(stream))
    _check(st)


def attn_check_index(seq, pos, strict: bool, stream=None) -> int:
    """Number of positions violating the (seq, pos) order (synchronises)."""
    torch = _torch()
    n = seq.shape[0]
    _need(seq, "seq", torch.int32, (n,))
    _need(pos, "pos", torch.int32, (n,))
    bad = torch.zeros(1, dtype=torch.int32, device=seq.device)
    st = _lib.load().attn_check_index(_ptr(seq), _ptr(pos), n, 1 if strict else 0, _ptr(bad),
                                      _stream(stream))
    _check(st)
    return int(bad.item())


def _mailbox(slots, stamps):
    torch = _torch()
    _need(slots, "slots")
    _need(stamps, "stamps", torch.int64)
    nslots = slots.shape[0]
    if stamps.shape != (nslots,):
        raise ValueError(f"stamps must have shape ({nslots},), got {tuple(stamps.shape)}")
    return nslots, slots[0].numel() * slots.element_size()


def tap_send(slots, stamps, slot: int, payload, seq: int, stream=None):
    """Copy `payload` into slot `slot` of the mailbox (slots [nslots, ...],
    stamps int64 [nslots]) and publish stamps[slot] = seq (include/bac.h)."""
    nslots, slot_bytes = _mailbox(slots, stamps)
    _need(payload, "payload")
    st = _lib.load().tap_send(_ptr(slots), _ptr(stamps), nslots, slot_bytes, int(slot),
                              _ptr(payload), payload.numel() * payload.element_size(), int(seq),
                              _stream(stream))
    _check(st)


def tap_recv(slots, stamps, slot: int, seq: int, out, status, spin_limit: int = 1 << 22,
             stream=None):
    """Wait (at most spin_limit polls) for stamps[slot] == seq, then copy the
    slot into `out`; status (int32 [1], device) receives 0 received, 1 gave
    up, 2 the slot holds a newer sequence."""
    torch = _torch()
    nslots, slot_bytes = _mailbox(slots, stamps)
    _need(out, "out")
    _need(status, "status", torch.int32, (1,))
    st = _lib.load().tap_recv(_ptr(slots), _ptr(stamps), nslots, slot_bytes, int(slot), int(seq),
                              int(spin_limit), _ptr(out), out.numel() * out.element_size(),
                              _ptr(status), _stream(stream))
    _check(st)
