"""Workload specifications (shapes, branch structure, seeds).

The workloads stand in for the pages' measurements, which used RL rollouts
that are not available here:

* the variable-length EAGLE-3 operator test whose longest case is 20,480
  tokens and the fixed 256K-token EAGLE-3 TTT scaling test ([R] section
  "长上下文才是系统设计的主场"; [G] 关键结果 and 结果分析);
* the three draft families whose branch patterns the method must serve:
  EAGLE-3 test-time training (a depth-D chain at every position), DFlash
  block diffusion (a whole block guessed at once, bidirectional inside) and
  DSpark's Markov head (a block corrected in order, causal inside)
  ([G] 深度分析 · 研究背景 and the 简单解释 section).

Every tensor is synthetic and seeded; nothing here is a dataset item.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

_MASK64 = (1 << 64) - 1


def splitmix64(seed: int):
    """Vigna's SplitMix64 generator (public-domain definition, 2015).

    state += 0x9E3779B97F4A7C15; z = state;
    z = (z ^ z>>30) * 0xBF58476D1CE4E5B9; z = (z ^ z>>27) * 0x94D049BB133111EB;
    return z ^ z>>31.
    """
    state = seed & _MASK64
    while True:
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        yield z ^ (z >> 31)


def varlen_lengths(total: int, lo: int, hi: int, seed: int) -> Tuple[int, ...]:
    """Split ``total`` tokens into sequences of length in [lo, hi].

    While more than ``hi`` tokens remain, draw L = lo + x mod (min(hi, rem-lo)
    - lo + 1) from SplitMix64; the remainder (<= hi) is the last sequence.
    """
    gen = splitmix64(seed)
    rem = total
    out = []
    while rem > hi:
        x = next(gen)
        span = min(hi, rem - lo) - lo + 1
        L = lo + x % span
        out.append(int(L))
        rem -= L
    out.append(int(rem))
    return tuple(out)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.

    branch: 'eagle3' (depth-D chain at every position), 'dflash' (block of B
    tokens every ``anchor_stride`` positions, bidirectional inside) or
    'dspark' (block of B tokens every ``anchor_stride`` positions, causal
    inside).  ``branch_len`` is D or B.
    'mixed' takes one (family, length, stride) per sequence from ``mix``.
    """
    name: str
    seqlens: Tuple[int, ...]
    hq: int
    hkv: int
    d: int
    dtype: str                 # 'f32' or 'bf16'
    branch: str
    branch_len: int
    anchor_stride: int
    value_scale: float
    seed_base: int
    cp: int = 1                # zigzag ring size whose rank-0 share is timed
    rank: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict, compare=False)
    # branch == 'mixed': one (family, length, stride) per sequence
    mix: Tuple[Tuple[str, int, int], ...] = ()

    @property
    def kind(self) -> str:
        if self.branch == "mixed":
            return "mixed"
        return "bidir" if self.branch == "dflash" else "causal"

    @property
    def n_main(self) -> int:
        return int(sum(self.seqlens))


VARLEN_20K = varlen_lengths(20480, 512, 8192, 0)

WORKLOADS = {
    w.name: w for w in [
        Workload("eagle3_tiny_fp32", (96, 160), 4, 2, 64, "f32", "eagle3", 3, 1,
                 1.0, 100, note="EAGLE-3 TTT depth 3, two packed sequences"),
        Workload("eagle3_varlen_20k", VARLEN_20K, 32, 8, 128, "bf16", "eagle3", 4,
                 1, 0.5, 200,
                 note="EAGLE-3 TTT depth 4, 20,480 packed tokens, lengths 512-8192"),
        Workload("dflash_32k", (32768,), 32, 8, 128, "bf16", "dflash", 16, 16,
                 1.0, 300, note="DFlash blocks of 16 every 16 positions"),
        Workload("dspark_4x16k", (16384,) * 4, 32, 8, 128, "bf16", "dspark", 8, 8,
                 1.0, 400, note="DSpark blocks of 8 every 8 positions"),
        Workload("eagle3_256k", (262144,), 32, 8, 128, "bf16", "eagle3", 3, 1,
                 1.0, 500, note="EAGLE-3 TTT depth 3, one 262,144-token sequence"),
        Workload("eagle3_256k_rank0_of_8", (262144,), 32, 8, 128, "bf16", "eagle3",
                 3, 1, 1.0, 500, cp=8, rank=0,
                 note="rank 0's share of the 256K sequence under a zigzag ring of 8"),
        # the 256K scale with the two block-draft families
        Workload("dflash_256k", (262144,), 32, 8, 128, "bf16", "dflash", 16, 16,
                 1.0, 600, note="DFlash blocks of 16 every 16 positions, one 262,144-token sequence"),
        Workload("dspark_256k", (262144,), 32, 8, 128, "bf16", "dspark", 8, 8,
                 1.0, 700, note="DSpark blocks of 8 every 8 positions, one 262,144-token sequence"),
        # one varlen pack mixing the three families, one family per sequence
        Workload("mixed_12k", (4096, 6144, 2048), 32, 8, 128, "bf16", "mixed", 16, 1, 1.0, 800,
                 note="EAGLE-3 depth 3 / DFlash B=16 / DSpark B=8 in one packed batch",
                 mix=(("eagle3", 3, 1), ("dflash", 16, 16), ("dspark", 8, 8))),
        # same length and branch rule as the 256K workload, small enough to
        # check in full against the oracle (unsharded and under a ring of 8)
        Workload("eagle3_32k", (32768,), 32, 8, 128, "bf16", "eagle3", 3, 1, 1.0, 900,
                 note="EAGLE-3 TTT depth 3, one 32,768-token sequence"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def small(name: str, seqlens, hq=4, hkv=2, d=64, dtype="f32", branch="eagle3",
          branch_len=3, anchor_stride=1, value_scale=1.0, seed_base=900, mix=()) -> Workload:
    """A custom small workload for tests (same recipe, other sizes)."""
    return Workload(name, tuple(int(x) for x in seqlens), hq, hkv, d, dtype, branch,
                    branch_len, anchor_stride, value_scale, seed_base, mix=tuple(mix))
