"""CPU oracle for branch-aware causal attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy implementation of what the method computes, written
from the pages and used to check the HIP library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``branch_aware_causal_amd`` and never
imports it; the only shared module is ``workloads`` (seeded inputs, none of
the method's arithmetic).

Page keys: [G] gptget.net summary of report 2609.07108, [AF] ai-feeds.com
page on the report, [R] rebasdaily.com article on the report.

Modes:
  * definition  (attention.forward / backward): one softmax per query row over
    the union of the main keys and its own branch keys under the mask.
  * brute       (brute.*): pure-Python loops with math.exp / math.fsum.
  * decomposed  (attention.forward_decomposed): main part and branch part
    computed separately and combined with the LSE merge of [G] 技术贡献.
  * zigzag      (zigzag.*): the oracle's own zigzag shard plan and a ring-order
    emulation of every rank, merged after each step.

Pins (tests/test_oracle.py): brute force, hand-written mask fixtures under
tests/golden/, the Q=0 closed form, one-hot V, closed-form pair counts,
torch SDPA on the purely causal case, finite differences, torch autograd,
gradient invariants and metamorphic shifts.  No function here is "parity
unpinned".
"""

from .problem import Problem
from .attention import (lse_merge, partial, grads, forward, backward,
                        forward_decomposed, forward_rows, backward_rows,
                        key_grads, delta)
from . import brute, zigzag

__all__ = ["Problem", "lse_merge", "partial", "grads", "forward", "backward",
           "forward_decomposed", "forward_rows", "backward_rows", "key_grads",
           "delta", "brute", "zigzag"]
