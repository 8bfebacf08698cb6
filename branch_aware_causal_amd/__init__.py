"""branch_aware_causal_amd -- branch-aware causal attention for MI355X (gfx950).

Merged main + branch attention for online draft co-training: packed
variable-length causal attention of the main sequence, rank-local branch
attention for EAGLE-3 TTT / DFlash / DSpark draft queries, and the
online-softmax merge, forward and backward, behind the C ABI of libbac.so
(include/bac.h).  Page keys in citations: [G] gptget.net summary of report
2609.07108, [R] rebasdaily.com article on it.
"""

from .api import (BacError, BAC_OK, BAC_EINVAL, BAC_EUNSUPPORTED, BAC_ESIZE, BAC_EHIP, F32, BF16,
                  WRITE, MERGE, CAUSAL, BIDIR, zigzag_shard_plan, attn_main_fwd, attn_branch_fwd,
                  lse_merge, attn_bwd_delta, attn_main_bwd, attn_main_bwd_dq, attn_main_bwd_dkdv,
                  attn_branch_bwd, attn_check_index, tap_send, tap_recv)
from . import ring, flops, accounting

__all__ = ["BacError", "BAC_OK", "BAC_EINVAL", "BAC_EUNSUPPORTED", "BAC_ESIZE", "BAC_EHIP",
           "F32", "BF16", "WRITE", "MERGE", "CAUSAL", "BIDIR", "zigzag_shard_plan",
           "attn_main_fwd", "attn_branch_fwd", "lse_merge", "attn_bwd_delta", "attn_main_bwd",
           "attn_main_bwd_dq", "attn_main_bwd_dkdv",
           "attn_branch_bwd", "attn_check_index", "tap_send", "tap_recv", "ring", "flops",
           "accounting"]
