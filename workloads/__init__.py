"""Seeded synthetic workloads for branch-aware causal attention.

This package only builds inputs: sequence lengths, anchor/branch structure and
random tensors.  It holds none of the attention arithmetic, so both the CPU
oracle (``oracle/``) and the HIP path (``branch_aware_causal_amd``) may use it
without sharing any of the method's code.

Page keys used in citations throughout the repository:

* [G]  gptget.net summary page of report 2609.07108 (Chinese summary that ends
       with the English abstract, section 原文摘要).
* [AF] ai-feeds.com page "大规模长上下文 RL 后训练中面向投机解码的 Online Draft
       Co-Training".
* [R]  rebasdaily.com news article on the same report (2026-09-10 topic page).
"""

from .specs import (WORKLOADS, Workload, get, splitmix64, varlen_lengths)
from .gen import Structure, make_structure, make_tensors, numpy_rows

__all__ = ["WORKLOADS", "Workload", "get", "splitmix64", "varlen_lengths",
           "Structure", "make_structure", "make_tensors", "numpy_rows"]
