"""Float64 CPU oracle for one learnable-channel-permutation (LCP) step.

TEST INFRASTRUCTURE. This package is the plain, slow, obviously correct
reference that the GPU library is checked against. Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does, and it shares no code with the HIP library.

Sources (cited by page title and section):

* [PermLLM summary] "PermLLM: Learnable Channel Permutation for N:M Sparse
  Large Language Models" (arXiv 2510.10136, summary page): task definition,
  Method 1 (soft permutation by Sinkhorn normalisation), Method 2 (hardening),
  Method 3 (block-wise channel permutation), the integration formula for the
  importance-based N:M mask, implementation details.
* [PermLLM blog] "PermLLM: 动态通道置换优化N:M稀疏大模型" (blog post):
  section 2.1 (N:M sparsity), section 2.2 (log-domain Sinkhorn, rows then
  columns), section 5.1 (P kept in FP32).

Every function is pinned by the CPU tests against closed forms, hand-worked
examples, brute force or finite differences; none is marked parity unpinned.
"""
from .lcp import *  # noqa: F401,F403
from .lcp import __all__  # noqa: F401
