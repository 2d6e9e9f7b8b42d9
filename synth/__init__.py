"""Seeded synthetic inputs for block-sparse paged attention.

This package builds inputs only: request lengths, block tables, top-k rows,
queries and paged K/V caches (encoded to bf16, fp8 E4M3FN or NVFP4).  It holds
none of the method's arithmetic: it never decodes codes, builds page tables,
masks or attends.  Both the HIP path's tests / benchmark and the CPU oracle's
tests draw their inputs from here.
"""

from .workloads import *  # noqa: F401,F403
from .workloads import __all__  # noqa: F401
