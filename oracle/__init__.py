"""Plain CPU oracle for MiniMax-M3 block-sparse paged attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package.  The product path (``block_sparse_paged_query_amd``) never imports it
and never falls back to it: the two share no code.

Everything here is written from the three vLLM API documentation pages the
method is described on, cited by page title and section:

* ``vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer`` (the FlashInfer
  attend, ``MiniMaxM3SparseFlashInferImpl.forward``)
* ``vllm.models.minimax_m3.amd.sparse_attention_nvfp4`` (the ROCm NVFP4 attend:
  ``customize_spec``, ``MiniMaxM3SparseRocmNvfp4Impl``,
  ``MiniMaxM3SparseRocmNvfp4MetadataBuilder.build``)
* ``vllm.models.minimax_m3.amd.ops.sparse_pa`` (the page-16 table helpers:
  ``_write_sparse_block_table_row_from_values``, the decode / prefill table
  builders, ``minimax_m3_insert_index_cache``,
  ``minimax_m3_rebase_block_table_to_page16``,
  ``minimax_m3_sparse_block_page_stride``)

Floating point is fp64 throughout.  Each function is pinned by a CPU test
under ``tests/`` against something other than itself (worked examples,
closed forms, library routines, brute force).  Two conventions the pages
leave open cannot be pinned and are marked "parity unpinned" where they are
defined:

* parity unpinned: the NVFP4 in-page byte order (``nvfp4_token_values``), a
  layout of ours; only the quantise -> dequantise error bound checks it;
* parity unpinned: the zero output of a row with an empty context
  (``attend_row``).

The grouped-query head mapping is a reading too, but it is pinned to torch's
``enable_gqa`` convention.
"""

from .msa_oracle import *  # noqa: F401,F403
from .msa_oracle import __all__  # noqa: F401
