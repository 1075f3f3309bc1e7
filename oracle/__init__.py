"""CPU float64 oracle for block-sparse attention forward and its metadata.

TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct reference.  Only
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
it.  It shares no code with the HIP library and never imports it.

Every function here is pinned by CPU tests (tests/test_oracle_*.py) against
page examples, closed forms, brute force and library routines; none is
"parity unpinned".
"""
from .attention import (MASK_CAUSAL, MASK_KV_VALID_COUNT, MASK_LOCAL, MASK_NONE,  # noqa: F401
                        block_sparsity, blocksparse_attention, dense_attention,
                        expand_element_mask, mask_mod_keep, softmax_weights,
                        varlen_blocksparse_attention)
from .metadata import (bitmask_to_index, bitmask_to_mask, cdiv,  # noqa: F401
                       expand_kv_blocks, index_to_mask, mask_to_index,
                       pack_varlen_lists, varlen_offsets)
from .proxy import block_summaries, proxy_attention, proxy_attention_bwd  # noqa: F401
from .backward import (blocksparse_attention_bwd, element_mask, kv_major_lists,  # noqa: F401
                       varlen_blocksparse_attention_bwd, varlen_kv_major_lists)
