"""paged_kv_attention_scatter_amd: paged KV attention, KV scatter and batched
sampling for MI355X (gfx950).

The product is libpkv.so (hand-written HIP kernels behind the C ABI of
include/pkv.h). This package is its thin Python binding:

* store_kv                  -- pkv_store_kv
* paged_attention_decode    -- pkv_paged_attention_decode
* paged_attention_decode_store -- pkv_paged_attention_decode_store (store_kv fused in)
* paged_attention_decode_noalloc -- pkv_paged_attention_decode_noalloc
* paged_attention_extend    -- pkv_paged_attention_extend
* qk_norm_rope_store_kv     -- pkv_qk_norm_rope_store_kv
* embedding_gather          -- pkv_embedding_gather
* sample                    -- pkv_sample
* num_pages, prepare_sampling, read_faults -- host helpers

Build the library with ``python -m paged_kv_attention_scatter_amd.build``.
"""

from .api import (HEAD_DIM, decode_workspace_size, embedding_gather, extend_workspace_size, make_pool, num_pages,
                  paged_attention_decode, paged_attention_decode_noalloc, paged_attention_decode_store,
                  paged_attention_extend, prepare_sampling,
                  qk_norm_rope_store_kv, read_faults, sample, sample_workspace, sample_workspace_size, store_kv,
                  version)
from ._lib import LIB_PATH, PkvError, lib

__all__ = [
    "HEAD_DIM", "LIB_PATH", "PkvError", "lib", "make_pool", "store_kv", "qk_norm_rope_store_kv", "embedding_gather", "paged_attention_decode",
    "paged_attention_decode_noalloc", "paged_attention_decode_store", "paged_attention_extend", "sample", "num_pages", "prepare_sampling", "read_faults",
    "decode_workspace_size", "extend_workspace_size", "sample_workspace", "sample_workspace_size", "version",
]
