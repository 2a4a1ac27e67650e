"""KV scatter into the paged pool (oracle side; test infrastructure only).

Follows "Mini-SGLang 完整剖析" section 4.4.3 (one pool tensor per K and V,
viewed per layer as [num_pages * page_size, kv_heads, head_dim]; store_kv
writes the new rows through out_loc) and section 4.9.4 (the store kernel's
contract: caches [-1, D'] and inputs [L, D'] with D' = kv_heads * head_dim,
indices [L] of int32 or int64): row i of k goes to pool slot out_loc[i], and
the same for v. It is a pure copy, so the result is bit-for-bit.
"""

import numpy as np


def store_kv(k_pool: np.ndarray, v_pool: np.ndarray, out_loc: np.ndarray,
             k: np.ndarray, v: np.ndarray):
    """Returns new (k_pool, v_pool) arrays with the rows written.

    Arrays may hold any element type (bf16 bit patterns or float32); slots
    must be unique (duplicates are only legal for the dummy slot, whose
    content is then unspecified)."""
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    idx = np.asarray(out_loc).astype(np.int64)
    kp[idx] = k
    vp[idx] = v
    return kp, vp
