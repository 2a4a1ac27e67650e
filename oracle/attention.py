"""Paged GQA attention, decode and extend (oracle side; test infrastructure only).

The definition is the dense reference ``attention`` function of
"第 0 步：一个能跑的最小推理引擎" (section 这份代码在做什么): the KV heads are
repeated to the query heads with repeat_interleave (query head h uses KV head
h // (HQ/HKV)), scores are q.k / sqrt(D), the query at row t of this step has
absolute position S - T + t and sees every key at a position <= its own, and
the output is the softmax-weighted sum of V.

Paging (O2) follows "核心数据结构：Req、Batch、Context" section Context (the
page table is always token-granular: entry j of a request's row is the pool
slot of its token j) and "Mini-SGLang 完整剖析" sections 4.4.3 and 4.6.4
(page_size > 1 keeps the token-granular table; a slot is page * page_size +
offset). The gather therefore needs no page arithmetic at all.

Decode is extend with one query row: store_kv has already written the new
token (section 4.6.7: store_kv runs first, then the kernel), so a decode
request attends to device_len keys including its own.

Readings where the pages are silent (listed in the design notes): scale
1/sqrt(head_dim), no soft-cap or window; the causal boundary is inclusive;
queries never attend to keys at or beyond device_len.
"""

import math

import numpy as np

from .numerics import widen


def gather_kv(pool: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Rows of a per-layer pool [num_slots, HKV, D] for the first n tokens of
    a request, in token order."""
    return pool[np.asarray(table_row[:n]).astype(np.int64)]


def attention_request(q: np.ndarray, K: np.ndarray, V: np.ndarray, cached_len: int,
                      scale: float | None = None, chunk: int = 256) -> np.ndarray:
    """q: [T, HQ, D] f64 (query t at absolute position cached_len + t);
    K, V: [S, HKV, D] f64 with S = cached_len + T. Returns [T, HQ, D] f64.

    Query rows are independent, so long extends are evaluated ``chunk`` rows
    at a time to bound the score matrix; each row is the same formula."""
    T, HQ, D = q.shape
    S, HKV, D2 = K.shape
    if D2 != D or V.shape != K.shape or HQ % HKV:
        raise ValueError("shape mismatch")
    if S != cached_len + T:
        raise ValueError("S must equal cached_len + T")
    G = HQ // HKV
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Kh = np.repeat(K, G, axis=1)          # [S, HQ, D], head h <- KV head h // G
    Vh = np.repeat(V, G, axis=1)
    out = np.empty((T, HQ, D), dtype=np.float64)
    key_pos = np.arange(S)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        scores = np.einsum("thd,shd->hts", q[t0:t1], Kh) * scale     # [HQ, t, S]
        visible = key_pos[None, :] <= (cached_len + np.arange(t0, t1))[:, None]
        scores = np.where(visible[None], scores, -np.inf)
        scores = scores - scores.max(axis=-1, keepdims=True)
        p = np.exp(scores)
        p = p / p.sum(axis=-1, keepdims=True)
        out[t0:t1] = np.einsum("hts,shd->thd", p, Vh)
    return out


def _row_of(r: int, table_idx) -> int:
    return r if table_idx is None else int(table_idx[r])


def attention_decode(q, k_pool, v_pool, page_table, cached_len, device_len, dtype: str,
                     table_idx=None, scale=None, requests=None) -> np.ndarray:
    """q: [bs, HQ, D]; pools [num_slots, HKV, D]; page_table [rows, width]
    token-granular int; device_len[r] keys per request. Inputs hold kernel
    data ("bf16" bit patterns or "f32"). Returns f64 [bs, HQ, D] (rows not in
    ``requests`` are left as NaN when a subset is requested)."""
    bs = q.shape[0]
    out = np.full(q.shape, np.nan, dtype=np.float64)
    reqs = range(bs) if requests is None else requests
    for r in reqs:
        S = int(device_len[r])
        row = page_table[_row_of(r, table_idx)]
        K = widen(gather_kv(k_pool, row, S), dtype)
        V = widen(gather_kv(v_pool, row, S), dtype)
        qr = widen(q[r:r + 1], dtype)
        out[r:r + 1] = attention_request(qr, K, V, S - 1, scale)
    return out


def cu_seqlens_q(cached_len, device_len) -> np.ndarray:
    """Exclusive prefix sum of extend_len = device_len - cached_len
    ("Mini-SGLang 完整剖析" section 4.6.5, the general branch)."""
    e = np.asarray(device_len, dtype=np.int64) - np.asarray(cached_len, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(e)])


def attention_extend(q, k_pool, v_pool, page_table, cached_len, device_len, dtype: str,
                     table_idx=None, scale=None, requests=None) -> np.ndarray:
    """q: [sum E, HQ, D] ragged in request order. Request r's queries are the
    new tokens at positions cached_len[r] .. device_len[r]-1 and read all
    device_len[r] keys from the pool. Returns f64 [sum E, HQ, D]."""
    cu = cu_seqlens_q(cached_len, device_len)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    reqs = range(len(device_len)) if requests is None else requests
    for r in reqs:
        C, S = int(cached_len[r]), int(device_len[r])
        row = page_table[_row_of(r, table_idx)]
        K = widen(gather_kv(k_pool, row, S), dtype)
        V = widen(gather_kv(v_pool, row, S), dtype)
        qr = widen(q[cu[r]:cu[r + 1]], dtype)
        out[cu[r]:cu[r + 1]] = attention_request(qr, K, V, C, scale)
    return out
