"""Python binding of libpkv with the C ABI's names (argument marshalling only).

Each function takes torch tensors that already live on the GPU, checks what
the C side cannot see (device placement, element type, contiguity of the
last dimensions), and passes raw pointers, sizes and the current HIP stream
to libpkv.so. All the work happens in the library's gfx950 kernels; there is
no PyTorch or CPU fallback. Workspaces not supplied by the caller are taken
from PyTorch's caching allocator.
"""

from ctypes import byref, c_float, c_int32, c_uint32

import numpy as np

from . import _lib
from ._lib import PKV_BF16, PKV_F32, PKV_I32, PKV_I64, PkvPool, PkvQNormRope, check, lib

HEAD_DIM = 128


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _cuda(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def make_pool(k_pool, v_pool, page_size: int = 1) -> PkvPool:
    """Pool descriptor from per-layer K/V views [num_slots, kv_heads, 128]
    whose last two dimensions are dense (views into a bigger pool tensor are
    fine)."""
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _cuda(t, n)
        if t.dim() != 3 or t.shape[2] != HEAD_DIM:
            raise ValueError(f"{n} must be [num_slots, kv_heads, {HEAD_DIM}]")
        if t.stride(2) != 1 or t.stride(1) != HEAD_DIM:
            raise ValueError(f"{n}: the last two dimensions must be dense")
    if k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype or k_pool.stride(0) != v_pool.stride(0):
        raise ValueError("k_pool and v_pool must have the same shape, dtype and slot stride")
    return PkvPool(k_pool.data_ptr(), v_pool.data_ptr(), k_pool.shape[0], k_pool.stride(0),
                   k_pool.shape[1], HEAD_DIM, page_size, _dtype_code(k_pool))


def _rows(t, name, width):
    """Row stride of a [n, heads, 128] (or [n, heads*128]) tensor with dense rows."""
    _cuda(t, name)
    flat = t.reshape(t.shape[0], -1) if t.dim() == 3 and t.stride(2) == 1 and t.stride(1) == HEAD_DIM else t
    if flat.dim() != 2 or flat.shape[1] != width or flat.stride(1) != 1:
        raise ValueError(f"{name} must be [n, {width // HEAD_DIM}, {HEAD_DIM}] with dense rows")
    return flat.stride(0)


def store_kv(k_pool, v_pool, out_loc, k, v, *, page_size: int = 1, stream=None) -> None:
    """k_pool[out_loc[i]] = k[i], v_pool[out_loc[i]] = v[i] (pkv_store_kv)."""
    pool = make_pool(k_pool, v_pool, page_size)
    width = pool.kv_heads * HEAD_DIM
    n = out_loc.shape[0]
    _cuda(out_loc, "out_loc")
    torch = _torch()
    if out_loc.dtype not in (torch.int32, torch.int64) or out_loc.dim() != 1 or out_loc.stride(0) != 1:
        raise ValueError("out_loc must be a dense 1-D int32 or int64 tensor")
    if k.dtype != k_pool.dtype or v.dtype != k_pool.dtype or k.shape[0] != n or v.shape[0] != n:
        raise ValueError("k, v must match the pool dtype and have len(out_loc) rows")
    ks, vs = _rows(k, "k", width), _rows(v, "v", width)
    loc_t = PKV_I32 if out_loc.dtype == torch.int32 else PKV_I64
    check(lib().pkv_store_kv(byref(pool), _ptr(out_loc), loc_t, n, k.data_ptr(), ks, v.data_ptr(), vs,
                             _stream(stream)))


def embedding_gather(weight, ids, *, vocab_start: int = 0, vocab_end=None, out=None, stream=None):
    """Rows of the vocab-parallel embedding (pkv_embedding_gather): out[i] =
    weight[ids[i] - vocab_start] for ids in [vocab_start, vocab_end), zero rows
    for the others. weight: [rows, hidden]; ids: int32 [n]. Returns out [n, hidden]."""
    torch = _torch()
    _cuda(weight, "weight")
    _cuda(ids, "ids")
    if weight.dim() != 2 or weight.stride(1) != 1:
        raise ValueError("weight must be [rows, hidden] with dense rows")
    if ids.dtype != torch.int32 or ids.dim() != 1 or ids.stride(0) != 1:
        raise ValueError("ids must be a dense 1-D int32 tensor")
    rows, hidden = weight.shape
    if vocab_end is None:
        vocab_end = vocab_start + rows
    n = ids.shape[0]
    if out is None:
        out = torch.empty((n, hidden), dtype=weight.dtype, device=weight.device)
    if out.dtype != weight.dtype or out.dim() != 2 or out.shape != (n, hidden) or out.stride(1) != 1:
        raise ValueError("out must be [len(ids), hidden] of the weight dtype with dense rows")
    check(lib().pkv_embedding_gather(weight.data_ptr(), _dtype_code(weight), rows, weight.stride(0), hidden,
                                     _ptr(ids), n, vocab_start, vocab_end, out.data_ptr(), out.stride(0),
                                     _stream(stream)))
    return out


def qk_norm_rope_store_kv(k_pool, v_pool, out_loc, q, k, v, positions, q_norm_weight, k_norm_weight, *,
                          eps: float = 1e-6, rope_theta: float = 1_000_000.0, page_size: int = 1, q_out=None,
                          stream=None):
    """Per-head RMSNorm of q and k, rotary embedding at `positions`, then the
    K/V store (pkv_qk_norm_rope_store_kv). Returns q_out ([n, num_q_heads,
    128], the normalised and rotated q; pass q_out=q to work in place).
    q=None: the k side only (q then goes through the attention call's own
    prologue, q_norm_weight=...); returns None."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool, page_size)
    width = pool.kv_heads * HEAD_DIM
    n = out_loc.shape[0]
    if q is None:
        for t, name in ((out_loc, "out_loc"), (positions, "positions"), (k, "k"), (v, "v"),
                        (k_norm_weight, "k_norm_weight")):
            _cuda(t, name)
        if k.dtype != k_pool.dtype or v.dtype != k_pool.dtype or k.shape[0] != n or v.shape[0] != n:
            raise ValueError("k, v must have the pool dtype and len(out_loc) rows")
        if positions.dtype != torch.int32 or positions.shape[0] != n or positions.stride(0) != 1:
            raise ValueError("positions must be a dense int32 tensor of len(out_loc) entries")
        if out_loc.dtype not in (torch.int32, torch.int64) or out_loc.dim() != 1 or out_loc.stride(0) != 1:
            raise ValueError("out_loc must be a dense 1-D int32 or int64 tensor")
        if k_norm_weight.dtype != k_pool.dtype or k_norm_weight.numel() != HEAD_DIM:
            raise ValueError(f"k_norm_weight must be a dense [{HEAD_DIM}] tensor of the pool dtype")
        ks, vs = _rows(k, "k", width), _rows(v, "v", width)
        loc_t = PKV_I32 if out_loc.dtype == torch.int32 else PKV_I64
        check(lib().pkv_qk_norm_rope_store_kv(byref(pool), _ptr(out_loc), loc_t, n, None, 0, None, 0, 0,
                                              k.data_ptr(), ks, v.data_ptr(), vs, _ptr(positions), None,
                                              k_norm_weight.data_ptr(), float(eps), float(rope_theta),
                                              _stream(stream)))
        return None
    for t, name in ((out_loc, "out_loc"), (positions, "positions"), (q, "q"), (k, "k"), (v, "v"),
                    (q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        _cuda(t, name)
    if out_loc.dtype not in (torch.int32, torch.int64) or out_loc.dim() != 1 or out_loc.stride(0) != 1:
        raise ValueError("out_loc must be a dense 1-D int32 or int64 tensor")
    if positions.dtype != torch.int32 or positions.dim() != 1 or positions.shape[0] != n or positions.stride(0) != 1:
        raise ValueError("positions must be a dense int32 tensor of len(out_loc) entries")
    if q.dtype != k_pool.dtype or k.dtype != k_pool.dtype or v.dtype != k_pool.dtype:
        raise ValueError("q, k, v must have the pool dtype")
    if q.shape[0] != n or k.shape[0] != n or v.shape[0] != n:
        raise ValueError("q, k, v must have len(out_loc) rows")
    for w, name in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        if w.dtype != k_pool.dtype or w.numel() != HEAD_DIM or not w.is_contiguous():
            raise ValueError(f"{name} must be a dense [{HEAD_DIM}] tensor of the pool dtype")
    hq = q.shape[1] if q.dim() == 3 else q.shape[-1] // HEAD_DIM
    qs = _rows(q, "q", hq * HEAD_DIM)
    if q_out is None:
        q_out = torch.empty_like(q)
    qos = _rows(q_out, "q_out", hq * HEAD_DIM)
    ks, vs = _rows(k, "k", width), _rows(v, "v", width)
    loc_t = PKV_I32 if out_loc.dtype == torch.int32 else PKV_I64
    check(lib().pkv_qk_norm_rope_store_kv(byref(pool), _ptr(out_loc), loc_t, n, q.data_ptr(), qs,
                                          q_out.data_ptr(), qos, hq, k.data_ptr(), ks, v.data_ptr(), vs,
                                          _ptr(positions), q_norm_weight.data_ptr(), k_norm_weight.data_ptr(),
                                          float(eps), float(rope_theta), _stream(stream)))
    return q_out


def decode_workspace_size(bs: int, num_q_heads: int, max_total_kv: int) -> int:
    return int(lib().pkv_decode_workspace_size(bs, num_q_heads, max_total_kv))


def _lengths(t, name, bs):
    torch = _torch()
    _cuda(t, name)
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] < bs or t.stride(0) != 1:
        raise ValueError(f"{name} must be a dense int32 tensor of >= {bs} entries")


def _table(page_table):
    torch = _torch()
    _cuda(page_table, "page_table")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.stride(1) != 1:
        raise ValueError("page_table must be a 2-D int32 tensor with dense rows")
    return page_table.shape[0], page_table.stride(0)


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if nbytes == 0:
        return workspace
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace


def _qnr(q_norm_weight, eps, rope_theta, pool_dtype):
    if q_norm_weight is None:
        return None
    _cuda(q_norm_weight, "q_norm_weight")
    if q_norm_weight.dtype != pool_dtype or q_norm_weight.numel() != HEAD_DIM or not q_norm_weight.is_contiguous():
        raise ValueError(f"q_norm_weight must be a dense [{HEAD_DIM}] tensor of the pool dtype")
    return PkvQNormRope(q_norm_weight.data_ptr(), float(eps), float(rope_theta))


def paged_attention_decode(q, k_pool, v_pool, page_table, cached_len, device_len, *, table_idx=None,
                           max_total_kv=None, sm_scale: float = 0.0, page_size: int = 1, out=None,
                           workspace=None, stream=None, q_norm_weight=None, eps: float = 1e-6,
                           rope_theta: float = 1_000_000.0):
    """GQA decode attention over the paged pool (pkv_paged_attention_decode).
    q: [bs, num_q_heads, 128]. Returns o with q's shape and dtype.
    With q_norm_weight, q is the raw projection and the call normalises and
    rotates it first (pkv_paged_attention_decode_qnr)."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool, page_size)
    bs, hq = q.shape[0], q.shape[1]
    qs = _rows(q, "q", hq * HEAD_DIM)
    if q.dtype != k_pool.dtype:
        raise ValueError("q must have the pool's dtype")
    if out is None:
        out = torch.empty((bs, hq, HEAD_DIM), dtype=q.dtype, device=q.device)
    os_ = _rows(out, "out", hq * HEAD_DIM)
    rows, pts = _table(page_table)
    _lengths(device_len, "device_len", bs)
    if table_idx is not None:
        _lengths(table_idx, "table_idx", bs)
    if max_total_kv is None:
        max_total_kv = bs * pts
    ws = _workspace(decode_workspace_size(bs, hq, max_total_kv), q.device, workspace)
    qnr = _qnr(q_norm_weight, eps, rope_theta, k_pool.dtype)
    common = (byref(pool), q.data_ptr(), qs, out.data_ptr(), os_, bs, hq, page_table.data_ptr(), rows, pts,
              _ptr(table_idx), _ptr(cached_len), device_len.data_ptr(), int(max_total_kv), sm_scale)
    wsa = (_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if qnr is None:
        check(lib().pkv_paged_attention_decode(*common, *wsa))
    else:
        check(lib().pkv_paged_attention_decode_qnr(*common, byref(qnr), *wsa))
    return out


def paged_attention_decode_store(q, k_pool, v_pool, page_table, cached_len, device_len, out_loc, k, v, *,
                                 table_idx=None, max_total_kv=None, sm_scale: float = 0.0, page_size: int = 1,
                                 out=None, workspace=None, stream=None):
    """store_kv fused into decode attention (pkv_paged_attention_decode_store):
    writes k[r] / v[r] to pool slot out_loc[r] and attends with the new row as
    key device_len - 1 of request r. Same result as store_kv followed by
    paged_attention_decode when out_loc holds each request's last page-table
    entry. k, v: [bs, kv_heads, 128] in the pool's dtype."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool, page_size)
    bs, hq = q.shape[0], q.shape[1]
    qs = _rows(q, "q", hq * HEAD_DIM)
    if q.dtype != k_pool.dtype or k.dtype != k_pool.dtype or v.dtype != k_pool.dtype:
        raise ValueError("q, k and v must have the pool's dtype")
    row = k_pool.shape[1] * HEAD_DIM
    ks, vs = _rows(k, "k", row), _rows(v, "v", row)
    if k.shape[0] != bs or v.shape[0] != bs or out_loc.shape[0] != bs:
        raise ValueError("k, v and out_loc need one row per request")
    loc_type = {torch.int32: PKV_I32, torch.int64: PKV_I64}.get(out_loc.dtype)
    if loc_type is None:
        raise ValueError("out_loc must be int32 or int64")
    if out is None:
        out = torch.empty((bs, hq, HEAD_DIM), dtype=q.dtype, device=q.device)
    os_ = _rows(out, "out", hq * HEAD_DIM)
    rows, pts = _table(page_table)
    _lengths(device_len, "device_len", bs)
    if table_idx is not None:
        _lengths(table_idx, "table_idx", bs)
    if max_total_kv is None:
        max_total_kv = bs * pts
    ws = _workspace(decode_workspace_size(bs, hq, max_total_kv), q.device, workspace)
    check(lib().pkv_paged_attention_decode_store(
        byref(pool), out_loc.data_ptr(), loc_type, k.data_ptr(), ks, v.data_ptr(), vs, q.data_ptr(), qs,
        out.data_ptr(), os_, bs, hq, page_table.data_ptr(), rows, pts, _ptr(table_idx), _ptr(cached_len),
        device_len.data_ptr(), int(max_total_kv), sm_scale, _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
    return out


def paged_attention_decode_noalloc(q, k_pool, v_pool, page_table, cached_len, device_len, *, table_idx=None,
                                   max_total_kv=None, sm_scale: float = 0.0, page_size: int = 1, out=None,
                                   stream=None):
    """Decode attention without a workspace (pkv_paged_attention_decode_noalloc):
    the library's per-GPU scratch holds the partials. `out` must be given to
    keep the call free of allocations (else it is created here). Calls that
    overlap in time on one GPU race."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool, page_size)
    bs, hq = q.shape[0], q.shape[1]
    qs = _rows(q, "q", hq * HEAD_DIM)
    if q.dtype != k_pool.dtype:
        raise ValueError("q must have the pool's dtype")
    if out is None:
        out = torch.empty((bs, hq, HEAD_DIM), dtype=q.dtype, device=q.device)
    os_ = _rows(out, "out", hq * HEAD_DIM)
    rows, pts = _table(page_table)
    _lengths(device_len, "device_len", bs)
    if table_idx is not None:
        _lengths(table_idx, "table_idx", bs)
    if max_total_kv is None:
        max_total_kv = bs * pts
    check(lib().pkv_paged_attention_decode_noalloc(
        byref(pool), q.data_ptr(), qs, out.data_ptr(), os_, bs, hq, page_table.data_ptr(), rows, pts,
        _ptr(table_idx), _ptr(cached_len), device_len.data_ptr(), int(max_total_kv), sm_scale,
        _stream(stream)))
    return out


def extend_workspace_size(bs: int, num_q_heads: int, total_q: int, dtype=PKV_BF16) -> int:
    """Workspace bytes of an extend call on a pool of `dtype` (PKV_BF16 or PKV_F32 code)."""
    return int(lib().pkv_extend_workspace_size(bs, num_q_heads, total_q, dtype))


def paged_attention_extend(q, k_pool, v_pool, page_table, cached_len, device_len, *, max_extend: int,
                           table_idx=None, sm_scale: float = 0.0, page_size: int = 1, out=None,
                           workspace=None, stream=None, q_norm_weight=None, eps: float = 1e-6,
                           rope_theta: float = 1_000_000.0):
    """Causal extend attention over a cached prefix (pkv_paged_attention_extend).
    q: ragged [total_q, num_q_heads, 128] in request order; max_extend bounds
    every request's extend_len. Returns o with q's shape and dtype.
    With q_norm_weight, q is the raw projection and the call normalises and
    rotates it first (pkv_paged_attention_extend_qnr)."""
    torch = _torch()
    pool = make_pool(k_pool, v_pool, page_size)
    total_q, hq = q.shape[0], q.shape[1]
    bs = device_len.shape[0]
    qs = _rows(q, "q", hq * HEAD_DIM)
    if q.dtype != k_pool.dtype:
        raise ValueError("q must have the pool's dtype")
    if out is None:
        out = torch.empty((total_q, hq, HEAD_DIM), dtype=q.dtype, device=q.device)
    os_ = _rows(out, "out", hq * HEAD_DIM)
    rows, pts = _table(page_table)
    _lengths(device_len, "device_len", bs)
    _lengths(cached_len, "cached_len", bs)
    if table_idx is not None:
        _lengths(table_idx, "table_idx", bs)
    ws = _workspace(extend_workspace_size(bs, hq, total_q, _dtype_code(k_pool)), q.device, workspace)
    qnr = _qnr(q_norm_weight, eps, rope_theta, k_pool.dtype)
    common = (byref(pool), q.data_ptr(), qs, out.data_ptr(), os_, bs, hq, page_table.data_ptr(), rows, pts,
              _ptr(table_idx), cached_len.data_ptr(), device_len.data_ptr(), total_q, int(max_extend), sm_scale)
    wsa = (_ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if qnr is None:
        check(lib().pkv_paged_attention_extend(*common, *wsa))
    else:
        check(lib().pkv_paged_attention_extend_qnr(*common, byref(qnr), *wsa))
    return out


def sample_workspace_size(bs: int, vocab: int) -> int:
    return int(lib().pkv_sample_workspace_size(bs, vocab))


def sample_workspace(bs: int, vocab: int, device):
    """A sampler workspace for calls of at most bs rows over this vocabulary."""
    torch = _torch()
    return torch.empty(max(1, sample_workspace_size(bs, vocab)), dtype=torch.uint8, device=device)


def sample(logits, temperature=None, top_k=None, top_p=None, uniforms=None, *, min_p=None, out=None,
           workspace=None, stream=None):
    """One token per row (pkv_sample). temperature None = all-greedy batch;
    min_p None = no min_p."""
    torch = _torch()
    _cuda(logits, "logits")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [bs, vocab] with dense rows")
    bs, vocab = logits.shape
    for t, n, dt in ((temperature, "temperature", torch.float32), (top_k, "top_k", torch.int32),
                     (top_p, "top_p", torch.float32), (min_p, "min_p", torch.float32),
                     (uniforms, "uniforms", torch.float32)):
        if t is not None:
            _cuda(t, n)
            if t.dtype != dt or t.dim() != 1 or t.shape[0] < bs or t.stride(0) != 1:
                raise ValueError(f"{n} must be a dense {dt} tensor of >= {bs} entries")
    if out is None:
        out = torch.empty(bs, dtype=torch.int32, device=logits.device)
    ws = _workspace(sample_workspace_size(bs, vocab), logits.device, workspace)
    check(lib().pkv_sample(logits.data_ptr(), _dtype_code(logits), bs, vocab, logits.stride(0),
                           _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(min_p), _ptr(uniforms),
                           out.data_ptr(),
                           _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
    return out


def num_pages(head_dim: int, kv_heads: int, page_size: int, itemsize: int, num_layers: int,
              free_before: int, model_bytes: int, memory_ratio: float = 0.9, tp_size: int = 1) -> int:
    """KV pool page count (pkv_num_pages); raises when fewer than two pages fit."""
    n = lib().pkv_num_pages(head_dim, kv_heads, tp_size, page_size, itemsize, num_layers, free_before,
                            model_bytes, memory_ratio)
    if n < 0:
        check(int(n))
    return int(n)


def prepare_sampling(temperature, top_k, top_p, vocab: int):
    """Batch sampling arguments from per-request parameters
    (pkv_prepare_sampling). Returns (T | None, top_k | None, top_p | None) as
    host numpy arrays: None where the batch does not need the array."""
    T = np.ascontiguousarray(temperature, dtype=np.float32)
    K = np.ascontiguousarray(top_k, dtype=np.int32)
    P = np.ascontiguousarray(top_p, dtype=np.float32)
    n = T.shape[0]
    To, Ko, Po = np.empty_like(T), np.empty_like(K), np.empty_like(P)
    flags = c_int32(0)
    fp = lambda a: a.ctypes.data_as(_lib._P_f32)
    ip = lambda a: a.ctypes.data_as(_lib._P_i32)
    check(lib().pkv_prepare_sampling(n, fp(T), ip(K), fp(P), vocab, fp(To), ip(Ko), fp(Po), byref(flags)))
    f = flags.value
    if f & _lib.PKV_PREP_ALL_GREEDY:
        return None, None, None
    return To, (Ko if f & _lib.PKV_PREP_USE_TOP_K else None), (Po if f & _lib.PKV_PREP_USE_TOP_P else None)


def read_faults(stream=None) -> int:
    """Reads and clears the device fault word (PKV_FAULT_* bits)."""
    v = c_uint32(0)
    check(lib().pkv_read_faults(_stream(stream), byref(v)))
    return int(v.value)


def version() -> str:
    return lib().pkv_version().decode()
