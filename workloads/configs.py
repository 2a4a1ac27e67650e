"""The five synthetic cases (seeded; random draws only -- see the package
docstring for the shared recipe).

1 "tiny"    fp32 decode, 4 requests, device_len {5, 9, 17, 33}, page_size 1,
            256-page pool; sampler logits [4, 1024] ~ N(0, 2^2) with mixed
            per-row parameters.
2 "decode64" bf16 decode, 64 requests, device_len ~ U[256, 2048], page_size 1;
            logits [64, 151936] ~ N(0, 3^2), every row greedy.
3 "decode256" bf16 decode, 256 requests, device_len ~ U[1024, 8192],
            page_size 1; logits [256, 151936] ~ N(0, 3^2); exactly 128 greedy
            rows (a seeded permutation picks them), the rest T=0.7, top_p=0.9.
4 "extend8" bf16 extend, 8 requests, extend_len E ~ U[512, 4096] over a cached
            prefix C = floor(f * E), f ~ U[0, 0.5).
5 "mixed242" bf16, page_size 16: 240 decode requests with device_len
            ~ U[4096, 32768] plus 2 extend chunks of E = 2048 over a cached
            prefix C = 2048 * j, j ~ U{0..7}; logits [242, 151936] ~ N(0, 3^2),
            every row T=1.0, top_k=50, top_p=0.95.

A decode request has cached_len = device_len - 1: its new token's K/V row is
written by store_kv and then attended to.
"""

import math
from dataclasses import dataclass

import numpy as np

HQ = 16
HKV = 8
HEAD_DIM = 128
VOCAB = 151936
LAYERS = 28

_STREAMS = ("lengths", "pages", "q", "kv", "logits", "params", "uniforms")


@dataclass(frozen=True)
class CaseConfig:
    cid: int
    name: str
    dtype: str                  # "f32" or "bf16"
    page_size: int
    n_decode: int               # decode rows (first in row order)
    n_extend: int               # extend rows (after the decode rows)
    vocab: int
    logit_sigma: float
    pool_pages: int | None      # fixed pool size (pages), or None = sized by the caller

    @property
    def rows(self) -> int:
        return self.n_decode + self.n_extend

    @property
    def seed(self) -> int:
        return self.cid


CONFIGS = {
    1: CaseConfig(1, "tiny", "f32", 1, 4, 0, 1024, 2.0, 256),
    2: CaseConfig(2, "decode64", "bf16", 1, 64, 0, VOCAB, 3.0, None),
    3: CaseConfig(3, "decode256", "bf16", 1, 256, 0, VOCAB, 3.0, None),
    4: CaseConfig(4, "extend8", "bf16", 1, 0, 8, VOCAB, 3.0, None),
    5: CaseConfig(5, "mixed242", "bf16", 16, 240, 2, VOCAB, 3.0, None),
}


def config(cid: int) -> CaseConfig:
    return CONFIGS[cid]


def _streams(seed: int) -> dict:
    return dict(zip(_STREAMS, np.random.SeedSequence(seed).spawn(len(_STREAMS))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _as_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def draw_lengths(cfg: CaseConfig):
    """-> (cached_len, device_len) int32 [rows]."""
    rng = np.random.default_rng(_streams(cfg.seed)["lengths"])
    if cfg.cid == 1:
        S = np.array([5, 9, 17, 33], dtype=np.int64)
        return (S - 1).astype(np.int32), S.astype(np.int32)
    if cfg.cid in (2, 3):
        lo, hi = (256, 2048) if cfg.cid == 2 else (1024, 8192)
        S = rng.integers(lo, hi + 1, size=cfg.n_decode)
        return (S - 1).astype(np.int32), S.astype(np.int32)
    if cfg.cid == 4:
        E = rng.integers(512, 4096 + 1, size=cfg.n_extend)
        f = rng.random(cfg.n_extend)
        C = np.floor(f * 0.5 * E).astype(np.int64)
        return C.astype(np.int32), (C + E).astype(np.int32)
    if cfg.cid == 5:
        S_dec = rng.integers(4096, 32768 + 1, size=cfg.n_decode)
        j = rng.integers(0, 7 + 1, size=cfg.n_extend)
        C_ext = 2048 * j
        C = np.concatenate([S_dec - 1, C_ext])
        S = np.concatenate([S_dec, C_ext + 2048])
        return C.astype(np.int32), S.astype(np.int32)
    raise ValueError(cfg.cid)


def default_num_pages(cfg: CaseConfig, device_len: np.ndarray) -> int:
    """Pool pages when the caller does not size the pool: the fixed size of
    case 1, else 1.25 x the pages the requests use (the dummy page excluded)."""
    if cfg.pool_pages is not None:
        return cfg.pool_pages
    used = int(np.sum((np.asarray(device_len, np.int64) + cfg.page_size - 1) // cfg.page_size))
    return int(math.ceil(1.25 * used))


def table_width(device_len: np.ndarray) -> int:
    m = int(np.max(device_len))
    return (m + 31) // 32 * 32


def draw_page_table(cfg: CaseConfig, device_len: np.ndarray, num_pages: int) -> np.ndarray:
    """Token-granular page table int32 [rows, align32(max device_len)]:
    entry t of a row is the pool slot of token t. Unused entries point at the
    dummy slot (num_pages * page_size)."""
    rng = np.random.default_rng(_streams(cfg.seed)["pages"])
    ps = cfg.page_size
    S = np.asarray(device_len, dtype=np.int64)
    need = int(np.sum((S + ps - 1) // ps))
    if need > num_pages:
        raise ValueError(f"pool too small: {need} pages needed, {num_pages} available")
    perm = rng.permutation(num_pages)
    dummy = num_pages * ps
    table = np.full((len(S), table_width(S)), dummy, dtype=np.int64)
    off = 0
    for r, s in enumerate(S):
        npg = (int(s) + ps - 1) // ps
        pages = perm[off:off + npg]
        off += npg
        t = np.arange(int(s))
        table[r, :s] = pages[t // ps] * ps + t % ps
    return table.astype(np.int32)


def draw_request_kv(cfg: CaseConfig, r: int, device_len: int, rows: int | None = None):
    """(K, V) fp32 [device_len, HKV, D] of request r (its own stream)."""
    kv_children = _streams(cfg.seed)["kv"].spawn(cfg.rows)
    rng = np.random.default_rng(kv_children[r])
    K = rng.standard_normal((device_len, HKV, HEAD_DIM), dtype=np.float32)
    V = rng.standard_normal((device_len, HKV, HEAD_DIM), dtype=np.float32)
    return K, V


def draw_q(cfg: CaseConfig, cached_len, device_len) -> np.ndarray:
    """q [sum(device_len - cached_len), HQ, D] in row order, in the case dtype."""
    rng = np.random.default_rng(_streams(cfg.seed)["q"])
    n = int(np.sum(np.asarray(device_len, np.int64) - np.asarray(cached_len, np.int64)))
    return _as_dtype(rng.standard_normal((n, HQ, HEAD_DIM), dtype=np.float32), cfg.dtype)


def draw_logits(cfg: CaseConfig, rows: int | None = None) -> np.ndarray:
    rng = np.random.default_rng(_streams(cfg.seed)["logits"])
    n = cfg.rows if rows is None else rows
    x = rng.standard_normal((n, cfg.vocab), dtype=np.float32) * np.float32(cfg.logit_sigma)
    return _as_dtype(x, cfg.dtype)


def draw_sampling_params(cfg: CaseConfig, literal: bool = False):
    """Per-row (temperature, top_k, top_p) as a request would carry them
    (before the batch argument builder). Case 1's third and fourth rows give
    no temperature; they use T = 1.0 unless ``literal`` asks for the default
    temperature 0."""
    rng = np.random.default_rng(_streams(cfg.seed)["params"])
    if cfg.cid == 1:
        t_default = 0.0 if literal else 1.0
        return [(0.0, -1, 1.0), (0.7, -1, 0.9), (t_default, 20, 1.0), (t_default, 5, 0.8)]
    if cfg.cid in (2, 4):
        return [(0.0, -1, 1.0)] * cfg.rows
    if cfg.cid == 3:
        greedy = set(rng.permutation(cfg.rows)[: cfg.rows // 2].tolist())
        return [(0.0, -1, 1.0) if r in greedy else (0.7, -1, 0.9) for r in range(cfg.rows)]
    if cfg.cid == 5:
        return [(1.0, 50, 0.95)] * cfg.rows
    raise ValueError(cfg.cid)


def draw_uniforms(cfg: CaseConfig, rows: int | None = None) -> np.ndarray:
    rng = np.random.default_rng(_streams(cfg.seed)["uniforms"])
    return rng.random(cfg.rows if rows is None else rows, dtype=np.float32)


def draw_case(cfg: CaseConfig, num_pages: int | None = None, with_pool: bool = True,
              sentinel_bits: int = 0x7FC0):
    """Everything one step of the path needs, on the host.

    Returns a dict: cached_len, device_len (int32 [rows]); page_table;
    num_pages, num_slots (= (num_pages + 1) * page_size, the +1 page being
    the dummy); q (case dtype, [sum E, HQ, D]); new_k, new_v ([sum E, HKV, D],
    the rows store_kv writes, in row order); out_loc (int32 [sum E]); and,
    when ``with_pool``, k_pool / v_pool [num_slots, HKV, D] holding every
    request's cached prefix rows, with every other slot set to a sentinel
    (bf16 NaN bits 0x7FC0, or fp32 NaN)."""
    C, S = draw_lengths(cfg)
    if num_pages is None:
        num_pages = default_num_pages(cfg, S)
    table = draw_page_table(cfg, S, num_pages)
    num_slots = (num_pages + 1) * cfg.page_size
    q = draw_q(cfg, C, S)
    E = (S.astype(np.int64) - C.astype(np.int64))
    L = int(E.sum())
    store_dtype = np.uint16 if cfg.dtype == "bf16" else np.float32
    new_k = np.empty((L, HKV, HEAD_DIM), dtype=store_dtype)
    new_v = np.empty_like(new_k)
    out_loc = np.empty(L, dtype=np.int32)
    case = dict(cfg=cfg, cached_len=C, device_len=S, page_table=table, num_pages=num_pages,
                num_slots=num_slots, q=q, new_k=new_k, new_v=new_v, out_loc=out_loc)
    if with_pool:
        if cfg.dtype == "bf16":
            k_pool = np.full((num_slots, HKV, HEAD_DIM), sentinel_bits, dtype=np.uint16)
        else:
            k_pool = np.full((num_slots, HKV, HEAD_DIM), np.nan, dtype=np.float32)
        v_pool = k_pool.copy()
        case.update(k_pool=k_pool, v_pool=v_pool)
    off = 0
    for r in range(cfg.rows):
        c, s = int(C[r]), int(S[r])
        K, V = draw_request_kv(cfg, r, s)
        Kd, Vd = _as_dtype(K, cfg.dtype), _as_dtype(V, cfg.dtype)
        slots = table[r, :s].astype(np.int64)
        if with_pool:
            case["k_pool"][slots[:c]] = Kd[:c]
            case["v_pool"][slots[:c]] = Vd[:c]
        new_k[off:off + s - c] = Kd[c:]
        new_v[off:off + s - c] = Vd[c:]
        out_loc[off:off + s - c] = slots[c:]
        off += s - c
    return case
