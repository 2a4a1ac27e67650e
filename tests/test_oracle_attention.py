"""Oracle pins for paged GQA attention.

(1) brute force against a textbook library routine (torch CPU fp64
scaled_dot_product_attention with an explicit boolean mask and
repeat_interleave, a different code path from the oracle's einsum);
(2) paged gather == contiguous KV; (3) closed forms that pin the scale, the
inclusive causal boundary row by row and the GQA head map; (4) consistency
between decode and extend and invisibility of a prefix-cache hit."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attention_request
from workloads import f32_to_bf16_bits


def _sdpa(q, K, V, cached_len):
    T, HQ, D = q.shape
    S, HKV, _ = K.shape
    G = HQ // HKV
    qt = torch.from_numpy(q).permute(1, 0, 2)                          # [HQ, T, D]
    kt = torch.from_numpy(K).repeat_interleave(G, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(V).repeat_interleave(G, dim=1).permute(1, 0, 2)
    mask = torch.zeros(T, S, dtype=torch.bool)
    for t in range(T):
        mask[t, : cached_len + t + 1] = True
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("T,C,HQ,HKV,D", [(1, 0, 4, 2, 16), (1, 7, 4, 2, 16), (5, 0, 4, 4, 8),
                                          (6, 9, 16, 8, 128), (3, 30, 8, 1, 32)])
def test_brute_force_vs_sdpa(T, C, HQ, HKV, D):
    rng = np.random.default_rng(T * 100 + C)
    S = C + T
    q = rng.standard_normal((T, HQ, D))
    K = rng.standard_normal((S, HKV, D))
    V = rng.standard_normal((S, HKV, D))
    np.testing.assert_allclose(attention_request(q, K, V, C), _sdpa(q, K, V, C),
                               rtol=1e-12, atol=1e-12)


def test_chunking_does_not_change_rows():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((40, 4, 16))
    K = rng.standard_normal((50, 2, 16))
    V = rng.standard_normal((50, 2, 16))
    a = attention_request(q, K, V, 10, chunk=7)
    b = attention_request(q, K, V, 10, chunk=1000)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def _paged_pools(K, V, perm):
    """Scatter contiguous per-request K/V to slots ``perm`` of a pool."""
    kp = np.full((len(perm) + 5, K.shape[1], K.shape[2]), np.nan)
    vp = kp.copy()
    kp[perm] = K
    vp[perm] = V
    return kp, vp


def test_paged_equals_contiguous_decode_and_extend():
    rng = np.random.default_rng(11)
    HQ, HKV, D = 16, 8, 128
    S = np.array([5, 9, 17, 33], np.int32)
    C = S - 1
    total = int(S.sum())
    K = rng.standard_normal((total, HKV, D)).astype(np.float32)
    V = rng.standard_normal((total, HKV, D)).astype(np.float32)
    q = rng.standard_normal((4, HQ, D)).astype(np.float32)
    width = 64
    ident = np.zeros((4, width), np.int32)
    perm_table = np.zeros((4, width), np.int32)
    perm = rng.permutation(total)
    off = 0
    for r, s in enumerate(S):
        ident[r, :s] = np.arange(off, off + s)
        perm_table[r, :s] = perm[off:off + s]
        off += s
    kp_c, vp_c = K, V
    kp_p = np.full((total + 3, HKV, D), np.nan, np.float32)
    vp_p = kp_p.copy()
    kp_p[perm] = K
    vp_p[perm] = V
    a = oracle.attention_decode(q, kp_c, vp_c, ident, C, S, "f32")
    b = oracle.attention_decode(q, kp_p, vp_p, perm_table, C, S, "f32")
    assert np.array_equal(a, b) and np.all(np.isfinite(a))
    # the same pair through extend with every request one query row long
    e = oracle.attention_extend(q, kp_p, vp_p, perm_table, C, S, "f32")
    assert np.array_equal(a, e)


def test_single_key_returns_v_exactly():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 16))
    K = rng.standard_normal((1, 2, 16))
    V = rng.standard_normal((1, 2, 16))
    o = attention_request(q, K, V, 0)
    assert np.array_equal(o[0, 0], V[0, 0]) and np.array_equal(o[0, 3], V[0, 1])


def test_zero_query_gives_mean_of_visible_rows():
    """q = 0 makes every visible key equally weighted, so row t is the mean of
    V[0 .. C+t]: this pins the inclusive causal boundary for every row."""
    rng = np.random.default_rng(6)
    C, T, HQ, HKV, D = 4, 6, 4, 2, 8
    q = np.zeros((T, HQ, D))
    K = rng.standard_normal((C + T, HKV, D))
    V = rng.standard_normal((C + T, HKV, D))
    o = attention_request(q, K, V, C)
    for t in range(T):
        for h in range(HQ):
            np.testing.assert_allclose(o[t, h], V[: C + t + 1, h // 2].mean(axis=0), atol=1e-13)


def test_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(7)
    S, HQ, HKV, D = 9, 4, 2, 16
    q = rng.standard_normal((1, HQ, D))
    K = np.broadcast_to(rng.standard_normal((1, HKV, D)), (S, HKV, D)).copy()
    V = rng.standard_normal((S, HKV, D))
    o = attention_request(q, K, V, S - 1)
    for h in range(HQ):
        np.testing.assert_allclose(o[0, h], V[:, h // 2].mean(axis=0), atol=1e-13)


def test_gqa_head_map_is_repeat_interleave():
    """V of KV head g is the constant g, so o_h = h // (HQ/HKV); the other map
    (h mod HKV) would give different values."""
    rng = np.random.default_rng(8)
    S, HQ, HKV, D = 12, 16, 8, 8
    q = rng.standard_normal((3, HQ, D))
    K = rng.standard_normal((S, HKV, D))
    V = np.broadcast_to(np.arange(HKV, dtype=np.float64)[None, :, None], (S, HKV, D)).copy()
    o = attention_request(q, K, V, S - 3)
    for h in range(HQ):
        np.testing.assert_allclose(o[:, h], h // 2, atol=1e-13)


def test_scale_is_inverse_sqrt_head_dim():
    """Two keys whose score difference is sqrt(D) * x give softmax weights
    in ratio e^x: pins the 1/sqrt(D) scale."""
    D = 128
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    K = np.zeros((2, 1, D))
    K[0, 0, 0] = math.sqrt(D) * 0.5
    V = np.zeros((2, 1, D))
    V[0, 0, 1] = 1.0
    V[1, 0, 2] = 1.0
    o = attention_request(q, K, V, 1)
    np.testing.assert_allclose(o[0, 0, 1] / o[0, 0, 2], math.exp(0.5), rtol=1e-13)


def test_extend_last_row_equals_decode_and_prefix_hit_invisible():
    rng = np.random.default_rng(9)
    HQ, HKV, D = 8, 4, 32
    C, E = 13, 7
    S = C + E
    q_full = rng.standard_normal((S, HQ, D))
    K = rng.standard_normal((S, HKV, D))
    V = rng.standard_normal((S, HKV, D))
    cold = attention_request(q_full, K, V, 0)                 # extend(0, C+E): no prefix hit
    warm = attention_request(q_full[C:], K, V, C)             # extend(C, E): prefix cached
    np.testing.assert_allclose(warm, cold[C:], rtol=1e-12, atol=1e-12)
    dec = attention_request(q_full[S - 1:], K, V, S - 1)      # decode at device_len = S
    np.testing.assert_allclose(dec[0], warm[-1], rtol=1e-12, atol=1e-12)


def test_bf16_widening_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, -0.0, 65280.0], np.float32)
    bits = f32_to_bf16_bits(x)
    back = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, ref)


def test_ragged_extend_offsets_several_requests():
    """attention_extend over four requests that each have several query rows
    (E > 1, unequal) and cached prefixes: request r's rows of the ragged
    output are SDPA brute force ("Mini-SGLang 完整剖析" section 4.6.5: q is
    laid end to end, request r starting at the sum of the earlier extend
    lengths; "第 0 步" section 这份代码在做什么: query t of a request sits at
    absolute position cached + t). The offsets, the gather and the reference
    are built here with plain loops, not with the oracle's helpers, so a
    padded layout, an off-by-one offset or a request mix-up fails."""
    rng = np.random.default_rng(41)
    HQ, HKV, D = 8, 4, 32
    C = [3, 0, 11, 6]
    E = [5, 2, 7, 4]
    S = [c + e for c, e in zip(C, E)]
    n_slots = sum(S) + 10
    perm = rng.permutation(n_slots)
    kp = rng.standard_normal((n_slots, HKV, D)).astype(np.float32).astype(np.float64)  # fp32 values
    vp = rng.standard_normal((n_slots, HKV, D)).astype(np.float32).astype(np.float64)
    width = max(S) + 3
    table = np.full((len(S), width), n_slots - 1, np.int64)
    pos = 0
    for r, s in enumerate(S):
        for j in range(s):
            table[r, j] = perm[pos]
            pos += 1
    q = rng.standard_normal((sum(E), HQ, D)).astype(np.float32).astype(np.float64)
    got = oracle.attention_extend(q, kp, vp, table, np.array(C, np.int32), np.array(S, np.int32), "f32")
    start = 0
    for r in range(len(S)):
        rows = list(range(start, start + E[r]))
        K = np.stack([kp[table[r, j]] for j in range(S[r])])
        V = np.stack([vp[table[r, j]] for j in range(S[r])])
        want = _sdpa(q[rows], K, V, C[r])
        np.testing.assert_allclose(got[rows], want, rtol=1e-12, atol=1e-12)
        start += E[r]
    assert start == got.shape[0]
