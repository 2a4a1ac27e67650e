"""Oracle pins: request lengths, page count, greedy rule and argument builder,
store_kv. Every expected value is printed on the pages (tests/golden/*.json,
each with its citation) or follows from the definition's invariants."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.sampling_params import SamplingParams
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- request lengths

def test_req_trace_prompt6():
    g = _golden("req_lengths.json")["trace_prompt6"]
    req = oracle.Req(g["prompt_len"], g["cached_len"], g["output_len"])
    rows = [list(req.lengths()) + [req.can_decode]]
    for _ in range(3):
        req.complete_one()
        rows.append(list(req.lengths()) + [req.can_decode])
    assert rows == g["rows"]


def test_req_prompt5():
    g = _golden("req_lengths.json")["prompt5"]
    req = oracle.Req(g["prompt_len"], g["cached_len"], g["output_len"])
    assert list(req.lengths()) == g["admitted"]
    req.complete_one()
    assert list(req.lengths()) == g["after_prefill"]
    req.complete_one()
    req.complete_one()
    assert req.remain_len == g["remain_after_two_more"] and not req.can_decode


def test_req_prompt100():
    g = _golden("req_lengths.json")["prompt100"]
    req = oracle.Req(g["prompt_len"], g["cached_len"], g["output_len"])
    pick = lambda r: [r.cached_len, r.device_len, r.remain_len]
    assert pick(req) == g["admitted"]
    req.complete_one()
    assert pick(req) == g["after_prefill"]
    for _ in range(10):
        req.complete_one()
    assert pick(req) == g["after_10_decodes"]


@pytest.mark.parametrize("prompt,cached,out", [(5, 5, 1), (5, -1, 1), (0, 0, 1)])
def test_req_rejects_bad_lengths(prompt, cached, out):
    with pytest.raises(ValueError):
        oracle.Req(prompt, cached, out)


# ---------------------------------------------------------------- page count

def test_bytes_per_page_printed():
    g = _golden("num_pages.json")
    for key in ("qwen3_bf16", "qwen3_fp32"):
        c = g[key]
        assert oracle.bytes_per_page(c["head_dim"], c["kv_heads"], c["page_size"],
                                     c["itemsize"], c["layers"]) == c["bytes_per_page"]
    l = g["llama3_8b"]
    assert oracle.bytes_per_page(l["head_dim"], l["kv_heads"], 1, l["itemsize"], l["layers"]) \
        == l["bytes_per_page_ps1"]
    assert oracle.bytes_per_page(l["head_dim"], l["kv_heads"], 64, l["itemsize"], l["layers"]) \
        == l["bytes_per_page_ps64"]


def test_num_pages_24gb_card():
    g = _golden("num_pages.json")
    c, q = g["card_24gb"], g["qwen3_bf16"]
    n = oracle.num_pages(q["head_dim"], q["kv_heads"], 1, q["itemsize"], q["layers"],
                         c["free_before"], c["model_bytes"], c["memory_ratio"])
    assert n == c["num_pages"]
    assert abs(n - c["about"]) / c["about"] < 0.02           # "about 180 thousand tokens"


def test_num_pages_llama_h100():
    l = _golden("num_pages.json")["llama3_8b"]
    avail = l["available_gib"] << 30
    # free_before chosen so that 0.9 * free - model = 54 GiB exactly
    free_before = avail * 10 // 9
    assert int(0.9 * free_before) == avail
    n1 = oracle.num_pages(l["head_dim"], l["kv_heads"], 1, l["itemsize"], l["layers"],
                          free_before, 0, 0.9)
    n64 = oracle.num_pages(l["head_dim"], l["kv_heads"], 64, l["itemsize"], l["layers"],
                           free_before, 0, 0.9)
    assert n1 == l["num_pages_ps1"]
    assert n64 == l["num_pages_ps64"]
    assert n64 * 64 == n1                                     # same token capacity


def test_num_pages_tp_split_and_error():
    # KV heads split across TP ranks: 8 heads over tp=2 halves the page size
    assert oracle.bytes_per_page(128, 8, 1, 2, 28, tp_size=2) * 2 == 114688
    # fewer heads than ranks: replicated, one head per rank
    assert oracle.bytes_per_page(128, 2, 1, 2, 28, tp_size=4) == 2 * 128 * 1 * 1 * 2 * 28
    with pytest.raises(ValueError):
        oracle.num_pages(128, 8, 1, 2, 28, free_before=114688, model_bytes=0, memory_ratio=1.0)


# ---------------------------------------------------------------- greedy rule and prepare

def test_is_greedy_cases():
    G = oracle.is_greedy
    assert G(SamplingParams())                                  # defaults are greedy
    assert not G(SamplingParams(temperature=1.0, top_k=2))
    assert not G(SamplingParams(temperature=1.0, top_p=0.5))
    assert not G(SamplingParams(temperature=0.0, top_p=0.9))    # top_p < 1 is never greedy
    assert G(SamplingParams(temperature=0.8, top_k=1))          # top_k == 1 greedy at any T
    assert not G(SamplingParams(temperature=0.8, top_k=1, top_p=0.99))
    assert G(SamplingParams(temperature=-1.0))


def test_prepare_all_greedy_gives_no_arrays():
    T, k, p = oracle.prepare([SamplingParams(), SamplingParams(temperature=2.0, top_k=1)], 6)
    assert T is None and k is None and p is None


def test_prepare_mixed_batch():
    params = [SamplingParams(temperature=1.0, top_k=2), SamplingParams(temperature=1.0, top_p=0.5),
              SamplingParams(), SamplingParams(temperature=0.0, top_p=1e-9)]
    T, k, p = oracle.prepare(params, 6)
    assert T.dtype == np.float32 and k.dtype == np.int32 and p.dtype == np.float32
    np.testing.assert_array_equal(T, np.float32([1.0, 1.0, 1e-6, 1e-6]))
    np.testing.assert_array_equal(k, [2, 6, 6, 6])              # top_k < 1 -> vocab
    np.testing.assert_array_equal(p, np.float32([1.0, 0.5, 1.0, 1e-6]))   # clamp to [1e-6, 1]


def test_prepare_arrays_only_when_used():
    T, k, p = oracle.prepare([SamplingParams(temperature=0.7, top_p=0.9), SamplingParams()], 10)
    assert k is None and p is not None
    T, k, p = oracle.prepare([SamplingParams(temperature=0.7, top_k=5), SamplingParams()], 10)
    assert k is not None and p is None
    T, k, p = oracle.prepare([SamplingParams(temperature=0.7)], 10)
    assert k is None and p is None and T is not None


# ---------------------------------------------------------------- store_kv

@pytest.mark.parametrize("itype", [np.int32, np.int64])
def test_store_kv_invariants(itype):
    rng = np.random.default_rng(0)
    slots, H, D, L = 64, 8, 128, 13
    sentinel = np.uint16(0x7FC0)
    kp = np.full((slots, H, D), sentinel, np.uint16)
    vp = kp.copy()
    loc = rng.permutation(slots)[:L].astype(itype)
    k = rng.integers(0, 1 << 16, (L, H, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (L, H, D), dtype=np.uint16)
    k2, v2 = oracle.store_kv(kp, vp, loc, k, v)
    untouched = np.setdiff1d(np.arange(slots), loc)
    assert np.all(k2[untouched] == sentinel) and np.all(v2[untouched] == sentinel)
    for i in range(L):                                          # row i landed at slot loc[i]
        assert np.array_equal(k2[int(loc[i])], k[i]) and np.array_equal(v2[int(loc[i])], v[i])
    assert np.all(kp == sentinel)                               # inputs not modified
