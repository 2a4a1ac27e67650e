"""The C ABI on the host (no GPU needed): libpkv.so loads, exports every
function include/pkv.h declares, its host helpers agree with the oracle, and
argument errors are reported before anything is launched."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT

pkv = pytest.importorskip("paged_kv_attention_scatter_amd")
from paged_kv_attention_scatter_amd import _lib  # noqa: E402
from paged_kv_attention_scatter_amd._lib import PkvPool  # noqa: E402

HEADER = os.path.join(ROOT, "include", "pkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpkv.so is not built: run python -m paged_kv_attention_scatter_amd.build")
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 12
    missing = [n for n in names if not hasattr(ctypes.CDLL(_lib.LIB_PATH), n)]
    assert not missing, missing
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_version(L):
    assert "gfx950" in pkv.version()


# ---------------------------------------------------------------- page count vs oracle

@pytest.mark.parametrize("args", [
    (128, 8, 1, 1, 2, 28, 24_000_000_000, 1_200_000_000, 0.9),
    (128, 8, 1, 1, 4, 28, 24_000_000_000, 1_200_000_000, 0.9),
    (128, 8, 1, 1, 2, 32, 60 << 30, 0, 0.9),
    (128, 8, 1, 64, 2, 32, 60 << 30, 0, 0.9),
    (128, 8, 2, 1, 2, 28, 288 << 30, 3 << 30, 0.9),
    (128, 2, 4, 16, 2, 28, 100 << 30, 0, 0.85),
])
def test_num_pages_matches_oracle(L, args):
    hd, kvh, tp, ps, isz, layers, free, model, ratio = args
    want = oracle.num_pages(hd, kvh, ps, isz, layers, free, model, ratio, tp_size=tp)
    assert pkv.num_pages(hd, kvh, ps, isz, layers, free, model, ratio, tp_size=tp) == want


def test_num_pages_errors(L):
    with pytest.raises(pkv.PkvError) as e:
        pkv.num_pages(128, 8, 1, 2, 28, 114688, 0, 1.0)
    assert e.value.status == -4 and "Not enough memory" in str(e.value)
    with pytest.raises(pkv.PkvError):
        pkv.num_pages(128, 6, 1, 2, 28, 1 << 40, 0, 0.9, tp_size=4)


# ---------------------------------------------------------------- sampling arguments vs oracle

def _params_cases():
    rng = np.random.default_rng(0)
    fixed = [
        [(0.0, -1, 1.0), (0.0, -1, 1.0)],
        [(1.0, 2, 1.0), (1.0, -1, 0.5), (0.0, -1, 1.0)],
        [(0.0, -1, 0.9)],
        [(0.8, 1, 1.0), (0.7, -1, 0.9)],
        [(0.7, 5, 1.0), (0.0, -1, 1.0)],
        [(-3.0, 0, 1.0), (2.0, 7, 1e-9), (1.5, 6, 1.0)],
    ]
    rand = [[(float(np.float32(rng.choice([0.0, 1e-7, 0.5, 1.0]))), int(rng.choice([-1, 0, 1, 3, 6, 9])),
              float(np.float32(rng.choice([1.0, 0.9, 1e-8, 0.3])))) for _ in range(7)] for _ in range(20)]
    return fixed + rand


@pytest.mark.parametrize("rows", _params_cases())
def test_prepare_sampling_matches_oracle(L, rows):
    vocab = 6
    T, K, P = zip(*rows)
    got = pkv.prepare_sampling(T, K, P, vocab)
    want = oracle.prepare([oracle.SamplingParams(t, k, p) for t, k, p in rows], vocab)
    for g, w in zip(got, want):
        assert (g is None) == (w is None)
        if g is not None:
            assert g.dtype == w.dtype and np.array_equal(g, w)


# ---------------------------------------------------------------- argument errors (host-side, pre-launch)

def _pool(**kw):
    d = dict(k=0x10000, v=0x20000, num_slots=100, row_stride=1024, kv_heads=8, head_dim=128,
             page_size=1, dtype=1)
    d.update(kw)
    return PkvPool(**d)


def _store(L, pool, n=4, loc=0x30000, loc_t=0, k=0x40000, ks=1024, v=0x50000, vs=1024):
    return L.pkv_store_kv(ctypes.byref(pool), loc, loc_t, n, k, ks, v, vs, None)


@pytest.mark.parametrize("pool,kw,status", [
    (dict(head_dim=64), {}, -3), (dict(dtype=7), {}, -2), (dict(k=None), {}, -1),
    (dict(row_stride=1000), {}, -3), (dict(k=0x10008), {}, -5), (dict(row_stride=1028), {}, -5),
    (dict(), dict(loc_t=5), -2), (dict(), dict(loc=None), -1), (dict(), dict(ks=512), -3),
    (dict(), dict(v=0x50004), -5), (dict(), dict(n=-1), -3), (dict(num_slots=0), {}, -3),
])
def test_store_kv_argument_errors(L, pool, kw, status):
    assert _store(L, _pool(**pool), **kw) == status
    assert L.pkv_last_error().decode()


def test_store_kv_zero_rows_is_noop(L):
    assert _store(L, _pool(), n=0, loc=None) == 0


def _qkr(L, pool, n=4, loc=0x30000, loc_t=0, q=0x60000, qs=0, qo=0x70000, qos=0, hq=16, k=0x40000, ks=1024,
         v=0x50000, vs=1024, pos=0x80000, wq=0xA0000, wk=0xB0000, eps=1e-6, theta=1e6):
    return L.pkv_qk_norm_rope_store_kv(ctypes.byref(pool), loc, loc_t, n, q, qs, qo, qos, hq, k, ks, v, vs, pos,
                                       wq, wk, eps, theta, None)


@pytest.mark.parametrize("pool,kw,status", [
    (dict(head_dim=64), {}, -3), (dict(dtype=7), {}, -2), (dict(k=None), {}, -1),
    (dict(), dict(loc_t=5), -2), (dict(), dict(loc=None), -1), (dict(), dict(pos=None), -1),
    (dict(), dict(wq=None), -1), (dict(), dict(wk=0xB0004), -5), (dict(), dict(hq=12), -3),
    (dict(), dict(hq=64), -3), (dict(), dict(eps=-1.0), -3), (dict(), dict(theta=0.5), -3),
    (dict(), dict(qs=1000), -3), (dict(), dict(qo=0x70008), -5), (dict(), dict(ks=512), -3),
    (dict(), dict(n=-1), -3), (dict(), dict(q=None), -1),
])
def test_qk_norm_rope_store_argument_errors(L, pool, kw, status):
    assert _qkr(L, _pool(**pool), **kw) == status
    assert L.pkv_last_error().decode()


def test_qk_norm_rope_store_zero_rows_is_noop(L):
    assert _qkr(L, _pool(), n=0, loc=None, pos=None) == 0


def _emb(L, w=0x10000, dt=1, rows=100, ws=1024, hidden=1024, ids=0x20000, n=4, a=0, b=100, out=0x30000, os_=1024):
    return L.pkv_embedding_gather(w, dt, rows, ws, hidden, ids, n, a, b, out, os_, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=9), -2), (dict(hidden=4), -3), (dict(hidden=1028), -3), (dict(n=-1), -3), (dict(a=-1), -3),
    (dict(a=10, b=5), -3), (dict(b=101), -3), (dict(ids=None), -1), (dict(w=None), -1), (dict(out=None), -1),
    (dict(ws=1000), -3), (dict(w=0x10008), -5), (dict(os_=1028), -5), (dict(rows=-1), -3),
])
def test_embedding_gather_argument_errors(L, kw, status):
    assert _emb(L, **kw) == status
    assert L.pkv_last_error().decode()


def test_embedding_gather_zero_rows_is_noop(L):
    assert _emb(L, n=0, ids=None) == 0


def _decode(L, pool, bs=4, hq=16, q=0x60000, o=0x70000, pt=0x80000, dl=0x90000, max_kv=100,
            ws=0xA0000, ws_bytes=1 << 30, rows=4, pts=64):
    return L.pkv_paged_attention_decode(ctypes.byref(pool), q, 0, o, 0, bs, hq, pt, rows, pts, None, None,
                                        dl, max_kv, 0.0, ws, ws_bytes, None)


@pytest.mark.parametrize("pool,kw,status", [
    (dict(head_dim=256), {}, -3), (dict(), dict(hq=12), -3), (dict(), dict(q=None), -1),
    (dict(), dict(o=0x70002), -5), (dict(), dict(pt=None), -1), (dict(), dict(dl=None), -1),
    (dict(), dict(max_kv=0), -4), (dict(), dict(ws_bytes=16), -6), (dict(), dict(ws=None), -6),
    (dict(), dict(bs=5000), -3), (dict(), dict(rows=0), -3), (dict(dtype=3), {}, -2),
])
def test_decode_argument_errors(L, pool, kw, status):
    assert _decode(L, _pool(**pool), **kw) == status


def _decode_store(L, pool, loc=0xB0000, lt=0, k=0xC0000, ks=0, v=0xD0000, vs=0, bs=4, q=0x60000, ws=0xA0000):
    return L.pkv_paged_attention_decode_store(ctypes.byref(pool), loc, lt, k, ks, v, vs, q, 0, 0x70000, 0, bs, 16,
                                              0x80000, 4, 64, None, None, 0x90000, 100, 0.0, ws, 1 << 30, None)


@pytest.mark.parametrize("kw,status", [
    (dict(loc=None), -1), (dict(lt=2), -2), (dict(k=None), -1), (dict(v=None), -1), (dict(k=0xC0008), -5),
    (dict(ks=100), -3), (dict(vs=1028), -5), (dict(q=None), -1), (dict(ws=None), -6),
])
def test_decode_store_argument_errors(L, kw, status):
    """The fused store + decode checks the store's arguments as store_kv does
    and the rest as decode does (no device work: every case fails on the host)."""
    assert _decode_store(L, _pool(), **kw) == status
    assert L.pkv_last_error().decode()


def test_decode_store_zero_rows_is_noop(L):
    assert _decode_store(L, _pool(), bs=0, loc=None, k=None, v=None) == 0


def test_decode_workspace_size_grows_with_batch(L):
    a = L.pkv_decode_workspace_size(4, 16, 1000)
    b = L.pkv_decode_workspace_size(256, 16, 1_200_000)
    assert 0 < a < b and L.pkv_decode_workspace_size(0, 16, 10) == 0


def _sample(L, logits=0x100000, dt=1, bs=4, V=1024, stride=1024, T=0x200000, K=None, P=None, u=0x300000,
            out=0x400000, ws=0x500000, ws_bytes=1 << 30, MP=None):
    return L.pkv_sample(logits, dt, bs, V, stride, T, K, P, MP, u, out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), -1), (dict(dt=7), -2), (dict(V=0), -3), (dict(bs=-1), -3), (dict(stride=1000), -3),
    (dict(stride=1028), -5), (dict(logits=0x100004), -5), (dict(out=None), -1), (dict(u=None), -1),
    (dict(V=2097153, stride=2097160), -3), (dict(dt=0, V=1048577, stride=1048580), -3),
    (dict(ws=None), -6), (dict(ws_bytes=1024), -6), (dict(ws=0x500008), -5),
])
def test_sample_argument_errors(L, kw, status):
    assert _sample(L, **kw) == status
    assert L.pkv_last_error().decode()


def test_sample_zero_rows_is_noop(L):
    assert _sample(L, bs=0) == 0


def test_sample_workspace_size(L):
    """bf16 rows need slice records, masses and histograms; the size grows with the batch."""
    a, b = L.pkv_sample_workspace_size(1, 151936), L.pkv_sample_workspace_size(256, 151936)
    assert 0 < a < b and L.pkv_sample_workspace_size(0, 151936) == 0


def _extend(L, pool, bs=2, hq=16, q=0x60000, o=0x70000, pt=0x80000, cl=0x88000, dl=0x90000, total_q=10,
            max_e=8, rows=2, pts=64):
    return L.pkv_paged_attention_extend(ctypes.byref(pool), q, 0, o, 0, bs, hq, pt, rows, pts, None, cl, dl,
                                        total_q, max_e, 0.0, None, 0, None)


@pytest.mark.parametrize("pool,kw,status", [
    (dict(dtype=0), {}, -6),                       # fp32: the decode-row path needs its workspace
    (dict(dtype=0), dict(total_q=5000), -3),       # fp32: at most 4096 rows
    (dict(dtype=0), dict(cl=None), -1), (dict(dtype=3), {}, -2),
    (dict(), dict(hq=12), -3), (dict(), dict(q=None), -1), (dict(), dict(o=0x70002), -5),
    (dict(), dict(cl=None), -1), (dict(), dict(max_e=0), -4), (dict(), dict(rows=0), -3),
    (dict(), dict(bs=1 << 28, max_e=8), -3),
])
def test_extend_argument_errors(L, pool, kw, status):
    assert _extend(L, _pool(**pool), **kw) == status
    assert L.pkv_last_error().decode()


def test_extend_empty_batch_is_noop(L):
    assert _extend(L, _pool(), bs=0) == 0 and _extend(L, _pool(), total_q=0) == 0


def test_extend_workspace_size(L):
    """bf16 extend needs no workspace; fp32 extend needs the rows' decode
    lengths and a decode workspace, growing with total_q, up to 4096 rows."""
    assert L.pkv_extend_workspace_size(8, 16, 20000, 1) == 0
    a, b = L.pkv_extend_workspace_size(2, 16, 10, 0), L.pkv_extend_workspace_size(2, 16, 4096, 0)
    assert 0 < a < b
    assert L.pkv_extend_workspace_size(2, 16, 4097, 0) == 0


def test_qk_norm_rope_store_k_side_only_validates(L):
    """q = q_out = NULL is the k-side-only call: q's arguments are not
    checked (num_q_heads 0, no q weight), the k side still is."""
    assert _qkr(L, _pool(), q=None, qo=None, hq=0, wq=None, ks=512) == -3
    assert _qkr(L, _pool(), q=None, qo=None, hq=0, wq=None, wk=None) == -1
