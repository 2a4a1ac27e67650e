"""GPU parity of pkv_paged_attention_extend (bf16 MFMA path) against the
oracle: max-abs 2e-2 and relative L2 1e-2 on every output row, the
full-size cases included (their oracle runs in a host process pool)."""

import zlib

import numpy as np
import pytest

import oracle
from workloads import config, draw_case, f32_to_bf16_bits
from gpu_util import check_attention, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
pkv = pytest.importorskip("paged_kv_attention_scatter_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.read_faults()


def _make(seed, C, E, HKV=8, G=2, ps=1, q_pad=0, table_idx=False, extra_slots=40):
    """Random extend batch: request r has cached C[r] and E[r] new tokens; the
    pool holds random rows everywhere (prefix and new rows alike)."""
    rng = np.random.default_rng(seed)
    C = np.asarray(C, np.int32)
    E = np.asarray(E, np.int32)
    S = C + E
    bs = len(S)
    HQ = HKV * G
    pages_per = (S + ps - 1) // ps
    n_pages = int(pages_per.sum()) + extra_slots
    perm = rng.permutation(n_pages)
    width = (int(S.max()) + 31) // 32 * 32
    table = np.full((bs + 2, width), (n_pages) * ps, np.int32)   # unused entries -> dummy slot
    rows = rng.permutation(bs + 2)[:bs].astype(np.int32) if table_idx else np.arange(bs, dtype=np.int32)
    off = 0
    for r in range(bs):
        pg = perm[off:off + pages_per[r]]
        off += pages_per[r]
        tt = np.arange(S[r])
        table[rows[r], :S[r]] = pg[tt // ps] * ps + tt % ps
    n_slots = (n_pages + 1) * ps
    kv = f32_to_bf16_bits(rng.standard_normal((2, n_slots, HKV, 128), dtype=np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((int(E.sum()), HQ * 128 + q_pad), dtype=np.float32))
    return dict(C=C, S=S, E=E, table=table, rows=rows if table_idx else None, kv=kv, q=q, HQ=HQ, HKV=HKV,
                ps=ps)


def _run(c, sm_scale=0.0):
    HQ = c["HQ"]
    n = c["q"].shape[0]
    qd = to_dev(c["q"], "bf16")[:, :HQ * 128].view(n, HQ, 128)
    o = pkv.paged_attention_extend(
        qd, to_dev(c["kv"][0], "bf16"), to_dev(c["kv"][1], "bf16"), to_dev(c["table"]), to_dev(c["C"]),
        to_dev(c["S"]), max_extend=int(c["E"].max()), page_size=c["ps"],
        table_idx=None if c["rows"] is None else to_dev(c["rows"]), sm_scale=sm_scale)
    torch.cuda.synchronize()
    return to_host(o)


def _oracle(c, rows=None, scale=None):
    qh = c["q"][:, :c["HQ"] * 128].reshape(-1, c["HQ"], 128)
    return oracle.attention_extend(qh, c["kv"][0], c["kv"][1], c["table"], c["C"], c["S"], "bf16",
                                   table_idx=c["rows"], requests=rows, scale=scale)


CASES = [
    ("fresh_prefill", dict(C=[0, 0], E=[64, 200])),
    ("prefix_hit", dict(C=[130, 7, 1000], E=[70, 129, 33])),
    ("tiny_rows", dict(C=[0, 5, 63, 64], E=[1, 2, 1, 3])),
    ("ragged_many", dict(C=list(range(0, 300, 37)), E=[1, 17, 64, 65, 128, 3, 255, 40, 99])),
    ("long_prefix", dict(C=[3000], E=[96])),
    ("mha_g1", dict(C=[40, 0], E=[100, 77], HKV=8, G=1)),
    ("g4_two_pairs", dict(C=[40, 10], E=[100, 77], HKV=4, G=4)),
    ("tp2_hkv4", dict(C=[200], E=[300], HKV=4, G=2)),
    ("strided_q_table_idx", dict(C=[33, 0, 500], E=[31, 90, 64], q_pad=256, table_idx=True)),
    ("page16_chunks", dict(C=[2048, 0], E=[300, 200], ps=16)),
]


@pytest.mark.parametrize("name,kw", CASES)
def test_extend_matches_oracle(name, kw):
    c = _make(zlib.crc32(name.encode()) % 10000, **kw)
    print(f"extend case {name}: C={c['C'].tolist()} E={c['E'].tolist()}", flush=True)
    got = _run(c)
    ref = _oracle(c)
    mx, rel = check_attention(got, ref, "bf16", name)
    print(f"  max|d|={mx:.3e} relL2={rel:.3e}")
    assert pkv.read_faults() == 0


@pytest.mark.parametrize("grow", [20.0, 60.0])
def test_extend_growing_scores(grow):
    """K rows after each request's first 64 keys scaled by `grow`: later scores
    sit far above the first tile's maximum, so the running maximum moves by
    large steps and the accumulators are rescaled (softmax stays exact)."""
    c = _make(11, C=[300, 0, 70], E=[200, 260, 129])
    K = oracle.widen(c["kv"][0], "bf16")
    for r in range(len(c["S"])):
        later = c["table"][r, 64:c["S"][r]]
        K[later] *= grow
    c["kv"] = np.stack([f32_to_bf16_bits(K.astype(np.float32)), c["kv"][1]])
    got = _run(c)
    ref = _oracle(c)
    mx, rel = check_attention(got, ref, "bf16", f"grow {grow}")
    print(f"  grow {grow}: max|d|={mx:.3e} relL2={rel:.3e}")
    assert pkv.read_faults() == 0


@pytest.mark.parametrize("scale,G", [(0.03, 2), (-0.0884, 2), (-0.0884, 1)])
def test_extend_explicit_scale(scale, G):
    """A softmax scale other than 1/sqrt(head_dim), negative ones included:
    the kernel's running maximum is over unscaled scores, so a negative
    scale must reach it through q's sign, not leave every weight at zero."""
    c = _make(23, C=[100, 0, 333], E=[150, 70, 65], G=G)
    print(f"extend scale {scale} G {G}", flush=True)
    got = _run(c, sm_scale=scale)
    ref = _oracle(c, scale=scale)
    mx, rel = check_attention(got, ref, "bf16", f"scale {scale}")
    print(f"  max|d|={mx:.3e} relL2={rel:.3e}")
    assert pkv.read_faults() == 0


def test_extend_out_of_pool_slot_reads_as_zero_row():
    """A page-table entry outside the pool: that key's K and V rows read as
    zeros and PKV_FAULT_TABLE_SLOT (0x4) is raised; every output row equals
    the oracle's over a pool in which the key's row is zero."""
    c = _make(41, C=[300, 70, 0], E=[150, 90, 40])
    n_slots = c["kv"].shape[1]
    bad_r, bad_j = 0, 123            # a cached key of request 0, seen by all its queries
    gpu_table = c["table"].copy()
    gpu_table[bad_r, bad_j] = n_slots + 5
    ref_table = c["table"].copy()
    ref_table[bad_r, bad_j] = n_slots
    zero = np.zeros((1,) + c["kv"].shape[2:], c["kv"].dtype)
    ref_kv = np.stack([np.concatenate([c["kv"][0], zero]), np.concatenate([c["kv"][1], zero])])
    got = _run(dict(c, table=gpu_table))
    ref = _oracle(dict(c, table=ref_table, kv=ref_kv))
    mx, rel = check_attention(got, ref, "bf16", "out-of-pool slot")
    print(f"  max|d|={mx:.3e} relL2={rel:.3e}")
    assert pkv.read_faults() == 0x4


def test_extend_bad_table_row_request_is_skipped():
    """bf16 pools: a request whose table_idx lies outside the page table is
    skipped and flagged (PKV_FAULT_TABLE_ROW), its output rows are not
    written, and the other requests' rows match the oracle."""
    c = _make(73, C=[40, 100, 7], E=[70, 33, 129], table_idx=True)
    n_rows = c["table"].shape[0]
    rows_ok = c["rows"].copy()
    c["rows"] = c["rows"].copy()
    c["rows"][1] = n_rows + 3
    HQ, n = c["HQ"], c["q"].shape[0]
    out = torch.full((n, HQ, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    qd = to_dev(c["q"], "bf16")[:, :HQ * 128].view(n, HQ, 128)
    pkv.paged_attention_extend(qd, to_dev(c["kv"][0], "bf16"), to_dev(c["kv"][1], "bf16"), to_dev(c["table"]),
                               to_dev(c["C"]), to_dev(c["S"]), max_extend=int(c["E"].max()),
                               table_idx=to_dev(c["rows"]), out=out)
    torch.cuda.synchronize()
    assert pkv.read_faults() == 0x8
    got = oracle.widen(to_host(out), "bf16")
    ref = _oracle(dict(c, rows=rows_ok), rows=[0, 2])
    E0, E1 = int(c["E"][0]), int(c["E"][1])
    keep = np.r_[0:E0, E0 + E1:n]
    check_attention(to_host(out)[keep], ref[keep], "bf16", "around a skipped request")
    assert np.all(got[E0:E0 + E1] == 7.0)


def test_extend_paged_equals_contiguous_bitwise():
    """The same rows through an identity page table and through a permuted one."""
    c = _make(77, C=[100, 0, 9], E=[150, 64, 300])
    got_perm = _run(c)
    # rebuild with rows laid out contiguously (identity table over a packed pool)
    S, rows = c["S"], c["table"]
    packed_k = np.concatenate([c["kv"][0][rows[r, :S[r]]] for r in range(len(S))])
    packed_v = np.concatenate([c["kv"][1][rows[r, :S[r]]] for r in range(len(S))])
    ident = np.zeros_like(c["table"])
    off = 0
    for r in range(len(S)):
        ident[r, :S[r]] = np.arange(off, off + S[r])
        off += S[r]
    c2 = dict(c, table=ident, kv=np.stack([packed_k, packed_v]))
    got_ident = _run(c2)
    assert np.array_equal(got_perm, got_ident)


def test_extend_single_row_matches_decode():
    """extend with E=1 per request and decode over the same batch: both are the
    same attention (different kernels, so compared within the bounds)."""
    c = _make(5, C=[10, 500, 2047, 0], E=[1, 1, 1, 1])
    got_ext = _run(c)
    qd = to_dev(c["q"], "bf16").view(4, c["HQ"], 128)
    got_dec = to_host(pkv.paged_attention_decode(
        qd, to_dev(c["kv"][0], "bf16"), to_dev(c["kv"][1], "bf16"), to_dev(c["table"]), to_dev(c["C"]),
        to_dev(c["S"]), max_total_kv=int(c["S"].sum())))
    torch.cuda.synchronize()
    ref = _oracle(c)
    check_attention(got_ext, ref, "bf16", "extend E=1")
    check_attention(got_dec, ref, "bf16", "decode")


def _pool_refs(requests, dtype):
    """requests: (q rows, K, V, cached) per request in kernel dtype. Returns
    the oracle's fp64 output of every query row, in order, computed in the
    host process pool one chunk of rows at a time."""
    import oracle_pool
    spans, jobs = [], []
    for q, K, V, C in requests:
        for t0, t1, job in oracle_pool.extend_jobs(q, K, V, int(C)):
            spans.append(t1 - t0)
            jobs.append(job)
    outs = list(oracle_pool.attention(jobs, dtype))
    assert [o.shape[0] for o in outs] == spans
    return np.concatenate(outs)


def test_extend_prefill_case_every_row():
    """The 8-request prefill case (extend_len ~ U[512, 4096] over a 0-50%
    cached prefix): the kernel runs on the whole batch after store_kv wrote the
    new rows; every query row of every request is compared with the oracle
    (run in a process pool on the host cores)."""
    cfg = config(4)
    case = draw_case(cfg)
    dt = cfg.dtype
    kp, vp = to_dev(case["k_pool"], dt), to_dev(case["v_pool"], dt)
    pkv.store_kv(kp, vp, to_dev(case["out_loc"]), to_dev(case["new_k"], dt), to_dev(case["new_v"], dt))
    C, S = case["cached_len"], case["device_len"]
    E = S - C
    print(f"extend8: C={C.tolist()} E={E.tolist()}", flush=True)
    o = pkv.paged_attention_extend(to_dev(case["q"], dt), kp, vp, to_dev(case["page_table"]), to_dev(C),
                                   to_dev(S), max_extend=int(E.max()))
    torch.cuda.synchronize()
    got = to_host(o)
    assert pkv.read_faults() == 0
    rk, rv = oracle.store_kv(case["k_pool"], case["v_pool"], case["out_loc"], case["new_k"], case["new_v"])
    cu = np.concatenate([[0], np.cumsum(E)])
    reqs = [(case["q"][cu[r]:cu[r + 1]], rk[case["page_table"][r, :S[r]]], rv[case["page_table"][r, :S[r]]],
             int(C[r])) for r in range(len(S))]
    refs = _pool_refs(reqs, dt)
    mx, rel = check_attention(got, refs, dt, "extend8 every row")
    print(f"  {got.shape[0]} rows: max|d|={mx:.3e} relL2={rel:.3e}", flush=True)
    worst = np.max(np.abs(oracle.widen(got, dt) - refs), axis=(1, 2))
    assert np.all(worst <= 2e-2)


def test_extend_mixed_batch_chunks_full_size():
    """The two 2048-token prefill chunks of the mixed batch (page_size 16,
    cached prefixes of 2048 j tokens) at full size, picked from the batch's
    page table through table_idx, in the launch configuration the benchmark
    times. The pool is drawn on the device; store_kv writes the chunks' new
    rows first; every row of both chunks is compared with the oracle, whose
    inputs are the pool rows read back after the store."""
    from workloads import default_num_pages, draw_lengths, draw_page_table, draw_q
    cfg = config(5)
    C, S = draw_lengths(cfg)
    nump = default_num_pages(cfg, S)
    table = draw_page_table(cfg, S, nump)
    q_all = draw_q(cfg, C, S)
    E = (S - C).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(E)])
    ext = np.nonzero(E > 1)[0].astype(np.int32)
    q = np.concatenate([q_all[cu[r]:cu[r + 1]] for r in ext])
    Ce, Se = C[ext], S[ext]
    num_slots = (nump + 1) * cfg.page_size
    print(f"extend mixed-batch chunks: C={Ce.tolist()} S={Se.tolist()} slots {num_slots}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(2005)
    kp = torch.randn((num_slots, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    vp = torch.randn((num_slots, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    n_new = int((Se - Ce).sum())
    nk = torch.randn((n_new, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    nv = torch.randn((n_new, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    out_loc = np.concatenate([table[r, C[r]:S[r]] for r in ext]).astype(np.int32)
    pkv.store_kv(kp, vp, to_dev(out_loc), nk, nv, page_size=cfg.page_size)
    o = pkv.paged_attention_extend(to_dev(q, "bf16"), kp, vp, to_dev(table), to_dev(Ce), to_dev(Se),
                                   table_idx=to_dev(ext), max_extend=int((Se - Ce).max()),
                                   page_size=cfg.page_size)
    torch.cuda.synchronize()
    got = to_host(o)
    assert pkv.read_faults() == 0
    cq = np.concatenate([[0], np.cumsum(Se - Ce)])
    reqs = []
    for i, r in enumerate(ext):
        slots = torch.from_numpy(table[r, :S[r]].astype(np.int64)).cuda()
        reqs.append((q[cq[i]:cq[i + 1]], to_host(kp.index_select(0, slots)), to_host(vp.index_select(0, slots)),
                     int(Ce[i])))
    refs = _pool_refs(reqs, "bf16")
    mx, rel = check_attention(got, refs, "bf16", "mixed-batch chunks every row")
    print(f"  {got.shape[0]} rows: max|d|={mx:.3e} relL2={rel:.3e}", flush=True)
    worst = np.max(np.abs(oracle.widen(got, "bf16") - refs), axis=(1, 2))
    assert np.all(worst <= 2e-2)


# ---------------------------------------------------------------- fp32 pools (rows as decode rows)

@pytest.mark.parametrize("name,C,E,hkv,g", [
    ("f32_small", [5, 0, 37], [4, 9, 30], 8, 2),
    ("f32_one_row_each", [16, 1, 2], [1, 1, 1], 8, 2),
    ("f32_long", [300, 0], [250, 700], 4, 2),
    ("f32_mha", [9, 33], [17, 5], 8, 1),
])
def test_extend_fp32_matches_oracle(name, C, E, hkv, g):
    """fp32 pools: every query row runs as a decode row of C + t + 1 keys (fp32
    throughout); max-abs 1e-5 against the oracle on every row. total_q one
    larger than the rows: the extra output row stays untouched."""
    c = _make(zlib.crc32(name.encode()) % 1000, C, E, HKV=hkv, G=g)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    n = int(c["E"].sum())
    kv = rng.standard_normal(c["kv"].shape, dtype=np.float32)
    q = rng.standard_normal((n + 1, c["HQ"], 128), dtype=np.float32)
    out = torch.full((n + 1, c["HQ"], 128), 7.0, dtype=torch.float32, device="cuda")
    print(f"extend fp32 case {name}", flush=True)
    o = pkv.paged_attention_extend(to_dev(q), to_dev(kv[0]), to_dev(kv[1]), to_dev(c["table"]), to_dev(c["C"]),
                                   to_dev(c["S"]), max_extend=int(c["E"].max()), out=out)
    torch.cuda.synchronize()
    got = to_host(o)
    assert np.all(got[n] == 7.0), "the row past the batch's rows was written"
    ref = oracle.attention_extend(q[:n], kv[0], kv[1], c["table"], c["C"], c["S"], "f32")
    mx, _ = check_attention(got[:n], ref, "f32", name)
    print(f"  {n} rows: max|d|={mx:.3e}", flush=True)
    assert pkv.read_faults() == 0


def test_extend_fp32_invalid_request_is_skipped():
    """A request with cached_len >= device_len is skipped and flagged; the
    other requests' rows are still computed."""
    c = _make(71, [3, 4, 10], [5, 6, 7])
    rng = np.random.default_rng(71)
    kv = rng.standard_normal(c["kv"].shape, dtype=np.float32)
    n = int(c["E"].sum())
    q = rng.standard_normal((n, c["HQ"], 128), dtype=np.float32)
    C_bad = c["C"].copy()
    C_bad[1] = c["S"][1]                                   # E = 0 and C == S: invalid
    out = torch.full((n, c["HQ"], 128), 7.0, dtype=torch.float32, device="cuda")
    print("extend fp32 invalid request", flush=True)
    pkv.paged_attention_extend(to_dev(q), to_dev(kv[0]), to_dev(kv[1]), to_dev(c["table"]), to_dev(C_bad),
                               to_dev(c["S"]), max_extend=7, out=out)
    torch.cuda.synchronize()
    assert pkv.read_faults() & 0x2
    got = to_host(out)
    # request 1 has no rows now; request 2's rows follow request 0's directly
    E0, E2 = int(c["E"][0]), int(c["E"][2])
    C2 = np.array([c["C"][0], c["C"][2]], np.int32)
    S2 = np.array([c["S"][0], c["S"][2]], np.int32)
    tab2 = c["table"][[0, 2]]
    q2 = np.concatenate([q[:E0], q[E0:E0 + E2]])
    ref = oracle.attention_extend(q2, kv[0], kv[1], tab2, C2, S2, "f32")
    check_attention(got[:E0 + E2], ref, "f32", "fp32 extend around an invalid request")
    assert np.all(got[E0 + E2:] == 7.0)
