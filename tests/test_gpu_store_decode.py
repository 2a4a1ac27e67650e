"""GPU parity: store_kv (bit-exact) and decode attention (fp32 max-abs 1e-5;
bf16 max-abs 2e-2 and relative L2 1e-2) against the oracle, through the C ABI."""

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
    pkv.read_faults()  # clear


def _upload_case(case):
    dt = case["cfg"].dtype
    return dict(
        k_pool=to_dev(case["k_pool"], dt), v_pool=to_dev(case["v_pool"], dt),
        new_k=to_dev(case["new_k"], dt), new_v=to_dev(case["new_v"], dt),
        out_loc=to_dev(case["out_loc"]), q=to_dev(case["q"], dt),
        page_table=to_dev(case["page_table"]), cached_len=to_dev(case["cached_len"]),
        device_len=to_dev(case["device_len"]))


def _store_and_check(case, d, loc_dtype=torch.int32):
    ps = case["cfg"].page_size
    print(f"store_kv case {case['cfg'].name} rows={len(case['out_loc'])}", flush=True)
    pkv.store_kv(d["k_pool"], d["v_pool"], d["out_loc"].to(loc_dtype), d["new_k"], d["new_v"], page_size=ps)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.store_kv(case["k_pool"], case["v_pool"], case["out_loc"], case["new_k"],
                                   case["new_v"])
    gk, gv = to_host(d["k_pool"]), to_host(d["v_pool"])
    assert np.array_equal(gk.view(np.uint8), ref_k.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), ref_v.view(np.uint8))
    assert pkv.read_faults() == 0
    return ref_k, ref_v


@pytest.mark.parametrize("cid,loc_dtype", [(1, torch.int32), (1, torch.int64), (2, torch.int32),
                                           (4, torch.int64)])
def test_store_kv_bit_exact(cid, loc_dtype):
    case = draw_case(config(cid))
    _store_and_check(case, _upload_case(case), loc_dtype)


def test_store_kv_strided_rows():
    """k and v as column slices of one fused [n, (HQ + 2 HKV) * 128] buffer."""
    rng = np.random.default_rng(3)
    n, HKV, slots = 37, 8, 300
    qkv = f32_to_bf16_bits(rng.standard_normal((n, (16 + 2 * HKV) * 128), dtype=np.float32))
    qkv_d = to_dev(qkv, "bf16")
    k = qkv_d[:, 16 * 128:24 * 128].view(n, HKV, 128)
    v = qkv_d[:, 24 * 128:].view(n, HKV, 128)
    pool_k = np.full((slots, HKV, 128), 0x7FC0, np.uint16)
    pool_v = pool_k.copy()
    loc = rng.permutation(slots)[:n].astype(np.int32)
    dk, dv = to_dev(pool_k, "bf16"), to_dev(pool_v, "bf16")
    pkv.store_kv(dk, dv, to_dev(loc), k, v)
    torch.cuda.synchronize()
    rk, rv = oracle.store_kv(pool_k, pool_v, loc, qkv[:, 16 * 128:24 * 128].reshape(n, HKV, 128),
                             qkv[:, 24 * 128:].reshape(n, HKV, 128))
    assert np.array_equal(to_host(dk), rk) and np.array_equal(to_host(dv), rv)


@pytest.mark.parametrize("cid", [1, 2])
def test_decode_after_store_matches_oracle(cid):
    case = draw_case(config(cid))
    d = _upload_case(case)
    ref_k, ref_v = _store_and_check(case, d)
    dt = case["cfg"].dtype
    print(f"decode case {case['cfg'].name} bs={len(case['device_len'])}", flush=True)
    o = pkv.paged_attention_decode(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["cached_len"],
                                   d["device_len"], max_total_kv=int(case["device_len"].sum()))
    torch.cuda.synchronize()
    ref = oracle.attention_decode(case["q"], ref_k, ref_v, case["page_table"], case["cached_len"],
                                  case["device_len"], dt)
    mx, rel = check_attention(to_host(o), ref, dt, case["cfg"].name)
    print(f"  max|d|={mx:.3e} relL2={rel:.3e}")
    assert pkv.read_faults() == 0


def _random_decode(seed, bs, lens, HKV=8, G=2, dtype="bf16", slots_extra=64, q_pad=0, table_idx=False,
                   ps=1):
    """A decode batch with explicit lengths, random slots, pool fully random."""
    rng = np.random.default_rng(seed)
    HQ = HKV * G
    S = np.asarray(lens, np.int32)
    total = int(S.sum())
    width = (int(S.max()) + 31) // 32 * 32
    n_slots = total + slots_extra
    perm = rng.permutation(n_slots)
    table = np.full((bs + 3, width), n_slots - 1, np.int32)
    rows = rng.permutation(bs + 3)[:bs].astype(np.int32) if table_idx else np.arange(bs, dtype=np.int32)
    off = 0
    for r in range(bs):
        table[rows[r], :S[r]] = perm[off:off + S[r]]
        off += S[r]
    kv = rng.standard_normal((2, n_slots, HKV, 128), dtype=np.float32)
    qf = rng.standard_normal((bs, HQ * 128 + q_pad), dtype=np.float32)
    if dtype == "bf16":
        kv, qf = f32_to_bf16_bits(kv), f32_to_bf16_bits(qf)
    return dict(S=S, C=S - 1, table=table, rows=rows if table_idx else None, kv=kv, q=qf, HQ=HQ, HKV=HKV)


def _run_decode(c, dtype, max_total_kv=None, sm_scale=0.0):
    dk, dv = to_dev(c["kv"][0], dtype), to_dev(c["kv"][1], dtype)
    qd = to_dev(c["q"], dtype)
    bs = len(c["S"])
    qv = qd[:, :c["HQ"] * 128].view(bs, c["HQ"], 128)
    o = pkv.paged_attention_decode(
        qv, dk, dv, to_dev(c["table"]), to_dev(c["C"]), to_dev(c["S"]),
        table_idx=None if c["rows"] is None else to_dev(c["rows"]),
        max_total_kv=int(c["S"].sum()) if max_total_kv is None else max_total_kv, sm_scale=sm_scale)
    torch.cuda.synchronize()
    qh = c["q"][:, :c["HQ"] * 128].reshape(bs, c["HQ"], 128)
    ref = oracle.attention_decode(qh, c["kv"][0], c["kv"][1], c["table"], c["C"], c["S"], dtype,
                                  table_idx=c["rows"], scale=sm_scale if sm_scale != 0.0 else None)
    return to_host(o), ref


@pytest.mark.parametrize("name,kw", [
    ("one_long", dict(bs=1, lens=[20000])),
    ("ragged_small", dict(bs=7, lens=[1, 2, 3, 64, 65, 127, 300])),
    ("many_tiny", dict(bs=300, lens=list(range(1, 301)))),
    ("tp2_shard_hkv4", dict(bs=5, lens=[100, 900, 33, 5000, 1], HKV=4, G=2)),
    ("mha_g1", dict(bs=3, lens=[50, 700, 129], HKV=8, G=1)),
    ("g4", dict(bs=3, lens=[50, 700, 129], HKV=4, G=4)),
    ("q_strided_table_idx", dict(bs=6, lens=[10, 400, 2000, 3, 77, 1024], q_pad=8 * 256, table_idx=True)),
    ("f32_hkv2", dict(bs=4, lens=[5, 9, 17, 333], HKV=2, G=2, dtype="f32")),
    ("f32_g1", dict(bs=4, lens=[5, 900, 17, 33], HKV=8, G=1, dtype="f32")),
    # every other (kv_heads, group) the library dispatches
    ("hkv8_g4_32heads", dict(bs=5, lens=[2, 3000, 257, 700, 1], HKV=8, G=4)),
    ("hkv4_g1", dict(bs=4, lens=[1, 640, 2049, 90], HKV=4, G=1)),
    ("f32_hkv8_g2", dict(bs=5, lens=[1, 1500, 256, 257, 40], HKV=8, G=2, dtype="f32")),
    ("f32_hkv8_g4", dict(bs=3, lens=[700, 3, 1200], HKV=8, G=4, dtype="f32")),
    ("f32_hkv4_g1", dict(bs=3, lens=[1, 900, 64], HKV=4, G=1, dtype="f32")),
    ("f32_hkv4_g2", dict(bs=4, lens=[800, 2, 333, 1025], HKV=4, G=2, dtype="f32")),
    ("f32_hkv4_g4", dict(bs=3, lens=[5, 1700, 260], HKV=4, G=4, dtype="f32")),
    ("f32_hkv2_g4", dict(bs=3, lens=[1000, 1, 77], HKV=2, G=4, dtype="f32")),
])
def test_decode_shapes(name, kw):
    dtype = kw.get("dtype", "bf16")
    c = _random_decode(zlib.crc32(name.encode()) % 1000, **kw)
    print(f"decode shape case {name}", flush=True)
    got, ref = _run_decode(c, dtype)
    check_attention(got, ref, dtype, name)
    assert pkv.read_faults() == 0


@pytest.mark.parametrize("dtype,scale", [("bf16", 0.03), ("bf16", -0.0884), ("f32", -0.2)])
def test_decode_explicit_scale(dtype, scale):
    """A softmax scale other than 1/sqrt(head_dim), negative ones included:
    the weights are those of the scaled scores, whatever the sign."""
    c = _random_decode(31, 5, [1, 700, 64, 3000, 129], dtype=dtype)
    print(f"decode scale {scale} ({dtype})", flush=True)
    got, ref = _run_decode(c, dtype, sm_scale=scale)
    check_attention(got, ref, dtype, f"scale {scale}")
    assert pkv.read_faults() == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_out_of_pool_slot_reads_as_zero_row(dtype):
    """A page-table entry outside the pool: that key's K and V rows read as
    zeros and PKV_FAULT_TABLE_SLOT (0x4) is raised; every output row equals
    the oracle's over a pool in which the key's row is zero."""
    c = _random_decode(43, 4, [700, 1, 65, 2000], dtype=dtype)
    n_slots = c["kv"].shape[1]
    bad_r, bad_j = 3, 1500
    ref_table = c["table"].copy()
    ref_table[bad_r, bad_j] = n_slots
    c["table"][bad_r, bad_j] = n_slots + 5
    zero = np.zeros((1,) + c["kv"].shape[2:], c["kv"].dtype)
    ref_kv = np.stack([np.concatenate([c["kv"][0], zero]), np.concatenate([c["kv"][1], zero])])
    qv = to_dev(c["q"], dtype).view(4, c["HQ"], 128)
    o = pkv.paged_attention_decode(qv, to_dev(c["kv"][0], dtype), to_dev(c["kv"][1], dtype), to_dev(c["table"]),
                                   to_dev(c["C"]), to_dev(c["S"]), max_total_kv=int(c["S"].sum()))
    torch.cuda.synchronize()
    got = to_host(o)
    qh = c["q"][:, :c["HQ"] * 128].reshape(4, c["HQ"], 128)
    ref = oracle.attention_decode(qh, ref_kv[0], ref_kv[1], ref_table, c["C"], c["S"], dtype)
    check_attention(got, ref, dtype, f"out-of-pool slot ({dtype})")
    assert pkv.read_faults() == 0x4


def test_decode_loose_bound_same_result():
    """A loose max_total_kv bound changes the work split, not the answer
    (beyond float reassociation)."""
    c = _random_decode(5, 9, [300, 1, 4000, 77, 2048, 9, 15, 1000, 600])
    a, ref = _run_decode(c, "bf16")
    b, _ = _run_decode(c, "bf16", max_total_kv=10_000_000)
    check_attention(a, ref, "bf16", "tight")
    check_attention(b, ref, "bf16", "loose")


def test_decode_paged_equals_contiguous_bitwise():
    """Identity page table over contiguous rows vs a random permutation of the
    same rows: the kernel's arithmetic must not depend on where rows sit."""
    rng = np.random.default_rng(9)
    S = np.array([700, 5, 1500, 64], np.int32)
    total, HKV, HQ = int(S.sum()), 8, 16
    K = f32_to_bf16_bits(rng.standard_normal((total, HKV, 128), dtype=np.float32))
    V = f32_to_bf16_bits(rng.standard_normal((total, HKV, 128), dtype=np.float32))
    q = to_dev(f32_to_bf16_bits(rng.standard_normal((4, HQ, 128), dtype=np.float32)), "bf16")
    width = 1536
    ident = np.zeros((4, width), np.int32)
    permt = np.zeros((4, width), np.int32)
    perm = rng.permutation(total + 100)[:total]
    Kp = np.zeros((total + 100, HKV, 128), np.uint16)
    Vp = np.zeros_like(Kp)
    Kp[perm], Vp[perm] = K, V
    off = 0
    for r, s in enumerate(S):
        ident[r, :s] = np.arange(off, off + s)
        permt[r, :s] = perm[off:off + s]
        off += s
    outs = []
    for table, kk, vv in ((ident, K, V), (permt, Kp, Vp)):
        outs.append(to_host(pkv.paged_attention_decode(
            q, to_dev(kk, "bf16"), to_dev(vv, "bf16"), to_dev(table), to_dev(S - 1), to_dev(S),
            max_total_kv=total)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])


def test_decode_single_key_returns_v():
    c = _random_decode(12, 3, [1, 1, 1])
    got, ref = _run_decode(c, "bf16")
    for r in range(3):
        slot = c["table"][r, 0]
        for h in range(16):
            assert np.array_equal(got[r, h], c["kv"][1][slot, h // 2])


@pytest.mark.parametrize("cid", [3, 5])
def test_decode_full_size_every_request(cid):
    """Decode at the full sizes of the 256-request batch (config 3, page_size 1)
    and of the 240 decode rows of the mixed batch (config 5, page_size 16,
    contexts up to 32768, rows picked through table_idx), in the launch
    configuration the benchmark times. The pool is filled on the device with
    torch draws (the inputs); store_kv writes each request's new row first;
    every request's output is compared with the oracle's, whose inputs are the
    request's pool rows read back after the store (the oracle runs in a
    process pool on the host cores)."""
    import oracle_pool
    from workloads import default_num_pages, draw_lengths, draw_page_table, draw_q
    cfg = config(cid)
    C, S = draw_lengths(cfg)
    nump = default_num_pages(cfg, S)
    table = draw_page_table(cfg, S, nump)
    q_all = draw_q(cfg, C, S)
    E = (S - C).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(E)])
    dec = np.nonzero(E == 1)[0].astype(np.int32)
    q = q_all[cu[dec]]
    Cd, Sd = C[dec], S[dec]
    num_slots = (nump + 1) * cfg.page_size
    print(f"decode full-size case {cfg.name}: {len(dec)} rows, sum S {int(Sd.sum())}, slots {num_slots}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(1000 + cid)
    kp = torch.randn((num_slots, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    vp = torch.randn((num_slots, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    nk = torch.randn((len(dec), 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    nv = torch.randn((len(dec), 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    out_loc = table[dec, Cd].astype(np.int32)
    pkv.store_kv(kp, vp, to_dev(out_loc), nk, nv, page_size=cfg.page_size)
    o = pkv.paged_attention_decode(to_dev(q, "bf16"), kp, vp, to_dev(table), to_dev(Cd), to_dev(Sd),
                                   table_idx=to_dev(dec), max_total_kv=int(Sd.sum()), page_size=cfg.page_size)
    torch.cuda.synchronize()
    got = to_host(o)
    assert pkv.read_faults() == 0

    def jobs():  # each request's rows, read back from the pool after the store
        for i in range(len(dec)):
            slots = torch.from_numpy(table[dec[i], :Sd[i]].astype(np.int64)).cuda()
            yield q[i:i + 1], to_host(kp.index_select(0, slots)), to_host(vp.index_select(0, slots)), int(Cd[i])

    refs = np.stack([r[0] for r in oracle_pool.attention(jobs(), "bf16")])
    assert refs.shape[0] == len(dec)
    mx, rel = check_attention(got, refs, "bf16", f"{cfg.name} every request")
    print(f"  {len(dec)} requests: max|d|={mx:.3e} relL2={rel:.3e}", flush=True)
    worst = np.max(np.abs(oracle.widen(got, "bf16") - refs), axis=(1, 2))
    assert np.all(worst <= 2e-2)


# ---------------------------------------------------------------- store_kv fused into decode

def _fused_vs_separate(case, loc_dtype=torch.int32):
    """pkv_paged_attention_decode_store on one copy of the pool, store_kv then
    decode on another: the outputs and the whole pools must be equal bit for
    bit; the separate path is itself held to the oracle above."""
    d1, d2 = _upload_case(case), _upload_case(case)
    ps = case["cfg"].page_size
    kw = dict(max_total_kv=int(case["device_len"].sum()), page_size=ps)
    loc = d1["out_loc"].to(loc_dtype)
    pkv.store_kv(d1["k_pool"], d1["v_pool"], loc, d1["new_k"], d1["new_v"], page_size=ps)
    o_sep = pkv.paged_attention_decode(d1["q"], d1["k_pool"], d1["v_pool"], d1["page_table"], d1["cached_len"],
                                       d1["device_len"], **kw)
    o_fus = pkv.paged_attention_decode_store(d2["q"], d2["k_pool"], d2["v_pool"], d2["page_table"],
                                             d2["cached_len"], d2["device_len"], loc, d2["new_k"], d2["new_v"], **kw)
    torch.cuda.synchronize()
    i16 = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    assert torch.equal(i16(o_fus), i16(o_sep)), f"{case['cfg'].name}: fused output differs"
    assert torch.equal(i16(d2["k_pool"]), i16(d1["k_pool"])) and torch.equal(i16(d2["v_pool"]), i16(d1["v_pool"]))
    assert pkv.read_faults() == 0


@pytest.mark.parametrize("cid,loc_dtype", [(1, torch.int32), (2, torch.int64)])
def test_decode_store_fused_equals_store_then_decode(cid, loc_dtype):
    print(f"decode_store case config {cid}", flush=True)
    _fused_vs_separate(draw_case(config(cid)), loc_dtype)


@pytest.mark.parametrize("cid", [3, 5])
def test_decode_store_fused_full_size(cid):
    """The fused call at the full sizes of the 256-request batch and of the
    mixed batch's 240 decode rows (page_size 16, rows through table_idx), pools
    drawn on the device: outputs and pools equal to store_kv then decode, bit
    for bit (the separate path is held to the oracle on every request above)."""
    from workloads import default_num_pages, draw_lengths, draw_page_table, draw_q
    cfg = config(cid)
    C, S = draw_lengths(cfg)
    nump = default_num_pages(cfg, S)
    table = draw_page_table(cfg, S, nump)
    q_all = draw_q(cfg, C, S)
    E = (S - C).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(E)])
    dec = np.nonzero(E == 1)[0].astype(np.int32)
    Cd, Sd = C[dec], S[dec]
    num_slots = (nump + 1) * cfg.page_size
    print(f"decode_store full-size case {cfg.name}: {len(dec)} rows, sum S {int(Sd.sum())}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(2000 + cid)
    kp = torch.randn((num_slots, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    vp = torch.randn((num_slots, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    kp2, vp2 = kp.clone(), vp.clone()
    nk = torch.randn((len(dec), 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    nv = torch.randn((len(dec), 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    q = to_dev(q_all[cu[dec]], "bf16")
    loc, dt, dC, dS, di = (to_dev(table[dec, Cd].astype(np.int32)), to_dev(table), to_dev(Cd), to_dev(Sd),
                           to_dev(dec))
    kw = dict(table_idx=di, max_total_kv=int(Sd.sum()), page_size=cfg.page_size)
    pkv.store_kv(kp, vp, loc, nk, nv, page_size=cfg.page_size)
    o_sep = pkv.paged_attention_decode(q, kp, vp, dt, dC, dS, **kw)
    o_fus = pkv.paged_attention_decode_store(q, kp2, vp2, dt, dC, dS, loc, nk, nv, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_fus.view(torch.int16), o_sep.view(torch.int16))
    assert torch.equal(kp2.view(torch.int16), kp.view(torch.int16))
    assert torch.equal(vp2.view(torch.int16), vp.view(torch.int16))
    assert pkv.read_faults() == 0


def test_decode_store_strided_rows_and_table_idx():
    """New rows as column slices of a fused qkv buffer; requests through
    table_idx; lengths from 1 to 3000 (items of every kind)."""
    c = _random_decode(41, 6, [1, 2, 700, 3000, 33, 129], table_idx=True)
    rng = np.random.default_rng(42)
    bs = 6
    S, rows, table = c["S"], c["rows"], c["table"]
    loc = table[rows, S - 1].astype(np.int32)
    qkv = f32_to_bf16_bits(rng.standard_normal((bs, (16 + 16) * 128), dtype=np.float32))
    qkv_d = to_dev(qkv, "bf16")
    k, v = qkv_d[:, 16 * 128:24 * 128].view(bs, 8, 128), qkv_d[:, 24 * 128:].view(bs, 8, 128)
    pools = [(to_dev(c["kv"][0], "bf16"), to_dev(c["kv"][1], "bf16")) for _ in range(2)]
    q = to_dev(c["q"], "bf16").view(bs, 16, 128)
    kw = dict(table_idx=to_dev(rows), max_total_kv=int(S.sum()))
    dt, dC, dS, dl = to_dev(table), to_dev(c["C"]), to_dev(S), to_dev(loc)
    pkv.store_kv(pools[0][0], pools[0][1], dl, k, v)
    o_sep = pkv.paged_attention_decode(q, pools[0][0], pools[0][1], dt, dC, dS, **kw)
    o_fus = pkv.paged_attention_decode_store(q, pools[1][0], pools[1][1], dt, dC, dS, dl, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_fus.view(torch.int16), o_sep.view(torch.int16))
    assert torch.equal(pools[1][0].view(torch.int16), pools[0][0].view(torch.int16))
    assert torch.equal(pools[1][1].view(torch.int16), pools[0][1].view(torch.int16))
    assert pkv.read_faults() == 0


def test_decode_store_fault_paths():
    """out_loc[r] off the table's last entry: the new row is still key S - 1
    (against the oracle with that row in place) and PKV_FAULT_OUT_LOC is set;
    out_loc[r] outside the pool: nothing written, PKV_FAULT_STORE_SLOT."""
    c = _random_decode(43, 3, [50, 300, 7], slots_extra=8)
    S, table = c["S"], c["table"]
    n_slots = c["kv"].shape[1]
    rng = np.random.default_rng(44)
    new = f32_to_bf16_bits(rng.standard_normal((2, 3, 8, 128), dtype=np.float32))
    loc = table[np.arange(3), S - 1].astype(np.int32)
    free = np.setdiff1d(np.arange(n_slots - 1), table[:3][table[:3] != n_slots - 1])
    loc[1] = int(free[0])                                   # not the table's entry for key S - 1
    dk, dv = to_dev(c["kv"][0], "bf16"), to_dev(c["kv"][1], "bf16")
    q = to_dev(c["q"], "bf16").view(3, 16, 128)
    o = pkv.paged_attention_decode_store(q, dk, dv, to_dev(table), to_dev(c["C"]), to_dev(S), to_dev(loc),
                                         to_dev(new[0], "bf16"), to_dev(new[1], "bf16"), max_total_kv=int(S.sum()))
    torch.cuda.synchronize()
    assert pkv.read_faults() == 0x20
    kp, vp = c["kv"][0].copy(), c["kv"][1].copy()
    kp[loc], vp[loc] = new[0], new[1]
    assert np.array_equal(to_host(dk), kp) and np.array_equal(to_host(dv), vp)
    # the reference: every request's key S - 1 is its new row, wherever out_loc points
    kr, vr = c["kv"][0].copy(), c["kv"][1].copy()
    kr[table[np.arange(3), S - 1]], vr[table[np.arange(3), S - 1]] = new[0], new[1]
    ref = oracle.attention_decode(c["q"].reshape(3, 16, 128), kr, vr, table, c["C"], S, "bf16")
    check_attention(to_host(o), ref, "bf16", "decode_store out_loc off the table")
    # out of the pool
    loc2 = table[np.arange(3), S - 1].astype(np.int64)
    loc2[2] = n_slots + 5
    before = to_host(dk).copy()
    pkv.paged_attention_decode_store(q, dk, dv, to_dev(table), to_dev(c["C"]), to_dev(S), to_dev(loc2),
                                     to_dev(new[0], "bf16"), to_dev(new[1], "bf16"), max_total_kv=int(S.sum()))
    torch.cuda.synchronize()
    assert pkv.read_faults() & 0x1
    after = to_host(dk)
    changed = np.nonzero(np.any(after != before, axis=(1, 2)))[0]
    assert set(changed.tolist()) <= set(loc2[:2].tolist())


def test_decode_store_skipped_request_stores_nothing():
    """A request skipped for an invalid table row (table_idx out of range) or
    an invalid length (device_len beyond the table width): its output row is
    zero, nothing is written at its out_loc, the fault bits are set, and the
    other requests equal store_kv then decode bit for bit."""
    c = _random_decode(45, 4, [40, 300, 9, 1000], table_idx=True)
    S, rows, table = c["S"].copy(), c["rows"].copy(), c["table"]
    loc = table[rows, S - 1].astype(np.int32)
    rng = np.random.default_rng(46)
    new = f32_to_bf16_bits(rng.standard_normal((2, 4, 8, 128), dtype=np.float32))
    bad = rows.copy()
    bad[1] = table.shape[0] + 7                      # request 1: table row out of range
    S_bad = S.copy()
    S_bad[3] = table.shape[1] + 1                    # request 3: longer than the table
    q = to_dev(c["q"], "bf16").view(4, 16, 128)
    dk, dv = to_dev(c["kv"][0], "bf16"), to_dev(c["kv"][1], "bf16")
    o = pkv.paged_attention_decode_store(q, dk, dv, to_dev(table), to_dev(S_bad - 1), to_dev(S_bad), to_dev(loc),
                                         to_dev(new[0], "bf16"), to_dev(new[1], "bf16"), table_idx=to_dev(bad),
                                         max_total_kv=int(S_bad.sum()))
    torch.cuda.synchronize()
    assert pkv.read_faults() == (0x8 | 0x2)
    got = to_host(o)
    assert not np.any(got[1]) and not np.any(got[3])
    kp, vp = c["kv"][0].copy(), c["kv"][1].copy()
    kp[loc[[0, 2]]], vp[loc[[0, 2]]] = new[0][[0, 2]], new[1][[0, 2]]
    assert np.array_equal(to_host(dk), kp) and np.array_equal(to_host(dv), vp)
    # requests 0 and 2 against the separate calls on a copy of the pool
    d2k, d2v = to_dev(c["kv"][0], "bf16"), to_dev(c["kv"][1], "bf16")
    keep = np.array([0, 2])
    pkv.store_kv(d2k, d2v, to_dev(loc[keep]), to_dev(new[0][keep], "bf16"), to_dev(new[1][keep], "bf16"))
    o2 = pkv.paged_attention_decode(to_dev(c["q"][keep], "bf16").view(2, 16, 128), d2k, d2v, to_dev(table),
                                    to_dev(S[keep] - 1), to_dev(S[keep]), table_idx=to_dev(rows[keep]),
                                    max_total_kv=int(S[keep].sum()))
    torch.cuda.synchronize()
    assert pkv.read_faults() == 0
    # equal values (the two calls merge the same partials; only a -0 could differ in bits)
    assert np.array_equal(oracle.widen(got[keep], "bf16"), oracle.widen(to_host(o2), "bf16"))
