"""GPU parity of pkv_qk_norm_rope_store_kv (per-head q/k RMSNorm, rotary
embedding, K/V store) against the oracle.

Tolerance, from the arithmetic: the kernel works in fp32 -- a few fp32
roundings (relative 2^-24 each) on values of the head's scale, fp32 sin/cos
of the same fp32 angle the oracle uses (a few ulp) -- so its fp32 result is
within ~1e-6 of the head's scale of the exact value; bf16 outputs are then
rounded to nearest even. Each element must lie within one bf16 ulp of the
fp64 oracle value plus 2^-20 times the largest |value| of its head (the
second term covers cancellation in the rotation); fp32 outputs within 2^-20
times that scale. V rows are copies and must be bit-exact, as must every pool
slot the call does not write."""

import zlib

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
pkv = pytest.importorskip("paged_kv_attention_scatter_amd")

THETA, EPS = 1_000_000.0, 1e-6
SENTINEL = 0x7FC0


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.read_faults()


def _rng(name):
    return np.random.default_rng(zlib.crc32(name.encode()))


def _case(name, n, hq, hkv, dtype, slots=None, max_pos=32768):
    rng = _rng(name)
    num_slots = slots or (n + 17)
    as_dt = (lambda x: f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    return dict(
        q=as_dt(rng.standard_normal((n, hq, 128), dtype=np.float32)),
        k=as_dt(rng.standard_normal((n, hkv, 128), dtype=np.float32) * 2.0),
        v=as_dt(rng.standard_normal((n, hkv, 128), dtype=np.float32)),
        wq=as_dt(rng.uniform(0.5, 1.5, 128).astype(np.float32)),
        wk=as_dt(rng.uniform(0.5, 1.5, 128).astype(np.float32)),
        pos=rng.integers(0, max_pos, n).astype(np.int32),
        loc=rng.permutation(num_slots)[:n].astype(np.int32),
        num_slots=num_slots, hq=hq, hkv=hkv, dtype=dtype)


def _pool(c):
    shape = (c["num_slots"], c["hkv"], 128)
    if c["dtype"] == "bf16":
        return np.full(shape, SENTINEL, np.uint16), np.full(shape, SENTINEL, np.uint16)
    return np.full(shape, np.nan, np.float32), np.full(shape, np.nan, np.float32)


def _check(got, ref, dtype, what):
    """got: kernel output (bf16 bits or fp32) [..., heads, 128]; ref: fp64."""
    g = oracle.widen(got, dtype)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    tol = scale * 2.0 ** -20
    if dtype == "bf16":
        e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126)))
        tol = tol + 2.0 ** (e - 7)
    err = np.abs(g - ref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} elements off, first {bad[:3].tolist()} err {err[tuple(bad[0])]:.3e}"
    return float(np.max(err / np.maximum(scale, 1e-30)))


def _bits(x):
    return np.ascontiguousarray(x).view(np.uint8)


def _run(c, loc_dtype=torch.int32, in_place=False, q_pad=0, kv_pad=0):
    dt = c["dtype"]
    kp_h, vp_h = _pool(c)
    kp, vp = to_dev(kp_h, dt), to_dev(vp_h, dt)
    n, hq, hkv = c["q"].shape[0], c["hq"], c["hkv"]

    def padded(x, pad, heads):  # rows with `pad` extra elements
        if not pad:
            return to_dev(x, dt)
        big = np.zeros((n, heads * 128 + pad), dtype=x.dtype)
        big[:, :heads * 128] = x.reshape(n, -1)
        return to_dev(big, dt)[:, :heads * 128].view(n, heads, 128)

    q = padded(c["q"], q_pad, hq)
    k, v = padded(c["k"], kv_pad, hkv), padded(c["v"], kv_pad, hkv)
    loc = to_dev(c["loc"]).to(loc_dtype)
    print(f"qk-rope case n={n} hq={hq} hkv={hkv} {dt} loc={loc_dtype} in_place={in_place} "
          f"pads={q_pad},{kv_pad}", flush=True)
    qo = pkv.qk_norm_rope_store_kv(kp, vp, loc, q, k, v, to_dev(c["pos"]), to_dev(c["wq"], dt), to_dev(c["wk"], dt),
                                   eps=EPS, rope_theta=THETA, q_out=q if in_place else None)
    torch.cuda.synchronize()
    w = lambda x: oracle.widen(x, dt)
    rq, rk = oracle.qk_norm_rope(w(c["q"]), w(c["k"]), c["pos"], w(c["wq"]), w(c["wk"]), EPS, THETA)
    eq = _check(to_host(qo), rq, dt, "q_out")
    kp_g, vp_g = to_host(kp), to_host(vp)
    ek = _check(kp_g[c["loc"]], rk, dt, "pool K rows")
    assert np.array_equal(_bits(vp_g[c["loc"]]), _bits(c["v"])), "pool V rows differ"
    untouched = np.setdiff1d(np.arange(c["num_slots"]), c["loc"])
    assert np.array_equal(_bits(kp_g[untouched]), _bits(kp_h[untouched])), "K slots outside out_loc written"
    assert np.array_equal(_bits(vp_g[untouched]), _bits(vp_h[untouched])), "V slots outside out_loc written"
    assert pkv.read_faults() == 0
    print(f"  max err / head scale: q {eq:.2e}, k {ek:.2e}")


@pytest.mark.parametrize("n,hq,hkv", [(37, 16, 8), (5, 8, 4), (9, 32, 8), (13, 4, 2), (3, 2, 1), (64, 16, 16)])
def test_matches_oracle_bf16(n, hq, hkv):
    _run(_case(f"bf16-{n}-{hq}-{hkv}", n, hq, hkv, "bf16"))


def test_matches_oracle_fp32():
    _run(_case("f32", 21, 16, 8, "f32"))


def test_int64_slots_strides_and_in_place():
    _run(_case("strided", 19, 16, 8, "bf16"), loc_dtype=torch.int64, in_place=True, q_pad=8, kv_pad=24)


def test_position_zero_normalises_only():
    """At position 0 the rotation is the identity: the output is the RMSNorm alone."""
    c = _case("pos0", 8, 16, 8, "bf16")
    c["pos"][:] = 0
    _run(c)


def test_bad_slot_skips_kv_and_raises_fault():
    c = _case("badslot", 6, 16, 8, "bf16")
    kp_h, vp_h = _pool(c)
    kp, vp = to_dev(kp_h, "bf16"), to_dev(vp_h, "bf16")
    loc = c["loc"].copy()
    loc[2] = c["num_slots"] + 5
    print("qk-rope case bad slot", flush=True)
    qo = pkv.qk_norm_rope_store_kv(kp, vp, to_dev(loc), to_dev(c["q"], "bf16"), to_dev(c["k"], "bf16"),
                                   to_dev(c["v"], "bf16"), to_dev(c["pos"]), to_dev(c["wq"], "bf16"),
                                   to_dev(c["wk"], "bf16"), eps=EPS, rope_theta=THETA)
    torch.cuda.synchronize()
    assert pkv.read_faults() & 0x1
    w = lambda x: oracle.widen(x, "bf16")
    rq, rk = oracle.qk_norm_rope(w(c["q"]), w(c["k"]), c["pos"], w(c["wq"]), w(c["wk"]), EPS, THETA)
    _check(to_host(qo), rq, "bf16", "q_out (all tokens)")
    good = np.array([i for i in range(6) if i != 2])
    _check(to_host(kp)[loc[good]], rk[good], "bf16", "K rows of the valid tokens")
    written = set(loc[good].tolist())
    rest = np.array([s for s in range(c["num_slots"]) if s not in written])
    assert np.array_equal(_bits(to_host(kp)[rest]), _bits(kp_h[rest]))


def test_prefill_token_count_every_token():
    """The 8-request prefill's token count (19,892 new tokens, 16 query and 8
    KV heads, positions cached_len + t), in the launch configuration the
    benchmark times; every token's q_out and K row is checked against the
    oracle, all V rows bit-exact."""
    from workloads import config, draw_lengths
    C, S = draw_lengths(config(4))
    pos = np.concatenate([np.arange(c, s) for c, s in zip(C, S)]).astype(np.int32)
    n = len(pos)
    rng = _rng("prefill")
    num_slots = n + 1000
    loc = rng.permutation(num_slots)[:n].astype(np.int32)
    gen = torch.Generator(device="cuda").manual_seed(44)
    q = torch.randn((n, 16, 128), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((n, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((n, 8, 128), generator=gen, device="cuda").to(torch.bfloat16)
    wq = (torch.rand(128, generator=gen, device="cuda") + 0.5).to(torch.bfloat16)
    wk = (torch.rand(128, generator=gen, device="cuda") + 0.5).to(torch.bfloat16)
    kp = torch.zeros((num_slots, 8, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    print(f"qk-rope prefill case n={n}", flush=True)
    qo = pkv.qk_norm_rope_store_kv(kp, vp, to_dev(loc), q, k, v, to_dev(pos), wq, wk, eps=EPS, rope_theta=THETA)
    torch.cuda.synchronize()
    assert pkv.read_faults() == 0
    w = lambda x: oracle.widen(x, "bf16")
    qh, kh, vh = to_host(q), to_host(k), to_host(v)
    rq, rk = oracle.qk_norm_rope(w(qh), w(kh), pos, w(to_host(wq)), w(to_host(wk)), EPS, THETA)
    _check(to_host(qo), rq, "bf16", "prefill q_out, every token")
    _check(to_host(kp)[loc], rk, "bf16", "prefill K rows, every token")
    assert np.array_equal(_bits(to_host(vp)[loc]), _bits(vh)), "prefill V rows differ"


# ---------------------------------------------------------------- q's norm + RoPE in the attention prologue
# ("第 0 步" layer function: q_norm and rope right before attention; "Mini-SGLang
# 完整剖析" section 4.6.7). The k side goes through the store call with q =
# None; the attention call normalises and rotates the raw q itself. Checked
# through oracle.qk_norm_rope followed by oracle attention over the pool rows
# the kernels wrote, and against the unfused chain (q_out through the store
# call, then plain attention).

def _paged(rng, lens, hkv, dtype, extra=50):
    """Pool with random rows everywhere, one table row per request."""
    S = np.asarray(lens, np.int32)
    n_slots = int(S.sum()) + extra
    perm = rng.permutation(n_slots)
    width = (int(S.max()) + 31) // 32 * 32
    table = np.full((len(S), width), n_slots - 1, np.int32)
    off = 0
    for r, s in enumerate(S):
        table[r, :s] = perm[off:off + s]
        off += s
    kv = rng.standard_normal((2, n_slots, hkv, 128), dtype=np.float32)
    if dtype == "bf16":
        kv = f32_to_bf16_bits(kv)
    return table, kv


def _attn_ref(q64, kp_h, vp_h, table, C, S, dtype):
    """fp64 attention of the rotated queries q64 (ragged, request order) over
    the pool rows as the kernels left them."""
    from oracle.attention import attention_request
    out, off = [], 0
    for r in range(len(S)):
        e = int(S[r] - C[r])
        rows = table[r, :S[r]]
        out.append(attention_request(q64[off:off + e], oracle.widen(kp_h[rows], dtype),
                                     oracle.widen(vp_h[rows], dtype), int(C[r])))
        off += e
    return np.concatenate(out)


@pytest.mark.parametrize("dtype,hkv,g", [("bf16", 8, 2), ("f32", 8, 2), ("bf16", 4, 4), ("f32", 4, 1)])
def test_decode_with_q_prologue(dtype, hkv, g):
    from gpu_util import check_attention
    rng = _rng(f"dec-qnr-{dtype}-{hkv}-{g}")
    hq = hkv * g
    S = rng.integers(1, 3000, 9).astype(np.int32)
    S[0] = 1
    C = S - 1
    table, kv = _paged(rng, S, hkv, dtype)
    as_dt = (lambda x: f32_to_bf16_bits(x)) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    q = as_dt(rng.standard_normal((len(S), hq, 128), dtype=np.float32) * 1.7)
    k = as_dt(rng.standard_normal((len(S), hkv, 128), dtype=np.float32) * 2.0)
    v = as_dt(rng.standard_normal((len(S), hkv, 128), dtype=np.float32))
    wq = as_dt(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    wk = as_dt(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    pos = (S - 1).astype(np.int32)
    loc = table[np.arange(len(S)), S - 1].astype(np.int32)
    d = lambda x: to_dev(x, dtype)
    outs = {}
    for mode in ("fused", "unfused"):
        kp, vp = d(kv[0]), d(kv[1])
        print(f"decode q-prologue case {dtype} hkv={hkv} g={g} {mode}", flush=True)
        if mode == "fused":
            pkv.qk_norm_rope_store_kv(kp, vp, to_dev(loc), None, d(k), d(v), to_dev(pos), None, d(wk),
                                      eps=EPS, rope_theta=THETA)
            o = pkv.paged_attention_decode(d(q), kp, vp, to_dev(table), to_dev(C), to_dev(S),
                                           max_total_kv=int(S.sum()), q_norm_weight=d(wq), eps=EPS,
                                           rope_theta=THETA)
        else:
            qo = pkv.qk_norm_rope_store_kv(kp, vp, to_dev(loc), d(q), d(k), d(v), to_dev(pos), d(wq), d(wk),
                                           eps=EPS, rope_theta=THETA)
            o = pkv.paged_attention_decode(qo, kp, vp, to_dev(table), to_dev(C), to_dev(S),
                                           max_total_kv=int(S.sum()))
        torch.cuda.synchronize()
        outs[mode] = (to_host(o), to_host(kp), to_host(vp))
    assert pkv.read_faults() == 0
    # the k side is the same call in both modes: identical pools
    assert np.array_equal(_bits(outs["fused"][1]), _bits(outs["unfused"][1]))
    w = lambda x: oracle.widen(x, dtype)
    rq, _ = oracle.qk_norm_rope(w(q), w(k), pos, w(wq), w(wk), EPS, THETA)
    ref = _attn_ref(rq, outs["fused"][1], outs["fused"][2], table, C, S, dtype)
    mx, rel = check_attention(outs["fused"][0], ref, dtype, f"decode with q prologue ({dtype})")
    print(f"  fused vs oracle: max|d|={mx:.3e} relL2={rel:.3e}", flush=True)
    check_attention(outs["unfused"][0], ref, dtype, f"unfused chain ({dtype})")


@pytest.mark.parametrize("hkv,g", [(8, 2), (4, 1)])
def test_extend_with_q_prologue(hkv, g):
    """Three requests over cached prefixes (several 128-row query blocks,
    ragged tails), bf16: the k side of the new tokens stored by the fused
    store call, then extend with the q prologue at positions C + t."""
    from gpu_util import check_attention
    rng = _rng(f"ext-qnr-{hkv}-{g}")
    hq = hkv * g
    C = np.array([5, 0, 300], np.int32)
    E = np.array([40, 257, 130], np.int32)
    S = C + E
    table, kv = _paged(rng, S, hkv, "bf16")
    n = int(E.sum())
    q = f32_to_bf16_bits(rng.standard_normal((n, hq, 128), dtype=np.float32) * 1.7)
    k = f32_to_bf16_bits(rng.standard_normal((n, hkv, 128), dtype=np.float32) * 2.0)
    v = f32_to_bf16_bits(rng.standard_normal((n, hkv, 128), dtype=np.float32))
    wq = f32_to_bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    wk = f32_to_bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    pos = np.concatenate([np.arange(c, s) for c, s in zip(C, S)]).astype(np.int32)
    loc = np.concatenate([table[r, C[r]:S[r]] for r in range(len(S))]).astype(np.int32)
    d = lambda x: to_dev(x, "bf16")
    outs = {}
    for mode in ("fused", "unfused"):
        kp, vp = d(kv[0]), d(kv[1])
        print(f"extend q-prologue case hkv={hkv} g={g} {mode}", flush=True)
        if mode == "fused":
            pkv.qk_norm_rope_store_kv(kp, vp, to_dev(loc), None, d(k), d(v), to_dev(pos), None, d(wk),
                                      eps=EPS, rope_theta=THETA)
            o = pkv.paged_attention_extend(d(q), kp, vp, to_dev(table), to_dev(C), to_dev(S),
                                           max_extend=int(E.max()), q_norm_weight=d(wq), eps=EPS, rope_theta=THETA)
        else:
            qo = pkv.qk_norm_rope_store_kv(kp, vp, to_dev(loc), d(q), d(k), d(v), to_dev(pos), d(wq), d(wk),
                                           eps=EPS, rope_theta=THETA)
            o = pkv.paged_attention_extend(qo, kp, vp, to_dev(table), to_dev(C), to_dev(S),
                                           max_extend=int(E.max()))
        torch.cuda.synchronize()
        outs[mode] = (to_host(o), to_host(kp), to_host(vp))
    assert pkv.read_faults() == 0
    assert np.array_equal(_bits(outs["fused"][1]), _bits(outs["unfused"][1]))
    w = lambda x: oracle.widen(x, "bf16")
    rq, _ = oracle.qk_norm_rope(w(q), w(k), pos, w(wq), w(wk), EPS, THETA)
    ref = _attn_ref(rq, outs["fused"][1], outs["fused"][2], table, C, S, "bf16")
    mx, rel = check_attention(outs["fused"][0], ref, "bf16", "extend with q prologue")
    print(f"  fused vs oracle: max|d|={mx:.3e} relL2={rel:.3e}", flush=True)
    check_attention(outs["unfused"][0], ref, "bf16", "unfused extend chain")
