"""GPU parity of pkv_sample against the oracle: sampled token ids must be
bit-exact on every row the oracle does not flag (argmax rows always), given
the same uniforms. Flagged rows (a top-p cut or draw boundary within the oracle's margin
of the decision) are counted and reported."""

import zlib

import numpy as np
import pytest

import oracle
from workloads import (config, draw_logits, draw_sampling_params, draw_uniforms, f32_to_bf16_bits)
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
pkv = pytest.importorskip("paged_kv_attention_scatter_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


FLAG_COUNTS = []  # (case, rows, flagged) of every comparison, printed as the tests run


def _check(got, lf, T, K, P, u, what, max_flag_frac, MP=None):
    """got: kernel tokens; lf: the logits as the kernel saw them, widened to
    fp64. Unflagged rows must equal the oracle's token; a flagged row's token
    must be one the oracle can return with its rounding-sensitive thresholds
    moved within the margin (oracle.admissible); at most max_flag_frac of the
    rows may be flagged."""
    want, flagged = oracle.sample(lf, T, K, P, u, min_p=MP)
    assert np.all((got >= 0) & (got < lf.shape[1])), f"{what}: token out of range"
    bad = np.nonzero((got != want) & ~flagged)[0]
    assert bad.size == 0, f"{what}: rows {bad[:10].tolist()} got {got[bad[:10]].tolist()} " \
                          f"want {want[bad[:10]].tolist()}"
    fr = np.nonzero(flagged)[0]
    adm = oracle.admissible(lf, T, K, P, u, fr.tolist(), min_p=MP)
    off = [int(r) for r in fr if int(got[r]) not in adm[int(r)]]
    assert not off, f"{what}: flagged rows {off[:10]} got tokens outside their admissible sets " \
                    f"{[(int(got[r]), sorted(adm[r])[:6]) for r in off[:5]]}"
    FLAG_COUNTS.append((what, len(got), int(flagged.sum())))
    print(f"  {what}: {len(got)} rows, {int(flagged.sum())} flagged (admissible), rest exact", flush=True)
    assert flagged.mean() <= max_flag_frac, f"{what}: {flagged.sum()} of {len(got)} rows flagged"
    return want, flagged


def _run(logits, dtype, T, K, P, u, what, max_flag_frac=0.05, MP=None):
    """logits: numpy in kernel dtype ([bs, V]); T/K/P/MP: prepared arrays or None."""
    print(f"sample case {what} shape={logits.shape} dtype={dtype}", flush=True)
    d = lambda x: None if x is None else to_dev(x)
    tok = pkv.sample(to_dev(logits, dtype), d(T), d(K), d(P), d(u), min_p=d(MP))
    torch.cuda.synchronize()
    got = to_host(tok)
    want, flagged = _check(got, oracle.widen(logits, dtype), T, K, P, u, what, max_flag_frac, MP)
    return got, want, flagged


def _prepared(rows, vocab):
    T, K, P = zip(*rows)
    return pkv.prepare_sampling(T, K, P, vocab)


@pytest.mark.parametrize("cid,literal", [(1, False), (1, True), (2, False), (3, False), (5, False)])
def test_sample_configs(cid, literal):
    cfg = config(cid)
    logits = draw_logits(cfg)
    T, K, P = _prepared(draw_sampling_params(cfg, literal), cfg.vocab)
    u = draw_uniforms(cfg)
    if cid == 2:
        assert T is None                       # all greedy -> argmax path
    _run(logits, cfg.dtype, T, K, P, u, f"{cfg.name}{'-literal' if literal else ''}")


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def _rng(name):
    return np.random.default_rng(zlib.crc32(name.encode()))


def test_argmax_ties_lowest_index():
    V = 151936
    rng = _rng("ties")
    x = rng.standard_normal((6, V)).astype(np.float32)
    for r, pos in enumerate([[5, 100, 151935], [0, 1], [151934, 151935], [77], [3000, 9000], [1, 2, 3]]):
        x[r, pos] = 9.0
    x[5, :] = 0.0                              # one row all equal (+0) ...
    x[5, 10:20] = -0.0                         # ... with some -0: still equal
    got, _, _ = _run(_bf16(x), "bf16", None, None, None, np.zeros(6, np.float32), "argmax-ties")
    assert got.tolist() == [5, 0, 151934, 77, 3000, 0]


def test_topk_ties_at_threshold():
    """Equal logits straddling the k-th rank: the lower indices are kept."""
    V, bs = 4096, 64
    rng = _rng("topk-ties")
    x = np.round(rng.standard_normal((bs, V)) * 2, 0).astype(np.float32)   # few distinct values
    T = np.full(bs, 1.0, np.float32)
    K = rng.integers(1, 300, bs).astype(np.int32)
    u = rng.random(bs, dtype=np.float32)
    _run(_bf16(x), "bf16", T, K, None, u, "topk-ties")
    _run(x, "f32", T, K, None, u, "topk-ties-f32")


def test_topp_ties_at_cut():
    V, bs = 2048, 64
    rng = _rng("topp-ties")
    x = np.round(rng.standard_normal((bs, V)) * 1.5, 0).astype(np.float32)
    T = np.full(bs, 0.8, np.float32)
    P = rng.uniform(0.05, 0.99, bs).astype(np.float32)
    u = rng.random(bs, dtype=np.float32)
    _run(_bf16(x), "bf16", T, None, P, u, "topp-ties")
    K = rng.integers(1, 50, bs).astype(np.int32)
    _run(_bf16(x), "bf16", T, K, P, u, "topk-topp-ties")


# The last field bounds the share of flagged rows (the oracle's counts on
# these seeded rows, bf16 / fp32: plain 10/10, flat-topp 1/2, deep-p 8/10,
# big-k 2/2, k9000 8/6, k3000-p999 15/16, p-only 5/6 of 32, the rest 0; flat
# distributions over many tokens put draw boundaries within the margin).
@pytest.mark.parametrize("name,V,T,k,p,maxf", [
    ("plain", 151936, 1.0, -1, 1.0, 0.4),          # no filter: full softmax sampling
    ("flat-topp", 1024, 50.0, -1, 0.5, 0.13),      # cut far below the 256-key window -> radix path
    ("deep-p", 1024, 1.5, -1, 0.98, 0.4),          # cut deep in the tail -> radix path
    ("big-k", 1024, 0.7, 600, 1.0, 0.13),          # top-k threshold below the window -> radix select
    ("big-k-p", 1024, 2.0, 500, 0.97, 0.07),
    ("k1", 151936, 0.9, 1, 0.3, 0.0),
    ("tiny-T", 151936, 2e-6, 20, 0.9, 0.0),
    ("k50-p95", 151936, 1.0, 50, 0.95, 0.07),
    ("k9000", 151936, 1.0, 9000, 1.0, 0.32),       # more candidates than the LDS list holds -> generic path
    ("k3000-p999", 151936, 1.0, 3000, 0.999, 0.57),
    ("p-only", 151936, 0.7, -1, 0.9, 0.25),        # top-p over the whole row's mass
])
def test_sample_paths(name, V, T, k, p, maxf):
    """Every path of the kernel. On the full vocabulary a flat distribution
    gives each token less mass than the oracle's margin, so the paths that
    only flat distributions reach are exercised on 1024 tokens."""
    bs = 32
    rng = _rng(name)
    x = (rng.standard_normal((bs, V)) * 3).astype(np.float32)
    Ta = np.full(bs, T, np.float32)
    Ka = None if k < 0 else np.full(bs, k, np.int32)
    Pa = None if p >= 1.0 else np.full(bs, p, np.float32)
    u = rng.random(bs, dtype=np.float32)
    u[0], u[1] = 0.0, np.float32(0.99999994)
    _run(_bf16(x), "bf16", Ta, Ka, Pa, u, name, max_flag_frac=maxf)
    # fp32 rows: candidate lists of at most 1024 tokens per slice; big-k, the
    # flat and deep top-p cases and k9000 cut below them (the row in memory)
    _run(x, "f32", Ta, Ka, Pa, u, name + "-f32", max_flag_frac=maxf)


def test_sample_fp32_large_vocab_and_odd_sizes():
    """fp32 rows too long for registers (re-read path); vocab not a multiple
    of the 16-byte chunk; row stride larger than the vocabulary."""
    rng = _rng("odd")
    for V, pad, dtype in ((151936, 0, "f32"), (1000, 0, "bf16"), (50257, 7, "bf16"), (777, 5, "f32")):
        bs = 12
        full = (rng.standard_normal((bs, V + pad)) * 2.5).astype(np.float32)
        if dtype == "bf16":
            pad2 = (-(V + pad)) % 8
            full = np.pad(full, ((0, 0), (0, pad2)))
            x = _bf16(full)
        else:
            pad2 = (-(V + pad)) % 4
            full = np.pad(full, ((0, 0), (0, pad2)))
            x = full
        T = rng.choice([1e-7, 0.5, 1.0, 1.7], bs).astype(np.float32)
        K = rng.choice([0, 1, 5, 40, V + 3], bs).astype(np.int32)
        P = rng.choice([1.0, 0.2, 0.9, 0.999], bs).astype(np.float32)
        u = rng.random(bs, dtype=np.float32)
        dev = to_dev(x, dtype)[:, :V]
        print(f"sample case odd-V{V}-{dtype}", flush=True)
        tok = pkv.sample(dev, to_dev(T), to_dev(K), to_dev(P), to_dev(u))
        torch.cuda.synchronize()
        _check(to_host(tok), oracle.widen(x, dtype)[:, :V], T, K, P, u, f"odd-V{V}-{dtype}", 0.25)


def test_mixed_batch_greedy_rows_exact():
    """Half the rows greedy (T = 1e-6 after the argument builder), half
    sampled: greedy rows are exact argmax whatever the uniforms."""
    cfg = config(3)
    logits = draw_logits(cfg)[:64]
    rows = draw_sampling_params(cfg)[:64]
    T, K, P = _prepared(rows, cfg.vocab)
    greedy = T <= np.float32(1e-6)
    assert greedy.any() and (~greedy).any()
    for u_val in (0.0, 0.5, 0.9999):
        u = np.full(64, u_val, np.float32)
        got, _, _ = _run(logits, "bf16", T, K, P, u, f"mixed-u{u_val}")
        lf = oracle.widen(logits, "bf16")
        assert np.array_equal(got[greedy], np.argmax(lf[greedy], axis=1))


@pytest.mark.parametrize("V", [4097, 32768, 32769, 163840, 163841])
def test_vocab_boundaries_and_masked_tokens(V):
    """Vocabularies at and just past the kernels' register-round limits (odd
    sizes leave half a word past the row); maxima in the last token; rows
    where every third token is masked to -inf."""
    rng = _rng(f"edge{V}")
    bs = 8
    x = (rng.standard_normal((bs, V)) * 3).astype(np.float32)
    x[0, -1] = 50.0
    x[1, -2:] = 50.0
    x[2:5, ::3] = -np.inf
    x[6, :V // 2] = -np.inf                             # whole slices masked
    T = np.array([0.0, 0.0, 0.8, 1.0, 0.5, 0.9, 0.9, 1.2], np.float32)
    K = np.array([0, 0, 0, 40, 5, 30, 0, 0], np.int32)
    P = np.array([1.0, 1.0, 0.9, 1.0, 0.5, 0.9, 0.95, 1.0], np.float32)
    u = rng.random(bs, dtype=np.float32)
    xb = _bf16(np.pad(x, ((0, 0), (0, (-V) % 8))))     # rows padded to 16 bytes, the kernel sees V tokens
    print(f"sample case edge-V{V}", flush=True)
    tok = pkv.sample(to_dev(xb, "bf16")[:, :V], to_dev(T), to_dev(K), to_dev(P), to_dev(u))
    torch.cuda.synchronize()
    got = to_host(tok)
    _check(got, oracle.widen(xb, "bf16")[:, :V], T, K, P, u, f"edge-V{V}", 0.25)
    assert got[0] == V - 1 and got[1] == V - 2
    xf = np.pad(x, ((0, 0), (0, (-V) % 4)))             # fp32 rows padded to 16 bytes
    print(f"sample case edge-V{V} fp32", flush=True)
    tok = pkv.sample(to_dev(xf)[:, :V], to_dev(T), to_dev(K), to_dev(P), to_dev(u))
    torch.cuda.synchronize()
    got = to_host(tok)
    _check(got, xf[:, :V].astype(np.float64), T, K, P, u, f"edge-V{V}-f32", 0.25)
    assert got[0] == V - 1 and got[1] == V - 2


def test_cut_deep_in_the_window():
    """A few dozen large logits spread over two binades above a low floor:
    top-k and top-p cuts land anywhere in the 256-key window of the row
    maximum, with margins far above the oracle's."""
    V, bs = 151936, 24
    rng = _rng("two-level")
    x = rng.standard_normal((bs, V)).astype(np.float32)
    for r in range(bs):
        idx = rng.choice(V, 40, replace=False)
        x[r, idx] = rng.uniform(3.0, 16.0, 40)
    T = rng.choice([1.0, 1.5, 2.5], bs).astype(np.float32)
    K = rng.choice([0, 7, 25, 39], bs).astype(np.int32)
    P = rng.choice([1.0, 0.5, 0.9, 0.97], bs).astype(np.float32)
    u = rng.random(bs, dtype=np.float32)
    _run(_bf16(x), "bf16", T, K, P, u, "two-level", max_flag_frac=0.25)


def test_workspace_reused_across_calls():
    """One workspace serves many calls of different batch sizes and
    parameter mixes (no state is carried from one call to the next)."""
    V = 151936
    ws = torch.full((pkv.sample_workspace_size(64, V),), 0xA5, dtype=torch.uint8, device="cuda")
    rng = _rng("reuse")
    for it, bs in enumerate((64, 17, 64, 1, 30)):
        x = (rng.standard_normal((bs, V)) * 3).astype(np.float32)
        T = rng.choice([0.0, 0.7, 1.0], bs).astype(np.float32)
        K = rng.choice([0, 50], bs).astype(np.int32)
        P = rng.choice([1.0, 0.9, 0.95], bs).astype(np.float32)
        u = rng.random(bs, dtype=np.float32)
        xb = _bf16(x)
        print(f"sample case reuse-{it} bs={bs}", flush=True)
        tok = pkv.sample(to_dev(xb, "bf16"), to_dev(T), to_dev(K), to_dev(P), to_dev(u), workspace=ws)
        torch.cuda.synchronize()
        _check(to_host(tok), oracle.widen(xb, "bf16"), T, K, P, u, f"reuse-{it}", 0.3)   # plain rows: 11 of 64 in the first call


def test_largest_bf16_vocabulary():
    """The bf16 limit (2^20 tokens: 128 slices per row), with
    top-p, top-k + top-p and plain rows; one token past it is refused."""
    V, bs = 1 << 20, 3
    rng = _rng("max-vocab")
    x = (rng.standard_normal((bs, V)) * 3).astype(np.float32)
    T = np.array([0.7, 1.0, 1.0], np.float32)
    K = np.array([0, 50, 0], np.int32)
    P = np.array([0.9, 0.95, 1.0], np.float32)
    u = rng.random(bs, dtype=np.float32)
    _run(_bf16(x), "bf16", T, K, P, u, "max-vocab", max_flag_frac=0.67)   # 2 of 3: flat rows over 2^20 tokens
    with pytest.raises(pkv.PkvError):
        pkv.sample(torch.zeros((1, V + 8), dtype=torch.bfloat16, device="cuda"),
                   to_dev(T[:1]), None, None, to_dev(u[:1]))


# ---------------------------------------------------------------- min_p
# ("Engine 与采样器", section 练习 and its answer: keep a token iff its
# probability is at least min_p times the largest, on the full tempered
# distribution; intersected with the top-k / top-p set)


# Flag bounds from the oracle's counts on these rows (bf16 / fp32 of 32):
# mp-only 0/1, mp-p 2/7, mp-1 1/0, mp-deep-p 4/6, the rest 0.
@pytest.mark.parametrize("name,V,T,k,p,mp,maxf", [
    ("mp-only", 151936, 1.0, -1, 1.0, 0.1, 0.1),        # cut inside the 256-key window
    ("mp-k50", 151936, 1.0, 50, 1.0, 0.05, 0.07),
    ("mp-p", 151936, 0.7, -1, 0.9, 0.2, 0.29),          # top-p over the whole row's mass, then min_p
    ("mp-k50-p95", 151936, 1.0, 50, 0.95, 0.1, 0.07),
    ("mp-loose-k", 151936, 1.0, 5, 1.0, 1e-4, 0.07),    # top-k is the tighter cut
    ("mp-1", 151936, 1.0, -1, 1.0, 1.0, 0.1),           # only the largest key survives
    ("mp-above-1", 151936, 0.8, 40, 0.9, 3.0, 0.07),    # acts as 1
    ("mp-deep", 1024, 1.5, -1, 1.0, 0.003, 0.07),       # cut below the window -> generic path
    ("mp-deep-bigk", 1024, 0.7, 600, 1.0, 0.01, 0.07),  # top-k below the window, min_p inside -> generic path
    ("mp-deep-p", 1024, 2.0, -1, 0.97, 0.004, 0.25),
])
def test_min_p_paths(name, V, T, k, p, mp, maxf):
    bs = 32
    rng = _rng(name)
    x = (rng.standard_normal((bs, V)) * 3).astype(np.float32)
    Ta = np.full(bs, T, np.float32)
    Ka = None if k < 0 else np.full(bs, k, np.int32)
    Pa = None if p >= 1.0 else np.full(bs, p, np.float32)
    MP = np.full(bs, mp, np.float32)
    MP[2] = 0.0                                   # rows without min_p in the same batch
    MP[3] = -1.0
    u = rng.random(bs, dtype=np.float32)
    u[0], u[1] = 0.0, np.float32(0.99999994)
    got, _, _ = _run(_bf16(x), "bf16", Ta, Ka, Pa, u, name, max_flag_frac=maxf, MP=MP)
    _run(x, "f32", Ta, Ka, Pa, u, name + "-f32", max_flag_frac=maxf, MP=MP)
    if mp >= 1.0:  # only the maximum's key group survives: on rows with one maximum, the argmax
        xb = oracle.widen(_bf16(x), "bf16")
        rows = (MP > 0) & ((xb == xb.max(axis=1, keepdims=True)).sum(axis=1) == 1)
        assert rows.sum() >= bs // 2
        assert np.array_equal(got[rows], np.argmax(xb, axis=1)[rows])


def test_min_p_closed_form():
    """Three tokens above a low floor at logits 0, -1, -2 (exact in bf16),
    T = 1: their probabilities over the largest are 1, e^-1, e^-2; the
    floor's e^-20 is below every min_p used and its total mass (4093 e^-20,
    under 1e-5) moves no boundary. The kept set and the drawn
    token follow by hand: min_p 0.2 keeps {10, 500} (W = 1 + e^-1),
    min_p 0.1 keeps {10, 500, 700}; top-k 2 or top-p 0.5 cut it further."""
    V = 4096
    base = np.full(V, -20.0, np.float32)
    base[[10, 500, 700]] = [0.0, -1.0, -2.0]
    e1, e2 = np.exp(-1.0), np.exp(-2.0)
    cases = [  # (min_p, top_k, top_p, u, token)
        (0.2, 0, 1.0, 0.5, 10), (0.2, 0, 1.0, 0.9, 500), (0.2, 0, 1.0, 1 / (1 + e1) + 1e-3, 500),
        (0.2, 0, 1.0, 1 / (1 + e1) - 1e-3, 10),
        (0.1, 0, 1.0, 0.9, 500), (0.1, 0, 1.0, 0.95, 700), (0.1, 0, 1.0, (1 + e1) / (1 + e1 + e2) + 1e-3, 700),
        (0.1, 2, 1.0, 0.95, 500), (0.1, 0, 0.5, 0.95, 10), (0.5, 0, 1.0, 0.99, 10), (0.3, 3, 0.9, 0.99, 500),
    ]
    bs = len(cases)
    x = np.tile(base, (bs, 1))
    MP = np.array([c[0] for c in cases], np.float32)
    K = np.array([c[1] for c in cases], np.int32)
    P = np.array([c[2] for c in cases], np.float32)
    u = np.array([c[3] for c in cases], np.float32)
    T = np.ones(bs, np.float32)
    want = [c[4] for c in cases]
    for dt, xx in (("bf16", _bf16(x)), ("f32", x)):
        got, _, flagged = _run(xx, dt, T, K, P, u, f"min_p-closed-form-{dt}", max_flag_frac=0.0, MP=MP)
        assert got.tolist() == want


def test_fp32_candidate_lists_and_fallback_mix():
    """fp32 rows of one batch, each with its own cut: some inside the slices'
    candidate lists, some below them (top-k beyond the lists, a nucleus
    larger than the lists, min_p alone with every listed token above it),
    plain and greedy rows, on a vocabulary with a ragged last slice."""
    V, bs = 50000, 40
    rng = _rng("f32-mix")
    x = (rng.standard_normal((bs, V)) * rng.choice([1.0, 3.0, 6.0], (bs, 1))).astype(np.float32)
    x[5, 100:400] = 2.5                               # many equal logits at a top-k threshold
    x[6, :] = np.round(x[6, :])                       # few distinct values: large tie groups
    T = rng.choice([0.0, 0.6, 1.0, 2.0, 8.0], bs).astype(np.float32)
    K = rng.choice([0, 1, 20, 300, 2000], bs).astype(np.int32)
    P = rng.choice([1.0, 0.5, 0.9, 0.99], bs).astype(np.float32)
    MP = rng.choice([0.0, 0.0, 0.001, 0.1], bs).astype(np.float32)
    u = rng.random(bs, dtype=np.float32)
    _run(x, "f32", T, K, P, u, "f32-mix", max_flag_frac=0.18, MP=MP)   # 5 of 40


def test_largest_fp32_vocabulary():
    """fp32 rows at the 2^20-token limit: 128 slices, so the finish kernel's
    two slices per lane and the lists' binary search reach their last slice;
    top-k, top-k + top-p, min_p, top-p alone and plain rows."""
    V, bs = 1 << 20, 5
    rng = _rng("max-vocab-f32")
    x = (rng.standard_normal((bs, V)) * 3).astype(np.float32)
    x[1, V - 3] = 40.0                                # the maximum in the last slice
    T = np.array([0.7, 1.0, 1.0, 0.8, 1.0], np.float32)
    K = np.array([50, 30, 0, 0, 0], np.int32)
    P = np.array([1.0, 0.95, 1.0, 0.9, 1.0], np.float32)
    MP = np.array([0.0, 0.0, 0.05, 0.0, 0.0], np.float32)
    u = rng.random(bs, dtype=np.float32)
    got, _, _ = _run(x, "f32", T, K, P, u, "max-vocab-f32", max_flag_frac=0.4, MP=MP)   # 2 of 5
    assert got[1] == V - 3                            # e^(40 - ~15) dwarfs the rest


@pytest.mark.parametrize("T", [0.05, 1e-3])
def test_low_temperature_large_logits(T):
    """Rows whose largest logits sit around 30-40 at T = 0.05 and 1e-3, where
    l * log2(e) / T is in the thousands: every weight must be taken relative
    to a maximum without an extra rounding of the reference (each token's
    weight is exp2((l - l_max) log2(e) / T)). Plain rows get a uniform placed
    2.5 margins past a running-mass boundary of the oracle's draw, so an
    error of a few 1e-5 in any slice's or thread's mass moves their token;
    top-p rows (p = 0.93, off the tie groups' exact fractions) draw at random
    uniforms. bf16 and fp32 rows."""
    V, bs = 151936, 64
    rng = _rng(f"lowT{T}")
    x = (rng.standard_normal((bs, V)) * 3).astype(np.float32)
    for r in range(bs):
        idx = rng.choice(V, 40, replace=False)
        x[r, idx] = rng.uniform(30.0, 40.0, 40) if r % 2 else 35.0 + rng.uniform(-8, 1, 40) * T
    Ta = np.full(bs, T, np.float32)
    P = np.where(np.arange(bs) < bs // 2, 1.0, 0.93).astype(np.float32)
    for dt, xx in (("bf16", _bf16(x)), ("f32", x)):
        lf = oracle.widen(xx, dt)
        u = rng.random(bs, dtype=np.float32)
        for r in range(bs // 2):  # plain rows: a uniform just past a boundary of a token with mass
            w = np.exp((lf[r] - lf[r].max()) / np.float64(Ta[r]))
            c = np.cumsum(w) / w.sum()
            big = np.nonzero(w / w.sum() > 1e-3)[0]
            if len(big) > 1:
                j = big[rng.integers(0, len(big) - 1)]
                u[r] = np.float32(min(c[j] + 2.5 * oracle.DELTA, 0.999))
        _run(xx, dt, Ta, None, P, u, f"lowT{T}-{dt}", max_flag_frac=0.1)
