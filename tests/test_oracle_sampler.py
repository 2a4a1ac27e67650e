"""Oracle pins for the sampler: the pages' closed forms, a brute-force
interval computation on tiny vocabularies, invariants, ties and margin flags."""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from conftest import GOLDEN

GRID = (np.arange(10000, dtype=np.float64) + 0.5) / 10000


def _golden():
    with open(os.path.join(GOLDEN, "sampler_pins.json")) as f:
        return json.load(f)


def _draw_all(logits, T, k, p, us=GRID):
    return np.array([oracle.sample_row(np.asarray(logits, float), T, k, p, float(np.float32(u)))[0]
                     for u in us])


def test_topk2_closed_form():
    g = _golden()["topk2"]
    p0 = math.exp(5) / (math.exp(5) + math.exp(4))
    assert abs(p0 - g["p_token0"]) < 1e-15 and round(p0, 3) == g["printed"]
    toks = _draw_all(g["logits"], g["temperature"], g["top_k"], g["top_p"])
    assert set(toks.tolist()) == set(g["support"])
    # inverse CDF in index order: token 0 iff u < P(0)
    u32 = GRID.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(toks == 0, u32 < p0)
    # the page's empirical check: 2000 seeded draws, frequency within 0.03
    u = np.random.default_rng(0).random(2000, dtype=np.float32)
    freq = np.mean(_draw_all(g["logits"], 1.0, 2, 1.0, u) == 0)
    assert abs(freq - g["printed"]) < 0.03


def test_topp05_keeps_only_top_token():
    g = _golden()["topp05"]
    probs = softmax(np.array(g["logits"]))
    assert probs[0] > g["top_p"]                               # 0.6564 > 0.5
    assert set(_draw_all(g["logits"], 1.0, -1, g["top_p"]).tolist()) == set(g["support"])


def test_greedy_row_in_mixed_batch():
    g = _golden()["greedy_row"]
    logits = np.array([g["logits"]] * 3)
    T = np.float32([1.0, 1.0, 1e-6])
    k = np.int32([2, 6, 6])
    p = np.float32([1.0, 0.5, 1.0])
    u = np.float32([0.999, 0.999, 0.999])
    toks, flags = oracle.sample(logits, T, k, p, u)
    assert toks.tolist() == [1, 0, 0] and not flags.any()


def test_renormalised_topk_example():
    g = _golden()["renorm_topk"]
    logits = np.log(np.array(g["probs"]))
    r0 = g["renormalised"][0]
    assert [round(x, 2) for x in g["renormalised"]] == g["printed"]
    toks = _draw_all(logits, 1.0, g["top_k"], 1.0)
    u32 = GRID.astype(np.float32).astype(np.float64)
    assert set(toks.tolist()) == {0, 1}
    np.testing.assert_array_equal(toks == 0, u32 < r0)


def test_topp_boundary_is_flagged():
    g = _golden()["topp_boundary"]
    logits = np.log(np.array(g["probs"]))
    info = {}
    _, flagged = oracle.sample_row(logits, 1.0, -1, g["top_p"], 0.3, info=info)
    assert flagged and info["top_p_margin"] < oracle.DELTA
    _, flagged = oracle.sample_row(logits, 1.0, -1, 0.95, 0.3)
    assert not flagged


def test_topk_applied_before_topp():
    """probs [0.5, 0.3, 0.2], k=2, p=0.6: top-k first renormalises to
    [0.625, 0.375], so the second token's prior mass 0.625 >= 0.6 and only
    token 0 survives. top-p first would keep tokens 0 and 1 (prior mass 0.5)."""
    g = _golden()["topk_before_topp"]
    logits = np.log(np.array(g["probs"]))
    assert set(_draw_all(logits, 1.0, g["top_k"], g["top_p"]).tolist()) == set(g["support"])


# ---------------------------------------------------------------- brute force

def _brute_intervals(logits, T, k, p):
    """Independent route: ranks by counting, kept sets by explicit loops,
    each token's draw interval [lo, hi) as a fraction of the kept mass."""
    V = len(logits)
    rank = [sum(1 for j in range(V) if logits[j] > logits[i] or (logits[j] == logits[i] and j < i))
            for i in range(V)]
    kk = V if (k <= 0 or k >= V) else k
    kept = [i for i in range(V) if rank[i] < kk]
    zmax = max(logits[i] / T for i in range(V))
    w = {i: math.exp(logits[i] / T - zmax) for i in kept}
    if p < 1.0:
        tot = sum(w.values())
        keep2 = []
        for i in kept:
            before = sum(w[j] for j in kept if rank[j] < rank[i]) / tot
            if before < max(p, 1e-6):
                keep2.append(i)
        kept = keep2
    W = sum(w[i] for i in kept)
    lo, out = 0.0, {}
    for i in range(V):
        if i in kept:
            out[i] = (lo / W, (lo + w[i]) / W)
            lo += w[i]
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny_vocab(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 9))
    logits = np.round(rng.standard_normal(V) * 2, 1)          # rounded: ties are likely
    T = float(np.float32(rng.choice([0.5, 1.0, 1.7])))
    k = int(rng.choice([-1, 1, 2, 3, V]))
    p = float(np.float32(rng.choice([1.0, 0.3, 0.6, 0.9])))
    iv = _brute_intervals(logits.tolist(), T, k, p)
    u32 = GRID.astype(np.float32)
    toks = _draw_all(logits, T, k, p, u32)
    n_checked = 0
    for u, tok in zip(u32.astype(np.float64), toks):
        inside = [i for i, (a, b) in iv.items() if a <= u < b]
        near_edge = any(min(abs(u - a), abs(u - b)) < 1e-9 for a, b in iv.values())
        if near_edge:
            continue
        assert inside == [tok]
        n_checked += 1
    assert n_checked > 9000


# ---------------------------------------------------------------- invariants

def test_no_filter_is_plain_softmax_sampling():
    rng = np.random.default_rng(21)
    V = 7
    logits = rng.standard_normal(V) * 1.5
    probs = softmax(logits / 0.8)
    u = rng.random(100000)
    toks = _draw_all(logits, 0.8, V, 1.0, u)
    counts = np.bincount(toks, minlength=V)
    chi2 = np.sum((counts - probs * len(u)) ** 2 / (probs * len(u)))
    assert chi2 < 30.0                                        # 6 dof; p-value ~ 4e-5


def test_top_k1_is_argmax_and_support_properties():
    rng = np.random.default_rng(22)
    V = 300
    logits = rng.standard_normal(V) * 3
    order = np.lexsort((np.arange(V), -logits))
    for u in rng.random(50):
        assert oracle.sample_row(logits, 0.7, 1, 1.0, u)[0] == order[0]
        tok = oracle.sample_row(logits, 0.7, 20, 1.0, u)[0]
        assert tok in order[:20]
        tok = oracle.sample_row(logits, 0.7, -1, 0.8, u)[0]
        q = softmax(logits / np.float32(0.7))[order]
        before = np.concatenate(([0], np.cumsum(q)[:-1]))
        assert tok in order[before < np.float32(0.8)]


def test_ties_go_to_lowest_indices():
    logits = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 2.0, -1.0])
    assert oracle.sample_row(logits, 1e-6, -1, 1.0, 0.5)[0] == 1      # argmax tie -> lowest index
    toks, _ = oracle.sample(logits[None], None, None, None, np.float32([0.1]))
    assert toks[0] == 1
    # k = 3 keeps both 3.0s and the lowest-index 2.0 (index 2), never 4 or 5
    seen = set(_draw_all(logits, 1.0, 3, 1.0).tolist())
    assert seen == {1, 2, 3}
    # -0.0 and +0.0 are equal logits: the lower index wins
    assert oracle.sample_row(np.array([-0.0, 0.0, -5.0]), 1e-6, -1, 1.0, 0.5)[0] == 0


def test_draw_is_monotone_in_u():
    rng = np.random.default_rng(23)
    logits = rng.standard_normal(50)
    toks = _draw_all(logits, 1.3, 10, 0.9)
    assert np.all(np.diff(toks) >= 0)                          # index-order inverse CDF


def test_sample_batch_all_greedy_path():
    rng = np.random.default_rng(24)
    logits = rng.standard_normal((5, 40))
    toks, flags = oracle.sample(logits, None, None, None, np.zeros(5, np.float32))
    assert np.array_equal(toks, np.argmax(logits, axis=1)) and not flags.any()


def test_topp_keeps_strictly_below_p():
    """Two equal logits give renormalised mass [0.5, 0.5] exactly; with
    top_p = 0.5 the second token's prior mass equals p, and the rule keeps a
    token only if the mass before it is strictly below p. The row sits on the
    boundary, so it is also flagged."""
    logits = np.array([0.0, 0.0, -50.0])
    for u in (0.1, 0.6, 0.99):
        tok, flagged = oracle.sample_row(logits, 1.0, 2, 0.5, u)
        assert tok == 0 and flagged


def test_zero_uniform_lands_on_a_kept_token():
    """u = 0 must give the first *kept* index, never an index whose weight is
    zero (the running mass must strictly exceed u * W)."""
    logits = np.array([0.0, 5.0, 4.0, -1.0])
    assert oracle.sample_row(logits, 1.0, 1, 1.0, 0.0)[0] == 1
    assert oracle.sample_row(logits, 1.0, 2, 1.0, 0.0)[0] == 1


# ---------------------------------------------------------------- min_p ("Engine 与采样器", 练习 2 and its answer)

def _draws_mp(logits, T, k, p, mp, us):
    return np.array([oracle.sample_row(np.asarray(logits, float), T, k, p, float(np.float32(u)), min_p=mp)[0]
                     for u in us])


def test_min_p_closed_form_matches_top_k2():
    """logits [5,4,3,0,0,0] at T = 1: the second token has e^-1 = 0.368 of the
    largest probability and the third e^-2 = 0.135, so min_p = 0.3 keeps exactly
    the first two, like top-k = 2: token 0 iff u < 1 / (1 + e^-1)."""
    us = np.linspace(0.0, 0.999, 2001)
    got = _draws_mp([5, 4, 3, 0, 0, 0], 1.0, -1, 1.0, 0.3, us)
    assert set(got.tolist()) == {0, 1}
    assert np.array_equal(got == 0, us < 1.0 / (1.0 + np.exp(-1.0)))
    assert np.array_equal(got, _draw_all([5, 4, 3, 0, 0, 0], 1.0, 2, 1.0, us))


def test_min_p_zero_is_no_filter_and_one_keeps_the_maximum():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal(50) * 2
    us = rng.random(200)
    assert np.array_equal(_draws_mp(logits, 0.8, -1, 0.9, 0.0, us), _draw_all(logits, 0.8, -1, 0.9, us))
    assert set(_draws_mp(logits, 0.8, -1, 1.0, 1.0, us).tolist()) == {int(np.argmax(logits))}
    tied = np.array([1.0, 3.0, 3.0, 2.0])          # min_p = 1 keeps both tied maxima
    assert set(_draws_mp(tied, 1.0, -1, 1.0, 1.0, np.linspace(0, 0.99, 100)).tolist()) == {1, 2}


def test_min_p_is_relative_to_the_tempered_maximum():
    """The threshold scales with the temperature: ratio e^(-(l0 - l1) / T)."""
    logits = np.array([2.0, 1.0, -10.0])
    us = np.linspace(0, 0.999, 500)
    assert set(_draws_mp(logits, 1.0, -1, 1.0, 0.5, us).tolist()) == {0}          # e^-1 < 0.5
    assert set(_draws_mp(logits, 2.0, -1, 1.0, 0.5, us).tolist()) == {0, 1}       # e^-0.5 >= 0.5


def test_min_p_mask_intersects_top_p_on_the_full_distribution():
    """Probabilities [0.4, 0.35, 0.25], min_p = 0.7 (drops the third: 0.625 <
    0.7), top_p = 0.5. The page's answer intersects masks computed on the full
    distribution: top-p keeps the first two (0.4 before the second is < 0.5),
    so token 1 is drawn with probability 0.35 / 0.75. Renormalising top-p over
    the min_p survivors first would keep token 0 alone."""
    logits = np.log([0.4, 0.35, 0.25])
    us = np.linspace(0.0, 0.999, 4001)
    got = _draws_mp(logits, 1.0, -1, 0.5, 0.7, us)
    assert set(got.tolist()) == {0, 1}
    assert np.array_equal(got == 0, us < 0.4 / 0.75)


def test_min_p_kept_set_is_the_intersection():
    rng = np.random.default_rng(9)
    for trial in range(30):
        logits = rng.standard_normal(300) * 3
        T, k, p, mp = 0.7, int(rng.choice([-1, 5, 40])), float(rng.choice([1.0, 0.9, 0.6])), float(rng.choice([0.01, 0.1, 0.4]))
        i_all, i_kp, i_mp = {}, {}, {}
        oracle.sample_row(logits, T, k, p, 0.5, info=i_all, min_p=mp)
        oracle.sample_row(logits, T, k, p, 0.5, info=i_kp)
        oracle.sample_row(logits, T, -1, 1.0, 0.5, info=i_mp, min_p=mp)
        assert i_all["kept"] == min(i_kp["kept"], i_mp["kept"]), trial


def test_min_p_boundary_is_flagged():
    """A token whose probability ratio sits on min_p is rounding-sensitive: flagged."""
    logits = np.array([0.0, np.log(0.25)])
    _, flagged = oracle.sample_row(logits, 1.0, -1, 1.0, 0.3, min_p=0.25)
    assert flagged
    _, flagged = oracle.sample_row(logits, 1.0, -1, 1.0, 0.3, min_p=0.2)
    assert not flagged


def test_min_p_one_at_the_maximum_is_exact():
    """min_p = 1 (or above, acting as 1) sits exactly on the ratio of every
    token at the maximum logit, which is 1 on any arithmetic: not flagged.
    A token just below the maximum is on the threshold's other side by its
    own (tiny) ratio gap: flagged."""
    for logits in (np.array([0.5, 2.0, -1.0]), np.array([1.0, 3.0, 3.0, 2.0])):
        for mp in (1.0, 3.0):
            _, flagged = oracle.sample_row(logits, 0.8, -1, 1.0, 0.7, min_p=mp)
            assert not flagged
    _, flagged = oracle.sample_row(np.array([3.0, 3.0 - 1e-9]), 1.0, -1, 1.0, 0.2, min_p=1.0)
    assert flagged


# ---------------------------------------------------------------- admissible sets of flagged rows

def test_admissible_of_an_unflagged_row_is_its_token():
    rng = np.random.default_rng(31)
    n_checked = 0
    for _ in range(300):
        V = int(rng.integers(2, 400))
        logits = np.round(rng.standard_normal(V) * rng.choice([0.5, 2.0, 4.0]), 2)
        T = float(np.float32(rng.choice([0.3, 0.7, 1.0, 2.5])))
        k = int(rng.choice([-1, 1, 3, 20, V]))
        p = float(np.float32(rng.choice([1.0, 0.2, 0.5, 0.9, 0.99])))
        mp = float(np.float32(rng.choice([0.0, 0.0, 0.05, 0.3])))
        u = float(rng.random(dtype=np.float32))
        tok, flagged = oracle.sample_row(logits, T, k, p, u, min_p=mp)
        if flagged:
            continue
        assert oracle.admissible_row(logits, T, k, p, u, min_p=mp) == {tok}
        n_checked += 1
    assert n_checked > 250


def test_admissible_at_the_pages_top_p_boundary():
    """[0.66, 0.24, 0.10] with p = 0.9 puts the third token's prior mass on
    the cut ("源码解析（四）" section 14.4's worked example): kept {0, 1} or
    {0, 1, 2}. With u = 0.95 the draw gives token 1 (target 0.855 of 0.9) or
    token 2 (target 0.95 of 1.0); both are admissible, token 0 is not."""
    g = _golden()["topp_boundary"]
    logits = np.log(np.array(g["probs"]))
    tok, flagged = oracle.sample_row(logits, 1.0, -1, g["top_p"], 0.95)
    assert flagged
    assert oracle.admissible_row(logits, 1.0, -1, g["top_p"], 0.95) == {1, 2}


def test_admissible_covers_perturbed_thresholds():
    """Rows built to sit on a top-p, min_p or draw boundary: the token drawn
    with every threshold moved by less than the margin is in the set, and the
    set stays small."""
    rng = np.random.default_rng(32)
    d = oracle.DELTA
    for trial in range(60):
        V = int(rng.integers(3, 60))
        logits = rng.standard_normal(V) * 1.5
        e = np.exp(logits - logits.max())
        order = np.lexsort((np.arange(V), -logits))
        q = e[order] / e.sum()
        kind = trial % 3
        p, mp, u = 1.0, 0.0, float(rng.random())
        if kind == 0:                                   # top-p threshold on a prior mass
            j = int(rng.integers(1, V))
            p = float(np.sum(q[:j]))
        elif kind == 1:                                 # min_p threshold on a ratio
            j = int(rng.integers(1, V))
            mp = float(e[order[j]])
        else:                                           # draw target on a running-mass boundary
            c = np.cumsum(e) / e.sum()
            u = float(c[int(rng.integers(0, V - 1))])
        adm = oracle.admissible_row(logits, 1.0, -1, p, np.float32(u), min_p=mp)
        assert 1 <= len(adm) <= 4
        for _ in range(20):
            e1, e2, e3 = rng.uniform(-0.9, 0.9, 3) * d
            pp = p + e1 if p < 1.0 else 1.0
            mm = mp * (1.0 + e3) if mp > 0.0 else 0.0
            uu = float(np.float32(u)) + e2
            tok, _ = _sample_exact(logits, pp, mm, uu)
            assert tok in adm, (trial, kind, tok, adm)


def _sample_exact(logits, p, mp, u):
    """sample_row's rule with thresholds taken as given (no float32 rounding
    of p, min_p or u): the perturbed reference for the test above."""
    l = np.asarray(logits, np.float64)
    V = len(l)
    e = np.exp(l - l.max())
    ranked = np.lexsort((np.arange(V), -l))
    if p < 1.0:
        q = e[ranked] / e[ranked].sum()
        before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
        ranked = ranked[:max(1, int(np.count_nonzero(before < p)))]
    if mp > 0.0:
        keep = (e[ranked] >= min(mp, 1.0)) | (l[ranked] == l.max())
        ranked = ranked[:int(np.count_nonzero(keep))]
    w = np.zeros(V)
    w[ranked] = e[ranked]
    c = np.cumsum(w)
    i = int(np.searchsorted(c, u * c[-1], side="right"))
    return (int(ranked.max()) if i >= V else i), False
