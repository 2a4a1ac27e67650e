"""Batched per-request sampler (oracle side; test infrastructure only).

Semantics follow "Engine 与采样器", section 采样器 (Sampler.sample and the
torch reference sample_torch), and "Mini-SGLang 源码解析（四）：GPU 计算引擎系统"
sections 14.3-14.4:

* no temperature array -> the whole batch is greedy -> argmax of the logits;
* otherwise per row: probabilities softmax(logits / T); rank tokens by
  probability; top-k keeps ranks < k; the kept mass is renormalised; top-p
  keeps a token iff the renormalised mass ranked *before* it is < p (so the
  most probable token always survives); top-k is applied before top-p; one
  token is drawn from what is left.
* min_p ("Engine 与采样器", section 练习 and its answer): a token survives iff
  its probability is at least min_p times the largest one, taken on the
  full temperature-scaled distribution; the mask is computed before top-k
  and top-p and intersected with their masks (top-p still renormalises over
  the top-k set alone). min_p <= 0 means no min_p; values above 1 act as 1.

Readings where the pages leave the step open (each listed in the design
notes):

* a row whose temperature is <= 1e-6 is an exact argmax (the pages give greedy
  rows of a mixed batch T = 1e-6 and say the effect is argmax);
* argmax ties go to the lowest index; ranking ties (equal logits) are broken
  by ascending index, so top-k keeps exactly k tokens; the ranking is taken on
  the logits, which orders tokens exactly like the probabilities for T > 0;
* top_k <= 0 or >= vocab means no top-k; top_p >= 1 means no top-p;
* the draw is inverse-CDF sampling with one caller-supplied uniform u in
  [0, 1) per row, scanning the kept weights in vocabulary index order: the
  token is the smallest index whose running kept mass exceeds u * (total kept
  mass), or the last kept index if rounding finds none (the pages fix only the
  distribution, via torch.multinomial or FlashInfer's rejection sampler);
* a row is *flagged* when a floating-point boundary lies within DELTA
  (relative to the kept mass) of the decision: the top-p cut or the draw, or
  (relative to min_p) a token's probability ratio to the largest one at the
  min_p threshold. The
  GPU computes those sums in another order and precision, so flagged rows are
  excluded from the bit-exact comparison and counted. Argmax and top-k are
  pure order comparisons and are never flagged. Three boundaries are exact on
  any hardware and never flag: the start of the first kept token (no kept
  mass precedes it), the end of the last kept token (running past it
  returns that same token), and min_p at a token whose logit equals the
  maximum (its ratio to the largest probability is exactly 1, and min_p is
  at most 1).

DELTA = 1e-5 leaves room for an implementation that computes each weight in
fp32 as 2^((l - l_max) * log2(e) / T) (relative error below ~2e-6 for every
weight above 1e-6 of the maximum) and sums in fp32 within small groups and
fp64 above: it can only move a decision whose boundary lies within a few
1e-6 of the target.
"""

import numpy as np

from .sampling_params import MIN_P, MIN_T

DELTA = 1e-5


def sample_row(logits: np.ndarray, T: float, top_k: int, top_p: float, u: float,
               delta: float = DELTA, info: dict | None = None, min_p: float = 0.0):
    """logits: f64 [V]. T, top_k, top_p, min_p are this row's device-side
    values (float32/int32 as the kernel sees them). Returns (token, flagged)."""
    l = np.asarray(logits, dtype=np.float64)
    V = l.shape[0]
    if np.float32(T) <= np.float32(MIN_T):
        return int(np.argmax(l)), False                      # first maximum = lowest index
    z = l / np.float64(np.float32(T))
    e = np.exp(z - z.max())                                  # unnormalised probabilities
    order = np.lexsort((np.arange(V), -l))                   # logit desc, index asc
    k = V if (top_k <= 0 or top_k >= V) else int(top_k)
    ranked = order[:k]                                       # top-k: ranks < k
    flagged = False
    p = np.float64(np.float32(top_p))
    if p < 1.0:
        p = max(p, MIN_P)
        q = e[ranked] / e[ranked].sum()                      # renormalise the kept mass
        before = np.concatenate(([0.0], np.cumsum(q)[:-1]))  # mass ranked before each token
        n_keep = int(np.count_nonzero(before < p))           # a prefix; >= 1 since before[0] = 0
        margin = p - before[n_keep - 1]
        if n_keep < k:
            margin = min(margin, before[n_keep] - p)
        if margin < delta:
            flagged = True
        ranked = ranked[:n_keep]
        if info is not None:
            info["top_p_margin"] = float(margin)
    mp = min(np.float64(np.float32(min_p)), 1.0)
    if mp > 0.0:
        # e is the probability over the largest one (e_max = 1); ranked is in
        # descending order, so the mask keeps a prefix of it
        keep = e[ranked] >= mp
        n_mp = int(np.count_nonzero(keep))
        margin = np.inf
        if n_mp > 0 and l[ranked[n_mp - 1]] < l.max():      # ratio exactly 1 at the maximum: exact
            margin = (e[ranked[n_mp - 1]] - mp) / mp
        if n_mp < len(ranked):
            margin = min(margin, (mp - e[ranked[n_mp]]) / mp)
        if margin < delta:
            flagged = True
        ranked = ranked[:n_mp]
        if info is not None:
            info["min_p_margin"] = float(margin)
    w = np.zeros(V, dtype=np.float64)
    w[ranked] = e[ranked]
    c = np.cumsum(w)
    W = c[-1]
    target = np.float64(np.float32(u)) * W
    i = int(np.searchsorted(c, target, side="right"))      # first index with c > target
    if i >= V:
        i = int(ranked.max())
    lo = c[i - 1] if i > 0 else 0.0
    lo_margin = (target - lo) if lo > 0.0 else np.inf          # no kept mass before: exact
    hi_margin = (c[i] - target) if i != int(ranked.max()) else np.inf   # last kept: exact
    draw_margin = min(lo_margin, hi_margin) / W
    if draw_margin < delta:
        flagged = True
    if info is not None:
        info.update(kept=int(len(ranked)), draw_margin=float(draw_margin), W=float(W))
    return i, flagged


def admissible_row(logits: np.ndarray, T: float, top_k: int, top_p: float, u: float,
                   delta: float = DELTA, min_p: float = 0.0) -> set:
    """Every token the sampling rule can return for this row when each
    rounding-sensitive decision is moved within its margin: the top-p
    threshold anywhere in [p - delta, p + delta], the min_p threshold anywhere
    in [min_p (1 - delta), min_p (1 + delta)] (capped at 1), and the draw
    target anywhere in [u W - delta W, u W + delta W] for the kept mass W of
    the resulting kept set. These are exactly the decisions whose margins the
    flag of ``sample_row`` measures, so an unflagged row's set is the single
    token ``sample_row`` returns. Argmax and top-k are exact order decisions
    and do not move."""
    l = np.asarray(logits, dtype=np.float64)
    V = l.shape[0]
    if np.float32(T) <= np.float32(MIN_T):
        return {int(np.argmax(l))}
    z = l / np.float64(np.float32(T))
    e = np.exp(z - z.max())
    order = np.lexsort((np.arange(V), -l))
    k = V if (top_k <= 0 or top_k >= V) else int(top_k)
    ranked = order[:k]
    # kept-set sizes reachable by the top-p threshold (a prefix of the ranking)
    n_p = [k, k]
    p = np.float64(np.float32(top_p))
    if p < 1.0:
        p = max(p, MIN_P)
        q = e[ranked] / e[ranked].sum()
        before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
        n_p = [int(np.count_nonzero(before < p - delta)), int(np.count_nonzero(before < p + delta))]
    # ... and by the min_p threshold (a prefix again: ranked is descending in e)
    n_m = [k, k]
    mp = min(np.float64(np.float32(min_p)), 1.0)
    if mp > 0.0:
        er = e[ranked]
        at_max = l[ranked] == l.max()                      # ratio exactly 1: never moves
        hi_thr, lo_thr = min(mp * (1.0 + delta), 1.0), mp * (1.0 - delta)
        n_m = [int(np.count_nonzero(at_max | (er >= hi_thr))), int(np.count_nonzero(at_max | (er >= lo_thr)))]
    n_lo = max(1, min(n_p[0], n_m[0]))
    n_hi = max(1, min(n_p[1], n_m[1]))
    out = set()
    for n in range(n_lo, n_hi + 1):
        kept = ranked[:n]
        w = np.zeros(V, dtype=np.float64)
        w[kept] = e[kept]
        c = np.cumsum(w)
        W = c[-1]
        target = np.float64(np.float32(u)) * W
        i_lo = int(np.searchsorted(c, target - delta * W, side="right"))
        i_hi = int(np.searchsorted(c, target + delta * W, side="right"))
        last = int(kept.max())
        for i in kept:
            if i_lo <= i <= i_hi:
                out.add(int(i))
        if i_hi >= V or i_lo > last:
            out.add(last)
    return out


def admissible(logits: np.ndarray, temperature, top_k, top_p, uniforms, rows, delta: float = DELTA,
               min_p=None) -> dict:
    """admissible_row for each row in ``rows`` of a batch (arguments as for
    ``sample``). Returns {row: set of tokens}."""
    out = {}
    for r in rows:
        if temperature is None:
            out[r] = {int(np.argmax(logits[r]))}
            continue
        k = -1 if top_k is None else int(top_k[r])
        p = 1.0 if top_p is None else float(top_p[r])
        mp = 0.0 if min_p is None else float(min_p[r])
        out[r] = admissible_row(logits[r], float(temperature[r]), k, p, float(uniforms[r]), delta, min_p=mp)
    return out


def sample(logits: np.ndarray, temperature, top_k, top_p, uniforms, delta: float = DELTA,
           rows=None, min_p=None):
    """logits: f64 [bs, V]; temperature / top_k / top_p / min_p: per-row
    device arrays or None (None temperature = all-greedy batch). Returns
    (tokens int32 [bs], flagged bool [bs])."""
    bs = logits.shape[0]
    tokens = np.full(bs, -1, dtype=np.int32)
    flagged = np.zeros(bs, dtype=bool)
    for r in (range(bs) if rows is None else rows):
        if temperature is None:
            tokens[r] = int(np.argmax(logits[r]))
            continue
        k = -1 if top_k is None else int(top_k[r])
        p = 1.0 if top_p is None else float(top_p[r])
        mp = 0.0 if min_p is None else float(min_p[r])
        tokens[r], flagged[r] = sample_row(logits[r], float(temperature[r]), k, p,
                                           float(uniforms[r]), delta, min_p=mp)
    return tokens, flagged
