"""Pins of the oracle's sampled-decoding functions against the mathematics.

The rejection rule is pinned by what makes it worth having: the tokens it
emits follow the target's distribution whatever the draft distribution is
("Medusa heads versus separate draft model", Training: rejection sampling
with the heads' probabilities keeps the target's distribution). Monte Carlo
frequencies over many seeded draws are compared with the exact laws by a
chi-square test at a one-in-a-million false-alarm level; the draws are fixed
by the seed, so each test is deterministic. A dropped renormalisation, a
residual taken the wrong way round or a wrong child order biases one of
these laws far beyond the test's threshold.
"""
import numpy as np
import pytest
from scipy.stats import chi2

import oracle

ALPHA = 1e-6


def _words(rng, *shape):
    return rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)


def _chi2_ok(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    n = counts.sum()
    keep = probs > 0
    assert counts[~keep].sum() == 0, "outcomes of zero probability occurred"
    exp = n * probs[keep]
    stat = float(((counts[keep] - exp) ** 2 / exp).sum())
    df = int(keep.sum()) - 1
    return stat, chi2.ppf(1 - ALPHA, df)


def test_unit_from_words_open_interval():
    u = oracle.unit_from_words(np.array([0, 1 << 9, 2 ** 32 - 1], dtype=np.uint32))
    assert u[0] == 2.0 ** -24
    assert u[1] == 1.5 * 2.0 ** -23
    assert u[2] == 1.0 - 2.0 ** -24
    g = oracle.gumbel_from_words(np.array([0, 2 ** 32 - 1], dtype=np.uint32))
    assert np.all(np.isfinite(g)) and g[0] < g[1]


def test_gumbel_top_k_is_sampling_without_replacement():
    # ordered pair (a, b) of a 2-draw sample without replacement: p_a p_b / (1 - p_a)
    T = 0.7
    lg = np.array([1.0, 0.3, -0.2, -1.0])
    p = np.exp(lg / T) / np.exp(lg / T).sum()
    n = 60000
    rng = np.random.default_rng(11)
    out = oracle.draft_sample(np.broadcast_to(lg, (n, 1, 4)).copy(), _words(rng, n, 1, 4), [2], T)
    tok = out["tok"][:, 0, :2]
    V = 4
    counts = np.zeros((V, V))
    np.add.at(counts, (tok[:, 0], tok[:, 1]), 1)
    probs = np.array([[p[a] * p[b] / (1 - p[a]) if a != b else 0.0 for b in range(V)] for a in range(V)])
    stat, lim = _chi2_ok(counts.ravel(), probs.ravel())
    assert stat < lim, (stat, lim)


def test_gumbel_top_k_at_low_temperature_is_the_top_k():
    # logits 0.05 apart at T = 1e-3 are 50 apart, more than the noise's whole range (about 19.4)
    rng = np.random.default_rng(3)
    V = 64
    lg = rng.permutation(V) * 0.05
    out = oracle.draft_sample(lg[None, None, :], _words(rng, 1, 1, V), [10], 1e-3)
    assert list(out["tok"][0, 0]) == list(np.argsort(-lg, kind="stable")[:10])


def test_log_sum_exp_closed_form():
    V, c, T = 1000, 2.5, 0.8
    out = oracle.draft_sample(np.full((1, 1, V), c), np.zeros((1, 1, V), dtype=np.uint32), [3], T)
    assert out["lse"][0, 0] == pytest.approx(np.log(V) + c / T, rel=1e-14)
    # equal logits, equal noise: the draw order falls back to the lowest index
    assert list(out["tok"][0, 0]) == [0, 1, 2]


# A small tree: the root has three children, the first of which has two.
PARENT = [-1, 0, 0, 0, 1, 1]
DEPTH = [0, 1, 1, 1, 2, 2]


def _trials(n, V, T, seed, head_scale):
    """Seeded walks where the target's distribution depends on the token
    prefix (a real model's does): L0 at the root, L1[x] after token x,
    L2[x][y] after (x, y). The heads' distributions are unrelated to it."""
    rng = np.random.default_rng(seed)
    L0 = rng.normal(size=V)
    L1 = rng.normal(size=(V, V))
    L2 = rng.normal(size=(V, V, V))
    H = rng.normal(size=(2, V)) * head_scale
    d = oracle.draft_sample(np.broadcast_to(H, (n, 2, V)).copy(), _words(rng, n, 2, V), [3, 2], T)
    tok = np.empty((n, 6), dtype=np.int32)
    tok[:, 0] = 0
    tok[:, 1:4] = d["tok"][:, 0, :3]
    tok[:, 4:6] = d["tok"][:, 1, :2]
    tl = np.empty((n, 6, V))
    tl[:, 0] = L0
    for j in (1, 2, 3):
        tl[:, j] = L1[tok[:, j]]
    for j in (4, 5):
        tl[:, j] = L2[tok[:, 1], tok[:, j]]
    out = oracle.verify_sampled(PARENT, tok, tl, np.broadcast_to(H, (n, 2, V)).copy(), T, _words(rng, n, 6),
                                _words(rng, n, V))
    return out["chosen"], tok, L0, L1


@pytest.mark.parametrize("T,head_scale,seed", [(1.0, 1.0, 5), (0.6, 2.0, 6), (1.0, 0.0, 7)])
def test_rejection_walk_emits_the_target_distribution(T, head_scale, seed):
    V, n = 5, 30000
    chosen, tok, L0, L1 = _trials(n, V, T, seed, head_scale)
    t1 = chosen[:, 0]
    stat, lim = _chi2_ok(np.bincount(t1, minlength=V), oracle.softmax_t(L0, T))
    assert stat < lim, ("first token", stat, lim)
    # when the first token is a child's, the walk went on: the second token
    # follows the target's distribution after that token
    stats, df = 0.0, 0
    for x in range(V):
        rows = []
        for r in np.nonzero(t1 == x)[0]:
            kids = [c for c in (1, 2, 3) if tok[r, c] == x]
            if kids:
                rows.append(chosen[r, kids[0]])
        if len(rows) < 200:
            continue
        p = oracle.softmax_t(L1[x], T)
        c = np.bincount(np.asarray(rows), minlength=V)
        stats += float(((c - len(rows) * p) ** 2 / (len(rows) * p)).sum())
        df += V - 1
    assert df > 0
    assert stats < chi2.ppf(1 - ALPHA, df), ("second token", stats, df)


def test_single_candidate_acceptance_is_the_overlap():
    # one draft token from q is accepted with probability sum_x min(p(x), q(x))
    rng = np.random.default_rng(21)
    V, T, n = 7, 1.0, 40000
    Lt = rng.normal(size=V) * 1.5
    Lh = rng.normal(size=V) * 1.5
    d = oracle.draft_sample(np.broadcast_to(Lh, (n, 1, V)).copy(), _words(rng, n, 1, V), [1], T)
    tok = np.stack([np.zeros(n, dtype=np.int32), d["tok"][:, 0, 0]], axis=1)
    tl = np.empty((n, 2, V))
    tl[:] = Lt
    out = oracle.verify_sampled([-1, 0], tok, tl, np.broadcast_to(Lh, (n, 1, V)).copy(), T, _words(rng, n, 2),
                                _words(rng, n, V))
    acc = (out["chosen"][:, 0] == tok[:, 1]).mean()
    a = np.minimum(oracle.softmax_t(Lt, T), oracle.softmax_t(Lh, T)).sum()
    assert abs(acc - a) < 5 * np.sqrt(a * (1 - a) / n), (acc, a)


def test_draft_equal_to_target_accepts_the_first_child():
    rng = np.random.default_rng(4)
    V, n = 50, 200
    L = rng.normal(size=V)
    tok = np.zeros((n, 6), dtype=np.int32)
    for r in range(n):
        tok[r, 1:4] = rng.choice(V, 3, replace=False)
        tok[r, 4:6] = rng.choice(V, 2, replace=False)
    tl = np.broadcast_to(L, (n, 6, V)).copy()
    hl = np.broadcast_to(L, (n, 2, V)).copy()
    out = oracle.verify_sampled(PARENT, tok, tl, hl, 1.0, _words(rng, n, 6), _words(rng, n, V))
    # p(x) / q(x) = 1: the first child and then its first child are accepted
    assert np.array_equal(out["chosen"][:, 0], tok[:, 1])
    assert np.array_equal(out["chosen"][:, 1], tok[:, 4])


def test_target_certain_of_another_token_rejects_every_child():
    rng = np.random.default_rng(8)
    V, n = 20, 100
    tl = np.zeros((n, 6, V))
    tl[:, 0, 17] = 80.0  # p(17) = 1 to double precision
    tok = np.zeros((n, 6), dtype=np.int32)
    for r in range(n):
        tok[r, 1:4] = rng.choice(np.arange(17), 3, replace=False)
        tok[r, 4:6] = rng.choice(V, 2, replace=False)
    out = oracle.verify_sampled(PARENT, tok, tl, np.zeros((n, 2, V)), 1.0, _words(rng, n, 6), _words(rng, n, V))
    assert np.all(out["chosen"][:, 0] == 17)
    assert np.all(out["chosen"][:, 1:] == -1)


def test_typical_thresholds_closed_forms():
    V, n = 16, 4
    rng = np.random.default_rng(9)
    tok = rng.integers(0, V, size=(n, 6)).astype(np.int32)
    gw = _words(rng, n, V)
    # uniform p: entropy log V, threshold min(eps, delta / V), p(token) = 1 / V
    tl = np.zeros((n, 6, V))
    out = oracle.typical_accept(PARENT, tok, tl, 1.0, 0.3, 0.5, gw)
    assert np.allclose(out["thr"][:, 1:], 0.5 / V)
    assert np.all(out["match"][:, 1:])  # 1/V > 0.5/V
    # every node matches: the deepest, lowest-index node (4) ends the step
    assert np.all(out["chosen"][:, 0] == tok[:, 1]) and np.all(out["chosen"][:, 1] == tok[:, 4])
    out = oracle.typical_accept(PARENT, tok, tl, 1.0, 0.3, 2.0, gw)
    assert not out["match"].any()  # 1/V < 2/V: nothing matches, the root ends the step
    assert np.all(out["chosen"][:, 1:] == -1)
    # eps = 0: nothing can exceed the threshold 0 ... except a positive probability, which every token has
    out = oracle.typical_accept(PARENT, tok, rng.normal(size=(n, 6, V)), 1.0, 0.0, 1.0, gw)
    assert np.all(out["thr"][:, 1:] == 0.0) and np.all(out["match"][:, 1:])


def test_typical_entropy_of_a_two_point_law():
    # p = (a, 1 - a) on two tokens (the rest at -inf weight): H = -a ln a - (1 - a) ln(1 - a)
    V, a = 8, 0.3
    tl = np.full((1, 6, V), -1e4)
    tl[0, 0, 2] = np.log(a)
    tl[0, 0, 5] = np.log(1 - a)
    tok = np.array([[0, 5, 2, 1, 0, 1]], dtype=np.int32)
    H = -a * np.log(a) - (1 - a) * np.log(1 - a)
    out = oracle.typical_accept(PARENT, tok, tl, 1.0, 1.0, 1.0, np.zeros((1, V), dtype=np.uint32))
    assert out["thr"][0, 1] == pytest.approx(np.exp(-H), rel=1e-12)
    assert out["ptok"][0, 1] == pytest.approx(1 - a, rel=1e-12) and out["ptok"][0, 2] == pytest.approx(a, rel=1e-12)
    assert list(out["match"][0, 1:4]) == [1 - a > np.exp(-H), a > np.exp(-H), False]
