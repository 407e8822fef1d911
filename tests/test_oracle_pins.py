"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
numbers the pages print (tests/golden), hand-derived worked examples,
closed forms, a library routine, invariants of the definition, or a
statistical theorem the pages state (the output marginal equals the target).
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle as O
import workloads as W


def _toy_rows(state):
    return np.log(W.TOY_DRAFT[state]), np.log(W.TOY_TARGET[state])


# --------------------------------------------------------------------------- inputs

def test_toy_tables_match_page(golden):
    rows = golden("toy_tables.txt")
    for model, state, *vals in rows:
        table = W.TOY_DRAFT if model == "draft" else W.TOY_TARGET
        np.testing.assert_array_equal(table[int(state)], np.array(vals, dtype=np.float64))
    # Each table is a distribution.
    np.testing.assert_allclose(W.TOY_DRAFT.sum(1), 1.0, atol=1e-15)
    np.testing.assert_allclose(W.TOY_TARGET.sum(1), 1.0, atol=1e-15)


# --------------------------------------------------------------------------- O1 softmax

def test_softmax_uniform_logits():
    for V in (1, 7, 1000):
        l = np.full((2, V), 3.25)
        p, m, lz = O.softmax_rows(l, 0.5)
        np.testing.assert_allclose(p, 1.0 / V, rtol=1e-15)
        np.testing.assert_allclose(m, 6.5, rtol=0)
        np.testing.assert_allclose(lz, 6.5 + math.log(V), rtol=1e-15)


def test_softmax_of_log_table_returns_table():
    for s in (0, 1):
        for table in (W.TOY_DRAFT[s], W.TOY_TARGET[s]):
            p, _, lz = O.softmax_rows(np.log(table)[None], 1.0)
            np.testing.assert_allclose(p[0], table, rtol=0, atol=1e-15)
            assert abs(lz[0]) < 1e-15


def test_softmax_shift_invariance_and_temperature():
    rng = np.random.default_rng(5)
    l = rng.normal(size=(4, 50)) * 3
    p1, _, _ = O.softmax_rows(l, 1.0)
    p2, _, _ = O.softmax_rows(l + 123.0, 1.0)
    np.testing.assert_allclose(p1, p2, rtol=1e-12)
    for T in (0.3, 0.8, 2.5):
        pT, _, _ = O.softmax_rows(l, T)
        ref = p1 ** (1.0 / T)
        ref /= ref.sum(-1, keepdims=True)
        np.testing.assert_allclose(pT, ref, rtol=1e-11)


def test_softmax_matches_scipy():
    rng = np.random.default_rng(6)
    l = rng.normal(size=(3, 32000)) * 4
    for T in (1.0, 0.8):
        p, m, lz = O.softmax_rows(l, T)
        np.testing.assert_allclose(p, scipy.special.softmax(l / T, axis=-1), rtol=1e-12)
        np.testing.assert_allclose(lz, scipy.special.logsumexp(l / T, axis=-1), rtol=1e-14)
        np.testing.assert_array_equal(m, (l / T).max(-1))


def test_row_validity():
    l = np.zeros((5, 4))
    l[1, 2] = np.nan
    l[2, 0] = np.inf
    l[3, :] = -np.inf
    l[4, 1:] = -np.inf
    np.testing.assert_array_equal(O.row_valid(l), [True, False, False, False, True])
    p, _, _ = O.softmax_rows(l, 1.0)
    np.testing.assert_array_equal(p[4], [1, 0, 0, 0])


# --------------------------------------------------------------------------- O5 choice

def test_choice_running_sum_semantics():
    pi = np.array([0.25, 0.25, 0.5])
    assert O.choice(pi, 0.0)[0] == 0
    assert O.choice(pi, 0.2499999)[0] == 0
    assert O.choice(pi, 0.25)[0] == 1          # strict u < C_j
    assert O.choice(pi, 0.5)[0] == 2
    assert O.choice(pi, 0.9999999)[0] == 2
    # zero-probability tokens are never returned
    assert O.choice(np.array([0.5, 0.0, 0.5]), 0.5)[0] == 2
    # fallback when the running sum never exceeds u: last index with pi > 0
    assert O.choice(np.array([0.5, 0.25, 0.0]), 0.9)[0] == 1
    j, lo, hi = O.choice(pi, 0.3)
    assert (j, lo, hi) == (1, 0.25, 0.5)


# --------------------------------------------------------------------------- worked toy example

def test_toy_worked_example(golden):
    for row in golden("toy_worked.txt"):
        key, state, eps, *vals = row
        s = int(state)
        p, q = W.TOY_DRAFT[s], W.TOY_TARGET[s]
        v = np.array(vals, dtype=np.float64)
        if key == "accept":
            assert abs(O.acceptance_probability(p, q) - v[0]) < 1e-15
        elif key == "residual":
            w = O.residual_weights(p, q)
            np.testing.assert_allclose(w / w.sum(), v, atol=1e-14)
        elif key == "saguaro":
            w = O.residual_weights(p, q)
            np.testing.assert_allclose(O.saguaro_distribution(p, w, float(eps)), v,
                                       rtol=1e-8, atol=1e-12)


def test_saguaro_invariants():
    rng = np.random.default_rng(7)
    p = rng.dirichlet(np.ones(20))
    w = np.maximum(rng.normal(size=20), 0)
    # eps = 0: the residual's normalisation cancels.
    np.testing.assert_allclose(O.saguaro_distribution(p, w, 0.0),
                               O.saguaro_distribution(p, 7.5 * w, 0.0), rtol=1e-14)
    # p proportional to the residual: the geometric mean is the residual itself.
    np.testing.assert_allclose(O.saguaro_distribution(w / w.sum(), w, 0.0), w / w.sum(), atol=1e-15)
    # eps large: every token gets sqrt(p * eps) -> proportional to sqrt(p)
    s = np.sqrt(p)
    np.testing.assert_allclose(O.saguaro_distribution(p, w, 10.0), s / s.sum(), rtol=1e-13)


# --------------------------------------------------------------------------- accept rule

def _one(draft, target, x, ua, us, T=1.0, mode="residual", eps=0.0, in_len=0):
    return O.verify_one(np.asarray(draft), np.asarray(target), np.asarray(x),
                        np.asarray(ua, dtype=np.float64), np.asarray(us, dtype=np.float64),
                        T, mode, eps, in_len)


def test_accept_threshold_on_toy():
    ld, lt = _toy_rows(0)
    d = np.stack([ld, ld])     # gamma = 1: draft row 0, (unused) draft row 1
    t = np.stack([lt, lt])
    # x = 1: q/p = .18/.15 > 1 -> always accepted, bonus from target row 1.
    r = _one(d, t, [1], [0.9999999], [0.0, 0.0])
    assert r.accepted == 1 and r.tokens.tolist() == [1, 0] and r.mask == 1
    # x = 0: a = .50/.55 = 10/11.
    a = 10.0 / 11.0
    r = _one(d, t, [0], [a - 1e-9], [0.0, 0.0])
    assert r.accepted == 1
    r = _one(d, t, [0], [a + 1e-9], [0.59, 0.0])
    assert r.accepted == 0 and r.first_reject == 0 and r.mask == 0
    assert abs(r.a[0] - a) < 1e-15
    # Rejected: draw from residual [0, .6, .2, .2, 0, 0, 0] with C = .6, .8, 1.0.
    for us, tok in [(0.0, 1), (0.59, 1), (0.61, 2), (0.79, 2), (0.81, 3), (0.9999, 3)]:
        r = _one(d, t, [0], [0.95], [us, 0.0])
        assert r.tokens.tolist() == [tok, -1], (us, tok)
        assert abs(r.resid_mass - 0.05) < 1e-15
    r = _one(d, t, [0], [0.95], [0.7, 0.0], in_len=10)
    assert r.out_len == 11
    assert abs(r.cdf_lo - 0.6) < 1e-14 and abs(r.cdf_hi - 0.8) < 1e-14
    assert abs(r.sample_margin - 0.1) < 1e-12
    assert abs(r.zero_margin - 0.05) < 1e-15   # the residual mass: far from the S = 0 fallback


def test_special_cases():
    rng = np.random.default_rng(3)
    g, V = 5, 11
    d = rng.normal(size=(g + 1, V))
    # p == q: every position accepts whatever u < 1 is.
    r = _one(d, d, rng.integers(0, V, g), np.full(g, 0.99999994), np.zeros(g + 1))
    assert r.accepted == g and r.mask == (1 << g) - 1
    # u = 0 accepts every position with q(x) > 0.
    t = rng.normal(size=(g + 1, V))
    r = _one(d, t, rng.integers(0, V, g), np.zeros(g), np.zeros(g + 1))
    assert r.accepted == g
    # q(x) = 0 at position 2 forces the first rejection there (u = 0 still rejects).
    x = np.array([1, 2, 3, 4, 5])
    t2 = t.copy()
    t2[2, 3] = -np.inf
    r = _one(d, t2, x, np.zeros(g), np.zeros(g + 1))
    assert r.accepted == 2 and r.first_reject == 2 and r.mask == (1 << g) - 1 - (1 << 2)
    assert r.tokens[:2].tolist() == [1, 2] and r.tokens[2] != 3 and (r.tokens[3:] == -1).all()
    # p(x) = 0 (draft logit -inf at x) with q(x) > 0: accepted.
    d2 = d.copy()
    d2[0, 1] = -np.inf
    r = _one(d2, t, x, np.full(g, 0.5), np.zeros(g + 1))
    assert r.a[0] == 1.0


def test_bonus_comes_from_target_row_gamma():
    # All drafts accepted (p == q on rows < gamma); target row gamma is one-hot at 5,
    # row gamma-1 one-hot at 2.  The bonus must be 5 for every u.
    g, V = 3, 8
    d = np.zeros((g + 1, V))
    t = np.zeros((g + 1, V))
    t[g - 1] = d[g - 1] = -np.inf
    t[g - 1, 2] = d[g - 1, 2] = 0.0
    t[g] = -np.inf
    t[g, 5] = 0.0
    for us in (0.0, 0.5, 0.999):
        r = _one(d, t, [0, 1, 2], [0.5, 0.5, 0.5], [0.1, 0.1, 0.1, us])
        assert r.accepted == g and r.tokens.tolist() == [0, 1, 2, 5]


def test_invalid_sequences():
    d = np.zeros((3, 4))
    t = np.zeros((3, 4))
    r = _one(d, t, [0, 4], [0.1, 0.1], [0, 0, 0], in_len=7)
    assert r.accepted == -1 and r.out_len == 7 and (r.tokens == -1).all()
    t2 = t.copy()
    t2[2, 1] = np.nan        # target row gamma is read (bonus row)
    assert _one(d, t2, [0, 1], [0.1, 0.1], [0, 0, 0]).accepted == -1
    d2 = d.copy()
    d2[2, 1] = np.nan        # draft row gamma is not read by verification
    assert _one(d2, t, [0, 1], [0.1, 0.1], [0, 0, 0]).accepted == 2


# --------------------------------------------------------------------------- closed forms

def test_speedup_table_matches_page(golden):
    rows = golden("speedup_table.txt")
    assert len(rows) == 16
    for alpha, c, gamma, printed, flag in rows:
        s = float(O.speedup(float(alpha), float(c), int(gamma)))
        if flag == "ok":
            assert round(s, 2) == float(printed), (alpha, c, gamma, s, printed)
        else:
            assert round(s, 2) != float(printed)
            assert abs(s - 1.96875 / 1.5) < 1e-15


def test_expected_tokens_special_values():
    assert O.expected_tokens(0.0, 4) == 1.0
    assert O.expected_tokens(1.0, 4) == 5.0
    assert abs(O.expected_tokens(0.5, 1) - 1.5) < 1e-15


def _fixed_row_rounds(ld, lt, gamma, n, seed, T=1.0, mode="residual", eps=0.0):
    """n independent rounds whose every position uses the same rows (ld, lt)."""
    d = np.broadcast_to(ld, (gamma + 1, ld.shape[0]))
    t = np.broadcast_to(lt, (gamma + 1, lt.shape[0]))
    x = W.gumbel_argmax(np.broadcast_to(ld, (n, gamma, ld.shape[0])), T, W.philox(seed, 1))
    ua = W.uniforms24(W.philox(seed, 2), (n, gamma))
    us = W.uniforms24(W.philox(seed, 3), (n, gamma + 1))
    return [O.verify_one(d, t, x[b], ua[b], us[b], T, mode, eps) for b in range(n)]


@pytest.mark.slow
def test_expected_tokens_monte_carlo():
    # alpha = 0.5 exactly: p = [1, 0], q = [.5, .5]; x is always 0 and a = 0.5.
    with np.errstate(divide="ignore"):
        ld = np.log(np.array([1.0, 0.0]))
    lt = np.log(np.array([0.5, 0.5]))
    n, g = 20000, 4
    res = _fixed_row_rounds(ld, lt, g, n, seed=11)
    N = np.array([r.accepted + 1 for r in res])
    se = N.std() / math.sqrt(n)
    assert abs(N.mean() - O.expected_tokens(0.5, g)) < 4 * se
    # Toy state 0 rows with x ~ p: alpha = 0.95.
    ld, lt = _toy_rows(0)
    res = _fixed_row_rounds(ld, lt, g, n, seed=12)
    N = np.array([r.accepted + 1 for r in res])
    se = N.std() / math.sqrt(n)
    assert abs(N.mean() - O.expected_tokens(0.95, g)) < 4 * se
    # Acceptance rate at position 0 is sum min(p, q) = 0.95.
    acc0 = np.array([r.mask & 1 for r in res])
    assert abs(acc0.mean() - 0.95) < 4 * math.sqrt(0.95 * 0.05 / n)


def _chi2_ok(counts, probs, pmin=1e-3):
    counts = np.asarray(counts, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    keep = probs > 0
    assert counts[~keep].sum() == 0, "a zero-probability outcome was observed"
    exp = probs[keep] * counts.sum()
    stat = ((counts[keep] - exp) ** 2 / exp).sum()
    dof = keep.sum() - 1
    return scipy.stats.chi2.sf(stat, dof) > pmin


@pytest.mark.slow
def test_brute_force_tiny_vocab():
    """Exact (K, y) law by enumerating draft tuples, against oracle frequencies.

    With fixed rows per position, P(K = k, y = t) =
      sum_x prod_i p_i(x_i) * prod_{i<k} a_i(x_i) * (1 - a_k(x_k)) * pi_k(t)   (k < gamma)
      sum_x prod_i p_i(x_i) * prod_{i<gamma} a_i(x_i) * q_gamma(t)              (k = gamma)
    and the emitted token at every position j is distributed as q_j.
    """
    import itertools
    rng = np.random.default_rng(21)
    for V, g in ((2, 2), (3, 2), (4, 3)):
        P = rng.dirichlet(np.ones(V), size=g + 1)
        Q = rng.dirichlet(np.ones(V), size=g + 1)
        exact = np.zeros((g + 1, V))
        for x in itertools.product(range(V), repeat=g):
            wx = np.prod([P[i, x[i]] for i in range(g)])
            a = [min(1.0, Q[i, x[i]] / P[i, x[i]]) for i in range(g)]
            reach = 1.0
            for k in range(g):
                res = np.maximum(Q[k] - P[k], 0)
                exact[k] += wx * reach * (1 - a[k]) * res / res.sum()
                reach *= a[k]
            exact[g] += wx * reach * Q[g]
        assert abs(exact.sum() - 1) < 1e-12
        n = 20000
        x = W.gumbel_argmax(np.broadcast_to(np.log(P[:g]), (n, g, V)), 1.0, W.philox(V, 1))
        ua = W.uniforms24(W.philox(V, 2), (n, g))
        us = W.uniforms24(W.philox(V, 3), (n, g + 1))
        counts = np.zeros((g + 1, V))
        emitted = np.zeros((g + 1, V))
        for b in range(n):
            r = O.verify_one(np.log(P), np.log(Q), x[b], ua[b], us[b], 1.0)
            counts[r.accepted, r.tokens[r.accepted]] += 1
            for j in range(r.accepted + 1):
                emitted[j, r.tokens[j]] += 1
        assert _chi2_ok(counts.ravel(), exact.ravel()), (V, g)
        for j in range(g + 1):
            assert _chi2_ok(emitted[j], Q[j]), (V, g, j)


# --------------------------------------------------------------------------- losslessness

def _toy_transitions(n_rounds, seed, bonus_row_offset=0):
    prev = np.arange(n_rounds) % 2          # alternate prev between 0 and 1
    batch = W.toy_batch(prev, seed)
    d, t = batch.draft64(), batch.target64()
    if bonus_row_offset:
        # the page's toy passes q[:-1] and draws the bonus from its last entry
        t = t.copy()
        t[:, -1] = t[:, -1 + bonus_row_offset]
    res = O.verify(d, t, batch.draft_tokens, batch.u_accept, batch.u_sample, 1.0)
    first = np.zeros((2, 7))
    trans = np.zeros((2, 7))
    for b, r in enumerate(res):
        seq = [int(prev[b])] + r.tokens[: r.accepted + 1].tolist()
        first[int(prev[b] != 0), seq[1]] += 1
        for u, v in zip(seq[:-1], seq[1:]):
            trans[int(u != 0), v] += 1
    return first, trans


@pytest.mark.slow
def test_losslessness_toy_200k():
    """The blog's section 3 check: 200k rounds; the output equals the target law."""
    first, trans = _toy_transitions(200_000, seed=1201)
    for s in (0, 1):
        assert _chi2_ok(first[s], W.TOY_TARGET[s]), s
        assert _chi2_ok(trans[s], W.TOY_TARGET[s]), s
        freq = trans[s] / trans[s].sum()
        se = np.sqrt(W.TOY_TARGET[s] * (1 - W.TOY_TARGET[s]) / trans[s].sum())
        assert (np.abs(freq - W.TOY_TARGET[s]) < 5 * se).all()
    # The same statistic detects the page's off-by-one bonus row.
    _, bad = _toy_transitions(200_000, seed=1201, bonus_row_offset=-1)
    assert not all(_chi2_ok(bad[s], W.TOY_TARGET[s]) for s in (0, 1))


@pytest.mark.slow
def test_saguaro_marginal_closed_form():
    """In the resampling role the Saguaro output law is min(p, q) + (1 - alpha) pi_sag
    (so, unlike the residual, it is not q)."""
    ld, lt = _toy_rows(0)
    n = 40000
    res = _fixed_row_rounds(ld, lt, 1, n, seed=31, mode="saguaro")
    counts = np.zeros(7)
    for r in res:
        counts[r.tokens[0]] += 1
    p, q = W.TOY_DRAFT[0], W.TOY_TARGET[0]
    pi = np.array([0, 0.535960299, 0.252654108, 0.211385593, 0, 0, 0])
    law = np.minimum(p, q) + 0.05 * pi
    assert _chi2_ok(counts, law)


# --------------------------------------------------------------------------- outcome prediction

def test_top3_against_repeated_argmax():
    rng = np.random.default_rng(8)
    for V in (3, 7, 100, 5000):
        for _ in range(5):
            l = np.round(rng.normal(size=V), 1)      # many ties
            ref = []
            m = l.copy()
            for _ in range(3):
                j = int(np.argmax(m))                # first occurrence = lowest id
                ref.append(j)
                m[j] = -np.inf
            assert O.top3(l).tolist() == ref
    l = np.array([0.0, -0.0, 0.0, -1.0])
    assert O.top3(l).tolist() == [0, 1, 2]           # -0.0 ties with +0.0
    assert O.top3(np.array([1.0, np.nan, 2.0])).tolist() == [-1, -1, -1]
    assert O.top3(np.array([1.0, 2.0])).tolist() == [1, 0, -1]


@pytest.mark.slow
def test_predict_hit_rate_closed_form():
    """P(hit) = sum_k sum_{t in top3_k} P(K = k, y = t), by enumeration (tiny V)."""
    import itertools
    rng = np.random.default_rng(41)
    V, g = 5, 2
    P = rng.dirichlet(np.ones(V), size=g + 1)
    Q = rng.dirichlet(np.ones(V), size=g + 1)
    lp = np.log(P)
    cand = O.predict_outcomes(lp[None])[0]
    exact = np.zeros((g + 1, V))
    for x in itertools.product(range(V), repeat=g):
        wx = np.prod([P[i, x[i]] for i in range(g)])
        a = [min(1.0, Q[i, x[i]] / P[i, x[i]]) for i in range(g)]
        reach = 1.0
        for k in range(g):
            res = np.maximum(Q[k] - P[k], 0)
            exact[k] += wx * reach * (1 - a[k]) * res / res.sum()
            reach *= a[k]
        exact[g] += wx * reach * Q[g]
    p_hit = sum(exact[k, cand[k]].sum() for k in range(g + 1))
    n = 20000
    x = W.gumbel_argmax(np.broadcast_to(lp[:g], (n, g, V)), 1.0, W.philox(4, 1))
    ua = W.uniforms24(W.philox(4, 2), (n, g))
    us = W.uniforms24(W.philox(4, 3), (n, g + 1))
    res = [O.verify_one(lp, np.log(Q), x[b], ua[b], us[b], 1.0) for b in range(n)]
    hit, idx = O.predict_hits(np.broadcast_to(cand, (n, g + 1, 3)),
                              [r.accepted for r in res], [r.tokens for r in res])
    assert abs(hit.mean() - p_hit) < 4 * math.sqrt(p_hit * (1 - p_hit) / n)
    for b in range(n):
        k = res[b].accepted
        if hit[b]:
            assert idx[b] // 3 == k and cand[k, idx[b] % 3] == res[b].tokens[k]
        else:
            assert idx[b] == -1


# --------------------------------------------------------------------------- greedy verification

def test_greedy_is_the_zero_temperature_limit():
    """With distinct row maxima (gaps >= 0.5) and draft tokens = the draft's own
    argmax, the sampled rule at T = 0.002 (every probability off the maximum is
    below e^-250) must give exactly the greedy result for uniforms in
    [1e-3, 1 - 1e-3): accept iff the target's argmax agrees, emit its argmax."""
    rng = np.random.default_rng(21)
    T = 0.002
    for trial in range(40):
        g = int(rng.integers(1, 6))
        V = int(rng.integers(5, 60))
        d = np.stack([rng.permutation(V) * 0.5 for _ in range(g + 1)])
        t = d.copy()
        for i in range(g + 1):            # move the target's maximum elsewhere sometimes
            if rng.random() < 0.35:
                a, b = np.argmax(t[i]), int(rng.integers(V))
                t[i, [a, b]] = t[i, [b, a]]
        x = np.argmax(d[:g], axis=1)
        ua = rng.uniform(1e-3, 1 - 1e-3, g)
        us = rng.uniform(1e-3, 1 - 1e-3, g + 1)
        s = O.verify_one(d, t, x, ua, us, T, in_len=3)
        r = O.verify_greedy_one(t, x, in_len=3)
        assert (r.accepted, r.mask, r.out_len) == (s.accepted, s.mask, s.out_len), trial
        np.testing.assert_array_equal(r.tokens, s.tokens)


def test_greedy_speculation_reproduces_target_greedy_decoding():
    """Greedy speculative decoding of a Markov chain (draft proposes its own
    argmax continuation of gamma tokens, the target verifies them) emits
    exactly the target's own greedy decode, whatever the draft."""
    rng = np.random.default_rng(5)
    V = 7
    for trial in range(20):
        Pd = rng.normal(size=(V, V))
        Qt = Pd + rng.normal(scale=1.0, size=(V, V))   # overlapping, not equal
        g = int(rng.integers(1, 7))
        prev, out = 0, []
        while len(out) < 64:
            x, c = [], prev
            for _ in range(g):                            # draft's greedy proposal
                c = int(np.argmax(Pd[c]))
                x.append(c)
            ctx = [prev] + x                              # target scores gamma+1 positions
            t = np.stack([Qt[c] for c in ctx])
            r = O.verify_greedy_one(t, np.array(x))
            emitted = r.tokens[: r.accepted + 1].tolist()
            assert len(emitted) >= 1
            out += emitted
            prev = out[-1]
        ref, c = [], 0
        while len(ref) < len(out):
            c = int(np.argmax(Qt[c]))
            ref.append(c)
        assert out == ref, trial


def test_greedy_ties_and_invalid_rows():
    # Ties go to the lowest id, as numpy's argmax does.
    rng = np.random.default_rng(8)
    for _ in range(50):
        row = rng.integers(0, 3, size=int(rng.integers(1, 40))).astype(np.float64)
        assert O.first_argmax(row) == int(np.argmax(row))
    assert O.first_argmax(np.array([-np.inf, -np.inf])) == 0
    assert O.first_argmax(np.array([1.0, np.inf, 3.0, np.inf])) == 1
    assert O.first_argmax(np.array([-0.0, 0.0])) == 0
    g, V = 2, 5
    t = np.zeros((g + 1, V))
    t[0, 3] = t[1, 1] = t[2, 4] = 1.0
    r = O.verify_greedy_one(t, [3, 1], in_len=4)
    assert (r.accepted, r.first_reject, r.mask, r.out_len) == (2, -1, 3, 7)
    assert r.tokens.tolist() == [3, 1, 4]
    r = O.verify_greedy_one(t, [3, 2])
    assert (r.accepted, r.first_reject, r.mask) == (1, 1, 1) and r.tokens.tolist() == [3, 1, -1]
    r = O.verify_greedy_one(t, [0, 1])          # a later acceptance still shows in the mask
    assert (r.accepted, r.mask) == (0, 2) and r.tokens.tolist() == [3, -1, -1]
    t2 = t.copy()
    t2[2, 0] = np.nan                            # row gamma: read only after gamma acceptances
    assert O.verify_greedy_one(t2, [3, 2]).accepted == 1
    assert O.verify_greedy_one(t2, [3, 1]).accepted == -1
    t3 = t.copy()
    t3[1, 2] = np.nan                            # rows < gamma are always read
    assert O.verify_greedy_one(t3, [0, 1]).accepted == -1
    r = O.verify_greedy_one(t, [3, 5], in_len=9)  # token outside [0, V)
    assert (r.accepted, r.out_len, r.mask) == (-1, 9, 0) and (r.tokens == -1).all()


# --------------------------------------------------------------------------- early-exit verification

def test_early_exit_loop_equals_all_tests_then_first_rejection():
    """The page's loop with its break (early exit) and the all-positions
    formulation (every test, then the first rejection) give the same round on
    valid inputs; the early loop's mask is the full mask cut below k."""
    rng = np.random.default_rng(31)
    for trial in range(200):
        g = int(rng.integers(1, 7))
        V = int(rng.integers(2, 40))
        d = rng.normal(size=(g + 1, V)) * 2
        t = d + rng.normal(size=(g + 1, V)) * rng.uniform(0.05, 2.0)
        x = rng.integers(0, V, size=g)
        ua = rng.random(g)
        us = rng.random(g + 1)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        mode, eps = [("residual", 0.0), ("saguaro", 0.0), ("saguaro", 1e-8)][trial % 3]
        f = O.verify_one(d, t, x, ua, us, T, mode, eps, in_len=2)
        e = O.verify_early_one(d, t, x, ua, us, T, mode, eps, in_len=2)
        assert (e.accepted, e.first_reject, e.out_len) == (f.accepted, f.first_reject, f.out_len)
        np.testing.assert_array_equal(e.tokens, f.tokens)
        assert e.mask == f.mask & ((1 << f.accepted) - 1)
        assert e.token_prob == f.token_prob and (e.cdf_lo, e.cdf_hi) == (f.cdf_lo, f.cdf_hi)
        k = f.accepted
        np.testing.assert_array_equal(e.px[: k + 1 if k < g else g], f.px[: k + 1 if k < g else g])
        assert np.isnan(e.px[k + 1:]).all()


def test_early_exit_reads_only_up_to_the_first_rejection():
    g, V = 3, 6
    d = np.zeros((g + 1, V))
    t = np.zeros((g + 1, V))
    t[1, 0] = -np.inf              # q_1(x_1 = 0) = 0: position 1 always rejects
    x = [1, 0, 2]
    u = [0.5, 0.5, 0.5]
    us = [0.3, 0.3, 0.3, 0.3]
    assert O.verify_early_one(d, t, x, u, us, 1.0).accepted == 1
    for bad in ("draft2", "target2", "target3", "token2"):
        d2, t2, x2 = d.copy(), t.copy(), list(x)
        if bad == "draft2":
            d2[2, 4] = np.nan
        elif bad == "target2":
            t2[2, 1] = np.inf
        elif bad == "target3":
            t2[3, :] = -np.inf
        else:
            x2[2] = V
        e = O.verify_early_one(d2, t2, x2, u, us, 1.0)
        f = O.verify_one(d2, t2, x2, u, us, 1.0)
        assert e.accepted == 1 and e.mask == 1 and f.accepted == -1, bad
    d3 = d.copy()
    d3[1, 3] = np.nan              # a row the loop does read
    assert O.verify_early_one(d3, t, x, u, us, 1.0).accepted == -1
    t4 = t.copy()
    t4[1, 0] = 0.0                 # now every position accepts (p == q) ...
    t4[3, 2] = np.nan              # ... and the bonus row is read
    assert O.verify_early_one(d, t4, x, u, us, 1.0).accepted == -1
    t4[3, 2] = 0.0
    r = O.verify_early_one(d, t4, x, u, us, 1.0, in_len=4)
    assert (r.accepted, r.mask, r.out_len) == (3, 7, 8)


def test_bad_temperature_makes_the_sequence_invalid():
    d = np.zeros((3, 4))
    for T in (0.0, -1.0, np.nan, np.inf):
        for fn in (O.verify_one, O.verify_early_one):
            r = fn(d, d, [0, 1], [0.1, 0.1], [0.2, 0.2, 0.2], T, in_len=5)
            assert r.accepted == -1 and r.out_len == 5 and (r.tokens == -1).all()
    assert O.verify_one(d, d, [0, 1], [0.1, 0.1], [0.2, 0.2, 0.2], 1e-3).accepted == 2


# --------------------------------------------------------------------------- top-p

def _nucleus_by_sorting(l, T, top_p):
    """The shortest prefix of the tokens sorted by probability (then id) whose
    mass reaches top_p, extended to every token tied with its last one."""
    prob, _, _ = O.softmax_rows(l, T)
    order = np.lexsort((np.arange(len(l)), -l))
    run, last = 0.0, None
    for j in order:
        run += prob[j]
        last = j
        if run >= top_p:
            break
    keep = l >= l[last]
    return keep, prob[keep].sum()


def _nucleus_by_values(l, T, top_p):
    """The definition: distinct logits from the largest down, adding the mass
    of each value's tokens, until the mass reaches top_p."""
    prob, _, _ = O.softmax_rows(l, T)
    run = 0.0
    for v in np.unique(l)[::-1]:
        run += prob[l == v].sum()
        if run >= top_p:
            return v, run
    return np.unique(l)[0], run


def test_nucleus_against_sorting():
    rng = np.random.default_rng(41)
    for trial in range(300):
        V = int(rng.integers(1, 30))
        l = np.round(rng.normal(size=V) * 2, int(rng.integers(0, 2)))   # ties
        T = float(rng.choice([0.5, 1.0, 2.0]))
        top_p = float(rng.choice([0.1, 0.5, 0.8, 0.9, 0.95, 0.999]))
        L, mass, _ = O.nucleus(l, T, top_p)
        keep, m2 = _nucleus_by_sorting(l, T, top_p)
        np.testing.assert_array_equal(l >= L, keep)
        assert abs(mass - m2) < 1e-12
        v, m3 = _nucleus_by_values(l, T, top_p)
        assert v == L and abs(mass - m3) < 1e-12
    L, mass, _ = O.nucleus(np.array([1.0, 2.0]), 1.0, 1.0)
    assert L == -np.inf and mass == 1.0


def test_top_p_one_is_no_cut():
    rng = np.random.default_rng(42)
    d = rng.normal(size=(4, 9))
    t = d + 0.5 * rng.normal(size=d.shape)
    a = O.verify_one(d, t, [1, 2, 3], [0.3, 0.6, 0.9], [0.1, 0.5, 0.7, 0.2], 1.0)
    b = O.verify_one(d, t, [1, 2, 3], [0.3, 0.6, 0.9], [0.1, 0.5, 0.7, 0.2], 1.0, top_p=1.0)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    assert a.mask == b.mask and a.token_prob == b.token_prob


def test_top_p_rule_emits_the_cut_target_distribution():
    """With draft tokens drawn from the cut draft distribution, the first
    emitted token follows the cut target distribution (the pages' unbiasedness
    claim, with top-p on both sides), by a chi-square test over 60k rounds."""
    rng = np.random.default_rng(43)
    V, T, top_p = 7, 1.0, 0.8
    d = np.log(np.array([[.30, .20, .15, .12, .10, .08, .05]] * 2))
    t = np.log(np.array([[.10, .28, .22, .16, .11, .08, .05]] * 2))
    pd, _, _ = O.softmax_rows(d[0], T)
    Ld, Pd, _ = O.nucleus(d[0], T, top_p)
    p_cut = O.cut_to_nucleus(pd, d[0], Ld, Pd)
    qt, _, _ = O.softmax_rows(t[0], T)
    Lt, Pt, _ = O.nucleus(t[0], T, top_p)
    q_cut = O.cut_to_nucleus(qt, t[0], Lt, Pt)
    n = 60000
    xs = rng.choice(V, size=n, p=p_cut)
    ua, us = rng.random(n), rng.random((n, 2))
    counts = np.zeros(V)
    for i in range(n):
        r = O.verify_one(d, t, [xs[i]], [ua[i]], us[i], T, top_p=top_p)
        counts[r.tokens[0]] += 1
    assert counts[q_cut == 0].sum() == 0
    nz = q_cut > 0
    chi = scipy.stats.chisquare(counts[nz], q_cut[nz] * n)
    assert chi.pvalue > 1e-3, (counts / n, q_cut)


def test_top_p_equal_one_token_nuclei_fall_back_to_q():
    """Closed form: both rows' nuclei are the same single token t and the draft
    token lies outside them, so p'(x) = q'(x) = 0 rejects (reading 3), the
    residual (q' - p')+ is zero, and the draw falls back to q' = one-hot(t)
    (reading C7) whatever u is."""
    V, t = 9, 4
    d = np.full((2, V), -3.0)
    q = np.full((2, V), -2.0)
    d[:, t] = 4.0     # p(t) = e^7 / (e^7 + 8) ~ 0.993 > top_p
    q[:, t] = 3.0
    for us in (0.0, 0.5, 0.999):
        r = O.verify_one(d, q, [1], [0.3], [us, 0.0], 1.0, top_p=0.9)
        assert r.accepted == 0 and r.tokens.tolist() == [t, -1]
        assert r.resid_mass == 0.0 and r.token_prob == 1.0 and r.zero_margin == np.inf
