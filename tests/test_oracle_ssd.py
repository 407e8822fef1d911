"""Pins of the pipeline reference (oracle/ssd.py): rounds of speculative
decoding with bigram models and the drafts prepared per predicted outcome.

* the draft's Gumbel-max step draws from softmax(row / T) (frequencies against
  the closed form);
* the rounds are lossless: the first two committed tokens are distributed as
  two autoregressive draws from the target model ([SD] section 3's guarantee),
  which fails for a wrong row index, position or commit;
* equal draft and target accept every draft (a_i = 1);
* the planted hit and miss tables give the outcomes they were built for;
* a hit's prepared drafts are the drafts the next round uses ([SSD] 4.1).
"""
import numpy as np
import pytest
from scipy import stats

import workloads as W
from oracle import ssd as S


def softmax(v, T):
    z = np.asarray(v, dtype=np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def test_draft_step_samples_the_tempered_softmax():
    rng = np.random.default_rng(11)
    V, T, n = 5, 0.7, 40000
    table = rng.normal(size=(V, V)).astype(np.float32)
    noise = (T * rng.gumbel(size=(n, V))).astype(np.float32)
    for t in (0, 3):
        first = np.array([S.bigram_draft(table, noise, t, pos, 1)[0] for pos in range(n)])
        counts = np.bincount(first, minlength=V)
        exp = softmax(table[t].astype(np.float64), T) * n
        assert stats.chisquare(counts, exp).pvalue > 1e-4, (counts, exp)
        # the untempered softmax is rejected: T matters
        assert stats.chisquare(counts, softmax(table[t].astype(np.float64), 1.0) * n).pvalue < 1e-6


def test_draft_step_ties_take_the_lower_id():
    table = np.zeros((3, 3), dtype=np.float32)
    noise = np.zeros((1, 3), dtype=np.float32)
    assert S.bigram_draft(table, noise, 0, 0, 2).tolist() == [0, 0]
    noise[0] = [0.0, 1.0, 1.0]
    assert S.bigram_draft(table, noise, 2, 5, 1).tolist() == [1]
    assert S.bigram_draft(table, noise, -1, 0, 2).tolist() == [-1, -1]


@pytest.mark.slow
@pytest.mark.parametrize("V,H", [(4, 4), (5, 3)])
def test_rounds_are_lossless(V, H):
    """First two committed tokens ~ q(y0 | last) q(y1 | y0), sampled over
    sequences that share no noise row (H < V: token t uses row t mod H)."""
    gamma, T, B = 2, 1.0, 6000
    rng = np.random.default_rng(5 + V)
    d = rng.normal(scale=1.0, size=(H, V)).astype(np.float32).astype(np.float64)
    t = rng.normal(scale=1.0, size=(H, V)).astype(np.float32).astype(np.float64)
    stride = 16
    noise = (T * rng.gumbel(size=(B * stride + 32, V))).astype(np.float32)
    last0 = np.zeros(B, dtype=np.int32)
    len0 = (np.arange(B) * stride).astype(np.int32)
    ua = W.uniforms24(rng, (2, B, gamma))
    us = W.uniforms24(rng, (2, B, gamma + 1))
    R = S.sd_rounds(d, t, noise, last0, len0, ua, us, T, 2)
    pairs = np.array([S.emitted(R, b)[:2] for b in range(B)])
    counts = np.bincount(pairs[:, 0] * V + pairs[:, 1], minlength=V * V)
    q0 = softmax(t[0], T)
    exp = np.array([q0[a] * softmax(t[a % H], T)[c] for a in range(V) for c in range(V)]) * B
    assert stats.chisquare(counts, exp).pvalue > 1e-4
    # the draft's own distribution is far from it: the verification matters
    p0 = softmax(d[0], T)
    expd = np.array([p0[a] * softmax(d[a % H], T)[c] for a in range(V) for c in range(V)]) * B
    assert stats.chisquare(counts, expd).pvalue < 1e-6


def test_equal_models_accept_every_draft():
    s = W.bigram_setup(6, 3, 256, 1.0, 5, 21, dtype="f32", kind="zipf")
    d = s.draft64()
    R = S.sd_rounds(d, d, s.noise, s.last0, s.len0, s.u_accept, s.u_sample, s.T, s.rounds)
    for r, rec in enumerate(R):
        for b in range(s.B):
            res = rec.results[b]
            assert res.accepted == s.gamma and res.mask == (1 << s.gamma) - 1
            assert res.tokens[:s.gamma].tolist() == rec.x[b].tolist()
            assert res.out_len == s.len0[b] + (r + 1) * (s.gamma + 1)


@pytest.mark.parametrize("kind", ["hit", "miss"])
def test_planted_outcomes(kind):
    s = W.bigram_setup(5, 4, 512, 1.0, 4, 23, kind=kind)
    d, t = s.draft64(), s.target64()
    R = S.sd_rounds(d, t, s.noise, s.last0, s.len0, s.u_accept, s.u_sample, s.T, s.rounds)
    for rec in R:
        for b in range(s.B):
            res = rec.results[b]
            if kind == "hit":
                assert res.accepted == s.gamma and rec.hit[b] == 1
                assert res.tokens[s.gamma] == int(np.argmax(d[rec.x[b][-1]]))
                assert rec.cand_idx[b] == 3 * s.gamma
            else:
                assert res.accepted == 0 and rec.hit[b] == 0 and rec.cand_idx[b] == -1
                planted = int(np.argmax(t[rec.last[b]]))
                assert res.tokens[0] == planted
                assert planted not in rec.cand[b, 0]


def test_hits_use_the_prepared_drafts():
    s = W.bigram_setup(12, 4, 1024, 1.0, 8, 29, kind="zipf", zipf=1.5)
    R = S.sd_rounds(s.draft64(), s.target64(), s.noise, s.last0, s.len0, s.u_accept, s.u_sample,
                    s.T, s.rounds)
    n_hit = 0
    for r in range(len(R) - 1):
        for b in range(s.B):
            if R[r].hit[b]:
                n_hit += 1
                assert R[r].prepared[b, R[r].cand_idx[b]].tolist() == R[r + 1].x[b].tolist()
    assert n_hit > 0
