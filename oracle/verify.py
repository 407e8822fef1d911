"""Float64 definition of speculative-sampling verification, one sequence at a time.

Sources (cited by page title and section):

* [SD] "Speculative Decoding: small model guesses, large model verifies"
  (feifeigd.github.io blog, 2026-08-24).  Section 2: each round emits between 1
  and gamma+1 tokens; the target scores gamma+1 positions in one pass.
  Section 3: the per-position rule - accept the draft token x when a uniform
  is below min(1, q(x)/p(x)), otherwise resample from (q-p)+ / sum (q-p)+ and
  stop; the acceptance probability is sum_x min(p, q); the ``choice`` helper
  draws by a running sum in token-id order.  Section 5.4: temperature must be
  the same on both sides.
* [SSD] "Speculative Speculative Decoding (Saguaro)" note
  (metaphor-xennon.pages.dev).  Section 3.2: Saguaro sampling,
  p_sag(x) proportional to sqrt(p_D(x) * p_residual(x)); its code clamps the
  residual probabilities at 1e-8 before the square root and renormalises.
  Section 3.1: the verification outcome (k accepted, bonus, tokens) and the
  bonus prediction from the draft's top-3 logits.
* [SSD-blog] SSD summary (yomxxx.com, 2026-06-12), "AMD MI300X" part: on a
  rejection only the valid-length pointer of the KV cache moves.

Readings where the pages are silent or garbled (each is listed in the design
notes with its justification):

* p = softmax(l_draft / T), q = softmax(l_target / T), same T ([SD] 5.4).
* Inputs are [gamma+1][V] per sequence for both models; draft row gamma is
  read only by outcome prediction.
* The bonus token is drawn from target row gamma.  (The page's toy passes
  q[:-1] and then draws from its last entry, i.e. row gamma-1; section 2's
  "at most gamma+1 tokens" and the one-pass target over gamma+1 positions fix
  row gamma.)
* The loop stops at the first rejection even if the residual mass were zero;
  a zero residual mass (impossible in exact arithmetic after a rejection)
  falls back to drawing from q_k.
* Caller-supplied uniforms: u_accept[i] for the test at position i,
  u_sample[k] for the draw at the stopping position k (k = gamma: bonus).
* ``choice`` falls back to the last index with nonzero probability when the
  running sum never exceeds u (rounding only).
* Saguaro: pi proportional to sqrt(p_k * max(w / S, eps)), w = (q_k - p_k)+,
  S = sum w; eps = 0 is the formula, eps = 1e-8 the page's code.  Used only on
  a rejection; the bonus stays q_gamma.  A zero normaliser (residual only
  where p_k = 0) falls back to the residual.
* A sequence whose rows read by the rule hold a NaN or +inf logit, or are all
  -inf, or whose draft token lies outside [0, V), is invalid: accepted = -1,
  tokens -1, mask 0, first_reject -1, out_len = in_len.
* p(x) = 0 at a draft token: accept iff q(x) > 0.
* out_len = in_len + k + 1 (tokens committed this round).
* A per-sequence temperature that is not finite and positive makes that
  sequence invalid (a batch-wide one is rejected before any work).
* Top-p ([SD] section 3, after the unbiasedness check: the rule stacks on
  top-p sampling unchanged, when both sides use the same setting, section
  5.4): each row's distribution is cut to its nucleus and renormalised, and
  the rule runs on the cut distributions.  The pages do not define the
  nucleus; here it is every token whose logit is at least L, where L is the
  largest logit value at which the mass of the tokens with logits >= L
  reaches top_p (equal logits are all in or all out, so no order among equal
  tokens is needed).  top_p >= 1 keeps every token.
* Greedy verification is the temperature -> 0 limit of the rule: accept x_i
  iff it is the target's most likely token at position i, and emit the
  target's most likely token at the stopping position (the correction after a
  rejection, the bonus after gamma acceptances).  Equal logits: the lowest
  token id.  It reads only target rows; one holding a NaN makes the sequence
  invalid when the rule reads it (rows 0..gamma-1 always, row gamma iff k =
  gamma); +-inf logits are ordinary values there.
"""
from __future__ import annotations

import dataclasses

import numpy as np


# ---------------------------------------------------------------------------
# O1: tempered softmax per row.

def row_valid(logits64: np.ndarray) -> np.ndarray:
    """A row can be normalised iff it has no NaN, no +inf and some finite-or-above value."""
    l = np.asarray(logits64, dtype=np.float64)
    return ~np.isnan(l).any(-1) & ~(l == np.inf).any(-1) & (l > -np.inf).any(-1)


def softmax_rows(logits64: np.ndarray, T: float):
    """softmax(l / T) over the last axis, in float64.

    Returns (probs, row_max, row_logZ) with row_max = max_j l_j / T and
    row_logZ = log sum_j exp(l_j / T) (the log normaliser), so that
    probs_j = exp(l_j / T - row_logZ).  Invalid rows come back as NaN.
    """
    l = np.asarray(logits64, dtype=np.float64)
    ok = row_valid(l)
    z = l / T
    with np.errstate(invalid="ignore", over="ignore"):
        m = np.where(ok, np.max(np.where(np.isnan(z), -np.inf, z), axis=-1), np.nan)
        e = np.exp(z - m[..., None])
        Z = e.sum(axis=-1)
        probs = e / Z[..., None]
        logZ = m + np.log(Z)
    probs[~ok] = np.nan
    return probs, m, logZ


# ---------------------------------------------------------------------------
# O5: the categorical draw.

def choice(pi: np.ndarray, u: float) -> tuple[int, float, float]:
    """Running sum in token-id order; the first j with u < C_j.

    Returns (j, C_{j-1}, C_j).  If no j qualifies (C_last <= u by rounding),
    returns the last index with pi > 0.
    """
    c = np.cumsum(pi)
    hits = np.nonzero(u < c)[0]
    if hits.size:
        j = int(hits[0])
    else:
        nz = np.nonzero(pi > 0)[0]
        j = int(nz[-1]) if nz.size else len(pi) - 1
    lo = float(c[j - 1]) if j > 0 else 0.0
    return j, lo, float(c[j])


# ---------------------------------------------------------------------------
# Top-p cut of one row.

def nucleus(logits64_row: np.ndarray, T: float, top_p: float):
    """(L, mass, margin): the nucleus threshold logit, the probability mass of
    the tokens with logit >= L, and the distance of top_p from the two running
    masses around the cut (the boundary margin).  top_p >= 1: (-inf, 1, inf).

    The tokens are sorted by logit (descending); the running mass is read at
    the end of each run of equal logits, and the first run end at which it
    reaches top_p gives L."""
    l = np.asarray(logits64_row, dtype=np.float64)
    if top_p >= 1.0:
        return -np.inf, 1.0, np.inf
    prob, _, _ = softmax_rows(l, T)
    order = np.argsort(-l, kind="stable")
    ls, run = l[order], np.cumsum(prob[order])
    ends = np.nonzero(np.append(ls[1:] != ls[:-1], True))[0]   # last index of each run
    at = run[ends]
    hit = np.nonzero(at >= top_p)[0]
    g = int(hit[0]) if hit.size else len(ends) - 1
    before = float(at[g - 1]) if g > 0 else 0.0
    return float(ls[ends[g]]), float(at[g]), abs(min(top_p - before, float(at[g]) - top_p))


def cut_to_nucleus(prob: np.ndarray, logits64_row: np.ndarray, L: float, mass: float) -> np.ndarray:
    return np.where(np.asarray(logits64_row) >= L, prob / mass, 0.0)


# ---------------------------------------------------------------------------
# O4: the distribution drawn from after a rejection.

def residual_weights(p_k: np.ndarray, q_k: np.ndarray) -> np.ndarray:
    """w = (q - p)+ over normalised distributions ([SD] section 3)."""
    return np.maximum(q_k - p_k, 0.0)


def saguaro_distribution(p_k: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """pi proportional to sqrt(p_D * max(w / sum w, eps)) ([SSD] section 3.2).

    If every product is zero (the residual lives only where p_D = 0 and
    eps = 0) the formula is 0/0; the normalised residual is returned instead.
    """
    r = w / w.sum()
    s = np.sqrt(p_k * np.maximum(r, eps))
    tot = s.sum()
    return s / tot if tot > 0 else r


# ---------------------------------------------------------------------------

@dataclasses.dataclass
class SeqResult:
    valid: bool
    accepted: int                 # k, or -1 when invalid
    first_reject: int             # k if k < gamma else -1
    mask: int                     # bit i = decision at position i (all gamma decisions)
    tokens: np.ndarray            # [gamma+1], x_0..x_{k-1}, y, then -1
    out_len: int
    a: np.ndarray                 # [gamma] min(1, q_i(x_i)/p_i(x_i))
    acc_margin: np.ndarray        # [gamma] |u_i - a_i|
    sample_margin: float          # min(u - C_{y-1}, C_y - u)
    row_max: np.ndarray           # [2 gamma + 1] p rows 0..gamma-1 then q rows 0..gamma
    row_logZ: np.ndarray
    px: np.ndarray                # [gamma] p_i(x_i)
    qx: np.ndarray                # [gamma] q_i(x_i)
    resid_mass: float             # S = sum (q_k - p_k)+ (0 when k == gamma)
    token_prob: float             # pi(y)
    cdf_lo: float                 # C_{y-1}
    cdf_hi: float                 # C_y
    zero_margin: float = np.inf   # S at a rejection with S > 0 (its distance from the S = 0 fallback)


def _zero_margin(S: float, k: int, gamma: int) -> float:
    """Distance of a rejection's residual mass S from the S = 0 fallback
    (reading C7: S = 0 draws from q_k).  S is the total-variation distance of
    p_k and q_k; a residual that small is within float rounding of zero, so
    the draw is a boundary case like a u within rounding of a running sum."""
    return S if (k < gamma and S > 0.0) else np.inf


def _invalid(gamma: int, in_len: int) -> SeqResult:
    nan = np.full(gamma, np.nan)
    return SeqResult(False, -1, -1, 0, np.full(gamma + 1, -1, dtype=np.int32), int(in_len),
                     nan, nan, np.nan, np.full(2 * gamma + 1, np.nan),
                     np.full(2 * gamma + 1, np.nan), nan, nan, np.nan, np.nan, np.nan, np.nan)


def verify_one(draft64, target64, tokens, u_accept, u_sample, T, mode="residual",
               eps=0.0, in_len=0, top_p=1.0) -> SeqResult:
    """Verify one sequence.

    draft64, target64: [gamma+1, V] float64 logits.  tokens: [gamma] draft tokens.
    u_accept: [gamma], u_sample: [gamma+1] uniforms in [0, 1).
    """
    draft64 = np.asarray(draft64, dtype=np.float64)
    target64 = np.asarray(target64, dtype=np.float64)
    gamma = len(tokens)
    V = draft64.shape[-1]
    x = np.asarray(tokens, dtype=np.int64)
    if not (np.isfinite(T) and T > 0) or ((x < 0) | (x >= V)).any():
        return _invalid(gamma, in_len)
    if not (row_valid(draft64[:gamma]).all() and row_valid(target64[:gamma + 1]).all()):
        return _invalid(gamma, in_len)

    # O1
    p, pm, plz = softmax_rows(draft64[:gamma], T)
    q, qm, qlz = softmax_rows(target64[:gamma + 1], T)
    topp_margin = np.inf
    if top_p < 1.0:   # the rule on the nucleus of every row ([SD] section 3)
        for i in range(gamma):
            L, P, m = nucleus(draft64[i], T, top_p)
            p[i] = cut_to_nucleus(p[i], draft64[i], L, P)
            topp_margin = min(topp_margin, m)
        for i in range(gamma + 1):
            L, P, m = nucleus(target64[i], T, top_p)
            q[i] = cut_to_nucleus(q[i], target64[i], L, P)
            topp_margin = min(topp_margin, m)

    # O2: every position's decision (the mask reports all gamma of them).
    idx = np.arange(gamma)
    px = p[idx, x]
    qx = q[idx, x]
    a = np.empty(gamma)
    for i in range(gamma):
        if px[i] > 0:
            a[i] = min(1.0, qx[i] / px[i])
        else:
            a[i] = 1.0 if qx[i] > 0 else 0.0
    ua = np.asarray(u_accept, dtype=np.float64)
    acc = ua < a
    mask = 0
    for i in range(gamma):
        if acc[i]:
            mask |= 1 << i

    # O3: the first rejection stops the round ([SD] section 3).
    k = gamma
    for i in range(gamma):
        if not acc[i]:
            k = i
            break

    # O4/O5
    us = float(np.asarray(u_sample, dtype=np.float64)[k])
    if k < gamma:
        w = residual_weights(p[k], q[k])
        S = float(w.sum())
        if S > 0:
            pi = w / S if mode == "residual" else saguaro_distribution(p[k], w, eps)
        else:
            pi = q[k]
    else:
        S = 0.0
        pi = q[gamma]
    y, lo, hi = choice(pi, us)

    out = np.full(gamma + 1, -1, dtype=np.int32)
    out[:k] = x[:k]
    out[k] = y
    return SeqResult(
        valid=True, accepted=k, first_reject=k if k < gamma else -1, mask=mask,
        tokens=out, out_len=int(in_len) + k + 1, a=a,
        acc_margin=np.minimum(np.abs(ua - a), topp_margin),
        sample_margin=min(us - lo, hi - us, topp_margin), zero_margin=_zero_margin(S, k, gamma),
        row_max=np.concatenate([pm, qm]), row_logZ=np.concatenate([plz, qlz]),
        px=px, qx=qx, resid_mass=S, token_prob=float(pi[y]), cdf_lo=lo, cdf_hi=hi)


def verify_early_one(draft64, target64, tokens, u_accept, u_sample, T, mode="residual",
                     eps=0.0, in_len=0) -> SeqResult:
    """Early-exit verification of one sequence: the page's loop exactly as
    written ([SD] section 3: test position i, stop at the first rejection),
    reading a position's rows only when every earlier position was accepted.

    Same arguments as verify_one.  What differs from verify_one:
    * validity only concerns what the loop reads - draft tokens x_0..x_k,
      draft rows 0..min(k, gamma-1), target rows 0..k (row gamma only when
      k = gamma);
    * the mask holds the decisions made, bits 0..k-1 (all set);
    * row statistics, p(x) and q(x) exist only for the rows and positions read
      (NaN elsewhere).
    """
    draft64 = np.asarray(draft64, dtype=np.float64)
    target64 = np.asarray(target64, dtype=np.float64)
    gamma = len(tokens)
    V = draft64.shape[-1]
    x = np.asarray(tokens, dtype=np.int64)
    if not (np.isfinite(T) and T > 0):
        return _invalid(gamma, in_len)
    ua = np.asarray(u_accept, dtype=np.float64)
    nan = np.full(gamma, np.nan)
    a = nan.copy()
    px, qx = nan.copy(), nan.copy()
    row_max = np.full(2 * gamma + 1, np.nan)
    row_logZ = np.full(2 * gamma + 1, np.nan)
    k = gamma
    p_k = q_k = None
    for i in range(gamma):
        if not (0 <= x[i] < V) or not (row_valid(draft64[i]) and row_valid(target64[i])):
            return _invalid(gamma, in_len)
        p, pm, plz = softmax_rows(draft64[i], T)
        q, qm, qlz = softmax_rows(target64[i], T)
        row_max[i], row_logZ[i] = pm, plz
        row_max[gamma + i], row_logZ[gamma + i] = qm, qlz
        px[i], qx[i] = p[x[i]], q[x[i]]
        if px[i] > 0:
            a[i] = min(1.0, qx[i] / px[i])
        else:
            a[i] = 1.0 if qx[i] > 0 else 0.0
        if not ua[i] < a[i]:
            k = i
            p_k, q_k = p, q
            break
    us = float(np.asarray(u_sample, dtype=np.float64)[k])
    if k < gamma:
        w = residual_weights(p_k, q_k)
        S = float(w.sum())
        if S > 0:
            pi = w / S if mode == "residual" else saguaro_distribution(p_k, w, eps)
        else:
            pi = q_k
    else:
        if not row_valid(target64[gamma]):
            return _invalid(gamma, in_len)
        q_g, qm, qlz = softmax_rows(target64[gamma], T)
        row_max[2 * gamma], row_logZ[2 * gamma] = qm, qlz
        S = 0.0
        pi = q_g
    y, lo, hi = choice(pi, us)
    out = np.full(gamma + 1, -1, dtype=np.int32)
    out[:k] = x[:k]
    out[k] = y
    return SeqResult(
        valid=True, accepted=k, first_reject=k if k < gamma else -1, mask=(1 << k) - 1,
        tokens=out, out_len=int(in_len) + k + 1, a=a, acc_margin=np.abs(ua - a),
        sample_margin=min(us - lo, hi - us), zero_margin=_zero_margin(S, k, gamma),
        row_max=row_max, row_logZ=row_logZ,
        px=px, qx=qx, resid_mass=S, token_prob=float(pi[y]), cdf_lo=lo, cdf_hi=hi)


def verify(draft64, target64, draft_tokens, u_accept, u_sample, T, mode="residual",
           eps=0.0, in_len=None) -> list[SeqResult]:
    """Verify a batch: [B, gamma+1, V] logits; one SeqResult per sequence."""
    B = len(draft_tokens)
    in_len = np.zeros(B, dtype=np.int64) if in_len is None else np.asarray(in_len)
    return [verify_one(draft64[b], target64[b], draft_tokens[b], u_accept[b], u_sample[b],
                       T, mode, eps, int(in_len[b])) for b in range(B)]


# ---------------------------------------------------------------------------
# Greedy verification: the temperature -> 0 limit ([SD] section 5.4 ties the
# rule to the sampling temperature; "SSSD: Simply-Scalable Speculative
# Decoding" (papernotes.org note), training-strategy section: speculation runs
# in greedy and in speculative-sampling mode).

def first_argmax(row64: np.ndarray) -> int:
    """The lowest token id among the row's largest logits (row without NaN)."""
    l = np.asarray(row64, dtype=np.float64)
    m = l.max()
    return int(np.nonzero(l == m)[0][0])


@dataclasses.dataclass
class GreedyResult:
    valid: bool
    accepted: int        # k, or -1 when invalid
    first_reject: int    # k if k < gamma else -1
    mask: int            # bit i: x_i is the target's argmax at position i
    tokens: np.ndarray   # [gamma+1]: x_0..x_{k-1}, argmax q_k, then -1
    out_len: int


def verify_greedy_one(target64, tokens, in_len=0) -> GreedyResult:
    """Greedy verification of one sequence: target64 [gamma+1, V] logits,
    tokens [gamma] draft tokens."""
    t = np.asarray(target64, dtype=np.float64)
    gamma = len(tokens)
    V = t.shape[-1]
    x = np.asarray(tokens, dtype=np.int64)
    bad = GreedyResult(False, -1, -1, 0, np.full(gamma + 1, -1, dtype=np.int32), int(in_len))
    if ((x < 0) | (x >= V)).any() or np.isnan(t[:gamma]).any():
        return bad
    g = [first_argmax(t[i]) for i in range(gamma)]
    mask = 0
    for i in range(gamma):
        if x[i] == g[i]:
            mask |= 1 << i
    k = gamma
    for i in range(gamma):
        if x[i] != g[i]:
            k = i
            break
    if k == gamma and np.isnan(t[gamma]).any():
        return bad
    out = np.full(gamma + 1, -1, dtype=np.int32)
    out[:k] = x[:k]
    out[k] = g[k] if k < gamma else first_argmax(t[gamma])
    return GreedyResult(True, k, k if k < gamma else -1, mask, out, int(in_len) + k + 1)


def verify_greedy(target64, draft_tokens, in_len=None) -> list[GreedyResult]:
    B = len(draft_tokens)
    in_len = np.zeros(B, dtype=np.int64) if in_len is None else np.asarray(in_len)
    return [verify_greedy_one(target64[b], draft_tokens[b], int(in_len[b])) for b in range(B)]


# ---------------------------------------------------------------------------
# Outcome prediction ([SSD] section 3.1): the draft's top-3 at each position.

def top3(logits64_row: np.ndarray) -> np.ndarray:
    """The three largest logits' token ids, descending; equal logits: lower id first.

    A row holding a NaN yields [-1, -1, -1].
    """
    l = np.asarray(logits64_row, dtype=np.float64)
    if np.isnan(l).any():
        return np.full(3, -1, dtype=np.int32)
    order = np.lexsort((np.arange(l.shape[0]), -l))
    out = np.full(3, -1, dtype=np.int32)
    n = min(3, l.shape[0])
    out[:n] = order[:n]
    return out


def predict_outcomes(draft64: np.ndarray) -> np.ndarray:
    """Candidates [B, gamma+1, 3]: for every outcome k = 0..gamma, the draft's
    top-3 tokens at position k (the token emitted after k acceptances)."""
    B, G1, _ = draft64.shape
    cand = np.empty((B, G1, 3), dtype=np.int32)
    for b in range(B):
        for k in range(G1):
            cand[b, k] = top3(draft64[b, k])
    return cand


def predict_hits(cand: np.ndarray, accepted, tokens) -> tuple[np.ndarray, np.ndarray]:
    """hit[b] = the emitted token y at position k = accepted[b] is one of cand[b, k];
    cand_idx[b] = 3k + rank of that candidate, or -1."""
    B = cand.shape[0]
    hit = np.zeros(B, dtype=np.int32)
    idx = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        k = int(accepted[b])
        if k < 0:
            continue
        y = int(tokens[b][k])
        for r in range(3):
            if cand[b, k, r] == y and y >= 0:
                hit[b] = 1
                idx[b] = 3 * k + r
                break
    return hit, idx
