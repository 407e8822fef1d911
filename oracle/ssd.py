"""Reference rounds of speculative decoding with synthetic bigram models, and
the drafts that speculative speculative decoding prepares for each predicted
outcome (test infrastructure: only the test-suite uses it).

Pages: the speculative-decoding note ([SD]), section 3 (one round: draft,
verify, stop at the first rejection, emit the residual or bonus token; the
rounds repeat from the committed sequence), and "Speculative Speculative
Decoding (Saguaro)" ([SSD]), section 3.1 (an outcome is k accepted drafts and
the token after them, predicted from the draft's top-3) and section 4.1 (while
round r verifies, the next round's drafts are prepared; a hit uses them).

The models: after token t a bigram model's logits are row t mod H of its
[H, V] table.  The draft draws the token at absolute position pos after token t
as argmax_j(table[t mod H][j] + noise[pos mod P][j]), evaluated in float32 (one
addition) with ties to the lower id: with noise = T x standard Gumbel this is a
draw from softmax(table[t mod H] / T).  Every decision of a round is verify_one's, in
float64, on the exact logits.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .verify import SeqResult, predict_hits, predict_outcomes, verify_one


def bigram_draft(table32: np.ndarray, noise: np.ndarray, tok: int, pos: int, gamma: int) -> np.ndarray:
    """The gamma tokens the draft draws at positions pos, pos+1, ... after token
    tok (a token outside [0, V) gives -1 from there on)."""
    H, V = table32.shape
    P = noise.shape[0]
    out = np.full(gamma, -1, dtype=np.int32)
    tok = int(tok)
    for i in range(gamma):
        if not 0 <= tok < V:
            break
        score = np.add(table32[tok % H], noise[(int(pos) + i) % P], dtype=np.float32)
        tok = int(np.argmax(score))          # first maximum: the lower id among equals
        out[i] = tok
    return out


def bigram_rows(table64: np.ndarray, last: int, x: np.ndarray) -> np.ndarray:
    """A round's logits [gamma+1, V]: row i follows the token before position i
    (last, then x_0 .. x_{gamma-1}), row t mod H of the [H, V] table; a row
    after an invalid token is NaN."""
    H, V = table64.shape
    prev = [int(last)] + [int(v) for v in x]
    rows = np.full((len(prev), V), np.nan)
    for i, t in enumerate(prev):
        if 0 <= t < V:
            rows[i] = table64[t % H]
    return rows


@dataclasses.dataclass
class RefRound:
    last: np.ndarray          # [B] last committed token before the round
    length: np.ndarray        # [B] committed length before the round
    x: np.ndarray             # [B, gamma] the round's drafts
    results: list             # [B] SeqResult of verify_one
    cand: np.ndarray          # [B, gamma+1, 3] the draft's top-3 at every position
    hit: np.ndarray           # [B]
    cand_idx: np.ndarray      # [B]
    prepared: np.ndarray      # [B, 3(gamma+1), gamma] drafts after each predicted outcome


def sd_rounds(draft64: np.ndarray, target64: np.ndarray, noise: np.ndarray, last0, len0,
              u_accept: np.ndarray, u_sample: np.ndarray, T: float, rounds: int,
              seqs=None) -> list[RefRound]:
    """``rounds`` rounds from the start state (last0, len0) for the sequences
    ``seqs`` (default: all).  draft64, target64: [H, V] float64 tables (exact
    values of the stored logits); u_accept [R, B, gamma], u_sample
    [R, B, gamma+1]."""
    B = len(last0)
    seqs = list(range(B)) if seqs is None else list(seqs)
    gamma = u_accept.shape[2]
    n_out = 3 * (gamma + 1)
    table32 = draft64.astype(np.float32)     # exact: the logits are stored as float32 or bf16
    last = np.asarray(last0, dtype=np.int64).copy()
    length = np.asarray(len0, dtype=np.int64).copy()
    x = {b: bigram_draft(table32, noise, last[b], length[b], gamma) for b in seqs}
    out = []
    for r in range(rounds):
        rec = RefRound(last.copy(), length.copy(), np.full((B, gamma), -1, np.int32), [None] * B,
                       np.full((B, gamma + 1, 3), -1, np.int32), np.zeros(B, np.int32),
                       np.full(B, -1, np.int32), np.full((B, n_out, gamma), -1, np.int32))
        for b in seqs:
            p = bigram_rows(draft64, last[b], x[b])
            q = bigram_rows(target64, last[b], x[b])
            res: SeqResult = verify_one(p, q, x[b], u_accept[r, b], u_sample[r, b], T,
                                        in_len=int(length[b]))
            rec.x[b] = x[b]
            rec.results[b] = res
            # [SSD] 3.1: the outcomes predicted for this round, and whether it hit.
            rec.cand[b] = predict_outcomes(p[None])[0]
            h, i = predict_hits(rec.cand[b:b + 1], [res.accepted], [res.tokens])
            rec.hit[b], rec.cand_idx[b] = h[0], i[0]
            # [SSD] 4.1: the drafts that follow each predicted outcome.
            for c in range(n_out):
                rec.prepared[b, c] = bigram_draft(table32, noise, rec.cand[b, c // 3, c % 3],
                                                  length[b] + c // 3 + 1, gamma)
            # [SD] 3: commit x_0..x_{k-1} and y; the next round drafts after y.
            if res.valid:
                last[b] = int(res.tokens[res.accepted])
                length[b] = res.out_len
            else:
                last[b] = -1
            x[b] = bigram_draft(table32, noise, last[b], length[b], gamma)
        out.append(rec)
    return out


def emitted(rounds: list[RefRound], b: int) -> list[int]:
    """The tokens sequence b committed over the rounds, in order."""
    seq = []
    for rec in rounds:
        r = rec.results[b]
        if r is None or not r.valid:
            break
        seq += [int(v) for v in r.tokens[:r.accepted + 1]]
    return seq
