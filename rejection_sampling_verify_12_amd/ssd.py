"""Speculative speculative decoding (SSD) around the verification, with
synthetic bigram models, on two HIP streams.

"Speculative Speculative Decoding (Saguaro)", sections 3.1 and 4.1, and the SSD
summary's pipeline part: while the target model scores and verifies round r,
the draft model predicts the round's outcome - k accepted drafts followed by
one of the draft's top-3 tokens at position k - and prepares round r+1's
drafts for every predicted outcome.  When the verification ends, a round whose
outcome was among the predictions (a hit) starts from the prepared drafts at
once; a miss drafts after the verification (the fallback).  The summary's AMD
MI300X part runs draft and target on separate HIP streams synchronised by
events, as here.

No model weights exist here.  The models are bigram tables (``spec_synth_*``):
after token t the logits are row t mod H of an [H, V] table, and the draft samples by Gumbel-max with a
per-position noise table, so its drafts are a function of the committed
sequence and the drafts prepared for an outcome are exactly those a fallback
would draw after it.  The time a real forward pass takes is modelled by
``spec_synthetic_busy`` kernels (one work-group each, as models on separate
devices would not take the verifier's compute units).  Everything that
decides a token runs on the device: the drafts, the rows, the verification,
the prediction with its hit flags, and the choice between prepared and fresh
drafts; nothing goes through the host between rounds.

* standard SD, one stream, round r: draft (t_draft) -> target rows and
  forward (t_target) -> verification -> commit and draft round r+1;
* SSD, round r: the target stream waits for round r's drafts, gathers the
  target rows, runs the target (t_target) and the verification with
  prediction, and records an event; meanwhile the draft stream predicts the
  outcomes (the draft's top-3 at every position), spends t_draft x fanout
  and prepares the drafts of every predicted outcome, then waits for that
  event, pays the fallback (t_draft, skipped when every sequence hit), and
  commits round r and takes round r+1's drafts (prepared on a hit, drawn
  afresh on a miss).

Both schedules emit the same tokens, round for round.
"""
from __future__ import annotations

import dataclasses
import time

from . import (PredictOut, VerifyOut, alloc_outputs, alloc_predict_outputs, new_workspace,
               spec_predict_outcomes, spec_predict_workspace_bytes, spec_ssd_advance,
               spec_ssd_prespeculate, spec_synth_draft, spec_synth_rows, spec_synthetic_busy,
               spec_verify, spec_verify_predict, spec_workspace_bytes, _dtype_code)


@dataclasses.dataclass
class Models:
    """Device inputs of a pipeline run.

    draft_table, target_table: [H, V] logits (float32 or bfloat16), row t mod H =
    the logits after token t.  noise: [P, V] float32, T-scaled Gumbel variates by
    absolute position (mod P).  last0, len0: [B] int32 start state (last
    committed token, committed length).  u_accept [R, B, gamma] and
    u_sample [R, B, gamma+1]: float32 uniforms of each round.  T: temperature.
    """
    draft_table: object
    target_table: object
    noise: object
    last0: object
    len0: object
    u_accept: object
    u_sample: object
    T: float

    @property
    def B(self) -> int:
        return int(self.last0.shape[0])

    @property
    def gamma(self) -> int:
        return int(self.u_accept.shape[2])

    @property
    def V(self) -> int:
        return int(self.draft_table.shape[1])


@dataclasses.dataclass
class Round:
    """One round as run: the state it started from, its drafts, the
    verification outputs and, under SSD, the prediction and prepared drafts."""
    last: object        # [B] last committed token before the round
    length: object      # [B] committed length before the round
    x: object           # [B, gamma] drafts
    out: VerifyOut
    pred: PredictOut | None = None
    prepared: object = None   # [B, 3(gamma+1), gamma]


class _Buffers:
    """Every device buffer a run needs, allocated before the timed loop (an
    allocation inside it could synchronise the device and undo the overlap).
    The logits rows of a round live in two-slot rings: slot r % 2 is
    rewritten only after the verification that read it two rounds earlier."""

    def __init__(self, m: Models, rounds: int, ssd: bool):
        import torch
        dev = m.draft_table.device
        B, g, V = m.B, m.gamma, m.V
        i32 = dict(dtype=torch.int32, device=dev)
        dt = _dtype_code(m.draft_table)
        self.ws = new_workspace(spec_workspace_bytes(B, g, V, dt), dev)
        self.last = [m.last0] + [torch.empty((B,), **i32) for _ in range(rounds)]
        self.length = [m.len0] + [torch.empty((B,), **i32) for _ in range(rounds)]
        self.x = [torch.empty((B, g), **i32) for _ in range(rounds + 1)]
        rows = lambda: torch.empty((B, g + 1, V), dtype=m.draft_table.dtype, device=dev)
        self.p = [rows(), rows()]
        self.q = [rows(), rows()]
        self.out = [alloc_outputs(B, g, dev) for _ in range(rounds)]
        if ssd:
            self.ws_p = new_workspace(spec_predict_workspace_bytes(B, g, V, dt), dev)
            self.pred = [alloc_predict_outputs(B, g, dev) for _ in range(rounds)]
            self.cand = [alloc_predict_outputs(B, g, dev) for _ in range(2)]
            self.prepared = [torch.empty((B, 3 * (g + 1), g), **i32) for _ in range(rounds)]
            self.ready = [torch.cuda.Event() for _ in range(rounds)]
            self.verified = [torch.cuda.Event() for _ in range(rounds)]

    def next_state(self, r: int):
        return self.last[r + 1], self.length[r + 1], self.x[r + 1]


def run_sd(m: Models, rounds: int, t_draft_ns: int, t_target_ns: int):
    """Standard speculative decoding on one stream.  Returns (seconds, [Round])."""
    import torch
    dev = m.draft_table.device
    st = torch.cuda.Stream(device=dev)
    bf = _Buffers(m, rounds, ssd=False)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    with torch.cuda.stream(st):
        spec_synth_draft(m.draft_table, m.noise, m.gamma, m.last0, m.len0, out=bf.x[0], stream=st)
        for r in range(rounds):
            p, q = bf.p[r % 2], bf.q[r % 2]
            spec_synthetic_busy(t_draft_ns, stream=st, device=dev)
            spec_synth_rows(m.draft_table, bf.last[r], bf.x[r], out=p, stream=st)
            spec_synth_rows(m.target_table, bf.last[r], bf.x[r], out=q, stream=st)
            spec_synthetic_busy(t_target_ns, stream=st, device=dev)
            out = spec_verify(p, q, bf.x[r], m.u_accept[r], m.u_sample[r], m.T,
                              in_len=bf.length[r], out=bf.out[r], workspace=bf.ws, stream=st)
            spec_ssd_advance(m.draft_table, m.noise, out, out=bf.next_state(r), stream=st)
    torch.cuda.synchronize(dev)
    dt = time.perf_counter() - t0
    return dt, [Round(bf.last[r], bf.length[r], bf.x[r], bf.out[r]) for r in range(rounds)]


def run_ssd(m: Models, rounds: int, t_draft_ns: int, t_target_ns: int, fanout: float = 1.0):
    """SSD on two streams (see the module docstring).  Returns (seconds, [Round])."""
    import torch
    dev = m.draft_table.device
    st_t = torch.cuda.Stream(device=dev)
    st_d = torch.cuda.Stream(device=dev)
    bf = _Buffers(m, rounds, ssd=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    with torch.cuda.stream(st_d):   # round 0 has no earlier round to speculate from
        spec_synth_draft(m.draft_table, m.noise, m.gamma, m.last0, m.len0, out=bf.x[0], stream=st_d)
        spec_synthetic_busy(t_draft_ns, stream=st_d, device=dev)
        spec_synth_rows(m.draft_table, bf.last[0], bf.x[0], out=bf.p[0], stream=st_d)
    for r in range(rounds):
        p, q = bf.p[r % 2], bf.q[r % 2]
        last, length, x = bf.last[r], bf.length[r], bf.x[r]
        bf.ready[r].record(st_d)
        with torch.cuda.stream(st_t):
            st_t.wait_event(bf.ready[r])
            spec_synth_rows(m.target_table, last, x, out=q, stream=st_t)
            spec_synthetic_busy(t_target_ns, stream=st_t, device=dev)
            out, pred = spec_verify_predict(p, q, x, m.u_accept[r], m.u_sample[r], m.T,
                                            in_len=length, out=bf.out[r], pred=bf.pred[r],
                                            workspace=bf.ws, stream=st_t)
            bf.verified[r].record(st_t)
        with torch.cuda.stream(st_d):
            cand = spec_predict_outcomes(p, out=bf.cand[r % 2], workspace=bf.ws_p, stream=st_d).cand
            spec_synthetic_busy(int(t_draft_ns * fanout), stream=st_d, device=dev)
            spec_ssd_prespeculate(m.draft_table, m.noise, cand, length, out=bf.prepared[r],
                                  stream=st_d)
            st_d.wait_event(bf.verified[r])
            spec_synthetic_busy(t_draft_ns, hit=pred.hit, stream=st_d)
            nl, nlen, nx = bf.next_state(r)
            spec_ssd_advance(m.draft_table, m.noise, out, pred, bf.prepared[r], out=(nl, nlen, nx),
                             stream=st_d)
            spec_synth_rows(m.draft_table, nl, nx, out=bf.p[(r + 1) % 2], stream=st_d)
    torch.cuda.synchronize(dev)
    dt = time.perf_counter() - t0
    return dt, [Round(bf.last[r], bf.length[r], bf.x[r], bf.out[r], bf.pred[r], bf.prepared[r])
                for r in range(rounds)]


def emitted_tokens(recs) -> int:
    """Tokens committed over the rounds: accepted + 1 per valid sequence."""
    import torch
    total = 0
    for rec in recs:
        a = rec.out.accepted
        total += int(torch.where(a >= 0, a + 1, torch.zeros_like(a)).sum().item())
    return total
