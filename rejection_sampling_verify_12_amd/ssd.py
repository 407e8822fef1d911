"""Speculative speculative decoding (SSD) around the verification, with timed
synthetic models, on two HIP streams.

"Speculative Speculative Decoding (Saguaro)", section 4.1, and the SSD
summary's pipeline part: while the target model scores and verifies round r,
the draft model speculates the outcome of that verification and prepares the
drafts of round r+1 ahead of time; when the verification ends, a round whose
outcome was predicted (a cache hit) starts at once, and a miss falls back to
drafting after the verification.  The summary's AMD MI300X part runs draft
and target on separate HIP streams synchronised by events.

No model weights exist here.  The models are ``spec_synthetic_busy`` kernels
that occupy their stream for a set time (one work-group each, as models on
separate devices would not take the verifier's compute units); the
verification and the outcome prediction are the real kernels on real
(synthetic) logits, and the hit flags that decide whether a round pays the
fallback come from ``spec_verify_predict`` on the device, without a host
round trip:

* standard SD, one stream, per round: draft (t_draft) -> target (t_target) ->
  verification;
* SSD, per round r: the target stream waits for round r's drafts, runs the
  target (t_target) and the verification with prediction, and records an
  event; the draft stream meanwhile prepares round r+1 (t_draft x fanout, the
  drafts for the predicted outcomes), then waits for that event and runs a
  fallback draft (t_draft) that returns at once when every sequence's
  outcome was among its predictions.

The round's batch is verified with the same inputs either way, so both
pipelines emit the same tokens; only the schedule differs.
"""
from __future__ import annotations

import time

from . import (alloc_outputs, alloc_predict_outputs, new_workspace, spec_synthetic_busy,
               spec_verify, spec_verify_predict, spec_workspace_bytes, SPEC_BF16, SPEC_F32)


def _ws(batch):
    d = batch[0]
    B, G1, V = d.shape
    dt = SPEC_BF16 if str(d.dtype) == "torch.bfloat16" else SPEC_F32
    return new_workspace(spec_workspace_bytes(B, G1 - 1, V, dt), d.device)


def run_sd(batches, T: float, t_draft_ns: int, t_target_ns: int, rounds: int):
    """Standard speculative decoding on one stream.  ``batches``: a list of
    (draft, target, tokens, u_accept, u_sample) device tensors, used in turn.
    Returns (seconds, [VerifyOut per round])."""
    import torch
    dev = batches[0][0].device
    st = torch.cuda.Stream(device=dev)
    ws = _ws(batches[0])
    seq = (batches * (rounds // len(batches) + 1))[:rounds]
    outs = [alloc_outputs(b[0].shape[0], b[0].shape[1] - 1, dev) for b in seq]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    with torch.cuda.stream(st):
        for r in range(rounds):
            d, t, x, ua, us = seq[r]
            spec_synthetic_busy(t_draft_ns, stream=st, device=dev)
            spec_synthetic_busy(t_target_ns, stream=st, device=dev)
            spec_verify(d, t, x, ua, us, T, out=outs[r], workspace=ws, stream=st)
    torch.cuda.synchronize(dev)
    return time.perf_counter() - t0, outs


def run_ssd(batches, T: float, t_draft_ns: int, t_target_ns: int, rounds: int,
            fanout: float = 1.0):
    """SSD on two streams (see the module docstring).  Returns (seconds,
    [VerifyOut per round], [PredictOut per round])."""
    import torch
    dev = batches[0][0].device
    st_t = torch.cuda.Stream(device=dev)
    st_d = torch.cuda.Stream(device=dev)
    ws = _ws(batches[0])
    seq = (batches * (rounds // len(batches) + 1))[:rounds]
    outs = [alloc_outputs(b[0].shape[0], b[0].shape[1] - 1, dev) for b in seq]
    preds = [alloc_predict_outputs(b[0].shape[0], b[0].shape[1] - 1, dev) for b in seq]
    ready = [torch.cuda.Event() for _ in range(rounds + 1)]
    verified = [torch.cuda.Event() for _ in range(rounds)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    with torch.cuda.stream(st_d):   # round 0 has nothing to speculate from
        spec_synthetic_busy(t_draft_ns, stream=st_d, device=dev)
        ready[0].record(st_d)
    for r in range(rounds):
        d, t, x, ua, us = seq[r]
        with torch.cuda.stream(st_t):
            st_t.wait_event(ready[r])
            spec_synthetic_busy(t_target_ns, stream=st_t, device=dev)
            spec_verify_predict(d, t, x, ua, us, T, out=outs[r], pred=preds[r], workspace=ws,
                                stream=st_t)
            verified[r].record(st_t)
        with torch.cuda.stream(st_d):
            spec_synthetic_busy(int(t_draft_ns * fanout), stream=st_d, device=dev)
            st_d.wait_event(verified[r])
            spec_synthetic_busy(t_draft_ns, hit=preds[r].hit, stream=st_d)
            ready[r + 1].record(st_d)
    torch.cuda.synchronize(dev)
    return time.perf_counter() - t0, outs, preds


def emitted_tokens(outs) -> int:
    """Tokens committed over the rounds: accepted + 1 per valid sequence."""
    import torch
    total = 0
    for o in outs:
        a = o.accepted
        total += int(torch.where(a >= 0, a + 1, torch.zeros_like(a)).sum().item())
    return total
