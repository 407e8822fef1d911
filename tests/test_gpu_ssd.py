"""The SSD pipeline (two streams, synthetic bigram models, timed busy kernels)
around the real verification and prediction kernels, checked round by round
against the reference rounds of oracle/ssd.py: each round's start state and
drafts, its verification outputs (with the boundary excusal of the parity
harness), and under SSD the predicted outcomes, the hit flags and every
prepared draft.  Round times are logged; the one timing assertion is loose.

Every case prints its name before touching the GPU.
"""
import types

import numpy as np
import pytest

import workloads as W
from oracle import ssd as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("gpu_harness")


def to_device(s: W.BigramSetup):
    from rejection_sampling_verify_12_amd import ssd
    dev = "cuda"
    tab = lambda a: H.logits_to_device(a, s.dtype, dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return ssd.Models(tab(s.draft_table), tab(s.target_table), f32(s.noise), i32(s.last0),
                      i32(s.len0), f32(s.u_accept), f32(s.u_sample), s.T)


def reference(s: W.BigramSetup):
    return S.sd_rounds(s.draft64(), s.target64(), s.noise, s.last0, s.len0, s.u_accept,
                       s.u_sample, s.T, s.rounds)


def check_rounds(s: W.BigramSetup, recs, ref, prespec: bool):
    """Compare every round; a sequence whose draw was excused at a boundary
    diverges from the reference and is not compared after that round."""
    assert len(recs) == len(ref)
    live = set(range(s.B))
    n_hits = 0
    for r, (g, o) in enumerate(zip(recs, ref)):
        seqs = sorted(live)
        last, length, x = (g.last.cpu().numpy(), g.length.cpu().numpy(), g.x.cpu().numpy())
        for b in seqs:
            assert last[b] == o.last[b] and length[b] == o.length[b], f"round {r} seq {b}: state"
            assert x[b].tolist() == o.x[b].tolist(), f"round {r} seq {b}: drafts {x[b]} vs {o.x[b]}"
        gpu = {"tokens": g.out.tokens.cpu().numpy(), "accepted": g.out.accepted.cpu().numpy(),
               "first_reject": g.out.first_reject.cpu().numpy(),
               "mask": g.out.accept_mask.cpu().numpy().view(np.uint64),
               "out_len": g.out.out_len.cpu().numpy()}
        ns = types.SimpleNamespace(gamma=s.gamma, in_len=o.length)
        rep = H.compare(ns, gpu, {b: o.results[b] for b in seqs}, check_diag=False)
        rep.check()
        for b in seqs:
            res = o.results[b]
            if int(gpu["accepted"][b]) != res.accepted or not np.array_equal(gpu["tokens"][b], res.tokens):
                live.discard(b)          # excused at a boundary: the sequences part here
        if prespec:
            cand, hit = g.pred.cand.cpu().numpy(), g.pred.hit.cpu().numpy()
            idx, prep = g.pred.cand_idx.cpu().numpy(), g.prepared.cpu().numpy()
            for b in seqs:
                assert np.array_equal(cand[b], o.cand[b]), f"round {r} seq {b}: candidates"
                assert np.array_equal(prep[b], o.prepared[b]), f"round {r} seq {b}: prepared drafts"
                if b in live:
                    assert (hit[b], idx[b]) == (o.hit[b], o.cand_idx[b]), f"round {r} seq {b}: hit"
                    n_hits += int(hit[b])
    return len(live), n_hits


CASES = [  # (B, gamma, V, H, T, rounds, dtype, seed)
    (16, 4, 4096, 4096, 1.0, 12, "bf16", 41),
    (9, 3, 1000, 1000, 0.8, 10, "f32", 43),      # V not a multiple of the vector width
    (4, 7, 6000, 6000, 1.0, 6, "bf16", 47),
    (8, 4, 128256, 64, 1.0, 6, "bf16", 59),      # the B=128 workload's vocabulary, 64 table rows
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_g{c[1]}_V{c[2]}_H{c[3]}_{c[6]}")
def test_pipeline_rounds_match_the_oracle(case):
    from rejection_sampling_verify_12_amd import ssd
    B, g, V, Hr, T, R, dt, seed = case
    s = W.bigram_setup(B, g, V, T, R, seed, dtype=dt, H=Hr)
    ref = reference(s)
    m = to_device(s)
    H.say(f"[ssd] oracle rounds B={B} gamma={g} V={V} {dt} rounds={R}: SD")
    _, sd = ssd.run_sd(m, R, 0, 0)
    live_sd, _ = check_rounds(s, sd, ref, prespec=False)
    H.say(f"[ssd]   SD matched ({live_sd}/{B} sequences to the end); SSD")
    _, sp = ssd.run_ssd(m, R, 0, 0)
    live_ssd, n_hits = check_rounds(s, sp, ref, prespec=True)
    n_ref_hits = int(sum(o.hit.sum() for o in ref))
    H.say(f"[ssd]   SSD matched ({live_ssd}/{B} to the end), hits {n_hits} (oracle {n_ref_hits} "
          f"of {B * R})")
    assert ssd.emitted_tokens(sp) == ssd.emitted_tokens(sd)


@pytest.mark.parametrize("kind", ["hit", "miss"])
def test_ssd_schedule_follows_the_hits(kind):
    """Planted tables where every outcome is predicted (hit) or none is (miss):
    the tokens match the oracle either way; with hits the draft's time hides
    behind the target's."""
    from rejection_sampling_verify_12_amd import ssd
    B, g, V, R = 4, 4, 1024, 16
    s = W.bigram_setup(B, g, V, 1.0, R, 53, kind=kind)
    H.say(f"[ssd] planted {kind}s B={B} gamma={g} V={V} rounds={R}")
    ref = reference(s)
    m = to_device(s)
    td, tt = 600_000, 900_000                   # ns: draft 0.6 ms, target 0.9 ms per round
    ssd.run_sd(m, 2, td, tt)                     # warm-up (first launches load code)
    ssd.run_ssd(m, 2, td, tt)
    t_sd, sd = ssd.run_sd(m, R, td, tt)
    t_ssd, sp = ssd.run_ssd(m, R, td, tt)
    check_rounds(s, sd, ref, prespec=False)
    check_rounds(s, sp, ref, prespec=True)
    hits = [int(rec.pred.hit.sum().item()) for rec in sp]
    assert hits == [B if kind == "hit" else 0] * R
    sd_round, ssd_round = t_sd / R * 1e6, t_ssd / R * 1e6
    H.say(f"[ssd]   round us: sd {sd_round:.0f}, ssd {ssd_round:.0f} "
          f"(draft {td / 1e3:.0f}, target {tt / 1e3:.0f})")
    if kind == "hit":
        assert ssd_round < sd_round
