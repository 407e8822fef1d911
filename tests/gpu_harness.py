"""Helpers for the GPU parity tests: move a workload to the device, run the
HIP library through its C ABI, and compare element by element with the oracle.

Comparison rule (tolerances of the verification contract):
* accepted counts, first-rejection index, accept mask, output tokens and
  committed lengths must equal the oracle's exactly;
* the one excuse is a draw whose uniform lies within 1e-6 of its threshold:
  the first differing decision of a sequence (an accept test, or the sampled
  token) is excused iff the oracle's margin there is below 1e-6, measured in
  the normalised units of the distribution drawn from; that sequence's later
  outputs are not compared.  Excusals are counted over the whole session
  (TOTALS), and the excused rate over every draw compared must stay at or
  below 1e-4 (asserted by the session's last parity test);
* normalised probabilities (p(x), q(x), residual mass, pi(y)) agree within
  1e-5 relative (pi(y) below 1e-4: 1e-9 absolute); log-normalisers within
  1e-5 absolute; the running sums C_{y-1}, C_y of the normalised distribution
  within 1e-6 absolute (the boundary window).
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import oracle as O
import rejection_sampling_verify_12_amd as R
import workloads as W

EXCUSE = 1e-6
PROB_RTOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def logits_to_device(arr: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


@dataclasses.dataclass
class DeviceBatch:
    draft: torch.Tensor
    target: torch.Tensor
    tokens: torch.Tensor
    u_accept: torch.Tensor
    u_sample: torch.Tensor
    in_len: torch.Tensor


def to_device(batch: W.Batch, dev="cuda") -> DeviceBatch:
    return DeviceBatch(
        logits_to_device(batch.draft, batch.dtype, dev), logits_to_device(batch.target, batch.dtype, dev),
        torch.from_numpy(np.ascontiguousarray(batch.draft_tokens, dtype=np.int32)).to(dev),
        torch.from_numpy(np.ascontiguousarray(batch.u_accept, dtype=np.float32)).to(dev),
        torch.from_numpy(np.ascontiguousarray(batch.u_sample, dtype=np.float32)).to(dev),
        torch.from_numpy(np.ascontiguousarray(batch.in_len, dtype=np.int32)).to(dev))


def run_gpu(batch: W.Batch, mode="residual", eps=0.0, diag=True, db: DeviceBatch | None = None,
            early=False, ws=None):
    db = db or to_device(batch)
    dt = R.SPEC_BF16 if batch.dtype == "bf16" else R.SPEC_F32
    if ws is None:
        ws = R.new_workspace(R.spec_workspace_bytes(batch.B, batch.gamma, batch.V, dt), db.draft.device)
    if early:
        out = R.spec_verify_early(db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T,
                                  in_len=db.in_len, diag=diag, workspace=ws,
                                  saguaro=mode == "saguaro", eps=eps)
    elif mode == "residual":
        out = R.spec_verify(db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T,
                            in_len=db.in_len, diag=diag, workspace=ws)
    else:
        out = R.spec_verify_saguaro(db.draft, db.target, db.tokens, db.u_accept, db.u_sample,
                                    batch.T, in_len=db.in_len, diag=diag, eps=eps, workspace=ws)
    torch.cuda.synchronize()
    # The workspace's first word records a timed-out wait; it must stay zero.
    assert batch.B == 0 or int(ws[:4].view(torch.int32).item()) == 0, "bounded wait timed out"
    if batch.B:
        assert int(ws.to(torch.int64).sum().item()) == 0, "workspace not left zeroed"
    host = {
        "tokens": out.tokens.cpu().numpy(), "accepted": out.accepted.cpu().numpy(),
        "first_reject": out.first_reject.cpu().numpy(),
        "mask": out.accept_mask.cpu().numpy().view(np.uint64),
        "out_len": out.out_len.cpu().numpy(),
    }
    if out.diag is not None:
        host["diag"] = {k: v.cpu().numpy() for k, v in out.diag.items()}
    return host


def run_oracle(batch: W.Batch, mode="residual", eps=0.0, seqs=None, early=False):
    seqs = range(batch.B) if seqs is None else seqs
    out = {}
    fn = O.verify_early_one if early else O.verify_one
    for b in seqs:
        db = W.decode_f64(batch.draft[b], batch.dtype)
        tb = W.decode_f64(batch.target[b], batch.dtype)
        out[b] = fn(db, tb, batch.draft_tokens[b], batch.u_accept[b], batch.u_sample[b],
                    batch.T, mode, eps, int(batch.in_len[b]))
    return out


@dataclasses.dataclass
class Report:
    n_seq: int = 0
    n_draws: int = 0
    excused: int = 0
    boundary_draws: int = 0
    max_a_err: float = 0.0        # |a_gpu - a_oracle| over compared decisions
    max_cdf_err: float = 0.0      # |C_gpu - C_oracle| at the drawn token
    max_prob_rel: float = 0.0
    max_token_prob_abs: float = 0.0
    failures: list = dataclasses.field(default_factory=list)

    def merge(self, o: "Report"):
        for f in ("n_seq", "n_draws", "excused", "boundary_draws"):
            setattr(self, f, getattr(self, f) + getattr(o, f))
        for f in ("max_a_err", "max_cdf_err", "max_prob_rel", "max_token_prob_abs"):
            setattr(self, f, max(getattr(self, f), getattr(o, f)))
        self.failures += o.failures

    def check(self):
        """No unexcused difference; the excusals join the session's totals."""
        TOTALS.merge(dataclasses.replace(self, failures=[]))
        assert not self.failures, "\n".join(self.failures[:20])

    def __str__(self):
        return (f"seqs={self.n_seq} draws={self.n_draws} excused={self.excused} "
                f"boundary={self.boundary_draws} max|a err|={self.max_a_err:.3g} "
                f"max|C err|={self.max_cdf_err:.3g} max prob rel={self.max_prob_rel:.3g} "
                f"max|pi(y) err|={self.max_token_prob_abs:.3g}")


# Every checked comparison of the session: the excused rate is a property of
# the whole suite, not of one test.
TOTALS = Report()


def _rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


def compare(batch: W.Batch, gpu: dict, ref: dict, check_diag: bool = True) -> Report:
    rep = Report()
    g = batch.gamma
    for b, r in ref.items():
        rep.n_seq += 1
        gt = gpu["tokens"][b]
        gk = int(gpu["accepted"][b])
        if not r.valid:
            ok = (gk == -1 and (gt == -1).all() and gpu["first_reject"][b] == -1
                  and int(gpu["mask"][b]) == 0 and gpu["out_len"][b] == batch.in_len[b])
            if not ok:
                rep.failures.append(f"seq {b}: oracle invalid, gpu k={gk} tokens={gt.tolist()}")
            continue
        gm = int(gpu["mask"][b])
        rep.n_draws += g + 1
        # A draw is a boundary case when u is within rounding of a running sum,
        # or when the residual mass is within rounding of the S = 0 fallback.
        zero_boundary = getattr(r, "zero_margin", np.inf) < EXCUSE
        draw_boundary = r.sample_margin < EXCUSE or zero_boundary
        rep.boundary_draws += int((r.acc_margin < EXCUSE).sum()) + int(draw_boundary)
        excused = False
        for i in range(g):
            if ((gm >> i) & 1) != ((r.mask >> i) & 1):
                if r.acc_margin[i] < EXCUSE:
                    excused = True
                    break
                rep.failures.append(f"seq {b}: decision {i} differs, margin {r.acc_margin[i]:.3g}")
                break
        if excused:
            rep.excused += 1
            continue
        if gm != r.mask:
            continue   # failure already recorded
        if gk != r.accepted:
            rep.failures.append(f"seq {b}: k gpu {gk} vs oracle {r.accepted} with equal masks")
            continue
        k = gk
        exp_tokens = r.tokens.copy()
        if int(gt[k]) != int(exp_tokens[k]):
            if draw_boundary:
                rep.excused += 1
                continue
            rep.failures.append(f"seq {b}: token gpu {int(gt[k])} vs oracle {int(exp_tokens[k])} "
                                f"(k={k}, margin {r.sample_margin:.3g})")
            continue
        if not np.array_equal(gt, exp_tokens):
            rep.failures.append(f"seq {b}: tokens {gt.tolist()} vs {exp_tokens.tolist()}")
        if int(gpu["first_reject"][b]) != r.first_reject:
            rep.failures.append(f"seq {b}: first_reject {gpu['first_reject'][b]} vs {r.first_reject}")
        if int(gpu["out_len"][b]) != r.out_len:
            rep.failures.append(f"seq {b}: out_len {gpu['out_len'][b]} vs {r.out_len}")
        if check_diag and "diag" in gpu:
            d = gpu["diag"]
            px, qx = d["px"][b], d["qx"][b]
            a_gpu = np.where(px > 0, np.minimum(1.0, qx / np.where(px > 0, px, 1)), (qx > 0) * 1.0)
            rep.max_a_err = max(rep.max_a_err, float(np.abs(a_gpu - r.a).max()))
            for name, gv, ov in (("px", px, r.px), ("qx", qx, r.qx)):
                rel = np.abs(gv - ov) / np.maximum(np.abs(ov), 1e-300)
                big = (ov > 1e-30) & (rel > PROB_RTOL)
                if big.any():
                    rep.failures.append(f"seq {b}: {name} rel err {rel[big].max():.3g}")
                if (ov > 1e-30).any():
                    rep.max_prob_rel = max(rep.max_prob_rel, float(rel[ov > 1e-30].max()))
            lz = np.abs(d["row_logZ"][b] - r.row_logZ)
            if (lz > 1e-5 * np.maximum(1, np.abs(r.row_logZ))).any():
                rep.failures.append(f"seq {b}: row_logZ err {lz.max():.3g}")
            rm = np.abs(d["row_max"][b] - r.row_max)
            if (rm > 1e-6 * np.maximum(1, np.abs(r.row_max))).any():
                rep.failures.append(f"seq {b}: row_max err {rm.max():.3g}")
            if zero_boundary:   # the GPU may have drawn from q_k: the draw's diagnostics differ
                continue
            if r.resid_mass > 0 and _rel(d["resid_mass"][b], r.resid_mass) > PROB_RTOL:
                rep.failures.append(f"seq {b}: resid_mass {d['resid_mass'][b]} vs {r.resid_mass}")
            # pi(y) relative to 1e-5 above 1e-4; below, absolute 1e-9 (the fp32 residual's
            # cancellation error, ~1e-7 of q_j, exceeds 1e-5 of such tiny probabilities)
            tp_err = abs(d["token_prob"][b] - r.token_prob)
            rep.max_token_prob_abs = max(rep.max_token_prob_abs, tp_err)
            if tp_err > (PROB_RTOL * r.token_prob if r.token_prob >= 1e-4 else 1e-9):
                rep.failures.append(f"seq {b}: token_prob {d['token_prob'][b]} vs {r.token_prob}")
            ce = max(abs(d["cdf_lo"][b] - r.cdf_lo), abs(d["cdf_hi"][b] - r.cdf_hi))
            rep.max_cdf_err = max(rep.max_cdf_err, ce)
            if ce > EXCUSE:
                rep.failures.append(f"seq {b}: running-sum error {ce:.3g}")
    return rep


def parity(batch: W.Batch, mode="residual", eps=0.0, seqs=None, check_diag=True,
           early=False) -> Report:
    say(f"[parity] {batch.name} B={batch.B} gamma={batch.gamma} V={batch.V} dtype={batch.dtype} "
        f"T={batch.T} mode={mode} eps={eps} early={early}")
    gpu = run_gpu(batch, mode, eps, diag=check_diag, early=early)
    ref = run_oracle(batch, mode, eps, seqs, early=early)
    rep = compare(batch, gpu, ref, check_diag)
    say(f"[parity]   {rep}")
    return rep
