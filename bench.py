#!/usr/bin/env python3
"""Benchmark: batched speculative-sampling verification on one MI355X.

A step is one call of the whole verification (row statistics of every draft
row i < gamma and target row i <= gamma, the accept tests, the first
rejection, the residual / Saguaro / bonus draw, the outputs) over one batch of
synthetic logits already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode residual]

Prints one JSON line.
* value = verified draft positions per second, B * gamma / ms_per_step, where
  ms_per_step is the wall time of the K timed calls (synchronised on both
  sides) over K.
* Before the timed calls: W untimed calls, then more until --warmup-ms of
  sustained work has passed (after idle, this GPU runs calls ~20% slower for
  the first ~20 ms of sustained work; see the design notes).
* roofline prices the call's algorithmic bytes against the MI355X HBM peak
  of 8 TB/s, over the mean HIP-event time of one call (achieved, frac) and
  over ms_per_step (achieved_per_step, frac_per_step: also the few
  microseconds between back-to-back calls); attainable_read is a plain read of
  the logits with the same loads.
* statistics: the observed mean tokens per round against the closed form
  E[N] of the speculative-decoding blog's section 4 for these rows, and with
  --predict the outcome-prediction hit rate against its enumerated value.
* cpu_baseline times the fp64 oracle on the same workload on this host's
  cores (one process, then a pool of processes over the sequences).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "B256_g8_V152064_bf16"
METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak) at B,gamma,V"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-ms", type=float, default=300.0,
                    help="untimed calls continue until this much wall time of sustained work has passed")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", choices=("residual", "saguaro", "greedy"), default="residual",
                    help="greedy: temperature -> 0 verification of the draft's own argmax tokens "
                         "(reads target rows only)")
    ap.add_argument("--eps", type=float, default=0.0)
    ap.add_argument("--predict", action="store_true",
                    help="each step also predicts outcomes (draft top-3 per position, hits), in "
                         "the same pass as the verification (spec_verify_predict)")
    ap.add_argument("--early", action="store_true",
                    help="early-exit verification (spec_verify_early): rows are read only up to the "
                         "first rejection; the roofline prices the rows the rule reads")
    ap.add_argument("--predict-separate", action="store_true",
                    help="with --predict: verification, then the stand-alone prediction call")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="cut every row to its top-p nucleus (spec_verify_ex); 0 = no cut")
    ap.add_argument("--ssd", action="store_true",
                    help="speculative speculative decoding pipeline with synthetic bigram models and "
                         "timed model passes: standard SD (one stream) against SSD (two streams)")
    ap.add_argument("--ssd-rounds", type=int, default=64)
    ap.add_argument("--ssd-batch", type=int, default=1, help="sequences per SSD round")
    ap.add_argument("--ssd-t", type=float, default=0.5, help="temperature of the SSD rounds")
    ap.add_argument("--ssd-draft-us", type=float, default=220.0,
                    help="draft model time per round (gamma draft steps)")
    ap.add_argument("--ssd-target-us", type=float, default=330.0, help="target model time per round")
    ap.add_argument("--timeline", action="store_true",
                    help="measurement build (python -m rejection_sampling_verify_12_amd.build --timeline): "
                         "after the timed calls, one more call's per-block timeline of the single kernel")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets to rotate through (0: enough for > 1 GB)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="wall-clock budget of each CPU oracle leg")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the pooled CPU oracle leg (0: min(16, os.cpu_count()))")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--lds-probe", action="store_true",
                    help="only time LDS atomic adds by lane-to-word pattern (spec_lds_atomic_probe)")
    return ap.parse_args()


LDS_PATTERNS = ("64 words, 64 banks", "8 words, 8 lanes each", "one word", "32 words on one bank")


def lds_probe(R, dev, iters: int = 2048, reps: int = 5) -> dict:
    """Clocks per wave-wide LDS atomic add per CU, by the lane-to-word
    pattern of spec_lds_atomic_probe: the kernel's event time (best of reps)
    times the 2.4 GHz peak engine clock over the 16 waves x 8 x iters adds
    each CU issues."""
    import torch
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for pat, name in enumerate(LDS_PATTERNS):
        for _ in range(2):
            R.spec_lds_atomic_probe(pat, iters, sink, stream=stream)
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            R.spec_lds_atomic_probe(pat, iters, sink, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out[name] = {"us": best * 1e3, "clocks_per_add": best * 1e-3 * 2.4e9 / (16 * 8 * iters)}
    return out


def _code_only(text: str) -> str:
    """C++ source without its comments, trailing blanks and empty lines:
    what the compiler sees of it, so that a comment edit keeps the digest."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":   # a string or character literal, escapes included
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line)


def source_digest() -> str:
    """sha256 prefix of the kernel sources (rejection_sampling_verify_12_amd/
    csrc/*) without their comments."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rejection_sampling_verify_12_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_record(workload: str, mode: str):
    """HBM bytes per call from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; None otherwise.  mode: residual,
    saguaro or greedy, with "_predict" for the fused prediction."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{mode}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_call")


_CPU_BATCH = None
_CPU_ARGS = None


def _oracle_seq(n):
    """One sequence through the fp64 oracle (a pool worker's task)."""
    import oracle as O
    import workloads as W
    batch, mode, eps, tokens = _CPU_ARGS
    if mode == "greedy":
        O.verify_greedy_one(W.decode_f64(batch.target[n], batch.dtype), tokens[n])
    else:
        O.verify_one(W.decode_f64(batch.draft[n], batch.dtype), W.decode_f64(batch.target[n], batch.dtype),
                     batch.draft_tokens[n], batch.u_accept[n], batch.u_sample[n], batch.T, mode, eps)
    return n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, mode: str, eps: float, budget_s: float, tokens, workers: int) -> dict:
    """The fp64 oracle on the same workload: one process on the first
    sequences (bounded by budget_s), then a pool of `workers` processes over
    every sequence (bounded likewise).  Runs before the GPU is touched (the
    pool forks)."""
    import multiprocessing as mp
    global _CPU_ARGS
    _CPU_ARGS = (batch, mode, eps, tokens)
    t0 = time.perf_counter()
    n1 = 0
    while n1 < batch.B and time.perf_counter() - t0 < budget_s:
        _oracle_seq(n1)
        n1 += 1
    dt1 = time.perf_counter() - t0
    one = n1 * batch.gamma / dt1
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_seq, range(min(workers, batch.B)))   # start-up outside the timing
        t0 = time.perf_counter()
        done = 0   # sequences verified (passes over the batch until min(2 s, budget) have elapsed)
        while time.perf_counter() - t0 < min(2.0, budget_s) or done == 0:
            for s0 in range(0, batch.B, 4 * workers):
                pool.map(_oracle_seq, range(s0, min(batch.B, s0 + 4 * workers)), chunksize=1)
                done += min(batch.B, s0 + 4 * workers) - s0
                if time.perf_counter() - t0 > budget_s:
                    break
        dtp = time.perf_counter() - t0
    return {"value": done * batch.gamma / dtp, "unit": "positions/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} sequences (passes over the {batch.B} of {batch.name}) over {workers} "
                      f"processes in {dtp:.1f} s; one process: first {n1} sequences in {dt1:.1f} s",
            "value_one_core": one, "cpu_count": os.cpu_count(), "cpu_model": cpu_model()}


def ssd_main(args):
    """SD against SSD rounds with synthetic bigram models: the workload's gamma
    and V, 64 table rows, --ssd-batch sequences per round, drafts drawn at
    --ssd-t, model times --ssd-draft-us and --ssd-target-us."""
    import numpy as np
    import torch

    import workloads as W
    from rejection_sampling_verify_12_amd import ssd

    name = args.workload if args.workload != DEFAULT_WORKLOAD else "B128_g4_V128256_bf16"
    _, gamma, V, _, dtype, _, seed = W.WORKLOADS[name]
    T, n, B = args.ssd_t, args.ssd_rounds, args.ssd_batch
    s = W.bigram_setup(B, gamma, V, T, n, seed, dtype=dtype, H=64)
    dev = torch.device("cuda:0")

    def tab(a):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    m = ssd.Models(tab(s.draft_table), tab(s.target_table), f32(s.noise), i32(s.last0),
                   i32(s.len0), f32(s.u_accept), f32(s.u_sample), T)
    td, tt = int(args.ssd_draft_us * 1e3), int(args.ssd_target_us * 1e3)
    ssd.run_sd(m, 4, td, tt)       # warm-up
    ssd.run_ssd(m, 4, td, tt)
    t_sd, sd = ssd.run_sd(m, n, td, tt)
    t_ssd, sp = ssd.run_ssd(m, n, td, tt)
    tokens = ssd.emitted_tokens(sd)
    same = all(torch.equal(a.out.tokens, b.out.tokens) for a, b in zip(sd, sp))
    hits = torch.stack([r.pred.hit for r in sp]).cpu().numpy()
    round_hit = float((hits != 0).all(axis=1).mean())     # rounds that need no fallback
    # rows, verification and commit alone, for the predicted round times
    t_v = ssd.run_sd(m, n, 0, 0)[0] / n
    sd_round, ssd_round = t_sd / n, t_ssd / n
    pred_ssd = max(td * 1e-9, tt * 1e-9 + t_v) + (1 - round_hit) * td * 1e-9
    print(json.dumps({
        "metric": "tokens/s of a speculative-decoding loop with synthetic bigram models and timed "
                  "model passes",
        "sd_tokens_per_s": tokens / t_sd, "ssd_tokens_per_s": tokens / t_ssd,
        "speedup": t_sd / t_ssd, "same_tokens": same, "hit_rate": float((hits != 0).mean()),
        "round_hit_rate": round_hit, "tokens": tokens, "rounds": n,
        "round_us": {"sd": sd_round * 1e6, "ssd": ssd_round * 1e6, "verify_only": t_v * 1e6,
                     "ssd_expected": pred_ssd * 1e6,
                     "sd_expected": (td + tt) * 1e-3 + t_v * 1e6},
        "config": {"workload": f"bigram models, gamma {gamma}, V {V}, 64 rows", "B_per_round": B,
                   "T": T, "draft_us": args.ssd_draft_us, "target_us": args.ssd_target_us},
        "data": "synthetic", "source_digest": source_digest()}), flush=True)


KINDS = ("stream", "decide", "mass", "sample", "draw", "last", "final", "test")


def timeline_report(args, batch, one_call, R):
    """One more call of the single kernel in the timeline build: per item
    kind, per XCC and for the sequence that finishes last, in microseconds
    from the kernel's first block (s_memrealtime, 100 MHz)."""
    import ctypes

    import numpy as np
    import torch
    lib = R.load_library()
    lib.spec_timeline_copy.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.spec_timeline_copy.restype = ctypes.c_int
    torch.cuda.synchronize()
    one_call()
    torch.cuda.synchronize()
    raw = np.zeros((1 << 17, 2, 4), dtype=np.uint32)
    if lib.spec_timeline_copy(raw.ctypes.data, 1 << 18) != 0:
        sys.exit("spec_timeline_copy failed")
    n = int((raw[:, 0, 1] != 0).sum())
    if n == 0:
        sys.exit("no timeline: this call does not run the single kernel")
    rec = raw[:n, 0, :].astype(np.int64)
    t0 = rec[:, 0].min()
    start, end = (rec[:, 0] - t0) / 100.0, (rec[:, 1] - t0) / 100.0
    kind, seq = rec[:, 2] & 0xFF, rec[:, 3]
    xcc = raw[:n, 1, 1].astype(np.int64) & 0xF
    r1 = lambda x: round(float(x), 1)
    kinds = {}
    for k in range(len(KINDS)):
        m = kind == k
        if m.any():
            d = end[m] - start[m]
            kinds[KINDS[k]] = {"n": int(m.sum()), "first_start": r1(start[m].min()),
                               "last_start": r1(start[m].max()), "last_end": r1(end[m].max()),
                               "dur_mean": r1(d.mean()), "dur_p50": r1(np.median(d)), "dur_max": r1(d.max())}
    per_xcc = {}
    for x in range(8):
        m = (kind == 0) & (xcc == x)
        if m.any():
            per_xcc[str(x)] = {"n": int(m.sum()), "dur_mean": r1((end[m] - start[m]).mean()),
                               "end_p50": r1(np.median(end[m])), "end_max": r1(end[m].max())}
    fin = kind == 6
    b_last = int(seq[fin][np.argmax(end[fin])]) if fin.any() else -1
    chain = {}
    for k in range(len(KINDS)):
        m = (kind == k) & (seq == b_last)
        if m.any():
            chain[KINDS[k]] = [r1(start[m].min()), r1(end[m].max())]
    edges = np.arange(0.0, end.max() + 2.0, 2.0)
    active = [int(((start < e + 2.0) & (end > e)).sum()) for e in edges]
    print(json.dumps({"timeline": {
        "workload": args.workload, "span_us": r1(end.max()), "blocks": n, "kinds": kinds,
        "stream_by_xcc": per_xcc, "last_sequence": b_last, "last_sequence_items": chain,
        "active_blocks_per_2us": active}, "source_digest": source_digest()}), flush=True)


_SMI = None


def gpu_clocks() -> dict:
    """Gfx and memory clocks (MHz) of GPU 0, if amdsmi can read them: the
    clock-info reading, and the GPU metrics table's per-XCC current and
    average gfx clocks (the clock-info value has read far below the clock the
    kernels run at, so the metrics are recorded beside it)."""
    global _SMI
    out = {}
    try:
        import amdsmi
        if _SMI is None:   # once: a later read then returns while the queued calls still run
            amdsmi.amdsmi_init()
            _SMI = amdsmi.amdsmi_get_processor_handles()[0]
        h = _SMI
    except Exception as e:   # a statistic, not a requirement
        return {"error": type(e).__name__}
    try:
        out["gfx_mhz"] = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk")
        out["mem_mhz"] = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM).get("clk")
    except Exception as e:
        out["clock_info_error"] = type(e).__name__
    try:
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        xcc = m.get("current_gfxclks")
        if isinstance(xcc, (list, tuple)):
            xcc = [v for v in xcc if isinstance(v, int) and 0 < v < 10000]
        out["metrics"] = {"current_gfxclks": xcc, "average_gfxclk_frequency": m.get("average_gfxclk_frequency"),
                          "current_uclk": m.get("current_uclk")}
    except Exception as e:
        out["metrics_error"] = type(e).__name__
    return out


def acceptance_statistics(d, t, T: float, gamma: int, chunk: int = 32):
    """alpha[b, i] = sum_j min(p_ij, q_ij), p = softmax(draft_i / T),
    q = softmax(target_i / T), for i < gamma, in fp64 on the GPU: the
    per-position acceptance probability when x_i ~ p_i (speculative-decoding
    blog, section 3).  A statistic of the workload; not on the measured path."""
    import torch
    B = d.shape[0]
    alpha = torch.empty((B, gamma), dtype=torch.float64, device=d.device)
    for b0 in range(0, B, chunk):
        p = torch.softmax(d[b0:b0 + chunk, :gamma].double() / T, -1)
        q = torch.softmax(t[b0:b0 + chunk, :gamma].double() / T, -1)
        alpha[b0:b0 + chunk] = torch.minimum(p, q).sum(-1)
    return alpha


def tokens_per_round(alpha, accepted):
    """Observed mean tokens per round (k + 1) against its expectation for these
    rows: E[N_b] = sum_{j=0..gamma} prod_{i<j} alpha_bi, which is the blog's
    section 4 closed form (1 - a^(gamma+1)) / (1 - a) when every alpha_bi = a."""
    import torch
    B, g = alpha.shape
    ones = torch.ones((B, 1), dtype=alpha.dtype, device=alpha.device)
    surv = torch.cat([ones, torch.cumprod(alpha, 1)], 1)          # P(N > j), j = 0..gamma
    j = torch.arange(g + 1, dtype=alpha.dtype, device=alpha.device)
    en = surv.sum(1)
    var = ((2 * j + 1) * surv).sum(1) - en * en
    k = torch.as_tensor(accepted, device=alpha.device)
    valid = k >= 0
    obs = (k[valid].double() + 1).mean().item()
    exp = en[valid].mean().item()
    se = (var[valid].sum().sqrt() / valid.sum()).item()
    a_bar = alpha[valid].mean().item()
    return {"observed": obs, "expected": exp, "se": se, "z": (obs - exp) / se if se > 0 else None,
            "closed_form_at_mean_alpha": (1 - a_bar ** (g + 1)) / (1 - a_bar), "mean_alpha": a_bar,
            "sequences": int(valid.sum().item())}


def hit_rate_statistics(d, t, T: float, gamma: int, alpha, cand, hit):
    """Outcome-prediction hit rate against its enumerated value ("Speculative
    Speculative Decoding (Saguaro)", section 3.1): with K the first rejection
    (x_i ~ p_i, uniforms uniform), P(hit) = sum_{k<gamma} P(K=k) sum over the
    draft's top-3 at k of the residual (q_k - p_k)+ / (1 - alpha_k), plus
    P(K=gamma) times q_gamma's mass on the top-3 at gamma.  Residual mode."""
    import torch
    B = d.shape[0]
    ones = torch.ones((B, 1), dtype=torch.float64, device=d.device)
    surv = torch.cat([ones, torch.cumprod(alpha, 1)], 1)
    pk = torch.cat([surv[:, :gamma] * (1 - alpha), surv[:, gamma:]], 1)   # P(K = k), k = 0..gamma
    mass = torch.zeros((B, gamma + 1), dtype=torch.float64, device=d.device)
    c = cand.long().clamp(min=0)
    for k in range(gamma + 1):
        q = torch.softmax(t[:, k].double() / T, -1)
        if k < gamma:
            p = torch.softmax(d[:, k].double() / T, -1)
            w = (q - p).clamp(min=0) / (1 - alpha[:, k:k + 1])
        else:
            w = q
        mass[:, k] = (w.gather(1, c[:, k]) * (cand[:, k] >= 0)).sum(1)
    ph = (pk * mass).sum(1)
    obs = hit.double().mean().item()
    exp = ph.mean().item()
    se = ((ph * (1 - ph)).sum().sqrt() / B).item()
    return {"observed": obs, "expected": exp, "se": se, "z": (obs - exp) / se if se > 0 else None}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported (sequences are "
              "independent; a multi-GPU run would shard B with no communication).", file=sys.stderr)
        sys.exit(2)
    if args.ssd:
        return ssd_main(args)

    import numpy as np

    import rejection_sampling_verify_12_amd as R
    import workloads as W

    if args.timeline:
        from rejection_sampling_verify_12_amd import build as BLD
        R._lib = None
        R.load_library(BLD.TIMELINE_LIB)

    t0 = time.perf_counter()
    batch = W.make_workload(args.workload, workers=min(16, os.cpu_count() or 1))
    print(f"[bench] generated {args.workload} in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
          flush=True)
    B, g, V = batch.B, batch.gamma, batch.V
    dt_code = R.SPEC_BF16 if batch.dtype == "bf16" else R.SPEC_F32
    if args.top_p > 0.0 and (args.predict or args.early or args.mode == "greedy"):
        sys.exit("--top-p combines with residual or Saguaro verification only")
    if (args.predict or args.early) and args.mode == "greedy":
        sys.exit("--predict and --early are not available with --mode greedy")
    if args.predict and args.early:
        sys.exit("--predict and --early do not combine")
    greedy = args.mode == "greedy"
    gtok = None
    if greedy:   # the draft's greedy tokens
        gtok = np.argmax(W.decode_f64(batch.draft[:, :g], batch.dtype), axis=-1).astype(np.int32)

    # The CPU oracle legs run first: the pool forks, which must happen before
    # anything touches the GPU.
    cpu = None
    if not args.no_cpu:
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(batch, args.mode, args.eps, args.cpu_seconds, gtok, workers)
        print(f"[bench] cpu baseline {cpu['value']:.0f} positions/s over {workers} processes", file=sys.stderr,
              flush=True)

    import torch
    dev = torch.device("cuda:0")
    if args.lds_probe:
        print(json.dumps({"lds_atomic_probe": lds_probe(R, dev), "iters": 2048, "waves_per_cu": 16,
                          "clock_ghz": 2.4, "source_digest": source_digest()}))
        return
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": args.steps}))
        return

    es = 2 if batch.dtype == "bf16" else 4
    if greedy:   # target rows, draft tokens, lengths and the outputs
        bytes_alg = (B * (g + 1) * V * es + B * g * 4 + B * 4 + B * (g + 1) * 4
                     + B * (4 + 4 + 8 + 4))
    else:
        bytes_alg = R.bytes_algorithmic(B, g, V, dt_code)
    if args.predict:   # draft row gamma, which only the prediction reads
        bytes_alg += B * V * es
    nsets = args.sets or max(1, -(-(1 << 30) // max(bytes_alg, 1)) + (1 if bytes_alg < (1 << 30) else 0))

    def dev_logits(a):
        if batch.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    base_d, base_t = dev_logits(batch.draft), dev_logits(batch.target)
    sets = [(base_d, base_t)]
    for s in range(1, nsets):   # extra copies so that successive calls miss the 256 MB cache
        sets.append((base_d.clone(), base_t.clone()))
    tok = torch.from_numpy(gtok if greedy else batch.draft_tokens).to(dev)
    ua = torch.from_numpy(batch.u_accept).to(dev)
    us = torch.from_numpy(batch.u_sample).to(dev)
    out = R.alloc_outputs(B, g, dev)
    ws = R.new_workspace((R.spec_greedy_workspace_bytes if greedy else R.spec_workspace_bytes)(
        B, g, V, dt_code), dev)
    stream = torch.cuda.current_stream(dev)
    sep = args.predict and args.predict_separate
    pws = R.new_workspace(R.spec_predict_workspace_bytes(B, g, V, dt_code), dev) if sep else None
    pout = R.alloc_predict_outputs(B, g, dev) if args.predict else None

    def call(i):
        nonlocal pout
        d, t = sets[i % nsets]
        if greedy:
            R.spec_verify_greedy(t, tok, out=out, workspace=ws, stream=stream)
        elif args.top_p > 0.0:
            R.spec_verify_ex(d, t, tok, ua, us, batch.T, out=out, workspace=ws, stream=stream,
                             saguaro=args.mode == "saguaro", eps=args.eps, top_p=args.top_p,
                             early=args.early)
        elif args.early:
            R.spec_verify_early(d, t, tok, ua, us, batch.T, out=out, workspace=ws, stream=stream,
                                saguaro=args.mode == "saguaro", eps=args.eps)
        elif args.predict and not sep:
            R.spec_verify_predict(d, t, tok, ua, us, batch.T, out=out, pred=pout, workspace=ws,
                                  stream=stream, saguaro=args.mode == "saguaro", eps=args.eps)
        elif args.mode == "residual":
            R.spec_verify(d, t, tok, ua, us, batch.T, out=out, workspace=ws, stream=stream)
        else:
            R.spec_verify_saguaro(d, t, tok, ua, us, batch.T, out=out, workspace=ws, stream=stream,
                                  eps=args.eps)
        if sep:
            pout = R.spec_predict_outcomes(d, out.accepted, out.tokens, out=pout, workspace=pws,
                                           stream=stream)

    gpu_clocks()   # opens the SMI handle before anything is timed
    # Untimed warm-up: W calls, then more until warmup_ms of wall time of
    # sustained work have passed (synchronising every 16 calls, so the host
    # does not queue far ahead of the GPU).
    w0 = time.perf_counter()
    nw = 0
    while nw < args.warmup or (time.perf_counter() - w0) * 1e3 < args.warmup_ms:
        call(nw)
        nw += 1
        if nw % 16 == 0:
            torch.cuda.synchronize()
    clk0 = gpu_clocks()   # read while the last warm-up calls still run
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - w0) * 1e3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        call(nw + i)
        ev[i][1].record(stream)
    t_enq = time.perf_counter()
    clk1 = gpu_clocks()   # read while the timed calls still run (they are queued)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    busy_at_clk1 = (t_enq - t_start) < wall
    if args.timeline:
        return timeline_report(args, batch, lambda: call(nw + args.steps), R)
    per_call_ms = np.array([a.elapsed_time(b) for a, b in ev])
    region_ms = ev[0][0].elapsed_time(ev[-1][1])
    ms_step = wall * 1e3 / args.steps
    ev_ms = float(per_call_ms.mean())
    acc = out.accepted.cpu().numpy()
    err_word = int(ws[:4].view(torch.int32).item())
    if args.early:   # the rows the loop reads: 2(k+1) rows before a rejection, 2 gamma + 1 after none
        rows = np.where(acc < g, 2 * (acc + 1), 2 * g + 1)
        small = R.bytes_algorithmic(B, g, V, dt_code) - (2 * g + 1) * B * V * es   # tokens, uniforms, outputs
        bytes_alg = int(rows.sum()) * V * es + small

    # Attainable read bandwidth: the same loads over the logits (both tensors).
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    read_bytes = (base_d.numel() + base_t.numel()) * es
    for _ in range(10):
        R.spec_read_bandwidth(base_d, sink, stream=stream)
        R.spec_read_bandwidth(base_t, sink, stream=stream)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nread = 20
    r0.record(stream)
    for _ in range(nread):
        R.spec_read_bandwidth(base_d, sink, stream=stream)
        R.spec_read_bandwidth(base_t, sink, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    read_gbps = read_bytes * nread / (r0.elapsed_time(r1) * 1e-3) / 1e9

    stats = {}
    if not greedy and not args.top_p:
        alpha = acceptance_statistics(base_d, base_t, batch.T, g)
        stats["tokens_per_round"] = tokens_per_round(alpha, acc)
        if args.predict and args.mode == "residual":
            stats["hit_rate"] = hit_rate_statistics(base_d, base_t, batch.T, g, alpha, pout.cand, pout.hit)
        del alpha
        torch.cuda.empty_cache()

    achieved = bytes_alg / (ev_ms * 1e-3) / 1e9
    achieved_step = bytes_alg / (ms_step * 1e-3) / 1e9
    name = ("spec_verify_greedy" if greedy else "spec_verify_early" if args.early
            else "spec_verify_ex" if args.top_p else "spec_verify_predict" if (args.predict and not sep)
            else "spec_verify_saguaro" if args.mode == "saguaro" else "spec_verify")
    result = {
        "metric": METRIC,
        "value": B * g / (ms_step * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "gamma": g, "V": V, "T": batch.T,
                   "logits": batch.dtype, "mode": args.mode, "eps": args.eps,
                   "input_sets": nsets, "alpha_target": [float(batch.alpha_target.min()),
                                                         float(batch.alpha_target.max())],
                   "mean_accepted": float(acc[acc >= 0].mean()) if (acc >= 0).any() else None,
                   "predict": ("separate" if sep else "fused") if args.predict else False,
                   "early_exit": bool(args.early), "top_p": args.top_p or None,
                   **({"hit_rate": float(pout.hit.float().mean().item())} if args.predict else {})},
        "warmup_calls": nw,
        "warmup_ms": warm_ms,
        "event_ms": {"mean": ev_ms, "p10": float(np.percentile(per_call_ms, 10)),
                     "p50": float(np.percentile(per_call_ms, 50)),
                     "p90": float(np.percentile(per_call_ms, 90)),
                     "region_per_step": region_ms / args.steps},
        # Identical readings at both points mean the SMI tables did not refresh
        # between them: then neither is the clock the timed calls ran at.
        "clocks": {"end_of_warmup": clk0, "during_timed_calls": clk1 if busy_at_clk1 else None,
                   "refreshed_between_reads": clk0 != clk1},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_record(
                         args.workload, args.mode + ("_predict" if args.predict and not sep else "")
                         + ("_early" if args.early else "") + ("_topp" if args.top_p else "")),
                     "kernel": f"one {name} call (every kernel it launches), event-timed on its stream",
                     "bytes_alg": bytes_alg,
                     "achieved_per_step": achieved_step, "frac_per_step": achieved_step / HBM_PEAK_GBPS,
                     "attainable_read": {"achieved": read_gbps, "frac": read_gbps / HBM_PEAK_GBPS,
                                         "bytes": read_bytes,
                                         "kernel": "spec_read_bandwidth over the draft and target logits"}},
        "statistics": stats,
        "error_word": err_word,
        "source_digest": source_digest(),
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
