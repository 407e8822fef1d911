"""GPU parity of spec_verify_ex options: per-sequence temperatures (with every
mode: residual, Saguaro, early exit, outcome prediction) against the fp64
oracle run at each sequence's own temperature.

Every case prints its name, shapes and seed before touching the GPU.
"""
import functools

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("gpu_harness")
from test_gpu_parity import random_batch  # noqa: E402


@functools.lru_cache(maxsize=None)
def workload(name):
    H.say(f"[gen] {name}")
    return W.make_workload(name, workers=8)


def run_ex(batch, temps, mode="residual", eps=0.0, early=False, predict=False, diag=True, top_p=0.0):
    import rejection_sampling_verify_12_amd as R
    H.say(f"[options] {batch.name} B={batch.B} gamma={batch.gamma} V={batch.V} {batch.dtype} "
          f"mode={mode} eps={eps} early={early} predict={predict} top_p={top_p}")
    db = H.to_device(batch)
    dt = R.SPEC_BF16 if batch.dtype == "bf16" else R.SPEC_F32
    ws = R.new_workspace(R.spec_workspace_bytes(batch.B, batch.gamma, batch.V, dt), "cuda")
    T = temps if np.isscalar(temps) else torch.from_numpy(np.asarray(temps, np.float32)).cuda()
    pred = R.alloc_predict_outputs(batch.B, batch.gamma, "cuda") if predict else None
    res = R.spec_verify_ex(db.draft, db.target, db.tokens, db.u_accept, db.u_sample, T,
                           in_len=db.in_len, diag=diag, workspace=ws, saguaro=mode == "saguaro",
                           eps=eps, early=early, pred=pred, top_p=top_p)
    out = res[0] if predict else res
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "bounded wait timed out"
    host = {"tokens": out.tokens.cpu().numpy(), "accepted": out.accepted.cpu().numpy(),
            "first_reject": out.first_reject.cpu().numpy(),
            "mask": out.accept_mask.cpu().numpy().view(np.uint64), "out_len": out.out_len.cpu().numpy()}
    if out.diag is not None:
        host["diag"] = {k: v.cpu().numpy() for k, v in out.diag.items()}
    if predict:
        host["cand"] = pred.cand.cpu().numpy()
        host["hit"] = pred.hit.cpu().numpy()
        host["cand_idx"] = pred.cand_idx.cpu().numpy()
    return host


def oracle_per_seq(batch, temps, mode="residual", eps=0.0, early=False, top_p=1.0):
    d64, t64 = batch.draft64(), batch.target64()
    if early:
        return {b: O.verify_early_one(d64[b], t64[b], batch.draft_tokens[b], batch.u_accept[b],
                                      batch.u_sample[b], float(temps[b]), mode, eps,
                                      int(batch.in_len[b])) for b in range(batch.B)}
    return {b: O.verify_one(d64[b], t64[b], batch.draft_tokens[b], batch.u_accept[b],
                            batch.u_sample[b], float(temps[b]), mode, eps, int(batch.in_len[b]),
                            top_p=top_p) for b in range(batch.B)}


TEMPS = [0.25, 0.7, 1.0, 1.6, 3.0, 0.0, -1.0, np.nan, np.inf, 0.9, 1.2, 0.5]


@pytest.mark.parametrize("mode,eps,early", [("residual", 0.0, False), ("saguaro", 0.0, False),
                                            ("saguaro", 1e-8, False), ("residual", 0.0, True)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_per_sequence_temperature(mode, eps, early, dtype):
    batch = random_batch(len(TEMPS), 4, 50000, dtype, 1.0, seed=6100)
    temps = np.array(TEMPS, np.float32)
    gpu = run_ex(batch, temps, mode, eps, early)
    ref = oracle_per_seq(batch, temps, mode, eps, early)
    assert [ref[b].valid for b in range(batch.B)] == [bool(np.isfinite(t) and t > 0) for t in temps]
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


def test_per_sequence_temperature_with_prediction():
    batch = random_batch(len(TEMPS), 4, 50000, "bf16", 1.0, seed=6101)
    temps = np.array(TEMPS, np.float32)
    gpu = run_ex(batch, temps, predict=True)
    ref = oracle_per_seq(batch, temps)
    H.compare(batch, gpu, ref).check()
    ref_cand = O.predict_outcomes(batch.draft64())
    np.testing.assert_array_equal(gpu["cand"], ref_cand)
    hit, idx = O.predict_hits(ref_cand, gpu["accepted"], gpu["tokens"])
    np.testing.assert_array_equal(gpu["hit"], hit)
    np.testing.assert_array_equal(gpu["cand_idx"], idx)


def test_temperature_ramp_on_the_b256_workload():
    """T_b from 0.5 to 2.0 across the 256 sequences, against the oracle."""
    batch = workload("B256_g8_V152064_bf16")
    temps = np.linspace(0.5, 2.0, batch.B).astype(np.float32)
    gpu = run_ex(batch, temps)
    ref = oracle_per_seq(batch, temps)
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


def test_equal_temperatures_match_the_scalar_call():
    """A per-sequence array of the batch temperature gives the scalar call's
    outputs and diagnostics bit for bit."""
    batch = workload("B128_g4_V128256_bf16")
    a = run_ex(batch, np.full(batch.B, batch.T, np.float32))
    b = run_ex(batch, float(batch.T))
    for k in ("tokens", "accepted", "first_reject", "mask", "out_len"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    for k, v in a["diag"].items():
        np.testing.assert_array_equal(v, b["diag"][k], err_msg=k)


# --------------------------------------------------------------------------- top-p

@pytest.mark.parametrize("top_p", [0.5, 0.9, 0.99])
@pytest.mark.parametrize("mode,eps", [("residual", 0.0), ("saguaro", 0.0), ("saguaro", 1e-8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_p(top_p, mode, eps, dtype):
    batch = random_batch(10, 4, 30000, dtype, 1.0, seed=6300, scale=2.0, sigma=0.4)
    temps = np.full(batch.B, 1.0, np.float32)
    gpu = run_ex(batch, 1.0, mode, eps, top_p=top_p)
    ref = oracle_per_seq(batch, temps, mode, eps, top_p=top_p)
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_p_ties_temperatures_and_prediction(dtype):
    """Rounded logits (many equal values at the cut), per-sequence
    temperatures and outcome prediction together."""
    batch = random_batch(8, 3, 20000, dtype, 1.0, seed=6301, scale=2.0, sigma=0.3)
    d64 = np.round(batch.draft64(), 1)
    t64 = np.round(batch.target64(), 1)
    batch = W.Batch(**{**batch.__dict__, "draft": W.encode(d64, dtype), "target": W.encode(t64, dtype),
                       "draft_tokens": W.gumbel_argmax(W.decode_f64(W.encode(d64, dtype), dtype)[:, :3],
                                                       1.0, W.philox(6301, 3))})
    temps = np.array([0.5, 0.8, 1.0, 1.2, 1.5, 2.0, 0.7, 1.1], np.float32)
    gpu = run_ex(batch, temps, top_p=0.85, predict=True)
    ref = oracle_per_seq(batch, temps, top_p=0.85)
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()
    np.testing.assert_array_equal(gpu["cand"], O.predict_outcomes(batch.draft64()))


def test_top_p_one_equals_no_cut():
    batch = workload("B64_g5_V128256_bf16")
    a = run_ex(batch, float(batch.T), top_p=1.0)
    b = run_ex(batch, float(batch.T))
    for k in ("tokens", "accepted", "first_reject", "mask", "out_len"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_top_p_on_the_b256_workload():
    batch = workload("B256_g8_V152064_bf16")
    gpu = run_ex(batch, float(batch.T), top_p=0.9)
    ref = oracle_per_seq(batch, np.full(batch.B, batch.T), top_p=0.9)
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


def counted_rows_batch(V, seed):
    """bfloat16 rows for the counting top-p path: values repeated 65536 times
    or more (16-bit counters wrap), constant rows, +0 and -0 at the cut, a
    near one-hot row, scattered -inf, and invalid rows (NaN, +inf, all -inf)."""
    B, g = 10, 3
    base = random_batch(B, g, V, "bf16", 1.0, seed=seed, scale=2.0, sigma=0.4)
    d64, t64 = base.draft64().copy(), base.target64().copy()
    rng = W.philox(seed, 11)
    heavy = rng.permutation(V)[:66000]
    d64[0, :, heavy] = -3.0                  # one value 66000 times in every row
    t64[0, :, heavy[:65536]] = 0.5           # exactly 65536 times
    d64[1], t64[1] = 1.5, 1.5                # constant rows: every token ties
    zeros = rng.permutation(V)[:V // 2]
    for r in range(g + 1):                   # half the row is zero, of either sign
        d64[2, r, zeros] = np.where(np.arange(zeros.size) % 2 == 0, 0.0, -0.0)
        t64[2, r, zeros] = np.where(np.arange(zeros.size) % 3 == 0, -0.0, 0.0)
    t64[6, :, 5] = 40.0                      # near one-hot target rows
    d64[7, :, rng.permutation(V)[:V // 3]] = -np.inf
    wide = rng.permutation(V)[:V // 2]       # thousands of distinct values (the in-place finish)
    t64[7][:, wide] = np.sign(rng.standard_normal((g + 1, wide.size))) * np.exp(rng.uniform(-40, 2.5, (g + 1, wide.size)))
    d = W.encode(d64, "bf16")
    t = W.encode(t64, "bf16")
    x = W.gumbel_argmax(W.decode_f64(d, "bf16")[:, :g], 1.0, W.philox(seed, 12))
    d[3, 1, 77] = np.uint16(0x7FC0)          # NaN in draft row 1
    t[4, 0, V - 1] = np.uint16(0x7F80)       # +inf in target row 0
    t[5, 2, :] = np.uint16(0xFF80)           # target row 2 all -inf
    t[8, 1, 3] = np.uint16(0xFFC1)           # a negative NaN (key below -inf)
    t[9, 1, :100] = np.uint16(0xFF80)        # -inf, and a NaN whose key shares its counter word
    t[9, 1, 100] = np.uint16(0xFF81)
    return W.Batch(**{**base.__dict__, "draft": d, "target": t, "draft_tokens": x,
                      "name": f"counted_V{V}"})


@pytest.mark.parametrize("V", [70000, 70001])   # aligned and unaligned rows
@pytest.mark.parametrize("top_p", [0.3, 0.95])
@pytest.mark.parametrize("mode,eps", [("residual", 0.0), ("saguaro", 1e-8)])
def test_top_p_counted_rows(V, top_p, mode, eps):
    batch = counted_rows_batch(V, seed=6400 + V % 2)
    d = batch.draft.view(np.uint16)
    assert (d[2] == 0x8000).any() and (d[2] == 0).any()
    gpu = run_ex(batch, 1.0, mode, eps, top_p=top_p)
    ref = oracle_per_seq(batch, np.full(batch.B, 1.0), mode, eps, top_p=top_p)
    assert [ref[b].valid for b in range(batch.B)] == [True] * 3 + [False] * 3 + [True] * 2 + [False] * 2
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


@pytest.mark.parametrize("V", [1, 5, 9, 1000, 2049])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_p_small_vocabularies(V, dtype):
    """Rows shorter than one 8-logit unit per thread, a single token, and
    lengths that leave a partial unit."""
    batch = random_batch(6, 3, V, dtype, 1.0, seed=6500 + V, scale=2.0, sigma=0.4)
    for top_p in (0.5, 0.9):
        gpu = run_ex(batch, 1.0, top_p=top_p)
        ref = oracle_per_seq(batch, np.full(batch.B, 1.0), top_p=top_p)
        rep = H.compare(batch, gpu, ref)
        H.say(f"[options]   {rep}")
        rep.check()


@pytest.mark.parametrize("mode,eps", [("residual", 0.0), ("saguaro", 0.0), ("saguaro", 1e-8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_p_equal_one_token_nuclei(mode, eps, dtype):
    """Both rows' nuclei are the same single token and the draft tokens lie
    outside them: every position rejects with a zero residual, and the draw
    falls back to the cut target, that token (the oracle pins the closed
    form).  The GPU's fp32 residual is rounding noise here and must count as
    zero."""
    B, g, V = 8, 3, 4099
    rng = W.philox(6600, 1)
    d64 = rng.standard_normal((B, g + 1, V)) * 0.5 - 4.0
    t64 = rng.standard_normal((B, g + 1, V)) * 0.5 - 4.0
    hot = rng.integers(0, V, B)
    for b in range(B):
        d64[b, :, hot[b]] = 6.0 + 0.1 * b
        t64[b, :, hot[b]] = 5.0 + 0.2 * b
    x = np.array([[(hot[b] + 1 + i) % V for i in range(g)] for b in range(B)], np.int32)
    batch = W.Batch(name=f"onehot_{dtype}", B=B, gamma=g, V=V, T=1.0, dtype=dtype,
                    draft=W.encode(d64, dtype), target=W.encode(t64, dtype), draft_tokens=x,
                    u_accept=W.uniforms24(W.philox(6600, 2), (B, g)),
                    u_sample=W.uniforms24(W.philox(6600, 3), (B, g + 1)),
                    in_len=np.zeros(B, np.int32), seed=6600)
    gpu = run_ex(batch, 1.0, mode, eps, top_p=0.5)
    ref = oracle_per_seq(batch, np.full(B, 1.0), mode, eps, top_p=0.5)
    assert all(ref[b].accepted == 0 and ref[b].tokens[0] == hot[b] and ref[b].resid_mass == 0.0
               for b in range(B))
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()
    assert rep.excused == 0


@pytest.mark.parametrize("top_p", [1e-6, 0.99999994])   # the largest float below 1
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_p_extremes(top_p, dtype):
    """A nucleus of the top value (and its ties) alone, and one that keeps
    all but a sliver of the mass."""
    batch = random_batch(8, 4, 20000, dtype, 1.0, seed=6700, scale=2.0, sigma=0.4)
    gpu = run_ex(batch, 1.0, top_p=top_p)
    ref = oracle_per_seq(batch, np.full(batch.B, 1.0), top_p=top_p)
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_top_p_with_per_sequence_temperatures(dtype):
    """Temperatures from 0.25 to 3 and invalid ones (0, -1, NaN, +inf: only
    their sequence is invalid) under a top-p cut."""
    batch = random_batch(len(TEMPS), 4, 50000, dtype, 1.0, seed=6701)
    temps = np.array(TEMPS, np.float32)
    gpu = run_ex(batch, temps, top_p=0.8)
    ref = oracle_per_seq(batch, temps, top_p=0.8)
    assert [ref[b].valid for b in range(batch.B)] == [bool(np.isfinite(t) and t > 0) for t in temps]
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


@pytest.mark.parametrize("V", [1 << 24, (1 << 24) + 8])
def test_top_p_longest_rows(V):
    """bfloat16 rows at the counting path's longest (2^24 logits: its hot
    values occur well over 65536 times, so the counters wrap) and just past
    it (the radix selection takes over)."""
    batch = random_batch(1, 1, V, "bf16", 1.0, seed=6800 + V % 7, scale=2.0, sigma=0.4)
    d, t = batch.draft.copy(), batch.target.copy()
    d[..., ::50] = np.uint16(0xBF80)   # -1.0, 335545 times a row
    t[..., ::40] = np.uint16(0xBFC0)   # -1.5
    batch = W.Batch(**{**batch.__dict__, "draft": d, "target": t, "name": f"long_V{V}"})
    gpu = run_ex(batch, 1.0, top_p=0.9)
    ref = oracle_per_seq(batch, np.full(batch.B, 1.0), top_p=0.9)
    rep = H.compare(batch, gpu, ref)
    H.say(f"[options]   {rep}")
    rep.check()


@pytest.mark.parametrize("V", [1 << 21, (1 << 21) + 8])
def test_top_p_band_limits(V):
    """bfloat16 rows at the longest the counting path takes with its band of
    per-lane copies (2^21 logits) and just past it (no band).  In the draft
    rows one value fills every other logit, so it is the rows' median and
    falls in the band, whose copies then sum past a 16-bit counter; in the
    target rows one value fills every 16th logit, away from the median."""
    batch = random_batch(1, 1, V, "bf16", 1.0, seed=6900 + V % 7, scale=2.0, sigma=0.4)
    d, t = batch.draft.copy(), batch.target.copy()
    d[..., ::2] = np.uint16(0xBF80)    # -1.0, 2^20 times a row
    t[..., ::16] = np.uint16(0xC040)   # -3.0, 2^17 times a row
    batch = W.Batch(**{**batch.__dict__, "draft": d, "target": t, "name": f"band_V{V}"})
    for top_p in (0.3, 0.9):
        gpu = run_ex(batch, 1.0, top_p=top_p)
        ref = oracle_per_seq(batch, np.full(batch.B, 1.0), top_p=top_p)
        rep = H.compare(batch, gpu, ref)
        H.say(f"[options]   {rep}")
        rep.check()


@pytest.mark.parametrize("V", [40000, 40003])   # the band (16-byte rows) and without it
@pytest.mark.parametrize("mu,sd,T", [(-8.0, 2.0, 0.7), (0.0, 0.5, 1.3), (3.0, 6.0, 1.0), (-1.0, 12.0, 0.8)])
def test_top_p_row_shapes(V, mu, sd, T):
    """bfloat16 rows whose logits centre on different values with different
    spreads, so the counting kernel's band lands on negative values, on
    both sides of zero (moved to one side) and on positive ones, and a wide
    spread leaves most logits outside it."""
    B, g = 4, 2
    rng = W.philox(7200 + int(10 * sd), 1)
    d64 = mu + sd * rng.standard_normal((B, g + 1, V))
    t64 = d64 + 0.4 * rng.standard_normal((B, g + 1, V))
    base = random_batch(B, g, 8, "bf16", T, seed=7201)
    d, t = W.encode(d64, "bf16"), W.encode(t64, "bf16")
    x = W.gumbel_argmax(W.decode_f64(d, "bf16")[:, :g], T, W.philox(7202, 2))
    batch = W.Batch(**{**base.__dict__, "V": V, "T": T, "draft": d, "target": t, "draft_tokens": x,
                       "name": f"shape_mu{mu}_sd{sd}_V{V}"})
    for top_p in (0.5, 0.95):
        gpu = run_ex(batch, T, top_p=top_p)
        ref = oracle_per_seq(batch, np.full(batch.B, T), top_p=top_p)
        rep = H.compare(batch, gpu, ref)
        H.say(f"[options]   {rep}")
        rep.check()


@pytest.mark.parametrize("kind", ["near", "past"])
def test_top_p_list_capacity(kind):
    """bfloat16 rows of V = 152064 whose distinct raw words (a value and its
    negation share one) come near the counting kernel's list of 1792 words
    (Gaussian logits, ~1550) or pass it (magnitudes over 11 binades, ~2000:
    the redo kernel finishes those rows)."""
    B, g, V = 2, 2, 152064
    batch = random_batch(B, g, V, "bf16", 1.0, seed=7100, scale=3.0, sigma=0.5)
    if kind == "past":
        rng = W.philox(7101, 1)
        mag = np.exp(rng.uniform(-8.0, 3.0, (B, g + 1, V)))
        d64 = np.sign(rng.standard_normal((B, g + 1, V))) * mag
        t64 = d64 * np.exp(0.1 * rng.standard_normal((B, g + 1, V)))
        d, t = W.encode(d64, "bf16"), W.encode(t64, "bf16")
        x = W.gumbel_argmax(W.decode_f64(d, "bf16")[:, :g], 1.0, W.philox(7101, 2))
        batch = W.Batch(**{**batch.__dict__, "draft": d, "target": t, "draft_tokens": x,
                           "name": f"list_past_V{V}"})
    words = [len(np.unique(r.view(np.uint16) & 0x7FFF)) for r in batch.draft.reshape(-1, V)]
    assert all(1000 < w <= 1792 for w in words) if kind == "near" else all(w > 1792 for w in words), words
    for top_p in (0.5, 0.95):
        gpu = run_ex(batch, 1.0, top_p=top_p)
        ref = oracle_per_seq(batch, np.full(batch.B, 1.0), top_p=top_p)
        rep = H.compare(batch, gpu, ref)
        H.say(f"[options]   {rep}")
        rep.check()


@pytest.mark.parametrize("V", [2, 8, 33])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,eps", [("residual", 0.0), ("saguaro", 1e-8)])
def test_top_p_small_peaked_rows(V, dtype, mode, eps):
    """Few tokens with one dominant under a cut: one-token nuclei, zero and
    small residuals."""
    batch = random_batch(24, 4, V, dtype, 1.0, seed=7400 + V, scale=6.0, sigma=0.3)
    for top_p in (0.3, 0.7):
        gpu = run_ex(batch, 1.0, mode, eps, top_p=top_p)
        ref = oracle_per_seq(batch, np.full(batch.B, 1.0), mode, eps, top_p=top_p)
        rep = H.compare(batch, gpu, ref)
        H.say(f"[options]   {rep}")
        rep.check()
