"""Every entry point writes only inside its outputs and workspace.

Each output array and workspace is placed in the middle of a larger device
buffer whose margins (4 KiB on each side) hold a byte pattern; after the call
the margins must still hold it, the inputs must equal copies taken before the
call, the workspace's error word must be clear (and the workspace all zero,
but after a top-p cut or outcome prediction, whose rows' statistics and lane
leaders stay until the next such call), and
the outputs must equal those of the same call on plainly allocated buffers.
Cases cover the short-call and long-call schedules, ragged vocabularies, both
dtypes and every mode and option.

Every case prints its name before touching the GPU.
"""
import functools
import math

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("gpu_harness")

MARGIN = 4096     # bytes of pattern on each side of a buffer
PATTERN = 0xA5


class Guarded:
    """Buffers carved from the middle of pattern-filled allocations."""

    def __init__(self):
        self.bufs = []

    def new(self, shape, dtype, fill=None):
        n = math.prod(shape)
        es = torch.empty((), dtype=dtype).element_size()
        g = MARGIN // es
        raw = torch.empty(n + 2 * g, dtype=dtype, device="cuda")
        raw.view(torch.uint8).fill_(PATTERN)
        view = raw[g:g + n].view(shape)
        if fill is not None:
            view.fill_(fill)
        self.bufs.append((raw, g, n, es))
        return view

    def check(self):
        torch.cuda.synchronize()
        for i, (raw, g, n, es) in enumerate(self.bufs):
            b = raw.view(torch.uint8)
            head, tail = b[:g * es], b[(g + n) * es:]
            assert bool((head == PATTERN).all()), f"buffer {i}: write before its start"
            assert bool((tail == PATTERN).all()), f"buffer {i}: write past its end"

    def workspace(self, nbytes):
        return self.new((max(int(nbytes), 1),), torch.uint8, fill=0)

    def verify_outputs(self, R, B, gamma, diag=False):
        d = None
        if diag:
            r = 2 * gamma + 1
            shapes = dict(row_max=(B, r), row_logZ=(B, r), px=(B, gamma), qx=(B, gamma),
                          resid_mass=(B,), token_prob=(B,), cdf_lo=(B,), cdf_hi=(B,))
            d = {k: self.new(shapes[k], torch.float64, fill=float("nan")) for k in R.DIAG_FIELDS}
        return R.VerifyOut(self.new((B, gamma + 1), torch.int32), self.new((B,), torch.int32),
                           self.new((B,), torch.int32), self.new((B,), torch.int64),
                           self.new((B,), torch.int32), d)


def _inputs_unchanged(db, snap):
    torch.cuda.synchronize()
    for k, v in snap.items():
        assert torch.equal(getattr(db, k), v), f"input {k} changed"


def _same(a, b):
    for k in ("tokens", "accepted", "first_reject", "accept_mask", "out_len"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    if a.diag is not None:
        for k in a.diag:
            np.testing.assert_array_equal(a.diag[k].cpu().numpy(), b.diag[k].cpu().numpy(), err_msg=k)


def _ws_clear(ws, zeroed=True):
    """The error word clear and (but after a top-p cut or outcome prediction,
    whose rows' statistics and lane leaders stay in the workspace until the
    next such call rewrites them) all zero."""
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "bounded wait timed out"
    if zeroed:
        assert int(ws.to(torch.int64).sum().item()) == 0, "workspace not left zeroed"


@functools.lru_cache(maxsize=None)
def _batch(kind):
    if kind == "B64_g5_V128256_bf16":
        return W.make_workload(kind)
    if kind == "B256_g8_V152064_bf16":
        return W.make_workload(kind)
    B, g, V, dt, seed = {"ragged_bf16": (17, 4, 2048 * 3 + 5, "bf16", 4401),
                         "ragged_f32": (9, 3, 30001, "f32", 4403),
                         "tiny": (3, 2, 7, "bf16", 4405)}[kind]
    from test_gpu_parity import random_batch
    return random_batch(B, g, V, dt, 1.0, seed=seed)


MODES = ["residual", "saguaro", "early", "topp", "temps", "predict", "noalloc"]
KINDS = ["tiny", "ragged_bf16", "ragged_f32", "B64_g5_V128256_bf16", "B256_g8_V152064_bf16"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kind", KINDS)
def test_verification_writes_stay_in_bounds(kind, mode):
    import rejection_sampling_verify_12_amd as R
    if mode == "noalloc" and kind == "B256_g8_V152064_bf16":
        pytest.skip("above the static scratch's batch limit")
    batch = _batch(kind)
    H.say(f"[guards] {batch.name} {mode}")
    db = H.to_device(batch)
    snap = {k: getattr(db, k).clone() for k in ("draft", "target", "tokens", "u_accept", "u_sample", "in_len")}
    dt = R.SPEC_BF16 if batch.dtype == "bf16" else R.SPEC_F32
    B, g, V = batch.B, batch.gamma, batch.V
    G = Guarded()
    diag = mode in ("residual", "saguaro", "early")
    out = G.verify_outputs(R, B, g, diag=diag)
    ws = G.workspace(R.spec_workspace_bytes(B, g, V, dt))
    args = (db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T)
    kw = dict(in_len=db.in_len)
    extra = {}
    if mode == "residual":
        call = lambda **k: R.spec_verify(*args, **kw, **k)
    elif mode == "saguaro":
        call = lambda **k: R.spec_verify_saguaro(*args, **kw, eps=1e-8, **k)
    elif mode == "early":
        call = lambda **k: R.spec_verify_early(*args, **kw, **k)
    elif mode == "topp":
        call = lambda **k: R.spec_verify_ex(*args, **kw, top_p=0.9, **k)
    elif mode == "temps":
        temps = G.new((B,), torch.float32)
        temps.copy_(torch.linspace(0.5, 1.5, B, device="cuda"))
        call = lambda **k: R.spec_verify_ex(db.draft, db.target, db.tokens, db.u_accept, db.u_sample,
                                            temps, **kw, **k)
    elif mode == "predict":
        pred = R.PredictOut(G.new((B, g + 1, 3), torch.int32), G.new((B,), torch.int32),
                            G.new((B,), torch.int32))
        extra["pred"] = pred
        call = lambda **k: R.spec_verify_predict(*args, **kw, **k)[0]
    else:
        call = lambda **k: R.spec_verify_noalloc(*args, **kw, **{x: y for x, y in k.items() if x != "workspace"})
    if mode == "predict":
        got = call(out=out, pred=extra["pred"], workspace=ws)
        ref_pred = R.alloc_predict_outputs(B, g, "cuda")
        ref = call(pred=ref_pred)
        for k in ("cand", "hit", "cand_idx"):
            assert torch.equal(getattr(extra["pred"], k), getattr(ref_pred, k)), k
    else:
        got = call(out=out, workspace=ws)
        ref = call(diag=diag) if mode != "temps" else call()
    G.check()
    _inputs_unchanged(db, snap)
    _ws_clear(ws, zeroed=mode not in ("topp", "predict"))
    _same(got, ref)


@pytest.mark.parametrize("kind", ["tiny", "ragged_bf16", "ragged_f32", "B64_g5_V128256_bf16"])
def test_greedy_and_prediction_writes_stay_in_bounds(kind):
    import rejection_sampling_verify_12_amd as R
    batch = _batch(kind)
    H.say(f"[guards] {batch.name} greedy and outcome prediction")
    db = H.to_device(batch)
    snap = {k: getattr(db, k).clone() for k in ("draft", "target", "tokens", "in_len")}
    dt = R.SPEC_BF16 if batch.dtype == "bf16" else R.SPEC_F32
    B, g, V = batch.B, batch.gamma, batch.V
    G = Guarded()
    out = G.verify_outputs(R, B, g)
    ws = G.workspace(R.spec_greedy_workspace_bytes(B, g, V, dt))
    got = R.spec_verify_greedy(db.target, db.tokens, in_len=db.in_len, out=out, workspace=ws)
    ref = R.spec_verify_greedy(db.target, db.tokens, in_len=db.in_len)
    pout = R.PredictOut(G.new((B, g + 1, 3), torch.int32), G.new((B,), torch.int32), G.new((B,), torch.int32))
    pws = G.workspace(R.spec_predict_workspace_bytes(B, g, V, dt))
    R.spec_predict_outcomes(db.draft, ref.accepted, ref.tokens, out=pout, workspace=pws)
    pref = R.spec_predict_outcomes(db.draft, ref.accepted, ref.tokens)
    G.check()
    _inputs_unchanged(db, snap)
    _ws_clear(ws)   # the prediction's workspace has no error word and keeps its records
    _same(got, ref)
    for k in ("cand", "hit", "cand_idx"):
        assert torch.equal(getattr(pout, k), getattr(pref, k)), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bigram_model_writes_stay_in_bounds(dtype):
    """The synthetic draft chain, target rows, pre-speculation and advance."""
    import rejection_sampling_verify_12_amd as R
    B, g, V, Hr = 6, 4, 3001, 97
    s = W.bigram_setup(B, g, V, 1.0, 2, 4411, dtype=dtype, H=Hr)
    H.say(f"[guards] bigram models B={B} gamma={g} V={V} H={Hr} {dtype}")
    tab = lambda a: H.logits_to_device(a, dtype)
    dtab, ttab = tab(s.draft_table), tab(s.target_table)
    noise = torch.from_numpy(np.ascontiguousarray(s.noise, dtype=np.float32)).cuda()
    last = torch.from_numpy(np.ascontiguousarray(s.last0, dtype=np.int32)).cuda()
    length = torch.from_numpy(np.ascontiguousarray(s.len0, dtype=np.int32)).cuda()
    G = Guarded()
    x = R.spec_synth_draft(dtab, noise, g, last, length, out=G.new((B, g), torch.int32))
    x_ref = R.spec_synth_draft(dtab, noise, g, last, length)
    rows = R.spec_synth_rows(ttab, last, x, out=G.new((B, g + 1, V), ttab.dtype))
    rows_ref = R.spec_synth_rows(ttab, last, x_ref)
    cand = R.spec_predict_outcomes(rows_ref).cand
    prep = R.spec_ssd_prespeculate(dtab, noise, cand, length, out=G.new((B, 3 * (g + 1), g), torch.int32))
    prep_ref = R.spec_ssd_prespeculate(dtab, noise, cand, length)
    vout = R.VerifyOut(G.new((B, g + 1), torch.int32, fill=-1), G.new((B,), torch.int32, fill=0),
                       None, None, G.new((B,), torch.int32), None)
    vout.tokens[:, 0] = last
    vout.out_len.copy_(length + 1)
    adv = R.spec_ssd_advance(dtab, noise, vout, out=(G.new((B,), torch.int32), G.new((B,), torch.int32),
                                                      G.new((B, g), torch.int32)))
    adv_ref = R.spec_ssd_advance(dtab, noise, vout)
    G.check()
    assert torch.equal(x, x_ref) and torch.equal(rows, rows_ref) and torch.equal(prep, prep_ref)
    for a, b in zip(adv, adv_ref):
        assert torch.equal(a, b)
