"""The checks build (SV_CHECKS=1): every index a kernel forms is tested against
its array's size, and a failed test records its site in the workspace's
second word (and clamps the index) instead of trapping.

Each case runs a call with the default library and with the checks build on
the same inputs and workspace layout: the check word must stay zero, the
error word too (but where the test sets it on purpose, as after a wait that
gave up), and the outputs and the workspaces the two builds leave must be
identical.  Cases cover
the short-call and long-call schedules, ragged vocabularies, both dtypes,
the refined residual draw, top-p (radix selection, counting and its redo
list), early exit, prediction, per-sequence temperatures and greedy.

Every case prints its name before touching the GPU.
"""
import functools

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("gpu_harness")


@pytest.fixture(scope="module")
def libs():
    """(default, checks) libraries; the default one is restored afterwards."""
    import rejection_sampling_verify_12_amd as R
    from rejection_sampling_verify_12_amd import build as BLD
    default = R.load_library()
    R._lib = None
    try:
        checks = R.load_library(BLD.CHECKS_LIB)
    finally:
        R._lib = default
    assert checks.spec_checks_build() == 1
    assert not hasattr(default, "spec_checks_build")
    yield default, checks
    R._lib = default


def _with(lib, fn):
    import rejection_sampling_verify_12_amd as R
    old = R._lib
    R._lib = lib
    try:
        return fn()
    finally:
        torch.cuda.synchronize()
        R._lib = old


def _words(ws):
    torch.cuda.synchronize()
    w = ws[:8].view(torch.int32).cpu().numpy()
    return int(w[0]), int(w[1])


def _site(word):
    return f"file {word >> 16}, line {word & 0xFFFF}"


def _host(o):
    if o is None:
        return None
    if hasattr(o, "_asdict"):
        return {k: _host(v) for k, v in o._asdict().items()}
    if isinstance(o, dict):
        return {k: _host(v) for k, v in o.items()}
    return o.cpu().numpy()


def _equal(a, b, path=""):
    if isinstance(a, dict):
        assert a.keys() == b.keys(), path
        for k in a:
            _equal(a[k], b[k], f"{path}.{k}")
    elif a is None:
        assert b is None, path
    else:
        np.testing.assert_array_equal(a, b, err_msg=path)


@functools.lru_cache(maxsize=None)
def _batch(kind):
    from test_gpu_parity import random_batch
    if kind in ("B64_g5_V128256_bf16", "B256_g8_V152064_bf16"):
        return W.make_workload(kind)
    if kind == "counted_rows":
        from test_gpu_options import counted_rows_batch
        return counted_rows_batch(70000, 8801)
    B, g, V, dt, seed, scale, sigma = {
        "tiny": (3, 2, 7, "bf16", 8803, 3.0, 0.7),
        "ragged_bf16": (17, 4, 2048 * 3 + 5, "bf16", 8805, 3.0, 0.7),
        "ragged_f32": (9, 3, 30001, "f32", 8807, 3.0, 0.7),
        "peaked_bf16": (24, 4, 64, "bf16", 8809, 6.0, 0.3),   # small residual masses: refined draws
        "peaked_f32": (24, 4, 5000, "f32", 8811, 6.0, 0.3),
    }[kind]
    return random_batch(B, g, V, dt, 1.0, seed=seed, scale=scale, sigma=sigma)


def _verify(batch, db, mode, ws):
    import rejection_sampling_verify_12_amd as R
    args = (db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T)
    kw = dict(in_len=db.in_len, workspace=ws)
    if mode == "residual":
        return R.spec_verify(*args, diag=True, **kw)
    if mode == "saguaro":
        return R.spec_verify_saguaro(*args, diag=True, eps=0.0, **kw)
    if mode == "saguaro_eps":
        return R.spec_verify_saguaro(*args, diag=True, eps=1e-8, **kw)
    if mode == "early":
        return R.spec_verify_early(*args, diag=True, **kw)
    if mode == "early_saguaro":
        return R.spec_verify_early(*args, diag=True, saguaro=True, eps=1e-8, **kw)
    if mode in ("topp", "topp_low"):
        return R.spec_verify_ex(*args, diag=True, top_p=0.9 if mode == "topp" else 0.3, **kw)
    if mode == "temps":
        temps = torch.linspace(0.5, 1.5, batch.B, device="cuda")
        return R.spec_verify_ex(db.draft, db.target, db.tokens, db.u_accept, db.u_sample, temps, diag=True, **kw)
    if mode == "predict":
        out, pred = R.spec_verify_predict(*args, diag=True, **kw)
        return {"out": out, "pred": pred}
    if mode == "greedy":
        return R.spec_verify_greedy(db.target, db.tokens, in_len=db.in_len, workspace=ws)
    raise ValueError(mode)


def _workspace(batch, mode):
    import rejection_sampling_verify_12_amd as R
    dt = R.SPEC_BF16 if batch.dtype == "bf16" else R.SPEC_F32
    if mode == "greedy":
        n = R.spec_greedy_workspace_bytes(batch.B, batch.gamma, batch.V, dt)
    else:
        n = R.spec_workspace_bytes(batch.B, batch.gamma, batch.V, dt)
    return R.new_workspace(n, "cuda")


MODES = ["residual", "saguaro", "saguaro_eps", "early", "early_saguaro", "topp", "temps", "predict",
         "greedy"]
KINDS = ["tiny", "ragged_bf16", "ragged_f32", "peaked_bf16", "peaked_f32", "B64_g5_V128256_bf16",
         "B256_g8_V152064_bf16"]


def _run_both(libs, batch, mode):
    db = H.to_device(batch)
    ws_d, ws_c = _workspace(batch, mode), _workspace(batch, mode)
    ref = _host(_with(libs[0], lambda: _verify(batch, db, mode, ws_d)))
    got = _host(_with(libs[1], lambda: _verify(batch, db, mode, ws_c)))
    err, chk = _words(ws_c)
    assert chk == 0, f"a check failed at {_site(chk)}"
    assert err == 0, "bounded wait timed out"
    assert _words(ws_d) == (0, 0)
    # Both builds leave the same workspace (all zero but for the top-p rows'
    # statistics and the prediction's lane leaders, which each such call
    # rewrites before reading).
    assert torch.equal(ws_c, ws_d), "the builds leave different workspaces"
    _equal(got, ref)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kind", KINDS)
def test_checks_build_matches_the_default_build(libs, kind, mode):
    batch = _batch(kind)
    H.say(f"[checks] {batch.name} {mode}")
    _run_both(libs, batch, mode)


@pytest.mark.parametrize("mode", ["topp", "topp_low"])
def test_checks_build_on_counted_top_p_rows(libs, mode):
    """Repeated values that wrap the counters: rows go to the redo list."""
    batch = _batch("counted_rows")
    H.say(f"[checks] counted rows V={batch.V} {mode}")
    _run_both(libs, batch, mode)


@pytest.mark.parametrize("mode", ["residual", "early", "saguaro_eps", "predict", "greedy"])
def test_checks_build_after_a_wait_gave_up(libs, mode):
    """The error word set before the call, as after a bounded wait that gave
    up: every wait gives up, no index is taken from a word that never
    arrived (the check word stays zero), and every sequence is invalid."""
    from test_gpu_parity import random_batch
    batch = random_batch(16, 4, 40000, "bf16", 1.0, seed=8813)
    H.say(f"[checks] give-up {mode} B={batch.B} gamma={batch.gamma} V={batch.V}")
    db = H.to_device(batch)
    ws = _workspace(batch, mode)
    ws[:4].view(torch.int32).fill_(1)
    out = _with(libs[1], lambda: _verify(batch, db, mode, ws))
    out = out["out"] if isinstance(out, dict) else out
    err, chk = _words(ws)
    assert chk == 0, f"a check failed at {_site(chk)}"
    assert err == 1
    assert (out.accepted.cpu().numpy() == -1).all()
    assert (out.tokens.cpu().numpy() == -1).all()
