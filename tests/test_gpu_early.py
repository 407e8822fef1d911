"""GPU parity of early-exit verification (spec_verify_early) against the fp64
oracle's loop with its break.

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


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_early_workloads(name):
    H.parity(workload(name), "residual", early=True).check()


@pytest.mark.parametrize("eps", [0.0, 1e-8])
def test_early_saguaro(eps):
    H.parity(workload("B256_g8_V152064_bf16"), "saguaro", eps, early=True).check()


def test_early_equals_full_verification_outputs():
    """On valid inputs the tokens, k and lengths equal spec_verify's; the mask
    is spec_verify's cut below k."""
    batch = workload("B128_g4_V128256_bf16")
    db = H.to_device(batch)
    e = H.run_gpu(batch, diag=False, db=db, early=True)
    f = H.run_gpu(batch, diag=False, db=db)
    for key in ("tokens", "accepted", "first_reject", "out_len"):
        np.testing.assert_array_equal(e[key], f[key], err_msg=key)
    k = f["accepted"].astype(np.uint64)
    np.testing.assert_array_equal(e["mask"], f["mask"] & ((np.uint64(1) << k) - np.uint64(1)))


@pytest.mark.parametrize("V", [50000, 50001, 2048 * 3 + 8, 7, 8, 1])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_early_ragged(V, dtype):
    batch = random_batch(6, 5, V, dtype, 0.9, seed=5200 + V % 89)
    H.parity(batch, "residual", early=True).check()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_early_bad_rows_after_the_stop(dtype):
    """NaN / +inf rows and out-of-range tokens after the first rejection do not
    invalidate a sequence here (they do in spec_verify); before it, they do.
    Forced rejections (q(x) = 0) put the stop where the test wants it; then a
    smaller call on the same workspace."""
    B, g, V = 8, 4, 30000
    rng = np.random.default_rng(17)
    d64 = np.round(rng.normal(size=(B, g + 1, V)) * 2, 2)
    t64 = d64 + 0.2 * rng.normal(size=d64.shape)
    tokens = rng.integers(0, V, size=(B, g)).astype(np.int32)
    stop = [1, 2, 0, 3, 1, 2, 4, 4]   # 4 = no forced rejection
    for b in range(B):
        if stop[b] < g:
            t64[b, stop[b], tokens[b, stop[b]]] = -np.inf
        for i in range(g):
            if i != stop[b]:
                t64[b, i] = d64[b, i]          # p == q: accepted whatever u
    t64[0, 3, 11] = np.inf                     # after the stop: ignored
    tokens[1, 3] = V                           # after the stop: ignored
    t64[4, 4, :] = -np.inf                     # target row gamma, stop at 1: ignored
    t64[5, 1, 5] = np.inf                      # before the stop (2): invalid
    t64[7, 4, :] = -np.inf                     # bonus row read (no stop): invalid
    draft, target = W.encode(d64, dtype), W.encode(t64, dtype)
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    draft[2, 2, 9] = nan                       # after the stop (0): ignored
    draft[6, 2, 9] = nan                       # no stop: invalid
    batch = W.Batch(name=f"early_bad_{dtype}", B=B, gamma=g, V=V, T=1.0, dtype=dtype, draft=draft,
                    target=target, draft_tokens=tokens,
                    u_accept=W.uniforms24(W.philox(33, 1), (B, g)),
                    u_sample=W.uniforms24(W.philox(33, 2), (B, g + 1)),
                    in_len=np.full(B, 3, np.int32))
    ref = H.run_oracle(batch, early=True)
    assert [ref[b].accepted for b in range(B)] == [1, 2, 0, 3, 1, -1, -1, -1]
    import rejection_sampling_verify_12_amd as R
    dt = R.SPEC_BF16 if dtype == "bf16" else R.SPEC_F32
    ws = R.new_workspace(R.spec_workspace_bytes(B, g, V, dt), "cuda")
    gpu = H.run_gpu(batch, early=True, ws=ws)
    H.compare(batch, gpu, ref).check()
    small = batch.subset(np.array([6, 0, 3]))
    gpu2 = H.run_gpu(small, early=True, ws=ws)
    H.compare(small, gpu2, H.run_oracle(small, early=True)).check()
