"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case prints its name, shapes and seed before touching the GPU.
"""
import dataclasses
import functools

import numpy as np
import pytest
import scipy.stats

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("gpu_harness")


@functools.lru_cache(maxsize=None)
def workload(name):
    H.say(f"[gen] {name}")
    return W.make_workload(name)


def random_batch(B, gamma, V, dtype, T, seed, scale=3.0, sigma=0.7):
    """Gaussian logits (draft) and a noisy copy (target); tokens ~ p by Gumbel-max."""
    rng = W.philox(seed, 7)
    d64 = rng.standard_normal((B, gamma + 1, V)) * scale
    t64 = d64 + sigma * rng.standard_normal((B, gamma + 1, V))
    draft, target = W.encode(d64, dtype), W.encode(t64, dtype)
    tokens = W.gumbel_argmax(W.decode_f64(draft, dtype)[:, :gamma], T, W.philox(seed, 8))
    return W.Batch(name=f"rand_B{B}_g{gamma}_V{V}_{dtype}", B=B, gamma=gamma, V=V, T=T,
                   dtype=dtype, draft=draft, target=target, draft_tokens=tokens,
                   u_accept=W.uniforms24(W.philox(seed, 9), (B, gamma)),
                   u_sample=W.uniforms24(W.philox(seed, 10), (B, gamma + 1)),
                   in_len=np.arange(B, dtype=np.int32) * 3, seed=seed)


# --------------------------------------------------------------------------- configured workloads

@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_residual(name):
    rep = H.parity(workload(name), "residual")
    rep.check()


@pytest.mark.parametrize("eps", [0.0, 1e-8])
def test_workload_saguaro(eps):
    rep = H.parity(workload("B256_g8_V152064_bf16"), "saguaro", eps)
    rep.check()


def test_alpha_spread_realised():
    """The B=256 workload's realised acceptance tracks its alpha ramp."""
    batch = workload("B256_g8_V152064_bf16")
    gpu = H.run_gpu(batch, diag=True)
    px, qx = gpu["diag"]["px"], gpu["diag"]["qx"]
    acc = np.minimum(1.0, qx / px).mean(1)   # E[accept | x] averaged over positions
    lo, hi = acc[:64].mean(), acc[-64:].mean()
    H.say(f"[alpha] mean a first quarter {lo:.3f} last quarter {hi:.3f}")
    assert hi > lo + 0.2


# --------------------------------------------------------------------------- toy (V = 7)

def test_toy_generation_64_tokens():
    """A 64-token toy generation, one B=1 call per round, GPU and oracle in lockstep."""
    out_g, out_o, prev, rnd = [0], [0], 0, 0
    while len(out_g) < 64:
        batch = W.toy_batch([prev], seed=1201, round_index=rnd)
        gpu = H.run_gpu(batch, diag=False)
        ref = H.run_oracle(batch)
        rep = H.compare(batch, gpu, ref, check_diag=False)
        assert rep.excused == 0
        rep.check()
        k = int(gpu["accepted"][0])
        out_g += gpu["tokens"][0][: k + 1].tolist()
        out_o += ref[0].tokens[: k + 1].tolist()
        prev = out_g[-1]
        rnd += 1
    assert out_g == out_o
    H.say(f"[toy64] rounds={rnd} tokens={out_g[:64]}")


def test_toy_200k_rounds():
    """200k independent toy rounds in one call: oracle parity on a slice, and the
    output law equals the target tables (speculative-decoding blog, section 3)."""
    n = 200_000
    prev = np.arange(n) % 2
    batch = W.toy_batch(prev, seed=1201)
    gpu = H.run_gpu(batch, diag=False)
    ref = H.run_oracle(batch, seqs=range(20_000))
    rep = H.compare(batch, gpu, ref, check_diag=False)
    H.say(f"[toy200k] {rep}")
    rep.check()
    trans = np.zeros((2, 7))
    for b in range(n):
        k = int(gpu["accepted"][b])
        seq = [int(prev[b])] + gpu["tokens"][b][: k + 1].tolist()
        for u, v in zip(seq[:-1], seq[1:]):
            trans[int(u != 0), v] += 1
    for s in (0, 1):
        exp = W.TOY_TARGET[s] * trans[s].sum()
        p = scipy.stats.chisquare(trans[s], exp).pvalue
        H.say(f"[toy200k] state {s} chi2 p={p:.3g} max dev "
              f"{np.abs(trans[s] / trans[s].sum() - W.TOY_TARGET[s]).max():.4f}")
        assert p > 1e-3


# --------------------------------------------------------------------------- shapes and edges

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,gamma,B", [(1, 3, 4), (5, 2, 9), (7, 4, 33), (2048 * 3 + 5, 3, 17),
                                      (16384 * 2 + 8, 2, 5), (4096, 63, 3), (50000, 1, 7),
                                      (65536, 6, 12)])
def test_shapes(dtype, V, gamma, B):
    batch = random_batch(B, gamma, V, dtype, 1.0, seed=V + gamma)
    H.parity(batch, "residual").check()
    H.parity(batch, "saguaro", 0.0).check()


@pytest.mark.parametrize("T", [0.25, 0.8, 2.0])
def test_temperatures(T):
    batch = random_batch(16, 4, 20000, "bf16", T, seed=77)
    H.parity(batch, "residual").check()


def test_forced_paths():
    """u = 0 accepts everything (bonus path); p == q accepts everything; q(x) = 0
    forces the rejection at a chosen position; p(x) = 0 with q(x) > 0 accepts."""
    B, g, V = 8, 5, 3000
    base = random_batch(B, g, V, "f32", 1.0, seed=5)
    b1 = W.Batch(**{**base.__dict__, "u_accept": np.zeros((B, g), np.float32), "name": "u0"})
    H.parity(b1, "residual").check()
    assert (H.run_gpu(b1, diag=False)["accepted"] == g).all()
    b2 = W.Batch(**{**base.__dict__, "target": base.draft.copy(), "name": "p_eq_q",
                    "u_accept": np.full((B, g), 1 - 2 ** -24, np.float32)})
    H.parity(b2, "residual").check()
    assert (H.run_gpu(b2, diag=False)["accepted"] == g).all()
    t3 = base.target.copy()
    for b in range(B):
        t3[b, b % g, base.draft_tokens[b, b % g]] = -np.inf
    b3 = W.Batch(**{**base.__dict__, "target": t3, "u_accept": np.zeros((B, g), np.float32),
                    "name": "q0"})
    H.parity(b3, "residual").check()
    gk = H.run_gpu(b3, diag=False)["accepted"]
    assert gk.tolist() == [b % g for b in range(B)]
    d4 = base.draft.copy()
    for b in range(B):
        d4[b, 0, base.draft_tokens[b, 0]] = -np.inf
    b4 = W.Batch(**{**base.__dict__, "draft": d4, "name": "p0"})
    H.parity(b4, "residual").check()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_invalid_sequences(dtype):
    B, g, V = 10, 3, 5000
    base = random_batch(B, g, V, dtype, 1.0, seed=6)
    d, t, x = base.draft.copy(), base.target.copy(), base.draft_tokens.copy()
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    inf = np.uint16(0x7F80) if dtype == "bf16" else np.float32(np.inf)
    ninf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    t[1, g, 17] = nan            # bonus row
    d[2, 0, 4999] = inf          # draft row 0
    t[3, 1, :] = ninf            # target row 1 all -inf
    x[4, 2] = V                  # token out of range
    x[5, 0] = -1
    d[6, g, 3] = nan             # draft row gamma: not read by the rule -> valid
    bad = W.Batch(**{**base.__dict__, "draft": d, "target": t, "draft_tokens": x, "name": "bad"})
    rep = H.parity(bad, "residual")
    rep.check()
    gpu = H.run_gpu(bad, diag=False)
    assert gpu["accepted"][[1, 2, 3, 4, 5]].tolist() == [-1] * 5
    assert gpu["accepted"][6] >= 0


def test_empty_batch_is_noop():
    import rejection_sampling_verify_12_amd as R
    z = torch.zeros((0, 5, 100), dtype=torch.bfloat16, device="cuda")
    i = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    u = torch.zeros((0, 4), dtype=torch.float32, device="cuda")
    us = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
    out = R.spec_verify(z, z, i, u, us, 1.0)
    assert out.tokens.shape == (0, 5)


@pytest.mark.parametrize("name", ["B64_g5_V128256_bf16", "B256_g8_V152064_bf16"])
def test_deterministic_replay(name):
    """Identical inputs give bit-identical outputs (including diagnostics) over
    100 replays."""
    batch = workload(name)
    H.say(f"[replay] {name} x100")
    db = H.to_device(batch)
    first = H.run_gpu(batch, db=db)
    for _ in range(100):
        again = H.run_gpu(batch, db=db)
        for k in ("tokens", "accepted", "mask", "out_len"):
            assert np.array_equal(first[k], again[k])
        for k, v in first["diag"].items():
            assert np.array_equal(v, again["diag"][k], equal_nan=True), k


def test_concurrent_calls_on_two_streams():
    """Calls on two streams with their own workspaces, launched back to back
    (a bf16 batch and a float32 one, several times each, no synchronisation
    in between), give the outputs the same calls give one at a time."""
    import rejection_sampling_verify_12_amd as R
    batches = [workload("B64_g5_V128256_bf16"), random_batch(9, 4, 30001, "f32", 0.9, seed=4321)]
    dbs = [H.to_device(b) for b in batches]
    dts = [R.SPEC_BF16, R.SPEC_F32]
    ws = [R.new_workspace(R.spec_workspace_bytes(b.B, b.gamma, b.V, dt), "cuda") for b, dt in zip(batches, dts)]
    alone = [H.run_gpu(b, db=db, diag=False) for b, db in zip(batches, dbs)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = [[], []]
    for _ in range(4):
        for i in (0, 1):
            b, db = batches[i], dbs[i]
            with torch.cuda.stream(streams[i]):
                outs[i].append(R.spec_verify(db.draft, db.target, db.tokens, db.u_accept, db.u_sample,
                                             b.T, in_len=db.in_len, workspace=ws[i], stream=streams[i]))
    torch.cuda.synchronize()
    for i in (0, 1):
        assert int(ws[i][:4].view(torch.int32).item()) == 0, "bounded wait timed out"
        for o in outs[i]:
            np.testing.assert_array_equal(o.tokens.cpu().numpy(), alone[i]["tokens"])
            np.testing.assert_array_equal(o.accepted.cpu().numpy(), alone[i]["accepted"])
            np.testing.assert_array_equal(o.out_len.cpu().numpy(), alone[i]["out_len"])


def test_calls_from_four_host_threads():
    """Four host threads, each with its own stream and workspace, call the
    library at once (ctypes releases the interpreter lock during a call):
    the plain rule in bf16 and float32, Saguaro with eps, and early exit.
    Every call's outputs equal the same call made alone."""
    import threading

    import rejection_sampling_verify_12_amd as R
    cases = [("residual", workload("B64_g5_V128256_bf16")),
             ("residual", random_batch(9, 4, 30001, "f32", 0.9, seed=4341)),
             ("saguaro", random_batch(12, 3, 20000, "bf16", 1.0, seed=4343)),
             ("early", random_batch(16, 5, 40000, "bf16", 0.8, seed=4347))]
    H.say("[threads] four host threads, eight calls each")
    dbs = [H.to_device(b) for _, b in cases]
    alone = [H.run_gpu(b, mode="saguaro" if m == "saguaro" else "residual", eps=1e-8 if m == "saguaro" else 0.0,
                       db=db, diag=False, early=m == "early") for (m, b), db in zip(cases, dbs)]
    torch.cuda.synchronize()
    results = [[] for _ in cases]
    errors = []

    def worker(i):
        try:
            m, b = cases[i]
            db = dbs[i]
            dt = R.SPEC_BF16 if b.dtype == "bf16" else R.SPEC_F32
            st = torch.cuda.Stream()
            ws = R.new_workspace(R.spec_workspace_bytes(b.B, b.gamma, b.V, dt), "cuda")
            torch.cuda.synchronize()
            with torch.cuda.stream(st):
                for _ in range(8):
                    args = (db.draft, db.target, db.tokens, db.u_accept, db.u_sample, b.T)
                    if m == "saguaro":
                        o = R.spec_verify_saguaro(*args, in_len=db.in_len, workspace=ws, stream=st, eps=1e-8)
                    elif m == "early":
                        o = R.spec_verify_early(*args, in_len=db.in_len, workspace=ws, stream=st)
                    else:
                        o = R.spec_verify(*args, in_len=db.in_len, workspace=ws, stream=st)
                    results[i].append(o)
            st.synchronize()
            assert int(ws[:4].view(torch.int32).item()) == 0, "bounded wait timed out"
        except Exception as e:   # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a calling thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(len(cases)):
        assert len(results[i]) == 8
        for o in results[i]:
            np.testing.assert_array_equal(o.tokens.cpu().numpy(), alone[i]["tokens"])
            np.testing.assert_array_equal(o.accepted.cpu().numpy(), alone[i]["accepted"])
            np.testing.assert_array_equal(o.out_len.cpu().numpy(), alone[i]["out_len"])


@pytest.mark.parametrize("early", [False, True])
def test_graph_capture_replays(early):
    """One call captured in a graph (outputs and workspace allocated
    beforehand) and replayed five times, with eager work and a
    synchronisation between the replays: every replay gives the eager call's
    outputs and leaves the workspace's error word clear."""
    import rejection_sampling_verify_12_amd as R
    batch = random_batch(24, 4, 50000, "bf16", 1.0, seed=4333)
    db = H.to_device(batch)
    ref = H.run_gpu(batch, db=db, diag=False, early=early)
    ws = R.new_workspace(R.spec_workspace_bytes(batch.B, batch.gamma, batch.V, R.SPEC_BF16), "cuda")
    out = R.alloc_outputs(batch.B, batch.gamma, "cuda")
    call = R.spec_verify_early if early else R.spec_verify
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        call(db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T, in_len=db.in_len,
             out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T, in_len=db.in_len,
             out=out, workspace=ws)
    for _ in range(5):
        out.tokens.fill_(-7)
        out.accepted.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0, "bounded wait timed out"
        np.testing.assert_array_equal(out.tokens.cpu().numpy(), ref["tokens"])
        np.testing.assert_array_equal(out.accepted.cpu().numpy(), ref["accepted"])
        np.testing.assert_array_equal(out.out_len.cpu().numpy(), ref["out_len"])


# --------------------------------------------------------------------------- outcome prediction

def _predict(batch, gpu=None):
    import rejection_sampling_verify_12_amd as R
    db = H.to_device(batch)
    acc = tok = None
    if gpu is not None:
        acc = torch.from_numpy(gpu["accepted"]).cuda()
        tok = torch.from_numpy(gpu["tokens"]).cuda()
    out = R.spec_predict_outcomes(db.draft, acc, tok)
    torch.cuda.synchronize()
    return out.cand.cpu().numpy(), out.hit.cpu().numpy(), out.cand_idx.cpu().numpy()


def test_predict_outcomes_workload():
    batch = workload("B128_g4_V128256_bf16")
    gpu = H.run_gpu(batch, diag=False)
    cand, hit, idx = _predict(batch, gpu)
    ref_cand = O.predict_outcomes(batch.draft64())
    np.testing.assert_array_equal(cand, ref_cand)
    ref_hit, ref_idx = O.predict_hits(ref_cand, gpu["accepted"], gpu["tokens"])
    np.testing.assert_array_equal(hit, ref_hit)
    np.testing.assert_array_equal(idx, ref_idx)
    H.say(f"[predict] hit rate {hit.mean():.3f} over {len(hit)} sequences")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_predict_edges(dtype):
    B, g, V = 6, 2, 20000
    rng = np.random.default_rng(3)
    d64 = np.round(rng.normal(size=(B, g + 1, V)), 1)   # many ties
    d64[0, 0, :] = 0.0
    d64[0, 0, 5] = -0.0
    d64[2, 2, 19999] = 50.0                               # max at the last id
    draft = W.encode(d64, dtype)
    draft[1, 1, 100] = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    batch = W.Batch(name="pred_edges", B=B, gamma=g, V=V, T=1.0, dtype=dtype, draft=draft,
                    target=draft, draft_tokens=np.zeros((B, g), np.int32),
                    u_accept=np.zeros((B, g), np.float32), u_sample=np.zeros((B, g + 1), np.float32),
                    in_len=np.zeros(B, np.int32))
    cand, _, _ = _predict(batch)
    np.testing.assert_array_equal(cand, O.predict_outcomes(W.decode_f64(draft, dtype)))
    small = W.Batch(**{**batch.__dict__, "V": 2, "draft": draft[:, :, :2].copy(),
                       "target": draft[:, :, :2].copy()})
    cand2, _, _ = _predict(small)
    np.testing.assert_array_equal(cand2, O.predict_outcomes(W.decode_f64(small.draft, dtype)))


# --------------------------------------------------------------------------- verification + prediction in one pass

def _verify_predict(batch, mode="residual", eps=0.0, db=None, ws=None):
    import rejection_sampling_verify_12_amd as R
    H.say(f"[verify_predict] {batch.name} B={batch.B} gamma={batch.gamma} V={batch.V} "
          f"{batch.dtype} mode={mode} eps={eps}")
    db = db or H.to_device(batch)
    if ws is None:
        dt = R.SPEC_BF16 if batch.dtype == "bf16" else R.SPEC_F32
        ws = R.new_workspace(R.spec_workspace_bytes(batch.B, batch.gamma, batch.V, dt), "cuda")
    out, pred = R.spec_verify_predict(db.draft, db.target, db.tokens, db.u_accept, db.u_sample,
                                      batch.T, in_len=db.in_len, workspace=ws,
                                      saguaro=(mode == "saguaro"), eps=eps)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "bounded wait timed out"
    return {"tokens": out.tokens.cpu().numpy(), "accepted": out.accepted.cpu().numpy(),
            "first_reject": out.first_reject.cpu().numpy(),
            "mask": out.accept_mask.cpu().numpy().view(np.uint64),
            "out_len": out.out_len.cpu().numpy(), "cand": pred.cand.cpu().numpy(),
            "hit": pred.hit.cpu().numpy(), "cand_idx": pred.cand_idx.cpu().numpy()}


def _check_verify_predict(batch, got, mode="residual", eps=0.0):
    """Verification outputs equal the verification-only call's; candidates equal
    the oracle's top-3; hit and index follow from them and the outputs."""
    alone = H.run_gpu(batch, mode, eps, diag=False)
    for k in ("tokens", "accepted", "first_reject", "mask", "out_len"):
        np.testing.assert_array_equal(got[k], alone[k], err_msg=k)
    ref_cand = O.predict_outcomes(batch.draft64())
    np.testing.assert_array_equal(got["cand"], ref_cand)
    ref_hit, ref_idx = O.predict_hits(ref_cand, got["accepted"], got["tokens"])
    np.testing.assert_array_equal(got["hit"], ref_hit)
    np.testing.assert_array_equal(got["cand_idx"], ref_idx)


@pytest.mark.parametrize("mode,eps", [("residual", 0.0), ("saguaro", 0.0)])
def test_verify_predict_workload(mode, eps):
    batch = workload("B128_g4_V128256_bf16")
    got = _verify_predict(batch, mode, eps)
    _check_verify_predict(batch, got, mode, eps)
    H.say(f"[verify_predict] hit rate {got['hit'].mean():.3f}")


@pytest.mark.parametrize("V", [50000, 50001, 2048 * 3 + 8, 8, 16, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_verify_predict_ragged(V, dtype):
    """Partial last chunks and partial lane periods (V = 50000, 6152), a V
    the packed path cannot take (50001), the smallest rows the single kernel
    takes (8, 16: one lane holds the whole row) and fewer tokens than
    candidates (2)."""
    batch = random_batch(5, 3, V, dtype, 1.0, seed=4100 + V % 97)
    _check_verify_predict(batch, _verify_predict(batch))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_verify_predict_many_chunks(dtype):
    """Rows of more than 21 chunks of 32768 logits (more candidate records
    than a wave holds three to a lane), each row's maximum planted in its
    last, partial chunk and its runner-up in the first."""
    V = 22 * 32768 - 4000
    batch = random_batch(2, 1, V, dtype, 1.0, seed=4177)
    d64 = W.decode_f64(batch.draft, dtype)
    d64[:, :, V - 3] = d64.max() + 2.0
    d64[:, :, 5] = d64.max() - 1.0
    batch = dataclasses.replace(batch, draft=W.encode(d64, dtype))
    got = _verify_predict(batch)
    assert (got["cand"][:, :, 0] == V - 3).all() and (got["cand"][:, :, 1] == 5).all()
    _check_verify_predict(batch, got)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_verify_predict_ties_and_bad_rows(dtype):
    """Heavy ties across lanes (logits rounded to 0.1), +-0, an all -inf draft
    row, the maximum at the last id, a NaN and a +inf draft logit; then a second,
    smaller call on the same workspace."""
    B, g, V = 6, 3, 40000
    rng = np.random.default_rng(11)
    d64 = np.round(rng.normal(size=(B, g + 1, V)), 1)
    d64[0, 0, :] = 0.0
    d64[0, 0, 5] = -0.0
    d64[2, 3, V - 1] = 50.0
    d64[3, 1, :] = -np.inf
    d64[4, 2, 7] = np.inf
    t64 = d64 + 0.3 * rng.normal(size=d64.shape)
    t64[3, 1, :] = 0.0
    draft, target = W.encode(d64, dtype), W.encode(np.nan_to_num(t64, posinf=50.0), dtype)
    draft[1, 1, 100] = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    tokens = rng.integers(0, V, size=(B, g)).astype(np.int32)
    batch = W.Batch(name=f"pred_ties_{dtype}", B=B, gamma=g, V=V, T=1.0, dtype=dtype,
                    draft=draft, target=target, draft_tokens=tokens,
                    u_accept=W.uniforms24(W.philox(12, 1), (B, g)),
                    u_sample=W.uniforms24(W.philox(12, 2), (B, g + 1)),
                    in_len=np.zeros(B, np.int32))
    import rejection_sampling_verify_12_amd as R
    dt = R.SPEC_BF16 if dtype == "bf16" else R.SPEC_F32
    ws = R.new_workspace(R.spec_workspace_bytes(B, g, V, dt), "cuda")
    _check_verify_predict(batch, _verify_predict(batch, ws=ws))
    small = W.Batch(**{**batch.__dict__, "B": 3, "draft": draft[3:].copy(), "target": target[3:].copy(),
                       "draft_tokens": tokens[3:].copy(), "u_accept": batch.u_accept[3:].copy(),
                       "u_sample": batch.u_sample[3:].copy(), "in_len": batch.in_len[3:].copy()})
    _check_verify_predict(small, _verify_predict(small, ws=ws))


def test_saguaro_eps_where_the_target_has_zero_probability():
    """Saguaro with eps > 0 gives a token with q = 0 and p > 0 the weight
    sqrt(p * eps) ("Speculative Speculative Decoding (Saguaro)", section 3.2
    code: the clamp applies to every token); half of each target row is -inf."""
    for dtype in ("bf16", "f32"):
        batch = random_batch(12, 3, 8192, dtype, 1.0, seed=7100, scale=1.0, sigma=0.5)
        t64 = batch.target64()
        t64[:, :, ::2] = -np.inf
        batch = W.Batch(**{**batch.__dict__, "target": W.encode(t64, dtype)})
        rep = H.parity(batch, "saguaro", 1e-3)
        rep.check()
        assert rep.n_draws > 0


# --------------------------------------------------------------------------- small, peaked rows

@pytest.mark.parametrize("V", [2, 3, 8, 16, 33])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,eps", [("residual", 0.0), ("saguaro", 0.0), ("saguaro", 1e-8)])
def test_small_peaked_rows(V, dtype, mode, eps):
    """Few tokens with one dominant: residual masses are small next to q_j,
    the regime where fp32 rounding weighs most."""
    batch = random_batch(24, 4, V, dtype, 1.0, seed=7300 + V, scale=6.0, sigma=0.3)
    H.parity(batch, mode, eps).check()
    H.parity(batch, mode, eps, early=True).check()


# --------------------------------------------------------------------------- a wait that gives up

@pytest.mark.parametrize("case", ["bf16", "f32", "early", "saguaro_eps", "predict", "greedy"])
def test_error_word_set_before_the_call(case):
    """The workspace's error word set from the host before the call (as after
    a bounded wait that gave up): every wait then gives up within 64 polls, so
    every kernel returns; no sequence is reported valid from a wait that gave
    up, and a decision taken with the word set reports its sequence invalid -
    so every sequence comes back invalid - and the word stays set."""
    import rejection_sampling_verify_12_amd as R
    dtype = "f32" if case == "f32" else "bf16"
    batch = random_batch(16, 4, 40000, dtype, 1.0, seed=4400)
    H.say(f"[give-up] case={case} B={batch.B} gamma={batch.gamma} V={batch.V} {dtype}")
    db = H.to_device(batch)
    dt = R.SPEC_F32 if dtype == "f32" else R.SPEC_BF16
    if case == "greedy":
        ws = R.new_workspace(R.spec_greedy_workspace_bytes(batch.B, batch.gamma, batch.V, dt), "cuda")
    else:
        ws = R.new_workspace(R.spec_workspace_bytes(batch.B, batch.gamma, batch.V, dt), "cuda")
    ws[:4].view(torch.int32).fill_(1)
    out = R.alloc_outputs(batch.B, batch.gamma, "cuda")
    for t in (out.tokens, out.accepted, out.first_reject, out.out_len):
        t.fill_(7)
    out.accept_mask.fill_(7)
    args = (db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T)
    if case in ("bf16", "f32"):
        R.spec_verify(*args, in_len=db.in_len, out=out, workspace=ws)
    elif case == "early":
        R.spec_verify_early(*args, in_len=db.in_len, out=out, workspace=ws)
    elif case == "saguaro_eps":
        R.spec_verify_saguaro(*args, in_len=db.in_len, out=out, workspace=ws, eps=1e-8)
    elif case == "predict":
        R.spec_verify_predict(*args, in_len=db.in_len, out=out, workspace=ws)
    else:
        R.spec_verify_greedy(db.target, db.tokens, in_len=db.in_len, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 1
    assert (out.accepted.cpu().numpy() == -1).all()
    assert (out.tokens.cpu().numpy() == -1).all()
    assert (out.first_reject.cpu().numpy() == -1).all()
    assert (out.accept_mask.cpu().numpy() == 0).all()
    np.testing.assert_array_equal(out.out_len.cpu().numpy(), batch.in_len)
