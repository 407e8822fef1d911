"""spec_verify_noalloc (the allocation-free entry point) against spec_verify:
two calls in a row through the C ABI, the second with a smaller input, each
equal to spec_verify's outputs on the same inputs."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("gpu_harness")

import workloads as W


def _batch(B, gamma, V, seed):
    rng = W.philox(seed, 7)
    d64 = rng.standard_normal((B, gamma + 1, V)) * 3.0
    t64 = d64 + 0.7 * rng.standard_normal((B, gamma + 1, V))
    draft, target = W.encode(d64, "bf16"), W.encode(t64, "bf16")
    tokens = W.gumbel_argmax(W.decode_f64(draft, "bf16")[:, :gamma], 1.0, W.philox(seed, 8))
    return W.Batch(name=f"noalloc_B{B}_g{gamma}_V{V}", B=B, gamma=gamma, V=V, T=1.0, dtype="bf16",
                   draft=draft, target=target, draft_tokens=tokens,
                   u_accept=W.uniforms24(W.philox(seed, 9), (B, gamma)),
                   u_sample=W.uniforms24(W.philox(seed, 10), (B, gamma + 1)),
                   in_len=np.arange(B, dtype=np.int32), seed=seed)


def test_noalloc_matches_spec_verify_twice():
    import rejection_sampling_verify_12_amd as R
    for batch in (_batch(40, 5, 60000, 4501), _batch(7, 3, 30000, 4502)):
        H.say(f"[noalloc] B={batch.B} gamma={batch.gamma} V={batch.V}")
        db = H.to_device(batch)
        ref = H.run_gpu(batch, db=db, diag=True)
        out = R.spec_verify_noalloc(db.draft, db.target, db.tokens, db.u_accept, db.u_sample, batch.T,
                                    in_len=db.in_len, diag=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.tokens.cpu().numpy(), ref["tokens"])
        np.testing.assert_array_equal(out.accepted.cpu().numpy(), ref["accepted"])
        np.testing.assert_array_equal(out.first_reject.cpu().numpy(), ref["first_reject"])
        np.testing.assert_array_equal(out.accept_mask.cpu().numpy().view(np.uint64), ref["mask"])
        np.testing.assert_array_equal(out.out_len.cpu().numpy(), ref["out_len"])
        for k, v in ref["diag"].items():
            np.testing.assert_array_equal(out.diag[k].cpu().numpy(), v, err_msg=k)
        # and the oracle agrees, as for spec_verify
        H.compare(batch, {"tokens": out.tokens.cpu().numpy(), "accepted": out.accepted.cpu().numpy(),
                          "first_reject": out.first_reject.cpu().numpy(),
                          "mask": out.accept_mask.cpu().numpy().view(np.uint64),
                          "out_len": out.out_len.cpu().numpy()},
                  H.run_oracle(batch), check_diag=False).check()
