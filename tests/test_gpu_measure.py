"""The measurement aids run and keep their sink untouched: the attainable-read
kernel over a buffer (with a ragged last work-group) and the LDS atomic probe
in every pattern.  Their argument checks are host-side."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("gpu_harness")


def test_read_bandwidth_and_lds_probe_run():
    import rejection_sampling_verify_12_amd as R
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    buf = torch.randn(3 * 16384 + 8, device="cuda")   # 196,640 bytes: a partial 64 KB chunk at the end
    H.say("[measure] spec_read_bandwidth")
    R.spec_read_bandwidth(buf, sink)
    for pat in range(4):
        H.say(f"[measure] spec_lds_atomic_probe pattern {pat}")
        R.spec_lds_atomic_probe(pat, 4, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    for bad in ((-1, 4), (4, 4), (0, 0), (0, (1 << 20) + 1)):
        with pytest.raises(R.SpecError):
            R.spec_lds_atomic_probe(*bad, sink)
