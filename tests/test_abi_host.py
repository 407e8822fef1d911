"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/spec_verify.h declares, sizes its workspace, and rejects bad
arguments with the documented status before anything is enqueued."""
import ctypes
import math
import os
import re

import pytest

import rejection_sampling_verify_12_amd as R

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "spec_verify.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(spec_\w+)\s*\(", src, re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(R.EXPORTED), names


def test_library_exports_every_declared_symbol():
    lib = R.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_checks_build_exports_the_same_abi():
    """The checks build (when built) exports every declared function and its
    marker; the default library has no marker."""
    from rejection_sampling_verify_12_amd import build as BLD
    assert not hasattr(R.load_library(), "spec_checks_build")
    if not os.path.exists(BLD.CHECKS_LIB):
        pytest.skip("checks build not built")
    lib = ctypes.CDLL(BLD.CHECKS_LIB)
    for n in declared_functions():
        assert hasattr(lib, n), n
    lib.spec_checks_build.restype = ctypes.c_int
    assert lib.spec_checks_build() == 1


def test_status_strings():
    for st in (R.SPEC_OK, R.SPEC_EINVAL, R.SPEC_EDTYPE, R.SPEC_EWORKSPACE, R.SPEC_ELAUNCH):
        assert R.spec_status_str(st) and R.spec_status_str(st) != "unknown status"
    assert R.spec_status_str(123) == "unknown status"


def test_workspace_bytes():
    assert R.spec_workspace_bytes(0, 4, 1000, R.SPEC_BF16) == 0
    assert R.spec_workspace_bytes(-1, 4, 1000, R.SPEC_BF16) == 0
    assert R.spec_workspace_bytes(2, 0, 1000, R.SPEC_BF16) == 0
    assert R.spec_workspace_bytes(2, 64, 1000, R.SPEC_BF16) == 0
    assert R.spec_workspace_bytes(2, 4, 0, R.SPEC_BF16) == 0
    assert R.spec_workspace_bytes(2, 4, 1000, 7) == 0
    a = R.spec_workspace_bytes(256, 8, 152064, R.SPEC_BF16)
    b = R.spec_workspace_bytes(512, 8, 152064, R.SPEC_BF16)
    assert 0 < a < b and a % 256 == 0
    # modest: far below the logits it verifies
    assert a < 0.01 * 256 * 17 * 152064 * 2
    assert R.spec_predict_workspace_bytes(128, 4, 128256, R.SPEC_BF16) > 0
    assert R.spec_predict_workspace_bytes(0, 4, 128256, R.SPEC_BF16) == 0


@pytest.mark.parametrize("gamma,V", [(4, 32000), (1, 7), (8, 152064), (4, 128256), (63, 40000)])
def test_workspace_serves_every_smaller_call(gamma, V):
    """Calls with few rows take shorter chunks (more per-chunk records per
    row); the workspace of a call still covers every call with fewer
    sequences, shorter rows or fewer positions."""
    for dt in (R.SPEC_BF16, R.SPEC_F32):
        sizes = [R.spec_workspace_bytes(B, gamma, V, dt) for B in range(1, 130)]
        assert all(x <= y for x, y in zip(sizes, sizes[1:])), (gamma, V, dt)
        for B in (1, 3, 17, 64):
            big = R.spec_workspace_bytes(B, gamma, V, dt)
            assert R.spec_workspace_bytes(B, gamma, max(V // 3, 1), dt) <= big
            assert R.spec_workspace_bytes(B, max(gamma // 2, 1), V, dt) <= big


FAKE = 4096   # never dereferenced: every call below fails validation first


def _verify(saguaro=False, eps=0.0, **kw):
    lib = R.load_library()
    a = dict(draft=FAKE, target=FAKE, dtype=R.SPEC_BF16, tokens=FAKE, ua=FAKE, us=FAKE, B=4,
             gamma=3, V=1000, T=1.0, in_len=None, out_tokens=FAKE, out_acc=FAKE, out_fr=None,
             out_mask=None, out_len=None, diag=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    args = list(a.values())
    return lib.spec_verify_saguaro(*args, eps) if saguaro else lib.spec_verify(*args)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), R.SPEC_EINVAL),
    (dict(gamma=0), R.SPEC_EINVAL),
    (dict(gamma=64), R.SPEC_EINVAL),
    (dict(V=0), R.SPEC_EINVAL),
    (dict(T=0.0), R.SPEC_EINVAL),
    (dict(T=-1.0), R.SPEC_EINVAL),
    (dict(T=math.nan), R.SPEC_EINVAL),
    (dict(T=math.inf), R.SPEC_EINVAL),
    (dict(dtype=2), R.SPEC_EDTYPE),
    (dict(draft=None), R.SPEC_EINVAL),
    (dict(target=None), R.SPEC_EINVAL),
    (dict(tokens=None), R.SPEC_EINVAL),
    (dict(ua=None), R.SPEC_EINVAL),
    (dict(us=None), R.SPEC_EINVAL),
    (dict(out_tokens=None), R.SPEC_EINVAL),
    (dict(out_acc=None), R.SPEC_EINVAL),
    (dict(ws=None), R.SPEC_EWORKSPACE),
    (dict(ws_bytes=16), R.SPEC_EWORKSPACE),
    (dict(B=0, draft=None, ws=None), R.SPEC_OK),
])
def test_verify_rejects_bad_arguments(kw, status):
    assert _verify(**kw) == status
    assert _verify(saguaro=True, **kw) == status


@pytest.mark.parametrize("eps", [-1e-8, math.nan, math.inf])
def test_saguaro_rejects_bad_eps(eps):
    assert _verify(saguaro=True, eps=eps) == R.SPEC_EINVAL


def test_predict_rejects_bad_arguments():
    lib = R.load_library()

    def call(**kw):
        a = dict(draft=FAKE, dtype=R.SPEC_BF16, B=4, gamma=3, V=1000, acc=None, tok=None,
                 cand=FAKE, hit=None, idx=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return lib.spec_predict_outcomes(*a.values())

    assert call(B=-1) == R.SPEC_EINVAL
    assert call(gamma=64) == R.SPEC_EINVAL
    assert call(dtype=9) == R.SPEC_EDTYPE
    assert call(draft=None) == R.SPEC_EINVAL
    assert call(cand=None) == R.SPEC_EINVAL
    assert call(acc=FAKE) == R.SPEC_EINVAL          # accepted without out_tokens
    assert call(ws_bytes=8) == R.SPEC_EWORKSPACE
    assert call(B=0, draft=None) == R.SPEC_OK


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(R, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        R.load_library(str(tmp_path / "absent.so"))


def test_greedy_rejects_bad_arguments():
    lib = R.load_library()

    def call(**kw):
        a = dict(target=FAKE, dtype=R.SPEC_BF16, tokens=FAKE, B=4, gamma=3, V=1000, in_len=None,
                 out_tokens=FAKE, out_acc=FAKE, out_fr=None, out_mask=None, out_len=None,
                 ws=FAKE, ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return lib.spec_verify_greedy(*a.values())

    assert call(B=-1) == R.SPEC_EINVAL
    assert call(gamma=0) == R.SPEC_EINVAL
    assert call(gamma=64) == R.SPEC_EINVAL
    assert call(V=0) == R.SPEC_EINVAL
    assert call(dtype=5) == R.SPEC_EDTYPE
    assert call(target=None) == R.SPEC_EINVAL
    assert call(tokens=None) == R.SPEC_EINVAL
    assert call(out_tokens=None) == R.SPEC_EINVAL
    assert call(out_acc=None) == R.SPEC_EINVAL
    assert call(ws=None) == R.SPEC_EWORKSPACE
    assert call(ws_bytes=8) == R.SPEC_EWORKSPACE
    assert call(B=0, target=None, ws=None) == R.SPEC_OK
    assert R.spec_greedy_workspace_bytes(256, 8, 152064, R.SPEC_BF16) > 0
    assert R.spec_greedy_workspace_bytes(0, 8, 152064, R.SPEC_BF16) == 0
    assert R.spec_greedy_workspace_bytes(4, 64, 100, R.SPEC_BF16) == 0


def test_verify_predict_rejects_bad_arguments():
    lib = R.load_library()

    def call(saguaro=0, eps=0.0, cand=FAKE, **kw):
        a = dict(draft=FAKE, target=FAKE, dtype=R.SPEC_BF16, tokens=FAKE, ua=FAKE, us=FAKE, B=4,
                 gamma=3, V=1000, T=1.0, in_len=None, out_tokens=FAKE, out_acc=FAKE, out_fr=None,
                 out_mask=None, out_len=None, diag=None)
        a.update(kw)
        return lib.spec_verify_predict(*a.values(), saguaro, eps, cand, None, None, FAKE, 1 << 30, None)

    assert call(cand=None) == R.SPEC_EINVAL
    assert call(saguaro=2) == R.SPEC_EINVAL
    assert call(saguaro=1, eps=-1.0) == R.SPEC_EINVAL
    assert call(T=0.0) == R.SPEC_EINVAL
    assert call(dtype=3) == R.SPEC_EDTYPE


def test_verify_ex_rejects_bad_options():
    lib = R.load_library()

    def call(T=1.0, **o):
        opts = R.SpecOptions(o.get("saguaro", 0), o.get("eps", 0.0), o.get("early", 0),
                             o.get("temps"), o.get("cand"), o.get("hit"), o.get("idx"))
        return lib.spec_verify_ex(FAKE, FAKE, R.SPEC_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, T, None,
                                  FAKE, FAKE, None, None, None, None, ctypes.byref(opts), FAKE,
                                  1 << 30, None)

    assert call(saguaro=2) == R.SPEC_EINVAL
    assert call(saguaro=1, eps=-1.0) == R.SPEC_EINVAL
    assert call(early=1, cand=FAKE) == R.SPEC_EINVAL
    assert call(hit=FAKE) == R.SPEC_EINVAL
    assert call(idx=FAKE) == R.SPEC_EINVAL
    assert call(T=0.0) == R.SPEC_EINVAL              # the scalar is checked without an array
    assert call(T=math.nan) == R.SPEC_EINVAL


def test_verify_ex_rejects_bad_top_p():
    lib = R.load_library()
    for top_p, early in ((-0.1, 0), (1.5, 0), (math.nan, 0), (0.9, 1)):
        opts = R.SpecOptions(0, 0.0, early, None, None, None, None, top_p)
        st = lib.spec_verify_ex(FAKE, FAKE, R.SPEC_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0, None,
                                FAKE, FAKE, None, None, None, None, ctypes.byref(opts), FAKE,
                                1 << 30, None)
        assert st == R.SPEC_EINVAL, (top_p, early)


def test_lost_decision_record_decodes_without_indices(tmp_path):
    """A decision record whose bounded wait gave up decodes as an invalid
    sequence with k = 0 (no index is derived from an unwritten word); a
    complete record decodes to what was stored.  The real device header is
    compiled host-only and run here (no GPU)."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "rec_decode_check")
    build = subprocess.run([hipcc, "--offload-host-only", "-std=c++17", "-x", "hip",
                            "-I", os.path.join(root, "include"),
                            "-I", os.path.join(root, "rejection_sampling_verify_12_amd", "csrc"),
                            os.path.join(root, "tests", "host", "rec_decode_check.hip"), "-o", exe],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True)
    assert run.returncode == 0, run.stdout + run.stderr


def test_launch_orders_only_wait_on_earlier_blocks(tmp_path):
    """The single kernel's launch orders (tests/host/sched_check.hip, the real
    header compiled host-only): over a sweep of sizes and slot counts every
    block decodes to one in-range item with both decoders, every item is
    dispatched exactly once, and every item a block waits for has a smaller
    block number (blocks start in order, so every wait ends)."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "sched_check")
    build = subprocess.run([hipcc, "--offload-host-only", "-std=c++17", "-O2", "-x", "hip",
                            "-I", os.path.join(root, "include"),
                            "-I", os.path.join(root, "rejection_sampling_verify_12_amd", "csrc"),
                            os.path.join(root, "tests", "host", "sched_check.hip"), "-o", exe],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True)
    assert run.returncode == 0 and run.stdout.startswith("ok"), run.stdout[-3000:] + run.stderr[-2000:]


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """spec_verify_noalloc checks sizes against its 16 MiB static scratch (and
    the usual arguments) before anything is enqueued or any device is used."""
    lib = R.load_library()

    def call(B, gamma, V, dtype=R.SPEC_BF16, T=1.0):
        return lib.spec_verify_noalloc(FAKE, FAKE, dtype, FAKE, FAKE, FAKE, B, gamma, V, T, None, FAKE,
                                       FAKE, None, None, None, None, None)
    assert R.spec_workspace_bytes(512, 8, 152064, R.SPEC_BF16) > 16 << 20
    assert call(512, 8, 152064) == R.SPEC_ESCRATCH
    # the boundary the header states for gamma = 8, V = 152064, bf16: B above 400
    assert R.spec_workspace_bytes(400, 8, 152064, R.SPEC_BF16) <= 16 << 20
    assert R.spec_workspace_bytes(401, 8, 152064, R.SPEC_BF16) > 16 << 20
    assert call(401, 8, 152064) == R.SPEC_ESCRATCH
    assert call(4, 3, 1000, dtype=9) == R.SPEC_EDTYPE
    assert call(4, 64, 1000) == R.SPEC_EINVAL
    assert call(0, 3, 1000) == R.SPEC_OK
    assert "16 MiB" in R.spec_status_str(R.SPEC_ESCRATCH)


def test_bigram_and_pipeline_calls_reject_bad_arguments():
    """The synthetic-model and pre-speculation calls check their arguments
    before anything is enqueued; empty batches are no-ops."""
    lib = R.load_library()
    bf = R.SPEC_BF16
    # spec_synth_draft(table, dtype, V, H, noise, P, gamma, n, start_tok, start_pos, out, stream)
    for kw in (dict(V=0), dict(H=0), dict(P=0), dict(gamma=0), dict(gamma=64), dict(n=-1),
               dict(dtype=7), dict(table=None), dict(noise=None), dict(tok=None), dict(out=None)):
        a = dict(table=FAKE, dtype=bf, V=100, H=10, noise=FAKE, P=8, gamma=4, n=3, tok=FAKE,
                 pos=None, out=FAKE, stream=None)
        a.update(kw)
        assert lib.spec_synth_draft(*a.values()) == R.SPEC_EINVAL, kw
    assert lib.spec_synth_draft(FAKE, bf, 100, 10, FAKE, 8, 4, 0, None, None, None, None) == R.SPEC_OK
    # spec_synth_rows(table, dtype, V, H, gamma, B, last, tokens, out, stream)
    for kw in (dict(V=0), dict(H=0), dict(gamma=64), dict(B=-1), dict(dtype=7), dict(last=None),
               dict(out=None)):
        a = dict(table=FAKE, dtype=bf, V=100, H=10, gamma=4, B=2, last=FAKE, tok=FAKE, out=FAKE,
                 stream=None)
        a.update(kw)
        assert lib.spec_synth_rows(*a.values()) == R.SPEC_EINVAL, kw
    assert lib.spec_synth_rows(FAKE, bf, 100, 10, 4, 0, None, None, None, None) == R.SPEC_OK
    # spec_ssd_prespeculate(table, dtype, V, H, noise, P, gamma, B, cand, len, prepared, stream)
    for kw in (dict(gamma=64), dict(B=-1), dict(cand=None), dict(prep=None), dict(noise=None)):
        a = dict(table=FAKE, dtype=bf, V=100, H=10, noise=FAKE, P=8, gamma=4, B=2, cand=FAKE,
                 len=None, prep=FAKE, stream=None)
        a.update(kw)
        assert lib.spec_ssd_prespeculate(*a.values()) == R.SPEC_EINVAL, kw
    # spec_ssd_advance(table, dtype, V, H, noise, P, gamma, B, out_tokens, accepted, out_len,
    #                  hit, cand_idx, prepared, next_last, next_len, next_tokens, stream)
    for kw in (dict(acc=None), dict(olen=None), dict(nl=None), dict(hit=FAKE),
               dict(hit=FAKE, idx=FAKE), dict(B=-1), dict(P=0)):
        a = dict(table=FAKE, dtype=bf, V=100, H=10, noise=FAKE, P=8, gamma=4, B=2, tok=FAKE,
                 acc=FAKE, olen=FAKE, hit=None, idx=None, prep=None, nl=FAKE, nlen=FAKE, nt=FAKE,
                 stream=None)
        a.update(kw)
        assert lib.spec_ssd_advance(*a.values()) == R.SPEC_EINVAL, kw


@pytest.mark.slow
def test_host_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The library's sources built with ASan and UBSan on the host code
    (device code compiled as usual, never launched) and driven through the
    size queries at the limits of int and every entry point's rejection of bad
    arguments (tests/host/abi_sanitize.hip).  Any sanitizer report fails."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "rejection_sampling_verify_12_amd", "csrc")
    srcs = [os.path.join(csrc, s) for s in ("verify.hip", "predict.hip", "greedy.hip",
                                            "synthetic.hip", "readbw.hip")]
    exe = str(tmp_path / "abi_sanitize")
    cmd = [hipcc, "--offload-arch=gfx950", "-std=c++17", "-x", "hip", "-g", "-O1",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(root, "include"), "-I", csrc, *srcs,
           os.path.join(root, "tests", "host", "abi_sanitize.hip"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert run.returncode == 0 and "ok (0 failures)" in run.stdout, run.stdout + run.stderr[-3000:]
