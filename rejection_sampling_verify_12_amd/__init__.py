"""Python binding of libspecverify (batched speculative-sampling verification, gfx950).

Argument marshalling only: every step of the verification runs in the HIP
kernels of ``libspecverify.so``; torch provides device memory and streams.
The names follow the C ABI in include/spec_verify.h.  Importing works
without a GPU; calling a compute entry point needs the built library and a
device, and fails loudly otherwise (there is no CPU fallback).
"""
from __future__ import annotations

import collections
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EWORKSPACE, SPEC_ELAUNCH, SPEC_ESCRATCH = 0, -1, -2, -3, -4, -5
SPEC_F32, SPEC_BF16 = 0, 1

EXPORTED = ("spec_workspace_bytes", "spec_verify", "spec_verify_saguaro",
            "spec_predict_workspace_bytes", "spec_predict_outcomes", "spec_verify_predict",
            "spec_greedy_workspace_bytes", "spec_verify_greedy", "spec_verify_early",
            "spec_verify_ex", "spec_synthetic_busy", "spec_verify_noalloc", "spec_read_bandwidth",
            "spec_lds_atomic_probe",
            "spec_synth_draft", "spec_synth_rows", "spec_ssd_prespeculate", "spec_ssd_advance",
            "spec_status_str")


class SpecOptions(ctypes.Structure):
    """struct spec_options (see spec_verify.h)."""
    _fields_ = [("saguaro", ctypes.c_int), ("eps", ctypes.c_float), ("early", ctypes.c_int),
                ("temperature", ctypes.c_void_p), ("cand", ctypes.c_void_p),
                ("hit", ctypes.c_void_p), ("cand_idx", ctypes.c_void_p), ("top_p", ctypes.c_float)]


class SpecDiag(ctypes.Structure):
    """struct spec_diag: optional device pointers (0 = not requested)."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("row_max", "row_logZ", "px", "qx", "resid_mass", "token_prob", "cdf_lo", "cdf_hi")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecverify.so and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m rejection_sampling_verify_12_amd.build` (no CPU fallback)")
    # torch first, so that the library binds to the HIP runtime torch loads:
    # the one that owns the device memory and streams handed to it.  Loaded
    # the other way round, the process holds two runtimes and launches fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    verify_args = [vp, vp, i32, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp,
                   ctypes.POINTER(SpecDiag), vp, sz, vp]
    lib.spec_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_workspace_bytes.restype = sz
    lib.spec_verify.argtypes = verify_args
    lib.spec_verify.restype = i32
    lib.spec_verify_saguaro.argtypes = verify_args + [f32]
    lib.spec_verify_saguaro.restype = i32
    lib.spec_predict_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_predict_workspace_bytes.restype = sz
    lib.spec_predict_outcomes.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_predict_outcomes.restype = i32
    lib.spec_verify_predict.argtypes = verify_args[:-3] + [i32, f32, vp, vp, vp] + verify_args[-3:]
    lib.spec_verify_predict.restype = i32
    lib.spec_verify_early.argtypes = verify_args[:-3] + [i32, f32] + verify_args[-3:]
    lib.spec_verify_ex.argtypes = verify_args[:-3] + [ctypes.POINTER(SpecOptions)] + verify_args[-3:]
    lib.spec_verify_ex.restype = i32
    lib.spec_synthetic_busy.argtypes = [ctypes.c_int64, vp, i32, vp]
    lib.spec_synthetic_busy.restype = i32
    lib.spec_synth_draft.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.spec_synth_draft.restype = i32
    lib.spec_synth_rows.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.spec_synth_rows.restype = i32
    lib.spec_ssd_prespeculate.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.spec_ssd_prespeculate.restype = i32
    lib.spec_ssd_advance.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32] + [vp] * 10
    lib.spec_ssd_advance.restype = i32
    lib.spec_verify_early.restype = i32
    lib.spec_greedy_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spec_greedy_workspace_bytes.restype = sz
    lib.spec_verify_greedy.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_greedy.restype = i32
    lib.spec_read_bandwidth.argtypes = [vp, sz, vp, vp]
    lib.spec_read_bandwidth.restype = i32
    lib.spec_lds_atomic_probe.argtypes = [i32, i32, vp, vp]
    lib.spec_lds_atomic_probe.restype = i32
    lib.spec_verify_noalloc.argtypes = verify_args[:-3] + [vp]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_status_str.argtypes = [i32]
    lib.spec_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


class SpecError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"spec status {status}: {spec_status_str(status)}")
        self.status = status


def spec_status_str(status: int) -> str:
    return load_library().spec_status_str(int(status)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def spec_workspace_bytes(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().spec_workspace_bytes(B, gamma, V, dtype))


def spec_predict_workspace_bytes(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().spec_predict_workspace_bytes(B, gamma, V, dtype))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check_dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("every tensor must be a contiguous device tensor")


def new_workspace(nbytes: int, device):
    """A zero-filled workspace (each call leaves it ready for the next: all
    zero again, but for the rows' statistics of a top-p cut and the lane
    leaders of outcome prediction, which every such call rewrites before it
    reads them)."""
    import torch
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


VerifyOut = collections.namedtuple(
    "VerifyOut", "tokens accepted first_reject accept_mask out_len diag")

DIAG_FIELDS = ("row_max", "row_logZ", "px", "qx", "resid_mass", "token_prob", "cdf_lo", "cdf_hi")


def alloc_outputs(B: int, gamma: int, device, diag: bool = False) -> VerifyOut:
    import torch
    i32 = dict(dtype=torch.int32, device=device)
    d = None
    if diag:
        R = 2 * gamma + 1
        shapes = dict(row_max=(B, R), row_logZ=(B, R), px=(B, gamma), qx=(B, gamma),
                      resid_mass=(B,), token_prob=(B,), cdf_lo=(B,), cdf_hi=(B,))
        d = {k: torch.full(shapes[k], float("nan"), dtype=torch.float64, device=device)
             for k in DIAG_FIELDS}
    return VerifyOut(torch.empty((B, gamma + 1), **i32), torch.empty((B,), **i32),
                     torch.empty((B,), **i32), torch.empty((B,), dtype=torch.int64, device=device),
                     torch.empty((B,), **i32), d)


def _verify_call(saguaro: bool, draft_logits, target_logits, draft_tokens, u_accept, u_sample,
                 temperature: float, in_len=None, out: VerifyOut | None = None, diag: bool = False,
                 workspace=None, stream=None, eps: float = 0.0, pred=None, early=False,
                 temps=None, ex=False, top_p: float = 0.0) -> VerifyOut:
    lib = load_library()
    B, G1, V = draft_logits.shape
    gamma = G1 - 1
    if target_logits.shape != draft_logits.shape or target_logits.dtype != draft_logits.dtype:
        raise ValueError("draft and target logits must share shape and dtype")
    _check_dev(draft_logits, target_logits, draft_tokens, u_accept, u_sample, in_len)
    dt = _dtype_code(draft_logits)
    dev = draft_logits.device
    if out is None:
        out = alloc_outputs(B, gamma, dev, diag)
    need = spec_workspace_bytes(B, gamma, V, dt)
    if workspace is None:
        workspace = new_workspace(need, dev)
    dg = None
    if out.diag is not None:
        dg = SpecDiag(*[out.diag[k].data_ptr() for k in DIAG_FIELDS])
    args = [draft_logits.data_ptr(), target_logits.data_ptr(), dt, draft_tokens.data_ptr(),
            u_accept.data_ptr(), u_sample.data_ptr(), B, gamma, V, float(temperature),
            _ptr(in_len), out.tokens.data_ptr(), out.accepted.data_ptr(),
            out.first_reject.data_ptr(), out.accept_mask.data_ptr(), out.out_len.data_ptr(),
            ctypes.byref(dg) if dg is not None else None, workspace.data_ptr(),
            workspace.numel(), _stream_handle(stream, dev)]
    if ex:
        _check_dev(temps)
        if pred is not None:
            _check_dev(*pred)
        opts = SpecOptions(int(saguaro), float(eps), int(early), _ptr(temps),
                           pred.cand.data_ptr() if pred is not None else None,
                           _ptr(pred.hit) if pred is not None else None,
                           _ptr(pred.cand_idx) if pred is not None else None, float(top_p))
        st = lib.spec_verify_ex(*args[:-3], ctypes.byref(opts), *args[-3:])
    elif early:
        st = lib.spec_verify_early(*args[:-3], int(saguaro), float(eps), *args[-3:])
    elif pred is not None:
        _check_dev(*pred)
        st = lib.spec_verify_predict(*args[:-3], int(saguaro), float(eps), pred.cand.data_ptr(),
                                     _ptr(pred.hit), _ptr(pred.cand_idx), *args[-3:])
    elif saguaro:
        st = lib.spec_verify_saguaro(*args, float(eps))
    else:
        st = lib.spec_verify(*args)
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def spec_verify(draft_logits, target_logits, draft_tokens, u_accept, u_sample, temperature,
                in_len=None, out=None, diag=False, workspace=None, stream=None) -> VerifyOut:
    """Residual-mode verification of a [B, gamma+1, V] batch (see spec_verify.h)."""
    return _verify_call(False, draft_logits, target_logits, draft_tokens, u_accept, u_sample,
                        temperature, in_len, out, diag, workspace, stream)


def spec_verify_noalloc(draft_logits, target_logits, draft_tokens, u_accept, u_sample, temperature,
                        in_len=None, out=None, diag=False, stream=None) -> VerifyOut:
    """spec_verify without a workspace: the library's static per-device
    scratch (see spec_verify.h; calls on one GPU must not overlap).  With
    ``out`` given, nothing is allocated here either."""
    lib = load_library()
    B, G1, V = draft_logits.shape
    gamma = G1 - 1
    if target_logits.shape != draft_logits.shape or target_logits.dtype != draft_logits.dtype:
        raise ValueError("draft and target logits must share shape and dtype")
    _check_dev(draft_logits, target_logits, draft_tokens, u_accept, u_sample, in_len)
    dev = draft_logits.device
    if out is None:
        out = alloc_outputs(B, gamma, dev, diag)
    dg = None
    if out.diag is not None:
        dg = SpecDiag(*[out.diag[k].data_ptr() for k in DIAG_FIELDS])
    st = lib.spec_verify_noalloc(draft_logits.data_ptr(), target_logits.data_ptr(),
                                 _dtype_code(draft_logits), draft_tokens.data_ptr(), u_accept.data_ptr(),
                                 u_sample.data_ptr(), B, gamma, V, float(temperature), _ptr(in_len),
                                 out.tokens.data_ptr(), out.accepted.data_ptr(), out.first_reject.data_ptr(),
                                 out.accept_mask.data_ptr(), out.out_len.data_ptr(),
                                 ctypes.byref(dg) if dg is not None else None, _stream_handle(stream, dev))
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def spec_verify_saguaro(draft_logits, target_logits, draft_tokens, u_accept, u_sample,
                        temperature, in_len=None, out=None, diag=False, workspace=None,
                        stream=None, eps: float = 0.0) -> VerifyOut:
    """Saguaro-mode verification (see spec_verify.h)."""
    return _verify_call(True, draft_logits, target_logits, draft_tokens, u_accept, u_sample,
                        temperature, in_len, out, diag, workspace, stream, eps)


PredictOut = collections.namedtuple("PredictOut", "cand hit cand_idx")


def spec_predict_outcomes(draft_logits, accepted=None, out_tokens=None, out=None,
                          workspace=None, stream=None) -> PredictOut:
    """Top-3 outcome candidates per position and, given a verification's
    outputs, the hit flag and candidate index (see spec_verify.h)."""
    import torch
    lib = load_library()
    B, G1, V = draft_logits.shape
    gamma = G1 - 1
    _check_dev(draft_logits, accepted, out_tokens)
    dt = _dtype_code(draft_logits)
    dev = draft_logits.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = PredictOut(torch.empty((B, G1, 3), **i32), torch.empty((B,), **i32),
                         torch.empty((B,), **i32))
    need = spec_predict_workspace_bytes(B, gamma, V, dt)
    if workspace is None:
        workspace = new_workspace(need, dev)
    st = lib.spec_predict_outcomes(draft_logits.data_ptr(), dt, B, gamma, V, _ptr(accepted),
                                   _ptr(out_tokens), out.cand.data_ptr(), _ptr(out.hit),
                                   _ptr(out.cand_idx), workspace.data_ptr(), workspace.numel(),
                                   _stream_handle(stream, dev))
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def spec_verify_early(draft_logits, target_logits, draft_tokens, u_accept, u_sample, temperature,
                      in_len=None, out=None, diag=False, workspace=None, stream=None,
                      saguaro: bool = False, eps: float = 0.0) -> VerifyOut:
    """Early-exit verification (residual, or Saguaro with ``saguaro=True``):
    rows are read only up to the first rejection (see spec_verify.h)."""
    return _verify_call(bool(saguaro), draft_logits, target_logits, draft_tokens, u_accept,
                        u_sample, temperature, in_len, out, diag, workspace, stream,
                        eps if saguaro else 0.0, None, True)


def spec_verify_ex(draft_logits, target_logits, draft_tokens, u_accept, u_sample, temperature,
                   in_len=None, out=None, diag=False, workspace=None, stream=None,
                   saguaro: bool = False, eps: float = 0.0, early: bool = False, pred=None,
                   top_p: float = 0.0):
    """Verification with options (see spec_verify.h): ``temperature`` is a float
    for the whole batch or a [B] float32 device tensor of per-sequence
    temperatures; ``pred`` (a PredictOut) asks for outcome prediction.
    Returns VerifyOut, or (VerifyOut, PredictOut) when ``pred`` is given."""
    import torch
    temps = temperature if isinstance(temperature, torch.Tensor) else None
    T = 1.0 if temps is not None else float(temperature)
    out = _verify_call(bool(saguaro), draft_logits, target_logits, draft_tokens, u_accept,
                       u_sample, T, in_len, out, diag, workspace, stream,
                       eps if saguaro else 0.0, pred, early, temps, ex=True, top_p=top_p)
    return (out, pred) if pred is not None else out


def spec_synthetic_busy(ns: int, hit=None, stream=None, device=None):
    """Keep one work-group of the stream busy for ns nanoseconds (a stand-in
    for a model forward pass); with ``hit``, only if some flag is 0."""
    import torch
    dev = hit.device if hit is not None else (device or torch.device("cuda"))
    _check_dev(hit)
    st = load_library().spec_synthetic_busy(int(ns), _ptr(hit), 0 if hit is None else hit.numel(),
                                            _stream_handle(stream, dev))
    if st != SPEC_OK:
        raise SpecError(st)


def _bigram(table, noise=None, ints=()):
    import torch
    for t in ints:
        if t is not None and t.dtype != torch.int32:
            raise TypeError(f"token, length and prediction arrays are int32, got {t.dtype}")
    if noise is not None and noise.dtype != torch.float32:
        raise TypeError(f"noise is float32, got {noise.dtype}")
    if table.dim() != 2:
        raise ValueError(f"a bigram table is [H, V], got {tuple(table.shape)}")
    H, V = table.shape
    if noise is not None and (noise.dim() != 2 or noise.shape[1] != V):
        raise ValueError(f"noise is [P, V], got {tuple(noise.shape)}")
    return _dtype_code(table), V, H, 0 if noise is None else noise.shape[0]


def spec_synth_draft(table, noise, gamma: int, start_tok, start_pos=None, out=None, stream=None):
    """gamma Gumbel-max draft steps of the bigram model ``table`` [H, V] after
    each start token (see spec_verify.h); returns out [n, gamma] int32."""
    import torch
    _check_dev(table, noise, start_tok, start_pos, out)
    dt, V, H, P = _bigram(table, noise, (start_tok, start_pos, out))
    n = start_tok.numel()
    if out is None:
        out = torch.empty((n, gamma), dtype=torch.int32, device=table.device)
    st = load_library().spec_synth_draft(table.data_ptr(), dt, V, H, noise.data_ptr(), P, gamma, n,
                                         start_tok.data_ptr(), _ptr(start_pos), out.data_ptr(),
                                         _stream_handle(stream, table.device))
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def spec_synth_rows(table, last, tokens, out=None, stream=None):
    """A round's logits [B, gamma+1, V] from the bigram ``table`` [H, V] (see spec_verify.h)."""
    import torch
    _check_dev(table, last, tokens, out)
    dt, V, H, _ = _bigram(table, None, (last, tokens))
    B, gamma = tokens.shape
    if out is None:
        out = torch.empty((B, gamma + 1, V), dtype=table.dtype, device=table.device)
    st = load_library().spec_synth_rows(table.data_ptr(), dt, V, H, gamma, B, last.data_ptr(),
                                        tokens.data_ptr(), out.data_ptr(),
                                        _stream_handle(stream, table.device))
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def spec_ssd_prespeculate(table, noise, cand, length=None, out=None, stream=None):
    """Drafts [B, 3(gamma+1), gamma] for every predicted outcome of a round
    (cand [B, gamma+1, 3] from spec_predict_outcomes; see spec_verify.h)."""
    import torch
    _check_dev(table, noise, cand, length, out)
    dt, V, H, P = _bigram(table, noise, (cand, length, out))
    B, G1, _ = cand.shape
    if out is None:
        out = torch.empty((B, 3 * G1, G1 - 1), dtype=torch.int32, device=table.device)
    st = load_library().spec_ssd_prespeculate(table.data_ptr(), dt, V, H, noise.data_ptr(), P, G1 - 1,
                                              B, cand.data_ptr(), _ptr(length), out.data_ptr(),
                                              _stream_handle(stream, table.device))
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def spec_ssd_advance(table, noise, vout, pred=None, prepared=None, out=None, stream=None):
    """The committed state and next drafts after a round (see spec_verify.h):
    returns (next_last [B], next_len [B], next_tokens [B, gamma])."""
    import torch
    _check_dev(table, noise, vout.tokens, prepared)
    dt, V, H, P = _bigram(table, noise, (vout.tokens, vout.accepted, vout.out_len, prepared))
    B, G1 = vout.tokens.shape
    if out is None:
        i32 = dict(dtype=torch.int32, device=table.device)
        out = (torch.empty((B,), **i32), torch.empty((B,), **i32), torch.empty((B, G1 - 1), **i32))
    hit = idx = None
    if pred is not None:
        hit, idx = pred.hit, pred.cand_idx
    st = load_library().spec_ssd_advance(
        table.data_ptr(), dt, V, H, noise.data_ptr(), P, G1 - 1, B, vout.tokens.data_ptr(),
        vout.accepted.data_ptr(), vout.out_len.data_ptr(), _ptr(hit), _ptr(idx), _ptr(prepared),
        out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(), _stream_handle(stream, table.device))
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def spec_read_bandwidth(buf, sink, nbytes=None, stream=None):
    """Read nbytes (default: all) of the device tensor ``buf`` with the stream
    items' loads (a measurement aid, see spec_verify.h); ``sink`` is a device
    int64 tensor of at least one element."""
    _check_dev(buf, sink)
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    st = load_library().spec_read_bandwidth(buf.data_ptr(), n, sink.data_ptr(),
                                            _stream_handle(stream, buf.device))
    if st != SPEC_OK:
        raise SpecError(st)


def spec_lds_atomic_probe(pattern: int, iters: int, sink, stream=None):
    """LDS atomic adds in a fixed lane-to-word pattern, one work-group per CU
    (a measurement aid, see spec_verify.h); ``sink`` is a device int64
    tensor of at least one element."""
    _check_dev(sink)
    st = load_library().spec_lds_atomic_probe(int(pattern), int(iters), sink.data_ptr(),
                                              _stream_handle(stream, sink.device))
    if st != SPEC_OK:
        raise SpecError(st)


def spec_greedy_workspace_bytes(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().spec_greedy_workspace_bytes(B, gamma, V, dtype))


def spec_verify_greedy(target_logits, draft_tokens, in_len=None, out=None, workspace=None,
                       stream=None) -> VerifyOut:
    """Greedy (temperature -> 0) verification of a [B, gamma+1, V] batch of
    target logits (see spec_verify.h)."""
    lib = load_library()
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    _check_dev(target_logits, draft_tokens, in_len)
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    if out is None:
        out = alloc_outputs(B, gamma, dev)
    if workspace is None:
        workspace = new_workspace(spec_greedy_workspace_bytes(B, gamma, V, dt), dev)
    st = lib.spec_verify_greedy(target_logits.data_ptr(), dt, draft_tokens.data_ptr(), B, gamma, V,
                                _ptr(in_len), out.tokens.data_ptr(), out.accepted.data_ptr(),
                                out.first_reject.data_ptr(), out.accept_mask.data_ptr(),
                                out.out_len.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream_handle(stream, dev))
    if st != SPEC_OK:
        raise SpecError(st)
    return out


def alloc_predict_outputs(B: int, gamma: int, device) -> "PredictOut":
    import torch
    i32 = dict(dtype=torch.int32, device=device)
    return PredictOut(torch.empty((B, gamma + 1, 3), **i32), torch.empty((B,), **i32),
                      torch.empty((B,), **i32))


def spec_verify_predict(draft_logits, target_logits, draft_tokens, u_accept, u_sample,
                        temperature, in_len=None, out=None, pred=None, diag=False, workspace=None,
                        stream=None, saguaro: bool = False, eps: float = 0.0):
    """Verification (residual, or Saguaro with ``saguaro=True``) and outcome
    prediction in one pass; returns (VerifyOut, PredictOut) (see spec_verify.h)."""
    B, G1, _ = draft_logits.shape
    if pred is None:
        pred = alloc_predict_outputs(B, G1 - 1, draft_logits.device)
    out = _verify_call(bool(saguaro), draft_logits, target_logits, draft_tokens, u_accept,
                       u_sample, temperature, in_len, out, diag, workspace, stream,
                       eps if saguaro else 0.0, pred)
    return out, pred


def bytes_algorithmic(B: int, gamma: int, V: int, dtype: int) -> int:
    """Bytes the method must move once per call: draft rows i < gamma and target
    rows i <= gamma, draft tokens, uniforms, lengths, and the outputs."""
    es = 2 if dtype == SPEC_BF16 else 4
    return ((B * gamma + B * (gamma + 1)) * V * es + B * gamma * 4 + B * gamma * 4
            + B * (gamma + 1) * 4 + B * 4 + B * (gamma + 1) * 4 + B * (4 + 4 + 8 + 4))
