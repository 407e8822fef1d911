"""Seeded synthetic inputs for batched speculative-sampling verification.

This module is the only code shared by the GPU path's tests/benchmark and the
CPU oracle's tests.  It holds input recipes only: it never normalises a
distribution, never forms a ratio q/p, a residual or a CDF.  The random numbers
the verification rule consumes (accept and sample uniforms) are produced here
and handed to both sides as plain buffers.

Recipes (all seeded; Philox counter-based streams, one per (seed, stream, sequence)):

* Toy (speculative-decoding blog, section 3 code, the two-state Markov toy):
  seven-token draft/target tables conditioned on ``prev == 0``; logits are
  ``float32(ln(table))``; draft tokens follow the Markov chain.
* Zipf-plus-Gaussian rows at LLM vocabulary sizes: draft logit of the token of
  rank r is ``-1.1 ln r`` over a fresh random permutation per row plus
  N(0, 0.5^2); target = draft + N(0, sigma^2).  sigma sets the overlap
  alpha = sum_x min(p, q); the sigma(alpha) relation is read from
  ``sigma_table.json`` (written by ``oracle/calibrate_sigma.py``).
* Draft tokens x_i ~ softmax(draft_i / T) by the Gumbel-max construction
  (argmax of l/T + Gumbel noise), which draws from the softmax without
  normalising it.
* Uniforms: ``integers(0, 2**24) * 2**-24`` stored as float32: exact in fp32
  and fp64, in [0, 1), never 1.0.
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# ---------------------------------------------------------------------------
# The toy model: speculative-decoding blog (feifeigd.github.io, 2026-08-24),
# section 3, the runnable toy (draft_dist / target_dist).  Index 0 is the
# "prev == 0" state, index 1 every other state.
TOY_DRAFT = np.array([[0.55, 0.15, 0.10, 0.07, 0.06, 0.04, 0.03],
                      [0.30, 0.20, 0.15, 0.12, 0.10, 0.08, 0.05]], dtype=np.float64)
TOY_TARGET = np.array([[0.50, 0.18, 0.11, 0.08, 0.06, 0.04, 0.03],
                       [0.28, 0.22, 0.16, 0.11, 0.09, 0.08, 0.06]], dtype=np.float64)
TOY_V = 7

DTYPES = ("f32", "bf16")

# Stream ids for the per-purpose Philox generators.
_S_LOGITS, _S_TOKENS, _S_UACC, _S_USAMP, _S_MISC = 1, 2, 3, 4, 5


def philox(seed: int, *key: int) -> np.random.Generator:
    """A Philox-4x64 generator keyed by (seed, *key)."""
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([int(seed), *map(int, key)])))


def uniforms24(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms on the 2^-24 grid in [0, 1), exact in float32."""
    return (rng.integers(0, 1 << 24, size=shape, dtype=np.int64).astype(np.float64)
            * (2.0 ** -24)).astype(np.float32)


# ---------------------------------------------------------------------------
# bfloat16 as raw uint16 bits (numpy has no bfloat16).

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.isnan(x).any():
        raise ValueError("NaN logits are planted as raw bits, not rounded")
    u = u + (((u >> 16) & 1) + np.uint32(0x7FFF))   # no overflow for finite or inf values
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact upcast of bfloat16 bits to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of logits stored as float32 or bfloat16 bits."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def encode(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Store float64 logits in the given dtype (float32 array or bf16 bits)."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


# ---------------------------------------------------------------------------
# Gumbel-max draws (draft-token sampling for the input recipe).

def gumbel(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.gumbel(size=shape)


def gumbel_argmax(logits64: np.ndarray, T: float, rng: np.random.Generator) -> np.ndarray:
    """argmax_j(l_j / T + G_j) over the last axis: a draw from softmax(l / T)."""
    g = gumbel(rng, logits64.shape)
    with np.errstate(invalid="ignore"):
        return np.argmax(logits64 / T + g, axis=-1).astype(np.int32)


# ---------------------------------------------------------------------------
# sigma(alpha) calibration table.

def load_sigma_table() -> dict:
    path = os.path.join(_HERE, "sigma_table.json")
    with open(path) as f:
        return json.load(f)


def sigma_for_alpha(alpha, V: int, T: float, dtype: str, table: dict | None = None) -> np.ndarray:
    """Noise scale sigma giving mean overlap ``alpha`` for Zipf rows at (V, T, dtype).

    Linear interpolation in the stored, monotone alpha(sigma) curve.
    """
    table = table or load_sigma_table()
    key = f"V{V}_T{T:g}_{dtype}"
    if key not in table["curves"]:
        raise KeyError(f"no sigma calibration for {key}; run oracle/calibrate_sigma.py")
    cur = table["curves"][key]
    sig = np.asarray(cur["sigma"], dtype=np.float64)
    alp = np.asarray(cur["alpha"], dtype=np.float64)
    # alpha decreases with sigma; np.interp needs increasing x.
    order = np.argsort(alp)
    return np.interp(np.asarray(alpha, dtype=np.float64), alp[order], sig[order])


def zipf_rows(rng: np.random.Generator, n_rows: int, V: int, draft_noise: float = 0.5) -> np.ndarray:
    """Draft logits: -1.1 ln(rank) over a random permutation per row, + N(0, draft_noise^2)."""
    base = -1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))
    out = np.empty((n_rows, V), dtype=np.float64)
    for r in range(n_rows):
        out[r, rng.permutation(V)] = base
    out += draft_noise * rng.standard_normal((n_rows, V))
    return out


# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Batch:
    """One verification call's inputs.

    draft, target: [B, gamma+1, V] logits, float32 array or bf16 bits (uint16).
    draft_tokens: [B, gamma] int32.  u_accept: [B, gamma] float32.
    u_sample: [B, gamma+1] float32.  in_len: [B] int32.
    """
    name: str
    B: int
    gamma: int
    V: int
    T: float
    dtype: str
    draft: np.ndarray
    target: np.ndarray
    draft_tokens: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray
    in_len: np.ndarray
    alpha_target: np.ndarray | None = None
    seed: int = 0

    def draft64(self) -> np.ndarray:
        return decode_f64(self.draft, self.dtype)

    def target64(self) -> np.ndarray:
        return decode_f64(self.target, self.dtype)

    def subset(self, idx) -> "Batch":
        idx = np.asarray(idx)
        return dataclasses.replace(
            self, B=len(idx), draft=self.draft[idx], target=self.target[idx],
            draft_tokens=self.draft_tokens[idx], u_accept=self.u_accept[idx],
            u_sample=self.u_sample[idx], in_len=self.in_len[idx],
            alpha_target=None if self.alpha_target is None else self.alpha_target[idx])

    @property
    def bytes_alg(self) -> int:
        """Bytes the method must read once: draft rows i<gamma, target rows i<=gamma,
        tokens, uniforms, lengths; plus the outputs written."""
        es = 2 if self.dtype == "bf16" else 4
        B, g, V = self.B, self.gamma, self.V
        return ((B * g + B * (g + 1)) * V * es + B * g * 4 + B * g * 4 + B * (g + 1) * 4
                + B * 4 + B * (g + 1) * 4 + B * (4 + 4 + 8 + 4))


def zipf_batch(name: str, B: int, gamma: int, V: int, T: float, dtype: str, alpha,
               seed: int, seqs=None, table: dict | None = None) -> Batch:
    """Zipf-plus-Gaussian workload.  ``alpha`` is a scalar or a per-sequence array.

    Every sequence b draws from its own Philox streams keyed by (seed, stream, b),
    so any subset ``seqs`` of a batch is reproduced exactly without the rest.
    """
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    alpha = np.broadcast_to(np.asarray(alpha, dtype=np.float64), (B,))
    sigma = sigma_for_alpha(alpha, V, T, dtype, table)
    n = len(seqs)
    es_dtype = np.uint16 if dtype == "bf16" else np.float32
    draft = np.empty((n, gamma + 1, V), dtype=es_dtype)
    target = np.empty((n, gamma + 1, V), dtype=es_dtype)
    tokens = np.empty((n, gamma), dtype=np.int32)
    u_acc = np.empty((n, gamma), dtype=np.float32)
    u_smp = np.empty((n, gamma + 1), dtype=np.float32)
    for j, b in enumerate(seqs):
        rl = philox(seed, _S_LOGITS, b)
        d64 = zipf_rows(rl, gamma + 1, V)
        t64 = d64 + sigma[b] * rl.standard_normal((gamma + 1, V))
        draft[j] = encode(d64, dtype)
        target[j] = encode(t64, dtype)
        d_stored = decode_f64(draft[j, :gamma], dtype)
        tokens[j] = gumbel_argmax(d_stored, T, philox(seed, _S_TOKENS, b))
        u_acc[j] = uniforms24(philox(seed, _S_UACC, b), gamma)
        u_smp[j] = uniforms24(philox(seed, _S_USAMP, b), gamma + 1)
    return Batch(name=name, B=n, gamma=gamma, V=V, T=float(T), dtype=dtype,
                 draft=draft, target=target, draft_tokens=tokens, u_accept=u_acc,
                 u_sample=u_smp, in_len=np.zeros(n, dtype=np.int32),
                 alpha_target=np.asarray(alpha)[seqs].copy(), seed=seed)


def toy_batch(prev, seed: int, round_index: int = 0, gamma: int = 4) -> Batch:
    """Toy Markov rounds, one sequence per entry of ``prev``.

    Row 0 of p and q is conditioned on ``prev``; row i >= 1 on draft token x_{i-1}
    (the toy's draft loop and its one-shot target pass).  Rounds are independent
    given ``prev``; (seed, round_index) keys the streams.
    """
    prev = np.asarray(prev, dtype=np.int64).reshape(-1)
    B = prev.shape[0]
    ln_d = np.log(TOY_DRAFT)
    rng_t = philox(seed, _S_TOKENS, round_index)
    tokens = np.empty((B, gamma), dtype=np.int32)
    states = np.empty((B, gamma + 1), dtype=np.int64)
    state = (prev != 0).astype(np.int64)
    g = gumbel(rng_t, (B, gamma, TOY_V))
    for i in range(gamma):
        states[:, i] = state
        x = np.argmax(ln_d[state] + g[:, i], axis=-1)
        tokens[:, i] = x
        state = (x != 0).astype(np.int64)
    states[:, gamma] = state
    draft = np.log(TOY_DRAFT)[states].astype(np.float32)
    target = np.log(TOY_TARGET)[states].astype(np.float32)
    return Batch(name="toy", B=B, gamma=gamma, V=TOY_V, T=1.0, dtype="f32",
                 draft=draft, target=target, draft_tokens=tokens,
                 u_accept=uniforms24(philox(seed, _S_UACC, round_index), (B, gamma)),
                 u_sample=uniforms24(philox(seed, _S_USAMP, round_index), (B, gamma + 1)),
                 in_len=np.zeros(B, dtype=np.int32), seed=seed)


# ---------------------------------------------------------------------------
# Named workloads.  Seeds are 1200 + the workload's position in the list.

WORKLOADS = {
    # name: (B, gamma, V, T, dtype, alpha, seed)
    "B1_g4_V32000_f32": (1, 4, 32000, 1.0, "f32", 0.8, 1202),
    "B64_g5_V128256_bf16": (64, 5, 128256, 0.8, "bf16", 0.7, 1203),
    "B256_g8_V152064_bf16": (256, 8, 152064, 1.0, "bf16", "spread", 1204),
    "B128_g4_V128256_bf16": (128, 4, 128256, 1.0, "bf16", 0.8, 1205),
}


def workload_alpha(name: str) -> np.ndarray:
    B, _, _, _, _, alpha, _ = WORKLOADS[name]
    if alpha == "spread":
        # alpha spread evenly over [0.5, 0.9] across the sequences.
        return 0.5 + 0.4 * np.arange(B) / max(B - 1, 1)
    return np.full(B, float(alpha))


def _make_part(args):
    name, seqs = args
    return make_workload(name, seqs=seqs)


def make_workload(name: str, seqs=None, table: dict | None = None, workers: int = 1) -> Batch:
    """A named workload (optionally a subset of its sequences).  ``workers`` > 1
    generates sequence blocks in worker processes; the result is identical."""
    B, gamma, V, T, dtype, _, seed = WORKLOADS[name]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    if workers > 1 and len(seqs) > 1:
        import concurrent.futures as cf
        import multiprocessing as mp
        blocks = [b for b in np.array_split(seqs, min(workers, len(seqs))) if len(b)]
        with cf.ProcessPoolExecutor(len(blocks), mp_context=mp.get_context("fork")) as ex:
            parts = list(ex.map(_make_part, [(name, b) for b in blocks]))
        cat = {f: np.concatenate([getattr(p, f) for p in parts])
               for f in ("draft", "target", "draft_tokens", "u_accept", "u_sample", "in_len",
                         "alpha_target")}
        return dataclasses.replace(parts[0], B=len(seqs), **cat)
    return zipf_batch(name, B, gamma, V, T, dtype, workload_alpha(name), seed, seqs=seqs, table=table)


# ---------------------------------------------------------------------------
# Bigram models for the speculative-speculative-decoding pipeline.

@dataclasses.dataclass
class BigramSetup:
    """Inputs of a multi-round pipeline run with synthetic bigram models.

    draft_table, target_table: [H, V] logits (float32 array or bf16 bits); row
    t mod H holds the logits after token t.  noise: [P, V] float32 T-scaled Gumbel
    variates, row = absolute position mod P.  last0, len0: [B] int32 start
    state.  u_accept: [R, B, gamma], u_sample: [R, B, gamma+1] float32.
    """
    name: str
    B: int
    gamma: int
    V: int
    T: float
    dtype: str
    rounds: int
    draft_table: np.ndarray
    target_table: np.ndarray
    noise: np.ndarray
    last0: np.ndarray
    len0: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray
    seed: int = 0

    def draft64(self) -> np.ndarray:
        return decode_f64(self.draft_table, self.dtype)

    def target64(self) -> np.ndarray:
        return decode_f64(self.target_table, self.dtype)


def bigram_setup(B: int, gamma: int, V: int, T: float, rounds: int, seed: int,
                 dtype: str = "bf16", kind: str = "zipf", zipf: float = 1.5,
                 draft_noise: float = 0.5, target_noise: float = 0.6, max_len0: int = 64,
                 P: int | None = None, len_stride: int = 0, H: int | None = None) -> BigramSetup:
    """Bigram tables, noise, start state and uniforms.

    kind "zipf": draft rows -zipf ln(rank) over a random permutation per row
    plus N(0, draft_noise^2); the target adds N(0, target_noise^2) to them.
    kind "hit": peaked draft rows (the top token 25 above a -2 ln(rank) tail)
    and the target equal to the draft: every draft is accepted and the bonus
    is the draft's top token, so every outcome is among the predictions.
    kind "miss": the same draft; the target raises the token the draft ranks
    V/2 to 60, so the first draft is rejected and the residual draw is that
    token, never among the draft's top-3.
    len_stride > 0 gives sequence b the start length b * len_stride (no two
    sequences share a noise row then, when P covers every position).  H rows
    (default V): token t's logits are row t mod H.
    """
    H = V if H is None else H
    rng = philox(seed, _S_LOGITS)
    if kind == "zipf":
        base = -zipf * np.log(np.arange(1, V + 1, dtype=np.float64))
    else:
        base = -2.0 * np.log(np.arange(1, V + 1, dtype=np.float64))
        base[0] += 25.0
    perm = rng.permuted(np.tile(np.arange(V), (H, 1)), axis=1)   # perm[row, rank] = token
    d = np.empty((H, V), dtype=np.float64)
    np.put_along_axis(d, perm, np.broadcast_to(base, (H, V)), axis=1)
    if kind == "zipf":
        d += draft_noise * rng.standard_normal((H, V))
        t = d + target_noise * rng.standard_normal((H, V))
    elif kind == "hit":
        t = d.copy()
    elif kind == "miss":
        t = d.copy()
        t[np.arange(H), perm[:, V // 2]] = 60.0
    else:
        raise ValueError(kind)
    misc = philox(seed, _S_MISC)
    last0 = misc.integers(0, V, size=B).astype(np.int32)
    if len_stride > 0:
        len0 = (np.arange(B) * len_stride).astype(np.int32)
    else:
        len0 = misc.integers(0, max_len0 + 1, size=B).astype(np.int32)
    if P is None:
        P = int(len0.max()) + rounds * (gamma + 1) + 2 * gamma + 2
    noise = (T * philox(seed, _S_TOKENS).gumbel(size=(P, V))).astype(np.float32)
    ua = uniforms24(philox(seed, _S_UACC), (rounds, B, gamma))
    us = uniforms24(philox(seed, _S_USAMP), (rounds, B, gamma + 1))
    return BigramSetup(f"bigram_{kind}_B{B}_g{gamma}_V{V}_{dtype}", B, gamma, V, T, dtype, rounds,
                       encode(d, dtype), encode(t, dtype), noise, last0, len0, ua, us, seed)
