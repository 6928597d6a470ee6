"""Seeded synthetic inputs for the gated-delta / gated-linear-attention scan.

This module holds random distributions, dtype casts and the named workload
shapes, and nothing of the scan's own arithmetic.  It is the one piece that the
CPU oracle's tests and the GPU path share: both draw their inputs here, so the
two sides see bit-identical operands.

Recipe (one independent stream per head):
  * ``numpy.random.default_rng(SeedSequence([seed, b, h]))`` draws, in this
    order, q (T x dk), k (T x dk), v (T x dv), the alpha source (T), the beta
    source (T) and S0 (dv x dk), all in float64;
  * q and k are divided by their per-token Euclidean norm in float64;
  * every value is then rounded float64 -> float32 (round to nearest even) and,
    for bfloat16 workloads, float32 -> bfloat16 (round to nearest even);
  * alpha and beta stay float32; S0 is float32.
Decode workloads draw each state ``n`` from ``SeedSequence([seed, n])``: the
initial state first, then all steps' q, k, v, alpha and beta (see
``decode_state_inputs``).

Diagonal-gate workloads (``diag_gates``) replace alpha by one decay per key
channel, [T, dk] from the alpha distribution, drawn from
``SeedSequence([seed, b, h, 4])``.

Fast-weight workloads (mode "lact") use q, k, v and S0 (as W0) of the recipe
above and draw learning rates ~ U(0, 1) dk / chunk from
``SeedSequence([seed, b, h, 3])``.

PRISM workloads (``prism_steps`` L > 0) add, per head (b, h), from
``SeedSequence([seed, b, h, 1])``: the anchor source x ~ N(0, 1) (T x dv) and
the step gates beta^(l) = sigmoid(N(0, 1)) (T x L); and per head index h,
shared over the batch, from ``SeedSequence([seed, 2**31, h])``: conv taps
~ N(0, 1/W) (W x dv, float32), W_k^(l) ~ N(0, 1/dv) (L x dk x dv) and
W_p^(l) ~ N(0, 1/dv) (L x dv x dv), cast like the data.  Split erase/write
strength tests draw a write plane ~ U(0, 1.5) from ``SeedSequence([seed, b, h, 2])``.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ---------------------------------------------------------------------------
# bfloat16 rounding on the host (round to nearest, ties to even)
# ---------------------------------------------------------------------------


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of ``x`` rounded from float32, RNE.

    Inputs are first rounded to float32.  Finite inputs only (the generators
    never produce NaN or Inf).
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    u = u.astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round to bfloat16 (RNE) and return the exact values as float32."""
    return bf16_to_f32(bf16_bits(x))


def cast(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 (RNE), then -> bfloat16 (RNE) when ``dtype == 'bf16'``.

    Always returns float32 arrays; bfloat16 values are held exactly in float32.
    """
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_round(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# distributions
# ---------------------------------------------------------------------------


def _draw_gate(rng: np.random.Generator, spec, n: int) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":            # x ~ U(lo, hi)
        return rng.uniform(spec[1], spec[2], size=n)
    if kind == "sigmoid_normal":     # x = 1 / (1 + exp(-z)), z ~ N(mu, sigma^2)
        z = rng.normal(spec[1], spec[2], size=n)
        return 1.0 / (1.0 + np.exp(-z))
    if kind == "exp_uniform":        # ln x ~ U(lo, hi)
        return np.exp(rng.uniform(spec[1], spec[2], size=n))
    if kind == "const":
        return np.full(n, float(spec[1]))
    raise ValueError(f"unknown gate distribution {spec!r}")


def _unit_rows(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    x = rng.standard_normal((rows, cols))
    n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
    n[n == 0.0] = 1.0
    return x / n


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value distribution of one synthetic scan workload."""

    name: str
    mode: str            # "gdn" or "gla"
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str           # element type of q, k, v, o: "f32" or "bf16"
    chunk: int
    alpha: tuple         # gate distribution, see _draw_gate
    beta: tuple | None   # None in gla mode
    s0_var: float | None  # None: zero initial state; else S0 ~ N(0, s0_var)
    seed: int
    path: str = "sequential"   # "sequential" or "blelloch"
    steps: int = 0       # decode workloads only: number of consecutive tokens
    prism_steps: int = 0   # PRISM workloads: L rank-1 corrections per token
    prism_window: int = 4  # PRISM workloads: taps W of the anchor convolution
    diag_gates: bool = False  # alpha is one decay per key channel ([T, dk])
    backward: bool = False  # the workload times the gradient (scan_bwd), not the forward

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Named workloads.  Shapes and distributions: q, k ~ N(0, 1) then unit norm per
# token; v ~ N(0, 1); gates and initial states as listed.
WORKLOADS = {
    "tiny-gdn": Workload("tiny-gdn", "gdn", 1, 1, 64, 16, 16, "f32", 16,
                         ("uniform", 0.9, 1.0), ("uniform", 0.0, 1.0), None, seed=1),
    "gla-b4h8t4096": Workload("gla-b4h8t4096", "gla", 4, 8, 4096, 128, 128, "bf16", 64,
                              ("exp_uniform", -0.05, 0.0), None, None, seed=2),
    "gdn-b8h16t8192": Workload("gdn-b8h16t8192", "gdn", 8, 16, 8192, 128, 128, "bf16", 64,
                               ("sigmoid_normal", 3.0, 1.0), ("sigmoid_normal", 0.0, 1.0), 0.01,
                               seed=3),
    # 256 sequences x 16 heads = 4096 independent 128x128 states, 100 tokens each.
    "decode-4096x100": Workload("decode-4096x100", "gdn", 256, 16, 1, 128, 128, "bf16", 1,
                                ("uniform", 0.9, 1.0), ("uniform", 0.0, 1.0), 0.01, seed=4,
                                path="decode", steps=100),
    "long-b2h8t262144": Workload("long-b2h8t262144", "gdn", 2, 8, 262144, 128, 128, "bf16", 64,
                                 ("uniform", 0.97, 1.0), ("sigmoid_normal", 0.0, 1.0), 0.01,
                                 seed=5, path="blelloch"),
    # PRISM: the training-shape gated delta rule with L = 2 corrections per token
    "prism-b8h16t8192-l2": Workload("prism-b8h16t8192-l2", "gdn", 8, 16, 8192, 128, 128, "bf16",
                                    64, ("sigmoid_normal", 3.0, 1.0), ("sigmoid_normal", 0.0, 1.0),
                                    0.01, seed=6, prism_steps=2, prism_window=4),
    "tiny-prism": Workload("tiny-prism", "gdn", 1, 2, 64, 16, 16, "f32", 16,
                           ("uniform", 0.9, 1.0), ("uniform", 0.0, 1.0), None, seed=7,
                           prism_steps=2, prism_window=4),
    # Large-chunk fast-weight update: chunk = 2048 tokens, W0 ~ N(0, 0.01); the
    # alpha field is unused (eta comes from lact_eta)
    "lact-b8h16t8192-m2048": Workload("lact-b8h16t8192-m2048", "lact", 8, 16, 8192, 128, 128,
                                      "bf16", 2048, ("const", 1.0), None, 0.01, seed=8),
    "tiny-lact": Workload("tiny-lact", "lact", 1, 2, 100, 16, 16, "f32", 16, ("const", 1.0),
                          None, 0.01, seed=9),
    # Diagonal (per-key-channel) gates: the training shape with alpha drawn per
    # channel from the gated-delta distribution
    "gdn-diag-b8h16t8192": Workload("gdn-diag-b8h16t8192", "gdn", 8, 16, 8192, 128, 128, "bf16",
                                    64, ("sigmoid_normal", 3.0, 1.0), ("sigmoid_normal", 0.0, 1.0),
                                    0.01, seed=10, diag_gates=True),
    "tiny-gla-diag": Workload("tiny-gla-diag", "gla", 1, 2, 77, 16, 16, "f32", 16,
                              ("uniform", 0.8, 1.0), None, 0.01, seed=11, diag_gates=True),
    # The gradient of the training shape: the inputs of gdn-b8h16t8192 (same
    # seed) and incoming gradients dO, dST from output_grads
    "gdn-bwd-b8h16t8192": Workload("gdn-bwd-b8h16t8192", "gdn", 8, 16, 8192, 128, 128, "bf16", 32,
                                   ("sigmoid_normal", 3.0, 1.0), ("sigmoid_normal", 0.0, 1.0),
                                   0.01, seed=3, backward=True),
}


@dataclasses.dataclass
class HeadInputs:
    q: np.ndarray      # [T, dk] float32 (bf16-exact for bf16 workloads)
    k: np.ndarray      # [T, dk]
    v: np.ndarray      # [T, dv]
    alpha: np.ndarray  # [T] float32
    beta: np.ndarray | None  # [T] float32, None in gla mode
    S0: np.ndarray | None    # [dv, dk] float32, None for a zero initial state


def head_inputs(w: Workload, b: int, h: int, T: int | None = None) -> HeadInputs:
    """Inputs of head (b, h) of workload ``w``; ``T`` overrides the sequence length.

    A shorter ``T`` is a fresh draw of that length from the same stream, not a
    prefix of the full-length head.
    """
    T = w.T if T is None else T
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, h]))
    q = cast(_unit_rows(rng, T, w.dk), w.dtype)
    k = cast(_unit_rows(rng, T, w.dk), w.dtype)
    v = cast(rng.standard_normal((T, w.dv)), w.dtype)
    alpha = cast(_draw_gate(rng, w.alpha, T), "f32")
    beta = cast(_draw_gate(rng, w.beta, T), "f32") if w.beta is not None else None
    S0 = None
    if w.s0_var is not None:
        S0 = cast(rng.normal(0.0, np.sqrt(w.s0_var), size=(w.dv, w.dk)), "f32")
    return HeadInputs(q, k, v, alpha, beta, S0)


@dataclasses.dataclass
class BatchInputs:
    q: np.ndarray      # [B, H, T, dk] float32
    k: np.ndarray
    v: np.ndarray      # [B, H, T, dv]
    alpha: np.ndarray  # [B, H, T]
    beta: np.ndarray | None
    S0: np.ndarray | None  # [B, H, dv, dk]

    def head(self, b: int, h: int) -> HeadInputs:
        return HeadInputs(self.q[b, h], self.k[b, h], self.v[b, h], self.alpha[b, h],
                          None if self.beta is None else self.beta[b, h],
                          None if self.S0 is None else self.S0[b, h])


def batch_inputs(w: Workload, threads: int = 8) -> BatchInputs:
    """All heads of ``w`` as [B, H, ...] float32 arrays (heads drawn in parallel)."""
    B, H, T = w.B, w.H, w.T
    q = np.empty((B, H, T, w.dk), np.float32)
    k = np.empty((B, H, T, w.dk), np.float32)
    v = np.empty((B, H, T, w.dv), np.float32)
    alpha = np.empty((B, H, T), np.float32)
    beta = np.empty((B, H, T), np.float32) if w.beta is not None else None
    S0 = np.empty((B, H, w.dv, w.dk), np.float32) if w.s0_var is not None else None

    def fill(bh):
        b, h = divmod(bh, H)
        x = head_inputs(w, b, h)
        q[b, h], k[b, h], v[b, h], alpha[b, h] = x.q, x.k, x.v, x.alpha
        if beta is not None:
            beta[b, h] = x.beta
        if S0 is not None:
            S0[b, h] = x.S0

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, range(B * H)))
    return BatchInputs(q, k, v, alpha, beta, S0)


# ---------------------------------------------------------------------------
# decode workloads
# ---------------------------------------------------------------------------


def decode_state_inputs(w: Workload, n: int, steps: int):
    """Initial state and ``steps`` consecutive tokens of decode state ``n``.

    One stream per state, ``SeedSequence([seed, n])``, drawn in the order
    S0 (dv x dk), q (steps x dk), k (steps x dk), v (steps x dv), alpha (steps),
    beta (steps).
    """
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, n]))
    S0 = cast(rng.normal(0.0, np.sqrt(w.s0_var), size=(w.dv, w.dk)), "f32")
    q = cast(_unit_rows(rng, steps, w.dk), w.dtype)
    k = cast(_unit_rows(rng, steps, w.dk), w.dtype)
    v = cast(rng.standard_normal((steps, w.dv)), w.dtype)
    alpha = cast(_draw_gate(rng, w.alpha, steps), "f32")
    beta = cast(_draw_gate(rng, w.beta, steps), "f32") if w.beta is not None else None
    return S0, q, k, v, alpha, beta


def decode_inputs(w: Workload, N: int | None = None, steps: int | None = None,
                  threads: int = 8):
    """Initial states [N, dv, dk] and per-step tokens [steps, N, ...] for ``w``."""
    N = w.B * w.H if N is None else N
    steps = w.steps if steps is None else steps
    S0 = np.empty((N, w.dv, w.dk), np.float32)
    q = np.empty((steps, N, w.dk), np.float32)
    k = np.empty((steps, N, w.dk), np.float32)
    v = np.empty((steps, N, w.dv), np.float32)
    alpha = np.empty((steps, N), np.float32)
    beta = np.empty((steps, N), np.float32) if w.beta is not None else None

    def fill(n):
        s0, tq, tk, tv, ta, tb = decode_state_inputs(w, n, steps)
        S0[n], q[:, n], k[:, n], v[:, n], alpha[:, n] = s0, tq, tk, tv, ta
        if beta is not None:
            beta[:, n] = tb

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, range(N)))
    return S0, q, k, v, alpha, beta


# ---------------------------------------------------------------------------
# split erase / write strengths and PRISM write inputs
# ---------------------------------------------------------------------------


def write_strengths(w: Workload, b: int, h: int, T: int | None = None) -> np.ndarray:
    """A write-strength plane for head (b, h): U(0, 1.5), float32."""
    T = w.T if T is None else T
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, h, 2]))
    return cast(rng.uniform(0.0, 1.5, T), "f32")


@dataclasses.dataclass
class PrismWeights:
    conv: np.ndarray  # [W, dv] float32
    Wk: np.ndarray    # [L, dk, dv] float32 (values of the data type)
    Wp: np.ndarray    # [L, dv, dv]


def prism_weights(w: Workload, h: int) -> PrismWeights:
    """Anchor taps and projections of head index h (shared by every batch row)."""
    L, W = w.prism_steps, w.prism_window
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 2**31, h]))
    conv = cast(rng.normal(0.0, np.sqrt(1.0 / W), size=(W, w.dv)), "f32")
    Wk = cast(rng.normal(0.0, np.sqrt(1.0 / w.dv), size=(L, w.dk, w.dv)), w.dtype)
    Wp = cast(rng.normal(0.0, np.sqrt(1.0 / w.dv), size=(L, w.dv, w.dv)), w.dtype)
    return PrismWeights(conv, Wk, Wp)


def prism_token_inputs(w: Workload, b: int, h: int, T: int | None = None):
    """Anchor source x [T, dv] (data type) and step gates beta^(l) [T, L] of head (b, h)."""
    T = w.T if T is None else T
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, h, 1]))
    x = cast(rng.standard_normal((T, w.dv)), w.dtype)
    z = rng.normal(0.0, 1.0, size=(T, w.prism_steps))
    beta_l = cast(1.0 / (1.0 + np.exp(-z)), "f32")
    return x, beta_l


def lact_eta(w: Workload, b: int, h: int, T: int | None = None) -> np.ndarray:
    """Learning rates of head (b, h) for a fast-weight workload: U(0, 1) * dk / chunk,
    float32, from ``SeedSequence([seed, b, h, 3])`` (so that |eta K^T K| stays
    near 1/2 and the chunk update is a contraction)."""
    T = w.T if T is None else T
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, h, 3]))
    return cast(rng.uniform(0.0, 1.0, T) * w.dk / w.chunk, "f32")


def diag_alpha(w: Workload, b: int, h: int, T: int | None = None) -> np.ndarray:
    """Per-key-channel decays [T, dk] of head (b, h) for a diagonal-gate workload,
    drawn from the workload's alpha distribution, float32, from
    ``SeedSequence([seed, b, h, 4])``."""
    T = w.T if T is None else T
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, h, 4]))
    return cast(_draw_gate(rng, w.alpha, T * w.dk).reshape(T, w.dk), "f32")


def output_grads(w: Workload, b: int, h: int, T: int | None = None):
    """Incoming gradients for the backward pass of head (b, h): dO [T, dv] ~ N(0, 1)
    cast like the data, and dST [dv, dk] ~ N(0, 1) float32, from
    ``SeedSequence([seed, b, h, 5])``."""
    T = w.T if T is None else T
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, b, h, 5]))
    dO = cast(rng.standard_normal((T, w.dv)), w.dtype)
    dST = cast(rng.standard_normal((w.dv, w.dk)), "f32")
    return dO, dST

