"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP path,
run the oracle on the same inputs, compare per head.

Gate (relative Frobenius error per head, max over heads): 1e-5 for float32
inputs, 5e-3 for bfloat16 inputs with float32 state.  o and S_T are compared
separately."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import scan_sequence_models_amd as gds
from scan_sequence_models_amd import inputs as I

TOL = {"f32": 1e-5, "bf16": 5e-3}


def say(msg: str):
    """Print a progress line (names the case before a GPU step)."""
    print(msg, flush=True)


def dev(x, dtype: str = "f32"):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t) -> np.ndarray:
    return t.float().cpu().numpy()


def gpu_scan(w: I.Workload, b: I.BatchInputs, chunk=None, path="auto", leaf_chunks=0,
             write_state=True):
    q, k, v = dev(b.q, w.dtype), dev(b.k, w.dtype), dev(b.v, w.dtype)
    alpha = dev(b.alpha)
    beta = dev(b.beta) if b.beta is not None else None
    S0 = dev(b.S0) if b.S0 is not None else None
    o, ST = gds.scan_fwd(q, k, v, alpha, beta, S0, chunk=chunk or w.chunk, path=path,
                         leaf_chunks=leaf_chunks, write_state=write_state)
    torch.cuda.synchronize()
    return host(o), (host(ST) if ST is not None else None)


def oracle_scan(w: I.Workload, b: I.BatchInputs, heads=None):
    """Oracle over all heads, or over the listed (b, h) pairs (stacked in that order)."""
    if heads is None:
        return oracle.scan(w.mode, b.q, b.k, b.v, b.alpha, b.beta,
                           None if b.S0 is None else b.S0.astype(np.float64))
    sel = lambda x: None if x is None else np.stack([x[bb, hh] for bb, hh in heads])  # noqa: E731
    S0 = sel(b.S0)
    return oracle.scan(w.mode, sel(b.q), sel(b.k), sel(b.v), sel(b.alpha), sel(b.beta),
                       None if S0 is None else S0.astype(np.float64))


def max_err(x, ref, head_dims):
    return float(np.max(oracle.rel_err_per_head(x, ref, head_dims)))


BLOCK = 64        # tokens per block of the local check
BLOCK_FACTOR = 4  # block gate = BLOCK_FACTOR x the head-wide gate


def block_err(x, ref, head_dims, block=BLOCK):
    """Local companion of the head-wide error, for outputs laid out
    [heads..., T, d]: the largest ||x_b - ref_b||_F over 64-token blocks b (a
    ragged last block holds the remaining tokens), divided by the head's RMS
    norm of a 64-token block, ||ref||_F sqrt(64 / T) (the absolute norm where
    a head's reference is zero).  With a uniform relative error e every block
    reads e, so the head-wide error is the RMS of these ratios; one wrong token
    in a long sequence moves the head-wide figure by 1/sqrt(T / 64) of what it
    moves its block's."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    T = ref.shape[-2]
    heads = ref.shape[:head_dims]
    nb = -(-T // block)
    pad = nb * block - T
    d2 = (x - ref) ** 2
    d2 = d2.reshape(*heads, T, -1).sum(axis=-1)
    if pad:
        d2 = np.concatenate([d2, np.zeros((*heads, pad))], axis=-1)
    blk = np.sqrt(d2.reshape(*heads, nb, block).sum(axis=-1))
    den = np.sqrt(np.sum(ref.reshape(*heads, -1) ** 2, axis=-1)) * np.sqrt(block / T)
    den = np.where(den > 0, den, 1.0)[..., None]
    return float(np.max(blk / den))


def assert_local(o, o_ref, head_dims, tol, what=""):
    """The block check alone, for tests that gate the head-wide error themselves."""
    eb = block_err(o, o_ref, head_dims)
    say(f"  {what} o worst 64-token block {eb:.3e} (block gate {BLOCK_FACTOR * tol:.0e})")
    assert eb <= BLOCK_FACTOR * tol, f"o block error {eb:.3e} > {BLOCK_FACTOR * tol:.0e}"
    return eb


def assert_parity(o, ST, o_ref, ST_ref, dtype, head_dims=2, tol=None, what=""):
    tol = TOL[dtype] if tol is None else tol
    eo = max_err(o, o_ref, head_dims)
    es = max_err(ST, ST_ref, head_dims) if ST is not None else 0.0
    # the block check needs a token axis: o laid out [heads..., T, d]
    eb = block_err(o, o_ref, head_dims) if np.ndim(o_ref) >= head_dims + 2 else 0.0
    say(f"  parity {what}: o {eo:.3e}  S_T {es:.3e}  o worst 64-token block {eb:.3e}  "
        f"(gate {tol:.0e}, block gate {BLOCK_FACTOR * tol:.0e})")
    assert eo <= tol, f"o error {eo:.3e} > {tol:.0e}"
    assert es <= tol, f"S_T error {es:.3e} > {tol:.0e}"
    assert eb <= BLOCK_FACTOR * tol, f"o block error {eb:.3e} > {BLOCK_FACTOR * tol:.0e}"
    return eo, es
