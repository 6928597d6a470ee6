#!/usr/bin/env python3
"""Throughput of the forward gated-delta scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one scan_fwd call over one batch of synthetic inputs that are
already resident in HBM: B=8 sequences x H=16 heads x T=8192 tokens, d=128,
bf16 q/k/v, fp32 state, chunk 64 (the gated-delta training-shape forward).
Prints one JSON line with tokens/s, the roofline of the dominant kernel and the
float64 CPU oracle timed on a bounded sample of the same workload.

Other workloads: --workload gla-b4h8t4096 (gated linear attention),
long-b2h8t262144 (the long-sequence path), decode-4096x100 (decode_step over
4096 states, one timed step per token), prism-b8h16t8192-l2 (the PRISM layer:
the factor rows, then the 3x longer element stream scanned in place) and
lact-b8h16t8192-m2048 (lact_fwd: the large-chunk fast-weight update, chunks of
2048 tokens), gdn-diag-b8h16t8192 (the gated delta rule with one decay per
key channel) and gdn-bwd-b8h16t8192 (scan_bwd: the gradient of the training
shape with respect to every input).  Timing: W untimed steps (by default
enough to cover the GPU's clock ramp), then two HIP events around K back-to-back
steps on the launch stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s fwd gated-delta scan (H=16,d=128,T=8192); % MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
FP32_MFMA_PEAK_TFS = 157.3   # MI355X dense fp32 MFMA
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def scan_bytes(w) -> int:
    """Algorithmic HBM bytes of one scan_fwd call: q, k, v read and o written
    once (dtype), alpha (+ beta) read once (fp32), S0 read and S_T written once
    (fp32).  Intermediates stay on chip."""
    es = 2 if w.dtype == "bf16" else 4
    ht = w.B * w.H * w.T
    b = ht * (2 * w.dk + 2 * w.dv) * es
    b += ht * 4 * {"gdn": 2, "gla": 1, "gdn_ew": 3}[w.mode]  # alpha and strength planes
    b += w.B * w.H * w.dv * w.dk * 4 * (2 if w.s0_var is not None else 1)
    return b


def scan_flops(w) -> float:
    """Dense-tile MFMA flops of the chunk algorithm per call, every C x C-sized
    product counted in full (the kernels skip tiles above the diagonal, so
    this is neither the executed nor the useful count; reported beside the
    algorithmic figure for comparison):
    gdn: 5 C^2-sized products (K K^T, Q K^T, W, U~, P U) = 10 C d per
    head-token, 3 state products (W S^T, Q S^T, U^T D K) = 6 d^2, UT solve C^2/3;
    gla: 2 C^2 products (Q K^T, P V) and 2 state products."""
    C, d = w.chunk, w.dk
    per = (10 * C * d + 6 * d * d + C * C / 3) if w.mode == "gdn" else (4 * C * d + 4 * d * d)
    return per * w.B * w.H * w.T


def scan_flops_alg(w) -> float:
    """Algorithmic flops per call: the triangular products counted at their
    useful size (half of each C x C-sized product), state products in full and
    the UT solve C^2/3 per head-token; gla: Q K^T and P V at half size plus the
    two state products."""
    C, d = w.chunk, w.dk
    per = (5 * C * d + 6 * d * d + C * C / 3) if w.mode == "gdn" else (2 * C * d + 4 * d * d)
    return per * w.B * w.H * w.T


def diag_mfma_flops(w) -> float:
    """Executed float32 MFMA flops of one diagonal-gate call: per 32-token chunk
    and 64-row value slice, X = R_v - R_w S^T and (Q gamma) S^T (2 * 32 * 64 * dk
    each), T X and P U (2 * 32 * 64 * 32 each) and the state update
    (2 * 64 * dk * 32); the linear-attention mode has no X and no T X.  The
    decayed Gram and scores (one exp2 per token pair and channel) run on the
    vector ALUs and are not counted."""
    C, S, d = 32, 64, w.dk
    per = 2 * C * S * (3 * d + 2 * C) if w.mode == "gdn" else 2 * C * S * (2 * d + C)
    return per * -(-w.T // C) * (w.dv // S) * w.B * w.H


def source_sha(paths) -> str:
    """First 16 hex digits of the SHA-256 of a source file (or of several,
    concatenated in the order given)."""
    h = hashlib.sha256()
    for path in [paths] if isinstance(paths, str) else paths:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def decode_bytes(w) -> int:
    """Algorithmic HBM bytes of one decode_step over all states: the fp32 state
    read and written once, q, k, v read and o written once, alpha (+ beta)."""
    es = 2 if w.dtype == "bf16" else 4
    N = w.B * w.H
    b = N * w.dv * w.dk * 4 * 2
    b += N * (2 * w.dk + 2 * w.dv) * es
    b += N * 4 * (2 if w.mode == "gdn" else 1)
    return b


def measured_traffic(kernel_src, summary: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken
    (``kernel_src``: one source file, or a list whose concatenation is hashed)."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_sha(kernel_src):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, heads: int):
    """The float64 oracle, as it stands, on the first ``heads`` heads of ``w``
    (full length each), using every host core it is given."""
    import numpy as np

    import oracle
    from scan_sequence_models_amd import inputs as I

    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:heads]
    hs = [I.head_inputs(w, b, h) for b, h in sel]
    st = lambda f: None if getattr(hs[0], f) is None else np.stack([getattr(x, f) for x in hs])  # noqa: E731
    q, k, v, a, be, S0 = st("q"), st("k"), st("v"), st("alpha"), st("beta"), st("S0")
    S0 = None if S0 is None else S0.astype(np.float64)
    mode = w.mode
    if w.diag_gates:
        a = np.stack([I.diag_alpha(w, b, h) for b, h in sel])
        mode = w.mode + "_diag"
    oracle.build(force=False)
    t0 = time.perf_counter()
    _, _, threads = oracle.scan(mode, q, k, v, a, be, S0, return_threads=True)
    sec = time.perf_counter() - t0
    head_tokens = len(sel) * w.T
    return {
        "value": head_tokens / w.H / sec,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(sel)} of {w.B * w.H} heads x {w.T} tokens ({head_tokens} head-tokens, "
                  f"= {head_tokens // w.H} tokens of all {w.H} heads), float64 token recurrence, "
                  f"{sec:.2f} s",
        "head_tokens_per_s": head_tokens / sec,
        "seconds": sec,
    }


def cpu_baseline_decode(w, states: int):
    """The float64 oracle's decode step on the first ``states`` states of ``w``,
    all of the workload's steps each."""
    import numpy as np

    import oracle
    from scan_sequence_models_amd import inputs as I

    S0, q, k, v, a, be = I.decode_inputs(w, N=states, threads=16)
    S = S0.astype(np.float64)
    oracle.build(force=False)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    for t in range(w.steps):
        oracle.decode_step(w.mode, q[t], k[t], v[t], a[t], None if be is None else be[t], S,
                           threads=threads)
    sec = time.perf_counter() - t0
    state_steps = states * w.steps
    return {
        "value": state_steps / w.H / sec,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{states} of {w.B * w.H} states x {w.steps} steps ({state_steps} state-steps "
                  f"= {state_steps // w.H} tokens of all {w.H} heads), float64, {sec:.2f} s",
        "seconds": sec,
    }


def timed(step, K: int, dev):
    """Run step(0..K-1) back to back on the current stream between two HIP
    events (after a device synchronize); returns (event span in ms, wall s)."""
    import torch

    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), time.perf_counter() - t0


def warm_up(step, W: int, min_ms: float) -> int:
    """W untimed calls of step(i), then more, in groups of 8, until at least
    ``min_ms`` of back-to-back work has run: the GPU raises its clock over the
    first ~15 ms of sustained load, so a fixed count alone can stop inside that
    ramp.  Returns the number of calls made."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(W):
        step(n)
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def rotation_sets(set_bytes: int, min_sets: int, min_total: int) -> int:
    """Input sets the timed calls cycle through so that no set is still in the
    256 MB MALL when it comes round again: at least ``min_sets`` and more than
    ``min_total`` bytes in all."""
    return max(min_sets, -(-(min_total + 1) // max(set_bytes, 1)))


MALL_BYTES = 256 << 20


def copy_probe(mib: int, dev):
    """One plain device copy of ``mib`` MiB (a kernel of known traffic that
    calibrates the rocprofv3 FETCH_SIZE / WRITE_SIZE counters)."""
    if not mib:
        return
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def bench_decode(args, w):
    """decode_step over all B*H states, ``steps`` launches back to back on the
    same states (in place), each with its own token."""
    import numpy as np
    import torch

    import scan_sequence_models_amd as gds
    from scan_sequence_models_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N = w.B * w.H
    nsteps = w.steps
    log(f"bench: generating {w.name} (N={N} states, d={w.dk}, {nsteps} tokens each)")
    S0, q, k, v, a, be = I.decode_inputs(w, threads=16)
    bf = w.dtype == "bf16"

    def up(x, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(torch.bfloat16) if bf16 else t

    # R disjoint state sets (more than twice the MALL in all) taken in turn,
    # so that a step never finds its states left in the MALL by the step
    # before; set r is a head-rolled copy of the generated states (the same
    # distribution, other addresses) and advances by one token every R steps
    R = args.rotate if args.rotate else rotation_sets(N * w.dv * w.dk * 4, 3, 2 * MALL_BYTES)
    S_sets = [up(np.roll(S0, r, axis=0)) for r in range(R)]
    del S0
    q, k, v, a = up(q, bf), up(k, bf), up(v, bf), up(a)
    be = up(be) if be is not None else None
    o_sets = [torch.empty((N, w.dv), dtype=q.dtype, device=dev) for _ in range(R)]

    def step(i):
        t, r = i % nsteps, i % R
        gds.decode_step(q[t], k[t], v[t], a[t], None if be is None else be[t], S_sets[r],
                        o=o_sets[r])

    copy_probe(args.copy_probe_mib, dev)

    warm_calls = warm_up(step, args.warmup, args.warmup_ms)
    K = args.steps if args.steps else nsteps
    span_ms, wall = timed(lambda i: step(warm_calls + i), K, dev)
    ms_per_step = span_ms / K
    kern_ms = ms_per_step  # one kernel launch per step
    log(f"bench: {warm_calls} warm-up steps, then {K} decode steps back to back over {R} "
        f"state sets, span {span_ms:.3f} ms ({kern_ms * 1e3:.2f} us per launch), "
        f"wall {wall * 1e3:.1f} ms")
    alg = decode_bytes(w)
    gbs = alg / (kern_ms / 1e3) / 1e9
    src = os.path.join(ROOT, "scan_sequence_models_amd", "csrc", "decode.hip")
    result = {
        "metric": "tokens/s decode_step (256 sequences x 16 heads, d=128); % HBM roofline",
        "value": w.B * 1 / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "states": N, "sequences": w.B, "H": w.H,
                   "dk": w.dk, "dv": w.dv, "io_dtype": w.dtype, "state_dtype": "f32",
                   "rotated_state_sets": R, "rotated_bytes": R * N * w.dv * w.dk * 4,
                   "warmup_calls_run": warm_calls},
        "roofline": {
            "bound": "hbm",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic(src, f"decode_{w.name}_traffic.txt"),
            "kernel": "decode_kernel",
            "algorithmic_bytes_per_launch": alg,
            "kernel_ms": kern_ms,
        },
    }
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle on {args.cpu_states} states")
        result["cpu_baseline"] = cpu_baseline_decode(w, args.cpu_states)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def cpu_baseline_prism(w, heads: int):
    """The float64 PRISM oracle (write factors, expansion, token recurrence) on
    the first ``heads`` heads of ``w``, full length each."""
    import numpy as np

    import oracle
    from oracle import prism as oprism
    from scan_sequence_models_amd import inputs as I

    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:heads]
    hs = [I.head_inputs(w, b, h) for b, h in sel]
    tok = [I.prism_token_inputs(w, b, h) for b, h in sel]
    wts = [I.prism_weights(w, h) for _, h in sel]
    rnd = (lambda z: I.cast(z, "bf16").astype(np.float64)) if w.dtype == "bf16" else None
    oracle.build(force=False)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    for x, (xs, bl), p in zip(hs, tok, wts):
        oprism.prism_scan(x.q, x.k, x.v, x.alpha, x.beta, xs, p.conv, p.Wk, p.Wp, bl,
                          None if x.S0 is None else x.S0.astype(np.float64), factor_round=rnd,
                          threads=threads)
    sec = time.perf_counter() - t0
    head_tokens = len(sel) * w.T
    return {
        "value": head_tokens / w.H / sec,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(sel)} of {w.B * w.H} heads x {w.T} tokens ({head_tokens} head-tokens), "
                  f"float64 write factors + token recurrence over {w.prism_steps + 1} elements "
                  f"per token, {sec:.2f} s",
        "seconds": sec,
    }


def prism_layer_bytes(w) -> int:
    """Algorithmic HBM bytes of one PRISM layer on the in-place path
    (prism_scan): q, k, v, x read and o written once (dtype); alpha, beta and
    beta^(l) read once (fp32); the factor rows k^(l), delta^(l) written once and
    read once (dtype); the per-head weights (L (dk + dv) dv elements, conv
    W dv fp32) read once; S0 read and S_T written once (fp32)."""
    es = 2 if w.dtype == "bf16" else 4
    L = w.prism_steps
    ht = w.B * w.H * w.T
    b = ht * (2 * w.dk + 3 * w.dv) * es + ht * 4 * (2 + L)
    b += 2 * ht * L * (w.dk + w.dv) * es
    b += w.H * (L * (w.dk + w.dv) * w.dv * es + w.prism_window * w.dv * 4)
    b += 2 * w.B * w.H * w.dv * w.dk * 4
    return b


def bench_prism(args, w):
    """The PRISM layer: prism_scan (the factor rows, then the element stream
    scanned in place); the materialised-stream path (prism_expand, then scan_fwd
    over the stream) is timed beside it for comparison."""
    import numpy as np
    import torch

    import scan_sequence_models_amd as gds
    from scan_sequence_models_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, T, L = w.B, w.H, w.T, w.prism_steps
    G = L + 1
    log(f"bench: generating {w.name} (B={B} H={H} T={T} d={w.dk} L={L})")
    b = I.batch_inputs(w, threads=16)
    bf = w.dtype == "bf16"
    xs = np.empty((B, H, T, w.dv), np.float32)
    bl = np.empty((B, H, T, L), np.float32)
    for bb in range(B):
        for hh in range(H):
            xs[bb, hh], bl[bb, hh] = I.prism_token_inputs(w, bb, hh)

    def up(x, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(torch.bfloat16) if bf16 else t

    def rolled(x, r, bf16=False):
        y = np.roll(x.reshape(B * H, *x.shape[2:]), r, axis=0).reshape(x.shape)
        return up(y, bf16)

    # input sets rotated across the timed calls (heads rolled), past the MALL
    es = 2 if bf else 4
    set_bytes = B * H * T * ((2 * w.dk + 2 * w.dv) * es + 4 * (2 + L))
    R = args.rotate or rotation_sets(set_bytes, 3, 2 * MALL_BYTES)
    sets = []
    for r in range(R):
        sets.append(dict(q=rolled(b.q, r, bf), k=rolled(b.k, r, bf), v=rolled(b.v, r, bf),
                         alpha=rolled(b.alpha, r), beta=rolled(b.beta, r), x=rolled(xs, r, bf),
                         beta_l=rolled(bl, r)))
    S0 = up(b.S0)
    del b, xs, bl
    wts = [I.prism_weights(w, hh) for hh in range(H)]
    conv = up(np.stack([p.conv for p in wts]))
    Wk = up(np.stack([p.Wk for p in wts]), bf)
    Wp = up(np.stack([p.Wp for p in wts]), bf)
    dt = sets[0]["q"].dtype
    o = torch.empty((B, H, T, w.dv), dtype=dt, device=dev)
    ST = torch.empty((B, H, w.dv, w.dk), dtype=torch.float32, device=dev)
    ws = torch.empty(gds.prism_scan_workspace_size(gds.SCAN_BF16 if bf else gds.SCAN_F32,
                                                   B, H, T, w.dk, w.dv, L),
                     dtype=torch.uint8, device=dev)

    def step(i):
        z = sets[i % R]
        gds.prism_scan(z["q"], z["k"], z["v"], z["alpha"], z["beta"], z["x"], z["beta_l"], conv, Wk, Wp,
                       S0, o=o, ST=ST, workspace=ws)

    copy_probe(args.copy_probe_mib, dev)
    warm_calls = warm_up(step, args.warmup, args.warmup_ms)
    span_ms, wall = timed(step, args.steps, dev)
    ms_per_step = span_ms / args.steps
    # the materialised-stream path, for comparison (its own buffers)
    T2 = T * G
    stream_bufs = (torch.empty((B, H, T2, w.dk), dtype=dt, device=dev),
                   torch.empty((B, H, T2, w.dk), dtype=dt, device=dev),
                   torch.empty((B, H, T2, w.dv), dtype=dt, device=dev),
                   torch.empty((B, H, T2), dtype=torch.float32, device=dev),
                   torch.empty((2, B, H, T2), dtype=torch.float32, device=dev))
    o2 = torch.empty((B, H, T2, w.dv), dtype=dt, device=dev)
    del ws

    def stream_step(i):
        z = sets[i % R]
        gds.prism_expand(z["q"], z["k"], z["v"], z["alpha"], z["beta"], z["x"], z["beta_l"], conv, Wk, Wp,
                         out=stream_bufs)
        gds.scan_fwd(*stream_bufs, S0, chunk=w.chunk, o=o2, ST=ST)

    warm_up(stream_step, 2, args.warmup_ms / 4)
    stream_ms = timed(stream_step, args.steps, dev)[0] / args.steps
    log(f"bench: {args.steps} layer steps, {ms_per_step:.4f} ms per step in place "
        f"({stream_ms:.4f} ms through the materialised stream), wall {wall * 1e3:.1f} ms")
    alg = prism_layer_bytes(w)
    scan_flops_alg_ = scan_flops_alg(w.replace(T=T2))
    csrc = os.path.join(ROOT, "scan_sequence_models_amd", "csrc")
    src_layer = [os.path.join(csrc, "prism.hip"), os.path.join(csrc, "chunk_bf16.hip")]
    result = {
        "metric": "tokens/s PRISM layer fwd (rank-L write, L=2; H=16, d=128, T=8192); "
                  "% MFMA / HBM roofline",
        "value": B * T / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": "gdn_ew (PRISM, element stream read in place)", "B": B,
                   "H": H, "T": T, "elements_per_token": G, "L": L, "W": w.prism_window, "dk": w.dk,
                   "dv": w.dv, "chunk": w.chunk, "io_dtype": w.dtype, "state_dtype": "f32",
                   "rotated_input_sets": R, "rotated_bytes": R * set_bytes, "warmup_calls_run": warm_calls},
        "roofline": {
            "bound": "hbm",
            "achieved": alg / (ms_per_step / 1e3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": alg / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic(src_layer, f"prism_layer_{w.name}_traffic.txt"),
            "kernel": "the layer: prism_mfma_kernel (factor rows) + chunk_mfma_kernel (in-place stream)",
            "algorithmic_bytes_per_launch": alg,
            "kernel_ms": ms_per_step,
            "alg_tflops": scan_flops_alg_ / (ms_per_step / 1e3) / 1e12,
            "alg_mfma_frac": scan_flops_alg_ / (ms_per_step / 1e3) / 1e12 / BF16_MFMA_PEAK_TFS,
        },
        "materialised_stream_ms": stream_ms,
    }
    if not args.no_cpu_baseline:
        heads = min(args.cpu_heads, 16)
        log(f"bench: timing the CPU PRISM oracle on {heads} heads")
        result["cpu_baseline"] = cpu_baseline_prism(w, heads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def lact_bytes(w) -> int:
    """Algorithmic HBM bytes of one lact_fwd call: q, k, v read and o written
    once (dtype), eta read once (fp32), W0 read and W_T written once (fp32)."""
    es = 2 if w.dtype == "bf16" else 4
    ht = w.B * w.H * w.T
    return ht * (2 * w.dk + 2 * w.dv) * es + ht * 4 + 2 * w.B * w.H * w.dv * w.dk * 4


def lact_flops(w) -> float:
    """Algorithmic flops of one lact_fwd call: per token G = K^T diag(eta) K,
    F = V^T diag(eta) K and the read-out (2 d^2 each), per chunk W G (2 d^3)."""
    d = w.dk
    nch = -(-w.T // w.chunk)
    return w.B * w.H * (w.T * 6 * d * d + nch * 2 * d ** 3)


def cpu_baseline_lact(w, heads: int):
    """The float64 fast-weight oracle on the first ``heads`` heads of ``w``."""
    import numpy as np

    from oracle import lact as olact
    from scan_sequence_models_amd import inputs as I

    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:heads]
    hs = [I.head_inputs(w, b, h) for b, h in sel]
    etas = [I.lact_eta(w, b, h) for b, h in sel]
    t0 = time.perf_counter()
    for x, e in zip(hs, etas):
        olact.lact(x.q, x.k, x.v, e, w.chunk, olact.UPDATE_THEN_APPLY, x.S0.astype(np.float64))
    sec = time.perf_counter() - t0
    head_tokens = len(sel) * w.T
    return {
        "value": head_tokens / w.H / sec,
        "unit": "tokens/s",
        "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{len(sel)} of {w.B * w.H} heads x {w.T} tokens ({head_tokens} head-tokens), "
                  f"float64 numpy chunk updates (BLAS threads), {sec:.2f} s",
        "seconds": sec,
    }


def bench_lact(args, w):
    """lact_fwd over the whole batch, inputs resident in HBM."""
    import numpy as np
    import torch

    import scan_sequence_models_amd as gds
    from scan_sequence_models_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: generating {w.name} (B={w.B} H={w.H} T={w.T} d={w.dk} chunk={w.chunk})")
    b = I.batch_inputs(w, threads=16)
    eta = np.stack([np.stack([I.lact_eta(w, bb, hh) for hh in range(w.H)]) for bb in range(w.B)])
    bf = w.dtype == "bf16"

    def up(x, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(torch.bfloat16) if bf16 else t

    q, k, v = up(b.q, bf), up(b.k, bf), up(b.v, bf)
    et, W0 = up(eta), up(b.S0)
    del b, eta
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=q.dtype, device=dev)
    WT = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)
    dcode = gds.SCAN_BF16 if bf else gds.SCAN_F32
    nws = gds.lact_fwd_workspace_size(dcode, w.B, w.H, w.T, w.dk, w.dv, w.chunk)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

    def step():
        gds.lact_fwd(q, k, v, et, W0, chunk=w.chunk, o=o, WT=WT, workspace=ws)

    copy_probe(args.copy_probe_mib, dev)
    warm_calls = warm_up(lambda i: step(), args.warmup, args.warmup_ms)
    span_ms, wall = timed(lambda i: step(), args.steps, dev)
    ms = span_ms / args.steps
    log(f"bench: {args.steps} lact_fwd calls, {ms:.4f} ms per call, wall {wall * 1e3:.1f} ms")
    alg = lact_bytes(w)
    flops = lact_flops(w)
    src = os.path.join(ROOT, "scan_sequence_models_amd", "csrc", "lact.hip")
    result = {
        "metric": "tokens/s large-chunk fast-weight update fwd (H=16, d=128, T=8192, chunk 2048); "
                  "% HBM / MFMA roofline",
        "value": w.B * w.T / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "order": "update_then_apply", "io_dtype": w.dtype,
                   "weight_dtype": "f32", "warmup_calls_run": warm_calls},
        "roofline": {
            "bound": "hbm",
            "achieved": alg / (ms / 1e3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic(src, f"lact_{w.name}_traffic.txt"),
            "kernel": "lact_fwd (stats + recursion + apply kernels)",
            "algorithmic_bytes_per_launch": alg,
            "kernel_ms": ms,
        },
        "mfma": {
            "alg_tflops": flops / (ms / 1e3) / 1e12,
            "peak_tflops": BF16_MFMA_PEAK_TFS,
            "alg_frac": flops / (ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFS,
            "alg_flops_per_launch": flops,
        },
    }
    if not args.no_cpu_baseline:
        heads = min(args.cpu_heads, 16)
        log(f"bench: timing the CPU oracle on {heads} heads")
        result["cpu_baseline"] = cpu_baseline_lact(w, heads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def bwd_mfma_flops(w) -> float:
    """Executed float32 MFMA flops of one scan_bwd call (32-token chunks, 64-row
    value slices; S = 64, C = 32, d = dk).  States pass per chunk and slice:
    K K^T (2 C^2 d), X (2 C S d), T X (2 C^2 S), state update (2 S d C).  Reverse
    pass: K K^T and Q K^T (2 C^2 d each), X, dO S, Kd dS'^T, U dS', dX S (2 C S d
    each), T X, dO U^T, P^T dO, T^T dU, dX U^T (2 C^2 S each), dQK K, dQK^T Q,
    (dKK + dKK^T) K (2 C^2 d each) and dS (two products, 4 S d C).  Linear
    attention drops K K^T, X, T X, dX S, T^T dU, dX U^T, dKK and one dS product."""
    C, S, d = 32, 64, w.dk
    if w.mode == "gdn":
        states = 2 * C * C * d + 2 * C * S * d + 2 * C * C * S + 2 * S * d * C
        rev = 5 * (2 * C * C * d) + 5 * (2 * C * S * d) + 5 * (2 * C * C * S) + 4 * S * d * C
    else:
        states = 2 * S * d * C
        rev = 3 * (2 * C * C * d) + 3 * (2 * C * S * d) + 2 * (2 * C * C * S) + 2 * S * d * C
    return (states + rev) * -(-w.T // C) * (w.dv // S) * w.B * w.H


def cpu_baseline_bwd(w, heads: int):
    """The float64 gradient oracle on the first ``heads`` heads of ``w``."""
    import numpy as np

    import oracle
    from scan_sequence_models_amd import inputs as I

    sel = [(b, h) for b in range(w.B) for h in range(w.H)][:heads]
    hs = [I.head_inputs(w, b, h) for b, h in sel]
    gs = [I.output_grads(w, b, h) for b, h in sel]
    st = lambda f: np.stack([f(x) for x in hs])  # noqa: E731
    dO = np.stack([g[0] for g in gs])
    dST = np.stack([g[1] for g in gs])
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.scan_bwd(w.mode, st(lambda x: x.q), st(lambda x: x.k), st(lambda x: x.v),
                    st(lambda x: x.alpha), st(lambda x: x.beta) if w.beta is not None else None,
                    st(lambda x: x.S0), dO, dST, threads=threads)
    sec = time.perf_counter() - t0
    head_tokens = len(sel) * w.T
    return {
        "value": head_tokens / w.H / sec,
        "unit": "tokens/s",
        "cores": min(threads, len(sel)),
        "kind": "oracle",
        "sample": f"{len(sel)} of {w.B * w.H} heads x {w.T} tokens ({head_tokens} head-tokens), "
                  f"float64 reverse sweep per state row, one thread per head, {sec:.2f} s",
        "head_tokens_per_s": head_tokens / sec,
        "seconds": sec,
    }


def bench_bwd(args, w):
    """scan_bwd over the whole batch (inputs and incoming gradients resident in HBM)."""
    import numpy as np
    import torch

    import scan_sequence_models_amd as gds
    from scan_sequence_models_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: generating {w.name} (B={w.B} H={w.H} T={w.T} d={w.dk})")
    b = I.batch_inputs(w, threads=16)
    dO = np.empty((w.B, w.H, w.T, w.dv), np.float32)
    dST = np.empty((w.B, w.H, w.dv, w.dk), np.float32)
    for bb in range(w.B):
        for hh in range(w.H):
            dO[bb, hh], dST[bb, hh] = I.output_grads(w, bb, hh)
    bf = w.dtype == "bf16"

    def up(x, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(torch.bfloat16) if bf16 else t

    q, k, v, g_o = up(b.q, bf), up(b.k, bf), up(b.v, bf), up(dO, bf)
    alpha, beta, S0, g_s = up(b.alpha), up(b.beta), up(b.S0), up(dST)
    del b, dO, dST
    f32 = torch.float32
    outs = [torch.empty((w.B, w.H, w.T, w.dk), dtype=f32, device=dev),
            torch.empty((w.B, w.H, w.T, w.dk), dtype=f32, device=dev),
            torch.empty((w.B, w.H, w.T, w.dv), dtype=f32, device=dev),
            torch.empty((w.B, w.H, w.T), dtype=f32, device=dev),
            torch.empty((w.B, w.H, w.T), dtype=f32, device=dev),
            torch.empty((w.B, w.H, w.dv, w.dk), dtype=f32, device=dev)]
    dcode = gds.SCAN_BF16 if bf else gds.SCAN_F32
    nws = gds.scan_bwd_workspace_size(gds.SCAN_GDN, dcode, w.B, w.H, w.T, w.dk, w.dv)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def step():
        gds.scan_bwd(q, k, v, alpha, beta, S0, g_o, g_s, workspace=ws, out=outs)

    copy_probe(args.copy_probe_mib, dev)
    warm_calls = warm_up(lambda i: step(), args.warmup, args.warmup_ms)
    span_ms, wall = timed(lambda i: step(), args.steps, dev)
    ms = span_ms / args.steps
    log(f"bench: {args.steps} scan_bwd calls, {ms:.4f} ms per call, wall {wall * 1e3:.1f} ms")
    flops = bwd_mfma_flops(w)
    tfs = flops / (ms / 1e3) / 1e12
    es = 2 if bf else 4
    ht = w.B * w.H * w.T
    # inputs and incoming gradients read once, gradients written once (float32);
    # the chunk states and slice partials are the workspace's round trips
    alg = ht * (2 * w.dk + 2 * w.dv) * es + ht * 8 + w.B * w.H * w.dv * w.dk * 4 * 3 \
        + ht * (2 * w.dk + w.dv + 2) * 4
    ws_bytes = 2 * nws
    csrc = os.path.join(ROOT, "scan_sequence_models_amd", "csrc")
    src = [os.path.join(csrc, f) for f in ("scan_bwd.hip", "mfma_f32.hpp", "solve.hpp")]
    result = {
        "metric": "tokens/s gradient of the gated-delta scan (H=16, d=128, T=8192); % MFMA roofline",
        "value": w.B * w.T / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk,
                   "dv": w.dv, "chunk": 32, "io_dtype": w.dtype, "grad_dtype": "f32",
                   "warmup_calls_run": warm_calls},
        "roofline": {
            "bound": "mfma",
            "achieved": tfs,
            "peak": FP32_MFMA_PEAK_TFS,
            "unit": "TFLOP/s",
            "frac": tfs / FP32_MFMA_PEAK_TFS,
            "traffic": measured_traffic(src, f"scan_bwd_{w.name}_traffic.txt"),
            "kernel": "scan_bwd (states + reverse chunk + slice reduction kernels)",
            "flops_per_launch": flops,
            "algorithmic_bytes_per_launch": alg,
            "workspace_round_trip_bytes": ws_bytes,
            "hbm_achieved_gbs": (alg + ws_bytes) / (ms / 1e3) / 1e9,
            "kernel_ms": ms,
        },
        "head_tokens_per_s": ht / (ms / 1e3),
    }
    if not args.no_cpu_baseline:
        heads = min(args.cpu_heads, 16)
        log(f"bench: timing the CPU gradient oracle on {heads} heads")
        result["cpu_baseline"] = cpu_baseline_bwd(w, heads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; decode workloads: the workload's token count)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: enough to cover the GPU's clock ramp, "
                         "~15 ms: 30 scan calls or 300 decode steps)")
    ap.add_argument("--warmup-ms", type=float, default=200.0,
                    help="after the --warmup calls, keep warming up until this much "
                         "back-to-back work has run (covers the clock ramp whatever --warmup is)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input (decode: state) sets the timed calls take in turn; 0 = enough "
                         "for at least 3 and more than twice the 256 MB MALL")
    ap.add_argument("--workload", default="gdn-b8h16t8192")
    ap.add_argument("--path", default="auto", choices=["auto", "sequential", "blelloch"])
    ap.add_argument("--leaf-chunks", type=int, default=0)
    ap.add_argument("--cpu-heads", type=int, default=128,
                    help="heads of the workload the CPU oracle is timed on")
    ap.add_argument("--cpu-states", type=int, default=4096,
                    help="decode workloads: states the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB before the timed "
                         "steps (a known-size kernel that calibrates rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads and sequences shard with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import scan_sequence_models_amd as gds
    from scan_sequence_models_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    if w.path == "decode":
        if args.warmup is None:
            args.warmup = 300
        return bench_decode(args, w)
    if args.steps is None:
        args.steps = 50
    if args.warmup is None:
        args.warmup = 30
    if w.prism_steps:
        return bench_prism(args, w)
    if w.mode == "lact":
        return bench_lact(args, w)
    if w.backward:
        return bench_bwd(args, w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"bench: generating {w.name} (B={w.B} H={w.H} T={w.T} d={w.dk})")
    b = I.batch_inputs(w, threads=16)
    if w.diag_gates:  # one decay per key channel replaces the scalar alpha
        b.alpha = np.stack([np.stack([I.diag_alpha(w, bb, hh) for hh in range(w.H)])
                            for bb in range(w.B)])

    def up(x, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        return t.to(torch.bfloat16) if bf16 else t

    bf = w.dtype == "bf16"
    # R input sets taken in turn by the timed calls (at least 3, more than
    # twice the 256 MB MALL in all), so that no call finds its inputs left in
    # the MALL by an earlier one; set r rolls the generated batch by r heads
    # (the same distribution at other addresses), each with its own o and S_T
    R = args.rotate if args.rotate else rotation_sets(scan_bytes(w), 3, 2 * MALL_BYTES)

    def rolled(x, r, bf16=False):
        if x is None:
            return None
        y = np.roll(x.reshape(w.B * w.H, *x.shape[2:]), r, axis=0).reshape(x.shape)
        return up(y, bf16)

    sets = []
    for r in range(R):
        sets.append(dict(q=rolled(b.q, r, bf), k=rolled(b.k, r, bf), v=rolled(b.v, r, bf),
                         alpha=rolled(b.alpha, r), beta=rolled(b.beta, r), S0=rolled(b.S0, r),
                         o=torch.empty((w.B, w.H, w.T, w.dv),
                                       dtype=torch.bfloat16 if bf else torch.float32, device=dev),
                         ST=torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)))
    del b
    mode = gds.SCAN_GDN if w.mode == "gdn" else gds.SCAN_GLA
    if w.diag_gates:
        mode = gds.SCAN_GDN_DIAG if w.mode == "gdn" else gds.SCAN_GLA_DIAG
    dcode = gds.SCAN_BF16 if bf else gds.SCAN_F32
    path = args.path if args.path != "auto" else w.path if w.path == "blelloch" else "auto"
    ws_bytes = gds.scan_fwd_workspace_size(mode, dcode, w.B, w.H, w.T, w.dk, w.dv, w.chunk, path,
                                           args.leaf_chunks)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None

    def step(i):
        x = sets[i % R]
        gds.scan_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], chunk=w.chunk,
                     path=path, leaf_chunks=args.leaf_chunks, o=x["o"], ST=x["ST"], workspace=ws)

    copy_probe(args.copy_probe_mib, dev)
    warm_calls = warm_up(step, args.warmup, args.warmup_ms)
    span_ms, wall = timed(lambda i: step(warm_calls + i), args.steps, dev)
    ms_per_step = span_ms / args.steps
    # the sequential path is one kernel launch per step; the long path's
    # figure covers all of its kernels
    kern_ms = ms_per_step
    tokens = w.B * w.T
    value = tokens / (ms_per_step / 1e3)
    log(f"bench: {warm_calls} warm-up calls, then {args.steps} calls back to back over {R} "
        f"input sets, span {span_ms:.3f} ms ({kern_ms:.4f} ms per step), wall {wall * 1e3:.1f} ms")

    alg_bytes = scan_bytes(w) + (w.B * w.H * w.T * (w.dk - 1) * 4 if w.diag_gates else 0)
    flops = scan_flops(w)
    flops_alg = scan_flops_alg(w)
    achieved_gbs = alg_bytes / (kern_ms / 1e3) / 1e9
    achieved_tfs = flops / (kern_ms / 1e3) / 1e12
    kernel_src = os.path.join(ROOT, "scan_sequence_models_amd", "csrc", "chunk_bf16.hip")
    traffic = None
    if w.diag_gates:
        kernel_src = [os.path.join(ROOT, "scan_sequence_models_amd", "csrc", f)
                      for f in ("chunk_diag.hip", "mfma_f32.hpp")]
        traffic = measured_traffic(kernel_src, f"chunk_diag_{w.name}_traffic.txt")
    elif path != "blelloch" and w.dk == 128 and w.chunk == 64 and bf:
        traffic = measured_traffic(kernel_src, f"chunk_mfma_{w.name}_traffic.txt")
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "B": w.B, "H": w.H, "T": w.T,
                   "dk": w.dk, "dv": w.dv, "chunk": w.chunk, "path": path,
                   "io_dtype": w.dtype, "state_dtype": "f32", "rotated_input_sets": R,
                   "rotated_bytes": R * scan_bytes(w), "warmup_calls_run": warm_calls},
    }
    if w.diag_gates:
        # float32 kernel: its products run on the fp32 MFMA, whose floor
        # (about 0.8 ms here) lies above the HBM floor (about 0.2 ms)
        dflops = diag_mfma_flops(w)
        dtfs = dflops / (kern_ms / 1e3) / 1e12
        result["dtype"] = "f32"
        result["config"]["io_dtype"] = w.dtype
        result["roofline"] = {
            "bound": "mfma",
            "achieved": dtfs,
            "peak": FP32_MFMA_PEAK_TFS,
            "unit": "TFLOP/s",
            "frac": dtfs / FP32_MFMA_PEAK_TFS,
            "traffic": traffic,
            "kernel": "chunk_diag_mfma_kernel",
            "flops_per_launch": dflops,
            "algorithmic_bytes_per_launch": alg_bytes,
            "hbm_achieved_gbs": achieved_gbs,
            "hbm_frac": achieved_gbs / HBM_PEAK_GBS,
            "kernel_ms": kern_ms,
        }
        result["head_tokens_per_s"] = w.B * w.H * w.T / (ms_per_step / 1e3)
    else:
        result.update(plain_scan_rooflines(path, achieved_gbs, traffic, alg_bytes, kern_ms,
                                           achieved_tfs, flops, flops_alg))
        result["head_tokens_per_s"] = w.B * w.H * w.T / (ms_per_step / 1e3)
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle on {args.cpu_heads} heads")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_heads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def plain_scan_rooflines(path, achieved_gbs, traffic, alg_bytes, kern_ms, achieved_tfs, flops, flops_alg):
    """The roofline and MFMA blocks of a scalar-gate scan line."""
    return {
        "roofline": {
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": "chunk_mfma_kernel" if path != "blelloch" else "blelloch path (all kernels)",
            "algorithmic_bytes_per_launch": alg_bytes,
            "kernel_ms": kern_ms,
        },
        "mfma": {
            "achieved_tflops": flops_alg / (kern_ms / 1e3) / 1e12,
            "peak_tflops": BF16_MFMA_PEAK_TFS,
            "frac": flops_alg / (kern_ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFS,
            "flops_per_launch": flops_alg,
            "count": "algorithmic flops: triangular C x C products at their useful size, "
                     "state products in full, UT solve C^2/3 per head-token",
            "dense_tile_tflops": achieved_tfs,
            "dense_tile_frac": achieved_tfs / BF16_MFMA_PEAK_TFS,
            "dense_tile_flops_per_launch": flops,
        },
    }


if __name__ == "__main__":
    main()
