"""Throughput of the Infini-attention layer forward on one MI355X.

A step is one ``infini_attn_forward_stream`` over the whole 32768-token stream of the
8-head, d=128, N=2048 workload (16 segments, linear update, bf16), preceded by a state
reset, with Q/K/V already resident in HBM.  The JSON line reports whole-step tokens/s,
the roofline of the dominant kernel (the fused local-attention + retrieval + gate kernel,
timed with HIP events on its own stream inside the timed region), and the CPU oracle's
throughput on a bounded sample of the same workload.

With --decode a step is one whole segment decoded token by token for --decode-batch
sequences (``infini_attn_decode_step`` N times; the last call writes the segment to the
memory), and the roofline is the decode kernel's HBM bandwidth.

With --layer a step is one ``infini_attn_forward_layer`` instead: the whole layer from
its input X [B, T, d_model] to O, the Q/K/V projection (Eq. 5) and the output projection
(Eq. 11) included; the roofline is then that of the kernel with the most time per step.

With --workload NAME the step runs another workload of the library's set (the delta-rule
32K streams at batch 1 and 4, the 512K-token 32-head stream, the 1M-token stream); streams
longer than 16 segments are built on the device from a pool of 16 distinct segments used
cyclically (the values do not change the kernels' work).  With --per-segment the 1M-token
stream is fed one ``infini_attn_forward_segment`` call per segment (the streaming path)
and the line also carries the device-memory evidence (used bytes after 1, 64, 256 and 512
segments).

Step time = the K timed steps back to back between one pair of HIP events on the launch
stream, divided by K (whole-job time); the median of the same K steps run once more, each
bracketed by its own events, is reported next to it.  Before the warmup steps the GPU runs bf16
matrix products for --spin-up-s seconds (0.5 by default): an idle MI355X raises its
clocks over the first ~10 ms of sustained load, and without the spin-up the first steps
after start run up to ~20% slower than the sustained rate that the line reports.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--layer]
       [--per-segment] [--decode] [--backward] [--local-qk]
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Infini-attention fwd tokens/sec per layer (H=8,d=128,N=2048) + % bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--local-qk", action="store_true",
                    help="separate (position-embedded) Q/K for the local attention: forward_stream_local")
    ap.add_argument("--layer", action="store_true",
                    help="the whole layer X -> O (Q/K/V and output projections included): forward_layer")
    ap.add_argument("--d-model", type=int, default=0, help="--layer: model width (default H * d)")
    ap.add_argument("--backward", action="store_true",
                    help="training: one step = infini_attn_backward over the stream (forward recomputed)")
    ap.add_argument("--decode", action="store_true",
                    help="incremental decoding: one step = one whole segment (N tokens) per sequence, token by token")
    ap.add_argument("--decode-batch", type=int, default=64, help="--decode: sequences decoded together")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--per-segment", action="store_true",
                    help="streaming: one forward_segment call per segment of the stream (default workload: 1M tokens)")
    ap.add_argument("--spin-up-s", type=float, default=0.5,
                    help="seconds of bf16 matrix products before the warmup steps (clock ramp; 0: none)")
    ap.add_argument("--pool-segments", type=int, default=16,
                    help="distinct segments drawn for streams longer than this (used cyclically)")
    return ap.parse_args()


def traffic_from_profiles(kernel_hash: str):
    """HBM bytes per attention launch from the committed counter summary, if it was taken
    from the kernel source that is built now; else None."""
    path = os.path.join(ROOT, "profiles", "attention_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source hash: `([0-9a-f]+)`", text)
    m_bytes = re.search(r"HBM bytes per launch \(scaled\): ([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash:
        return None
    return float(m_bytes.group(1))


def _blas_info():
    """(library description, threads) of the BLAS numpy uses here."""
    try:
        from threadpoolctl import threadpool_info
        infos = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if infos:
            p = infos[0]
            return f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer', '')})", int(p.get("num_threads", 1))
    except Exception:
        pass
    return "unknown", 1


def _oracle_worker_init():
    import numpy  # noqa: F401
    from compressive_memory_transformer_segment_amd import workloads  # noqa: F401
    from oracle import infini_oracle  # noqa: F401


def _oracle_worker_ready(_):
    return os.getpid()


def _oracle_unit(job):
    """One (batch element, head) of a workload through the oracle with one BLAS thread (the
    process-pool worker); see _oracle_pair.  Returns the seconds spent in the oracle."""
    from threadpoolctl import threadpool_limits
    w, b, h, segs, synthetic_state = job
    with threadpool_limits(1):
        return _oracle_pair(w, b, h, segs, synthetic_state)


def cpu_baseline(w, budget_s: float):
    """The oracle (numpy float64, as written), timed on the host cores:
    * value: all cores, a process pool over the (batch, head) pairs with one BLAS thread per
      worker (the pairs' chains are independent), wall time of the pool;
    * single_core: one (batch, head) pair on one core, scaled to all pairs;
    * blas_threaded: whole heads in this process with the BLAS library's own threads.
    Streams of up to 32 segments run in full from the zero state; longer ones run a seeded
    sample of segments (first 2, last 2, 4 random) from a synthetic state and the rate is
    extrapolated (a segment's cost does not depend on the state).  Tokens/s of the layer
    (all heads)."""
    import multiprocessing as mp
    import numpy as np
    blas, blas_threads = _blas_info()
    cores = len(os.sched_getaffinity(0))
    S = w.n_segments
    if S <= 32:
        segs, synthetic, sample = list(range(S)), False, "the full stream"
    else:
        rng = np.random.default_rng(w.seed)
        mid = sorted(rng.choice(np.arange(2, S - 2), size=4, replace=False).tolist())
        segs, synthetic = [0, 1] + mid + [S - 2, S - 1], True
        sample = f"segments {segs} (extrapolated to all {S})"
    seg_tokens = sum(w.segment_len_of(s) for s in segs)
    units = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    # single core: one pair
    t_one = _oracle_unit((w, 0, 0, segs, synthetic))
    single = {"value": w.batch * w.n_tokens / (t_one * (w.n_tokens / seg_tokens) * len(units)), "cores": 1,
              "sample": f"one (batch, head) pair, {sample}, {t_one:.1f} s, scaled to {len(units)} pairs"}
    # all cores: pool over the pairs (as many as fit the budget, at least one round)
    workers = max(1, min(cores, len(units), 16))
    per_unit = t_one
    n_units = max(workers, min(len(units), int(budget_s * workers / max(per_unit, 1e-9)) // workers * workers))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_oracle_worker_init) as pool:
        pool.map(_oracle_worker_ready, range(workers))   # workers started, modules imported
        t0 = time.perf_counter()
        pool.map(_oracle_unit, [(w, b, h, segs, synthetic) for b, h in units[:n_units]], chunksize=1)
        wall = time.perf_counter() - t0
    value = w.batch * w.n_tokens / (wall * (w.n_tokens / seg_tokens) * (len(units) / n_units))
    return {"value": value, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "affinity_cores": cores, "blas": blas,
            "sample": (f"process pool of {workers} workers (one BLAS thread each) over {n_units} of "
                       f"{len(units)} (batch, head) pairs, {sample}, {wall:.1f} s wall (input generation "
                       "included, worker start-up not)" + ("" if n_units == len(units) else ", scaled to all pairs")),
            "single_core": single,
            "blas_threaded": cpu_baseline_threaded(w, min(budget_s, 6.0), blas_threads, segs, synthetic, sample)}


def cpu_baseline_threaded(w, budget_s, blas_threads, segs, synthetic, sample):
    """Whole (batch, head) pairs in this process, BLAS with its own threads."""
    done, el = 0, 0.0
    for h in range(w.heads):
        el += _oracle_pair(w, 0, h, segs, synthetic)
        done += 1
        if el >= budget_s:
            break
    seg_tokens = sum(w.segment_len_of(s) for s in segs)
    per_unit = el / done * (w.n_tokens / seg_tokens)
    return {"value": w.batch * w.n_tokens / (per_unit * w.batch * w.heads), "cores": blas_threads,
            "sample": f"{done} (batch, head) pairs, {sample}, {el:.1f} s, scaled to all pairs"}


def _oracle_pair(w, b, h, segs, synthetic_state):
    """segment_forward on the listed segments of pair (b, h) in order, the state carried
    from M0, z0: zero (the exact stream from its start) or, for a sample of segments, a
    synthetic state (a segment's cost does not depend on the state's values).  Returns the
    seconds spent in the oracle (input generation excluded)."""
    import numpy as np
    from compressive_memory_transformer_segment_amd import workloads as wl
    from oracle import infini_oracle as orc
    beta = wl.beta_for(w)[h]
    scale = 1.0 / np.sqrt(w.head_dim)
    d = w.head_dim
    M = np.full((d, d), 1e-3) if synthetic_state else np.zeros((d, d))
    z = np.full(d, 1.0) if synthetic_state else np.zeros(d)
    el = 0.0
    for s in segs:
        q, k, v = (x[0].astype(np.float64) for x in wl.segment_inputs(w, b, s, heads=[h]))
        t0 = time.perf_counter()
        _, M, z, _, _ = orc.segment_forward(q, k, v, M, z, beta, w.update, w.eps, scale)
        el += time.perf_counter() - t0
    return el


def cpu_baseline_layer(w, d_model: int, budget_s: float):
    """The oracle's whole layer (projections included) on the stream's first segments,
    doubling the sample until about budget_s seconds of CPU work; tokens/s."""
    import numpy as np
    from compressive_memory_transformer_segment_amd import workloads as wl
    from oracle import infini_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    X, w_qkv, w_o = wl.layer_inputs(w.with_tokens(min(w.n_tokens, 4 * w.segment_len)), d_model)
    beta = wl.beta_for(w)
    n_seg, elapsed = 1, 0.0
    while True:
        n = min(n_seg * w.segment_len, X.shape[1])
        t0 = time.perf_counter()
        orc.layer_forward(X[:, :n], w_qkv, w_o, beta, w.segment_len, w.heads, w.head_dim, w.update, eps=w.eps)
        elapsed = time.perf_counter() - t0
        if 2 * elapsed > budget_s or n >= X.shape[1]:
            break
        n_seg *= 2
    return {"value": w.batch * n / elapsed, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"oracle.layer_forward on the first {n} tokens (all heads, d_model={d_model}), {elapsed:.1f} s"}


def decode_bytes(batch, heads, d, segment_len, es):
    """Algorithmic HBM bytes of the decode launches over one segment: per (b, h) and token
    at position p, the p cached key and value rows, M_{s-1} (fp32) and z_{s-1}, this
    token's q, k, v in and its output out, and the key and value appended to the cache."""
    per_bh = 0
    for p in range(segment_len):
        per_bh += 2 * p * d * es + 4 * d * d + 4 * d + 3 * d * es + d * es + 2 * d * es
    return batch * heads * per_bh


def cpu_baseline_decode(w, batch, budget_s: float):
    """The oracle's token-by-token decoding on one sequence of the same shape (all heads)
    until about budget_s seconds; tokens/s scaled to the batch is not claimed (it is one
    sequence's rate)."""
    import numpy as np
    from compressive_memory_transformer_segment_amd import workloads as wl
    from oracle import infini_oracle as orc
    n = min(w.segment_len, 256)
    ws = w.with_tokens(n).with_batch(1)
    Q, K, V = wl.stream_inputs(ws)
    beta = wl.beta_for(w)
    scale = 1.0 / np.sqrt(w.head_dim)
    t0 = time.perf_counter()
    done = 0
    M = np.zeros((w.head_dim, w.head_dim))
    z = np.zeros(w.head_dim)
    for t in range(n):
        for h in range(w.heads):
            orc.decode_token(Q[0, h, t], K[0, h, t], V[0, h, t], K[0, h, :t], V[0, h, :t], M, z, beta[h],
                             w.eps, scale)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": (f"oracle.decode_token for the first {done} tokens of one sequence, all {w.heads} heads "
                       f"({el:.1f} s); per-sequence rate, positions 0..{done - 1} of a segment (short caches)")}


def main_decode(args):
    import torch
    from compressive_memory_transformer_segment_amd import binding, profiling
    from compressive_memory_transformer_segment_amd import workloads as wl

    base = wl.WORKLOADS[args.workload or wl.THROUGHPUT_WORKLOAD]
    B, H, d, N = args.decode_batch, base.heads, base.head_dim, base.segment_len
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(base.seed)
    # one segment of tokens per sequence, resident in HBM: [N, B, H, d] so a token is contiguous
    Q, K, V = ((torch.randn((N, B, H, d), generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
               for _ in range(3))
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    layer = binding.InfiniAttention(B, H, d, N, update=base.update, io_dtype="bf16", eps=base.eps,
                                    beta=wl.beta_for(base))
    stream = torch.cuda.current_stream()
    copy_probe(args.copy_probe_mib, dev)

    def step():   # one whole segment token by token; the last token closes it into the memory
        for t in range(N):
            layer.decode_step(Q[t], K[t], V[t], out=out, stream=stream)

    spin_up(args.spin_up_s, torch.device("cuda", 0))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] decode B={B}: warmup {args.warmup} done, timing {args.steps} segments", file=sys.stderr,
          flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms = ev0.elapsed_time(ev1) / args.steps

    layer.profile_enable(True)
    step()
    prof = layer.profile_read()
    layer.profile_enable(False)
    torch.cuda.synchronize()
    dec_ms, dec_n = prof["decode"]
    bytes_seg = decode_bytes(B, H, d, N, 2)
    achieved = bytes_seg / (dec_ms / 1e3) / 1e9
    tokens = B * N
    rec = {
        "metric": METRIC + " [incremental decoding]",
        "value": tokens / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spin_up_s": args.spin_up_s,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode-b{B}-h{H}-d{d}-n{N}-{base.update}", "batch": B, "heads": H,
                   "head_dim": d, "segment_len": N, "tokens_per_step": tokens,
                   "step": "one segment per sequence, token by token, incl. the memory write at its end",
                   "parallelism": "none"},
        "roofline": {
            "kernel": "k_decode (one token per (batch, head))",
            "bound": "hbm",
            "achieved": achieved,
            "peak": profiling.PEAK_HBM_BYTES / 1e9,
            "unit": "GB/s",
            "frac": achieved / (profiling.PEAK_HBM_BYTES / 1e9),
            "traffic": None,
            "algorithmic_bytes": bytes_seg / dec_n,
            "avg_launch_us": dec_ms / dec_n * 1e3,
        },
        "kernels_avg_us": {k: (t / n * 1e3 if n else None) for k, (t, n) in prof.items()},
        "kernels_total_ms_per_step": {k: t for k, (t, n) in prof.items()},
        "wall_ms_per_step": wall_ms / args.steps,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_decode(base, B, args.cpu_budget_s)
    else:
        rec["cpu_baseline"] = None
    layer.close()
    print(json.dumps(rec), flush=True)


def backward_flops(batch, heads, d, segment_len, n_tokens, update):
    """Matrix-class FLOPs of the gradient kernels (the recomputed forward not included):
    local attention 5 causal n x n x d products (scores, dP, dV, dQ, dK), the retrieval
    gradient 2 n x d x d products (du, sigma(Q)^T dnum) and the update gradient 2 (linear:
    sigma(K) G, G v) or 4 (delta: also R and M dW) per segment and head, plus the chain's
    d x d x d product per segment for the delta rule."""
    import compressive_memory_transformer_segment_amd.profiling as pf
    tot = 0.0
    for n in pf.segment_lengths(n_tokens, segment_len):
        tot += 2.5 * pf.local_attention_flops(n, d)
        tot += (2 + (4 if update == "delta" else 2)) * 2.0 * n * d * d
        if update == "delta":
            tot += 2.0 * d * d * d
    return tot * batch * heads


def main_backward(args):
    import numpy as np
    import torch
    from compressive_memory_transformer_segment_amd import binding, profiling
    from compressive_memory_transformer_segment_amd import workloads as wl

    w = wl.WORKLOADS[args.workload or wl.THROUGHPUT_WORKLOAD]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    shape = (w.batch, w.heads, w.n_tokens, w.head_dim)
    Q, K, V = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(3))
    for b in range(w.batch):
        for s in range(w.n_segments):
            lo = s * w.segment_len
            for x, p in zip((Q, K, V), wl.segment_inputs(w, b, s)):
                x[b, :, lo:lo + p.shape[1]] = torch.from_numpy(p).to(dev, torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    dO = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    layer = binding.InfiniAttention(w.batch, w.heads, w.head_dim, w.segment_len, update=w.update, io_dtype="bf16",
                                    eps=w.eps, beta=wl.beta_for(w))
    stream = torch.cuda.current_stream()
    outs = None

    def step():
        nonlocal outs
        outs = layer.backward(Q, K, V, dO, stream=stream)

    spin_up(args.spin_up_s, torch.device("cuda", 0))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] backward {w.name}: warmup {args.warmup} done, timing {args.steps} steps", file=sys.stderr,
          flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms = ev0.elapsed_time(ev1) / args.steps
    layer.profile_enable(True)
    step()
    prof = layer.profile_read()
    layer.profile_enable(False)
    torch.cuda.synchronize()
    bwd_ms, bwd_n = prof["backward"]
    fl = backward_flops(w.batch, w.heads, w.head_dim, w.segment_len, w.n_tokens, w.update)
    achieved = fl / (bwd_ms / bwd_n / 1e3) / 1e12
    tokens = w.batch * w.n_tokens
    rec = {
        "metric": METRIC + " [backward]",
        "value": tokens / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spin_up_s": args.spin_up_s,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + "-backward", "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "segment_len": w.segment_len, "n_tokens": w.n_tokens, "update": w.update,
                   "step": "infini_attn_backward: forward recomputed, then all gradients", "parallelism": "none"},
        "roofline": {
            "kernel": "gradient kernels of one backward call (bf16 matrix-core products, fp32 chains)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": profiling.PEAK_BF16_FLOPS / 1e12,
            "unit": "TFLOP/s",
            "frac": achieved / (profiling.PEAK_BF16_FLOPS / 1e12),
            "traffic": None,
            "algorithmic_flops": fl,
            "avg_launch_us": bwd_ms / bwd_n * 1e3,
        },
        "kernels_total_ms_per_step": {k: t for k, (t, n) in prof.items()},
        "wall_ms_per_step": wall_ms / args.steps,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import infini_backward as ob
        n = w.segment_len
        ws = w.with_tokens(2 * n)
        Qh, Kh, Vh = wl.stream_inputs(ws)
        dOh = np.random.default_rng(1).standard_normal(Qh.shape)
        t0 = time.perf_counter()
        ob.gradients(Qh[:, :2], Kh[:, :2], Vh[:, :2], wl.beta_for(w)[:2], dOh[:, :2], n, w.update)
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": w.batch * 2 * n * 2 / w.heads / el, "unit": "tokens/s",
                               "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": f"oracle gradients (float64 autograd) of 2 heads x {2 * n} tokens, "
                                         f"{el:.1f} s, scaled to all {w.heads} heads"}
    layer.close()
    print(json.dumps(rec), flush=True)


def spin_up(seconds: float, dev) -> None:
    """Bring the GPU from idle to its sustained clocks before the warmup steps: bf16
    matrix products (not part of any step) for `seconds`."""
    if seconds <= 0:
        return
    import torch
    x = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            y = x @ x
        torch.cuda.synchronize()
    del x, y
    torch.cuda.synchronize()


def copy_probe(mib: int, dev) -> None:
    """One device copy of `mib` MiB before timing (calibrates the HBM byte counters)."""
    if mib <= 0:
        return
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def device_inputs(w, dev, pool_segments: int):
    """Q, K, V [B, H, L, d] bf16 on the device.  Streams of at most pool_segments segments
    are drawn exactly; longer ones repeat the first pool_segments segments cyclically (the
    kernels' work does not depend on the values), with the planted pair, if any, written at
    its place (token 0 of segment 0; the query at the last token).  Returns the tensors and
    a description."""
    import torch
    from compressive_memory_transformer_segment_amd import workloads as wl
    shape = (w.batch, w.heads, w.n_tokens, w.head_dim)
    Q, K, V = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(3))
    S, N = w.n_segments, w.segment_len
    exact = S <= pool_segments
    for b in range(w.batch):
        for s in range(S if exact else pool_segments):
            lo = s * N
            for x, p in zip((Q, K, V), wl.segment_inputs(w, b, s, plant=False)):
                x[b, :, lo:lo + p.shape[1]] = torch.from_numpy(p).to(dev, torch.bfloat16)
        if not exact:   # segments pool_segments .. S - 1 repeat the pool
            span = pool_segments * N
            for lo in range(span, w.n_tokens, span):
                n = min(span, w.n_tokens - lo)
                for x in (Q, K, V):
                    x[b, :, lo:lo + n] = x[b, :, :n]
    if w.plant:
        k_star, v_star = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in wl.planted_pair(w))
        K[:, :, 0], V[:, :, 0], Q[:, :, w.n_tokens - 1] = k_star, v_star, k_star
    torch.cuda.synchronize()
    desc = ("exact seeded draws" if exact else
            f"first {pool_segments} segments drawn (seeded), repeated cyclically over the {S} segments")
    return Q, K, V, desc


def timed_steps(step, steps: int, stream):
    """The timed region: K steps back to back between one pair of HIP events on the launch
    stream, between two synchronisations (whole-job time, no event between steps).  Then the
    same K steps once more, each between an event pair of its own, for the per-step spread
    (those records leave ~10 us of idle GPU between steps, outside each step's bracket).
    Returns (mean milliseconds per step of the region, per-step milliseconds of the second
    pass, wall milliseconds of the region)."""
    import torch
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    region_ms = e_start.elapsed_time(e_end) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    return region_ms, [e0.elapsed_time(e1) for e0, e1 in evs], wall_ms


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def main_per_segment(args):
    """The streaming path: the stream fed one infini_attn_forward_segment call per segment
    (as a caller streaming segment by segment would), against forward_stream on the same
    stream; plus the device-memory evidence of constant memory in the stream length."""
    import torch
    from compressive_memory_transformer_segment_amd import binding, profiling
    from compressive_memory_transformer_segment_amd import workloads as wl

    w = wl.WORKLOADS[args.workload or "h8-d128-n2048-l1m-linear-planted"]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    Q, K, V, desc = device_inputs(w, dev, args.pool_segments)
    out = torch.empty_like(Q)
    N, S = w.segment_len, w.n_segments
    seg_views = [tuple(x[:, :, s * N:min((s + 1) * N, w.n_tokens)].contiguous() for x in (Q, K, V))
                 for s in range(min(S, args.pool_segments))]   # contiguous [B, H, n, d] per call
    seg_out = torch.empty_like(seg_views[0][0])
    layer = binding.InfiniAttention(w.batch, w.heads, w.head_dim, N, update=w.update, io_dtype="bf16",
                                    eps=w.eps, beta=wl.beta_for(w))
    stream = torch.cuda.current_stream()
    copy_probe(args.copy_probe_mib, dev)
    mem = {}

    def step_segments(record_mem=False):
        layer.reset_state(stream)
        for s in range(S):
            q, k, v = seg_views[s % len(seg_views)]
            layer.forward_segment(q, k, v, out=seg_out, stream=stream)
            if record_mem and (s + 1) in (1, 64, 256, 512):
                torch.cuda.synchronize()
                free, total = torch.cuda.mem_get_info()
                mem[s + 1] = total - free

    def step_stream():
        layer.reset_state(stream)
        layer.forward_stream(Q, K, V, out=out, stream=stream)

    step_segments(record_mem=True)
    spin_up(args.spin_up_s, torch.device("cuda", 0))
    for _ in range(args.warmup):
        step_segments()
        step_stream()
    torch.cuda.synchronize()
    steps = max(3, args.steps // 4)
    print(f"[bench] {w.name} per segment: timing {steps} streams of {S} forward_segment calls", file=sys.stderr,
          flush=True)
    ms, seg_ms, wall_ms = timed_steps(step_segments, steps, stream)
    str_region, str_ms, _ = timed_steps(step_stream, steps, stream)
    layer.profile_enable(True)
    step_segments()
    prof = layer.profile_read()
    layer.profile_enable(False)
    torch.cuda.synchronize()
    tokens = w.batch * w.n_tokens
    att_ms, att_n = prof["attention"]
    seg_flops = profiling.attention_kernel_flops(w.batch, w.heads, w.head_dim, N, N)
    achieved = seg_flops / (att_ms / att_n / 1e3) / 1e12
    rec = {
        "metric": METRIC + " [streamed: one forward_segment call per segment]",
        "value": tokens / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "spin_up_s": args.spin_up_s,
        "ms_per_step": ms,
        "median_ms_per_step_evented": median(seg_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + "-per-segment", "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "segment_len": N, "n_tokens": w.n_tokens, "update": w.update, "inputs": desc,
                   "step": f"reset_state + {S} forward_segment calls of {N} tokens", "parallelism": "none"},
        "roofline": {
            "kernel": "k_attn_bf16 (local attention + retrieval + gate), one segment per launch",
            "bound": "mfma",
            "achieved": achieved,
            "peak": profiling.PEAK_BF16_FLOPS / 1e12,
            "unit": "TFLOP/s",
            "frac": achieved / (profiling.PEAK_BF16_FLOPS / 1e12),
            "traffic": None,
            "algorithmic_flops": seg_flops,
            "avg_launch_us": att_ms / att_n * 1e3,
        },
        "forward_stream_same_stream": {"ms_per_step": str_region, "value": tokens / (str_region / 1e3),
                                       "median_ms_per_step_evented": median(str_ms),
                                       "per_segment_over_windowed": ms / str_region},
        "kernels_avg_us": {k: (t / n * 1e3 if n else None) for k, (t, n) in prof.items()},
        "wall_ms_per_step": wall_ms / steps,
        "memory": {"device_bytes": layer.device_bytes(),
                   "used_bytes_after_segments": {str(k): v for k, v in sorted(mem.items())},
                   "constant": len(set(mem.values())) == 1},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget_s),
    }
    layer.close()
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.decode:
        return main_decode(args)
    if args.backward:
        return main_backward(args)
    if args.per_segment:
        return main_per_segment(args)

    import numpy as np
    import torch
    from compressive_memory_transformer_segment_amd import binding, profiling
    from compressive_memory_transformer_segment_amd import workloads as wl

    w = wl.WORKLOADS[args.workload or wl.THROUGHPUT_WORKLOAD]
    if w.io_dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    # inputs resident in HBM before the timed region
    d_model = args.d_model or w.heads * w.head_dim
    if args.layer:   # the layer's input X and its weights
        Xh, Wqh, Woh = wl.layer_inputs(w, d_model)
        X, Wq, Wo = (torch.from_numpy(a).to(dev, torch.bfloat16).contiguous() for a in (Xh, Wqh, Woh))
        del Xh, Wqh, Woh
        out_l = torch.empty_like(X)
    else:            # per-head Q, K, V
        Q, K, V, inputs_desc = device_inputs(w, dev, args.pool_segments)
        out = torch.empty_like(Q)
    layer = binding.InfiniAttention(w.batch, w.heads, w.head_dim, w.segment_len, update=w.update,
                                    io_dtype="bf16", eps=w.eps, beta=wl.beta_for(w))
    stream = torch.cuda.current_stream()

    copy_probe(args.copy_probe_mib, dev)

    if args.local_qk and not args.layer:   # distinct buffers; the values do not change the kernels' work
        Ql, Kl = Q.clone(), K.clone()

    def step():
        layer.reset_state(stream)
        if args.layer:
            layer.forward_layer(X, Wq, Wo, out=out_l, stream=stream)
        elif args.local_qk:
            layer.forward_stream_local(Q, K, V, Ql, Kl, out=out, stream=stream)
        else:
            layer.forward_stream(Q, K, V, out=out, stream=stream)

    spin_up(args.spin_up_s, torch.device("cuda", 0))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: warmup {args.warmup} done, timing {args.steps} steps", file=sys.stderr, flush=True)

    # timed region: K steps between two synchronisations and one pair of events
    ms, step_ms, wall_ms = timed_steps(step, args.steps, stream)

    # the same K steps with every kernel bracketed by HIP events on the launch stream
    layer.profile_enable(True)
    for _ in range(args.steps):
        step()
    prof = layer.profile_read()
    layer.profile_enable(False)
    torch.cuda.synchronize()

    tokens = w.batch * w.n_tokens
    value = tokens / (ms / 1e3)
    flops_step = profiling.layer_flops(w.batch, w.heads, w.head_dim, w.segment_len, w.n_tokens, w.update)
    attn_flops = profiling.attention_kernel_flops(w.batch, w.heads, w.head_dim, w.segment_len, w.n_tokens)
    mfma_kernels = {"attention": ("k_attn_bf16 (local attention + retrieval + gate)", attn_flops)}
    if args.layer:
        f_qkv, f_out = profiling.projection_flops(w.batch, w.n_tokens, d_model, w.heads, w.head_dim)
        flops_step += f_qkv + f_out
        mfma_kernels["proj_qkv"] = ("k_gemm (Q/K/V projection)", f_qkv)
        mfma_kernels["proj_out"] = ("k_gemm (output projection)", f_out)
    rooflines = {}
    for kind, (kname, flops) in mfma_kernels.items():
        t_ms, n = prof[kind]
        avg_s = t_ms / n / 1e3
        ach = flops * args.steps / n / avg_s / 1e12
        rooflines[kind] = {"kernel": kname, "achieved": ach, "frac": ach / (profiling.PEAK_BF16_FLOPS / 1e12),
                           "avg_launch_us": avg_s * 1e6, "total_ms_per_step": t_ms / args.steps}
    dominant = max(rooflines, key=lambda k: rooflines[k]["total_ms_per_step"])
    achieved = rooflines[dominant]["achieved"]
    traffic = traffic_from_profiles(profiling.kernel_source_hash()) if dominant == "attention" else None

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spin_up_s": args.spin_up_s,
        "ms_per_step": ms,
        "median_ms_per_step_evented": median(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name + ("-layer" if args.layer else ""), "batch": w.batch, "heads": w.heads,
                   "head_dim": w.head_dim, "segment_len": w.segment_len, "n_tokens": w.n_tokens,
                   "update": w.update, "local_qk": bool(args.local_qk),
                   "projections": bool(args.layer), "d_model": d_model if args.layer else None,
                   "inputs": "exact seeded draws" if args.layer else inputs_desc,
                   "step_time": "K steps between one pair of events, mean", "parallelism": "none"},
        "pct_bf16_peak": 100.0 * flops_step / (ms / 1e3) / profiling.PEAK_BF16_FLOPS,
        "roofline": {
            "kernel": rooflines[dominant]["kernel"],
            "bound": "mfma",
            "achieved": achieved,
            "peak": profiling.PEAK_BF16_FLOPS / 1e12,
            "unit": "TFLOP/s",
            "frac": achieved / (profiling.PEAK_BF16_FLOPS / 1e12),
            "traffic": traffic,
            "algorithmic_bytes": (profiling.attention_kernel_bytes(
                w.batch, w.heads, w.head_dim, w.segment_len, w.n_tokens) if dominant == "attention" else None),
            "avg_launch_us": rooflines[dominant]["avg_launch_us"],
        },
        "mfma_kernels": rooflines,
        "kernels_avg_us": {k: (t / n * 1e3 if n else None) for k, (t, n) in prof.items()},
        "wall_ms_per_step": wall_ms / args.steps,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = (cpu_baseline_layer(w, d_model, args.cpu_budget_s) if args.layer
                               else cpu_baseline(w, args.cpu_budget_s))
    else:
        rec["cpu_baseline"] = None
    layer.close()
    del np
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
