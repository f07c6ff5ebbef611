"""Measurement helpers: FLOP/byte accounting of the layer and rocprofv3 summaries.

* ``layer_flops`` / ``attention_kernel_flops`` / ``attention_kernel_bytes``: algorithmic
  work of one forward pass (what the method must do, not what the kernels execute).
* ``python -m compressive_memory_transformer_segment_amd.profiling stats <kernel_stats.csv>``
  prints a short markdown table of a ``rocprofv3 --kernel-trace --stats`` run.
* ``python -m ... pmc <counter_collection.csv> <counter>`` prints per-kernel averages of one
  PMC counter (FETCH_SIZE or WRITE_SIZE, KiB per dispatch).
* ``kernel_source_hash`` identifies the attention kernel's source, so a stored counter
  summary can be matched with the kernel that is built now.
"""

from __future__ import annotations

import csv
import hashlib
import re
import os
import sys
from collections import defaultdict

PKG_DIR = os.path.dirname(os.path.abspath(__file__))

# MI355X published peaks
PEAK_BF16_FLOPS = 2.5e15
PEAK_HBM_BYTES = 8.0e12


def segment_lengths(n_tokens: int, segment_len: int):
    full, tail = divmod(n_tokens, segment_len)
    return [segment_len] * full + ([tail] if tail else [])


def local_attention_flops(n: int, d: int) -> float:
    """Causal QK^T and PV over one segment of n tokens: 2d multiply-adds per (query, key)
    pair with key <= query, two products: 2 * d * n * (n + 1)."""
    return 2.0 * d * n * (n + 1)


def retrieval_flops(n: int, d: int) -> float:
    return 2.0 * n * d * d


def update_flops(n: int, d: int, update: str) -> float:
    return (4.0 if update == "delta" else 2.0) * n * d * d


def layer_flops(batch, heads, head_dim, segment_len, n_tokens, update) -> float:
    """Matrix-class FLOPs of one layer forward over the stream (all heads)."""
    tot = 0.0
    for n in segment_lengths(n_tokens, segment_len):
        tot += local_attention_flops(n, head_dim) + retrieval_flops(n, head_dim) + update_flops(n, head_dim, update)
    return tot * batch * heads


def attention_kernel_flops(batch, heads, head_dim, segment_len, n_tokens) -> float:
    """Algorithmic FLOPs of the fused attention kernel (local attention + retrieval)."""
    tot = 0.0
    for n in segment_lengths(n_tokens, segment_len):
        tot += local_attention_flops(n, head_dim) + retrieval_flops(n, head_dim)
    return tot * batch * heads


def attention_kernel_bytes(batch, heads, head_dim, segment_len, n_tokens) -> float:
    """Algorithmic HBM bytes of the fused attention kernel: Q, K, V read once (bf16),
    out written once (bf16), M^T (bf16) and z (fp32) read once per segment."""
    d = head_dim
    segs = len(segment_lengths(n_tokens, segment_len))
    return batch * heads * (n_tokens * d * 2 * 4 + segs * (d * d * 2 + d * 4))


def projection_flops(batch, n_tokens, d_model, heads, head_dim):
    """(Q/K/V projection, output projection) FLOPs: 2 B T d_model (3 H d) and 2 B T (H d) d_model."""
    hd = heads * head_dim
    return 2.0 * batch * n_tokens * d_model * 3 * hd, 2.0 * batch * n_tokens * hd * d_model


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("attention.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(PKG_DIR, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------- rocprofv3 summaries

def _short(name: str) -> str:
    """Kernel name without namespaces and argument list, template arguments kept."""
    m = re.search(r"infini::(?:\(anonymous namespace\)::)?(k_\w+(?:<[^>]*>)?)", name)
    if m:
        return m.group(1)
    if "copyBuffer" in name:
        return "__amd_rocclr_copyBuffer"
    if "direct_copy_kernel" in name:
        return "torch direct_copy_kernel (input staging)"
    if "distribution" in name:
        return "torch random fill (bench inputs, spin-up operand)"
    return (name.split("(")[0] or "(unnamed)")[:80]


def stats_table(path: str) -> str:
    """Kernel table of a rocprofv3 --stats summary.  The library's bf16 products that
    bench.py runs before its warmup steps to bring the clocks up (hipBLASLt ``Cijk_`` kernels)
    are left out, and the percentages are of the remaining kernels' time."""
    rows = [r for r in csv.DictReader(open(path)) if "Cijk_" not in (r.get("Name") or r.get("KernelName") or "")]
    total = sum(float(r.get("TotalDurationNs", 0)) for r in rows) or 1.0
    out = ["| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or ""
        calls = int(r.get("Calls", 0))
        tot = float(r.get("TotalDurationNs", 0)) / 1e6
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        pct = 100.0 * float(r.get("TotalDurationNs", 0)) / total
        out.append(f"| `{_short(name)}` | {calls} | {tot:.3f} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.1f} |")
    return "\n".join(out)


def pmc_table(path: str, counter: str) -> str:
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        vals[r.get("Kernel_Name", "")].append(float(r["Counter_Value"]))
    out = [f"| kernel | dispatches | avg {counter} (KiB) |", "|---|---|---|"]
    for name, v in vals.items():
        out.append(f"| `{_short(name)}` | {len(v)} | {sum(v) / len(v):.1f} |")
    return "\n".join(out)


def _per_kernel(path: str, counter: str, grid: int | None = None):
    """Counter values (KiB) per dispatch of each kernel; optionally only dispatches whose
    grid size (work items) is ``grid``."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        if grid is not None and int(r.get("Grid_Size", -1)) != grid:
            continue
        vals[_short(r.get("Kernel_Name", ""))].append(float(r["Counter_Value"]))
    return vals


def hbm_summary(fetch_csv: str, write_csv: str, copy_mib: int, algorithmic_bytes: float) -> str:
    """Markdown summary of the attention kernel's HBM traffic from two counter passes.

    Each counter is calibrated on the device copy of ``copy_mib`` MiB that bench.py runs
    before timing (``--copy-probe-mib``): factor = known bytes / counter reading, taken
    from the largest copy dispatch.  The attention kernel's readings are scaled by the
    same factors."""
    known = copy_mib * 1024.0   # KiB read and written by the copy
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    f_copy = max(fetch["__amd_rocclr_copyBuffer"])
    w_copy = max(write["__amd_rocclr_copyBuffer"])
    kf, kw = known / f_copy, known / w_copy
    key = next(k for k in fetch if k.startswith("k_attn_bf16"))
    fa = sum(fetch[key]) / len(fetch[key])
    wa = sum(write[key]) / len(write[key])
    total = (fa * kf + wa * kw) * 1024.0
    lines = [
        f"kernel: `{key}`; kernel source hash: `{kernel_source_hash()}`",
        "",
        "| counter | copy probe reading (KiB) | known (KiB) | factor | attention avg per dispatch (KiB) | scaled (MB) |",
        "|---|---|---|---|---|---|",
        f"| FETCH_SIZE | {f_copy:.1f} | {known:.0f} | {kf:.4f} | {fa:.1f} ({len(fetch[key])} dispatches) | {fa * kf * 1024 / 1e6:.1f} |",
        f"| WRITE_SIZE | {w_copy:.1f} | {known:.0f} | {kw:.4f} | {wa:.1f} ({len(write[key])} dispatches) | {wa * kw * 1024 / 1e6:.1f} |",
        "",
        f"HBM bytes per launch (scaled): {total:.6e}",
        f"Algorithmic bytes per launch: {algorithmic_bytes:.6e} (ratio {total / algorithmic_bytes:.2f})",
    ]
    return "\n".join(lines)


def _stats_avg_us(stats_csv: str):
    """Average duration (us) per kernel (short name) from a --kernel-trace --stats csv."""
    out = {}
    for r in csv.DictReader(open(stats_csv)):
        name = r.get("Name") or r.get("KernelName") or ""
        out[_short(name)] = float(r.get("AverageNs", 0)) / 1e3
    return out


def traffic_table(fetch_csv: str, write_csv: str, copy_mib: int, stats_csv: str, algorithmic=None) -> str:
    """Markdown table of the HBM bytes per dispatch of every library kernel in two counter
    passes (FETCH_SIZE, WRITE_SIZE), each scaled by the factor the same counter reads for
    the device copy of ``copy_mib`` MiB, with the achieved bandwidth over the kernel's
    average duration from a kernel-trace run of the same command, against 8 TB/s.
    ``algorithmic``: optional {kernel short name: algorithmic bytes per dispatch}."""
    known = copy_mib * 1024.0
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    kf = known / max(fetch["__amd_rocclr_copyBuffer"])
    kw = known / max(write["__amd_rocclr_copyBuffer"])
    avg_us = _stats_avg_us(stats_csv)
    algorithmic = algorithmic or {}
    lines = [f"copy-probe factors: FETCH_SIZE x{kf:.4f}, WRITE_SIZE x{kw:.4f}", "",
             "| kernel | dispatches | read MB | write MB | total MB | avg us | GB/s | of 8 TB/s | algorithmic MB | ratio |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for name in fetch:
        if not name.startswith("k_") or name not in write:
            continue
        fr = sum(fetch[name]) / len(fetch[name]) * kf * 1024 / 1e6
        wr = sum(write[name]) / len(write[name]) * kw * 1024 / 1e6
        tot = fr + wr
        us = avg_us.get(name)
        gbs = tot * 1e6 / (us * 1e-6) / 1e9 if us else None
        alg = algorithmic.get(name)
        lines.append(f"| `{name}` | {len(fetch[name])} | {fr:.1f} | {wr:.1f} | {tot:.1f} | "
                     + (f"{us:.1f} | {gbs:.0f} | {gbs / (PEAK_HBM_BYTES / 1e9):.2f}" if us else "- | - | -")
                     + (f" | {alg / 1e6:.1f} | {tot * 1e6 / alg:.2f} |" if alg else " | - | - |"))
    return "\n".join(lines)


def state_kernel_bytes(batch, heads, head_dim, segment_len, n_tokens, update, chunks):
    """Algorithmic HBM bytes of the state pass and the chain over one window holding the
    whole stream (S segments, `chunks` partial slots per segment): the state pass reads K
    and V once (bf16) and writes its partial sums once (fp32: key sums, (sigma(K)^T V)^T and,
    delta, the Gram term); the chain reads the partials and the state, writes the state,
    the bf16 M^T_{s-1} and the z_{s-1} of every segment.  Returns {kernel: bytes}."""
    d, S = head_dim, len(segment_lengths(n_tokens, segment_len))
    bh = batch * heads
    kv = bh * n_tokens * d * 2 * 2
    part = d * 4 + d * d * 4 + (d * d * 4 if update == "delta" else 0)
    parts = bh * S * chunks * part
    state = bh * (d * d + d) * 4
    chain = parts + 2 * state + bh * S * (d * d * 2 + d * 4)
    out = {}
    if update == "delta":
        out["k_keysum_bf16<128>"] = bh * n_tokens * d * 2 + bh * S * chunks * d * 4
        out["k_state_delta_bf16<128>"] = kv + parts
    else:
        out["k_state_lin_bf16<128>"] = kv + parts
    out["chain"] = chain
    return out


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "stats":
        print(stats_table(sys.argv[2]))
    elif what == "pmc":
        print(pmc_table(sys.argv[2], sys.argv[3]))
    elif what == "hbm":
        # hbm <fetch csv> <write csv> <copy MiB> : the C1-shaped attention launch
        alg = attention_kernel_bytes(1, 8, 128, 2048, 32768)
        print(hbm_summary(sys.argv[2], sys.argv[3], int(sys.argv[4]), alg))
    elif what == "traffic":
        # traffic <fetch csv> <write csv> <copy MiB> <kernel stats csv>
        print(traffic_table(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5]))
    elif what == "hash":
        print(kernel_source_hash())
    else:
        raise SystemExit(f"unknown command {what}")
