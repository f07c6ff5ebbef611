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


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("attention.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(PKG_DIR, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------- rocprofv3 summaries

def _short(name: str) -> str:
    """Kernel name without namespaces and argument list, template arguments kept."""
    for key in ("k_attn_bf16", "k_attn_f32", "k_state_bf16", "k_state_f32", "k_keysum_f32",
                "k_chain_linear", "k_chain_delta", "k_zero_f32"):
        i = name.find(key)
        if i >= 0:
            rest = name[i:]
            j = rest.find("(")
            return rest[:j] if j >= 0 else rest
    if "copyBuffer" in name:
        return "__amd_rocclr_copyBuffer"
    if "direct_copy_kernel" in name:
        return "torch direct_copy_kernel (input staging)"
    return (name.split("(")[0] or "(unnamed)")[:80]


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or ""
        calls = int(r.get("Calls", 0))
        tot = float(r.get("TotalDurationNs", 0)) / 1e6
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        pct = float(r.get("Percentage", 0))
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


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "stats":
        print(stats_table(sys.argv[2]))
    elif what == "pmc":
        print(pmc_table(sys.argv[2], sys.argv[3]))
    elif what == "hash":
        print(kernel_source_hash())
    else:
        raise SystemExit(f"unknown command {what}")
