"""Helpers that tie measured figures to the sources they were taken on.

`source_hash(kernel)` fingerprints the HIP sources a kernel (by its timing name)
is built from; bench.py only reports an HBM traffic figure whose recorded hash
still matches. `traffic_from_counters` turns two rocprofv3 `--pmc` runs
(FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into bytes per launch, scaling each
counter by what it reads for a plain copy kernel of known size in the same run.

    python -m padding_free_packed_amd.profiling --fetch F.csv --write W.csv \\
        --kernel bwd_dkdv --workload graph_transformer --copy-bytes 1073741824 \\
        --command "<the rocprofv3 commands>" --out profiles/traffic_bwd_dkdv_graph_transformer.json
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

KERNEL_SOURCES = {
    "attn_fwd": ["attn_fwd.hip", "attn_fwd_bf16.hip", "attn_fwd_w64b.hip", "attn_fwd_short.hip",
                 "attn_f32_wave.hip", "attn_common.h", "common.h"],
    "attn_fwd_first": ["attn_fwd.hip", "common.h"],
    "attn_bwd_first": ["attn_first_bwd.hip", "attn_common.h", "common.h"],
    "bwd_delta": ["attn_bwd.hip", "attn_bwd_seq.hip", "attn_common.h", "common.h"],
    "bwd_dkdv": ["attn_bwd.hip", "attn_bwd_seq.hip", "attn_f32_wave.hip", "attn_common.h", "common.h"],
    "bwd_dq": ["attn_bwd.hip", "attn_bwd_seq.hip", "attn_f32_wave.hip", "attn_common.h", "common.h"],
    "bwd_short": ["attn_bwd_seq.hip", "attn_common.h", "common.h"],
    "pack_rows": ["pack.hip", "common.h"],
    "unpack_rows": ["pack.hip", "common.h"],
    "scan": ["pack.hip", "common.h"],
    "worklist": ["pack.hip", "common.h"],
    "plan": ["pack.hip", "common.h"],
}

# device kernel names behind each timing name, as the profiler prints them:
# demangled ("attn_fwd_kernel<float, 64>") or, where its demangler does not know
# the __bf16 mangling, mangled ("...15attn_fwd_kernelIDF16bLi64E...")
KERNEL_PATTERNS = {
    "attn_fwd": r"attn_fwd(_bf16|_w64b|_short|_f32)?_kernel(<|I)",
    "attn_fwd_first": r"attn_fwd_first_kernel(<|I)",
    "attn_bwd_first": r"attn_bwd_first_kernel(<|I)",
    "bwd_delta": r"bwd_(delta|seq_prep)_kernel(<|I)",
    "bwd_dkdv": r"bwd_(dkdv(_f32)?|kv_seq)_kernel(<|I)",
    "bwd_dq": r"bwd_(dq(_ds)?(_f32)?|q_seq)_kernel(<|I)",
    "bwd_short": r"bwd_short_kernel(<|I)",
    "pack_rows": r"(?<!un)pack_rows_kernel(<|I)",
    "unpack_rows": r"unpack_rows_kernel(<|I)",
    "scan": r"scan_lengths_kernel",
    "worklist": r"worklist_kernel",
    "plan": r"plan_kernel",
}
# the copy probe: bench.py's 1 GiB device-to-device tensor copy, which the runtime runs as
# its blit kernel (torch's own elementwise kernels, e.g. the bf16 conversion of the input
# draws, also read and write gigabytes and must not be taken for it)
COPY_PATTERN = r"__amd_rocclr_copyBuffer"


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def per_dispatch(path: str, counter: str, pattern: str) -> tuple[float, int]:
    """Mean value of `counter` over the dispatches whose kernel name matches `pattern`."""
    tot = collections.defaultdict(float)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or not re.search(pattern, r["Kernel_Name"]):
                continue
            tot[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not tot:
        raise SystemExit(f"{path}: no {counter} rows for /{pattern}/")
    return sum(tot.values()) / len(tot), len(tot)


def traffic_from_counters(fetch_csv, write_csv, kernel, copy_bytes):
    pat = KERNEL_PATTERNS[kernel]
    f_k, nf = per_dispatch(fetch_csv, "FETCH_SIZE", pat)
    w_k, nw = per_dispatch(write_csv, "WRITE_SIZE", pat)
    # the largest copy dispatches are the probe (torch's own small copies are far smaller)
    f_c, _ = per_dispatch_largest(fetch_csv, "FETCH_SIZE", COPY_PATTERN)
    w_c, _ = per_dispatch_largest(write_csv, "WRITE_SIZE", COPY_PATTERN)
    kf = copy_bytes / (f_c * 1024.0)
    kw = copy_bytes / (w_c * 1024.0)
    return {
        "kernel": kernel,
        "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k, "dispatches": [nf, nw],
        "copy_bytes": copy_bytes, "copy_fetch_kib": f_c, "copy_write_kib": w_c,
        "fetch_scale": kf, "write_scale": kw,
        "bytes_per_launch": f_k * 1024.0 * kf + w_k * 1024.0 * kw,
    }


def per_dispatch_largest(path: str, counter: str, pattern: str) -> tuple[float, int]:
    vals = collections.defaultdict(float)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and re.search(pattern, r["Kernel_Name"]):
                vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"{path}: no copy dispatch with {counter}")
    top = max(vals.values())
    big = [v for v in vals.values() if v >= 0.5 * top]
    return sum(big) / len(big), len(big)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--kernel", required=True, choices=sorted(KERNEL_PATTERNS))
    ap.add_argument("--workload", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    t = traffic_from_counters(a.fetch, a.write, a.kernel, a.copy_bytes)
    t.update({"workload": a.workload, "source_hash": source_hash(a.kernel), "command": a.command})
    with open(a.out, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t))


if __name__ == "__main__":
    main()
