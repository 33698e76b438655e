#!/usr/bin/env python3
"""Benchmark of the packed-attention path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM:

    pe_pack (lengths -> cu_seqlens, flat_index, packed rows of the padded grid;
             its one host read included)
    pe_varlen_attn_fwd (work list + forward with log-sum-exp; _local with --window)
    pe_varlen_attn_fwd_first_token
    pe_varlen_attn_bwd (when the workload carries dO; _local with --window)
    pe_varlen_attn_bwd_first_token (when the workload carries dO: the readout's
             gradient is dO at the first rows)
    pe_unpack (attention output back to the padded grid)

The default workload is the graph-transformer shape: 4096 sequences of at most
256 tokens, lengths round(N(90, 40)) clipped to [1, 256], 8 heads x 64, fp32,
padded grid [4096, 256, 512]. `value` is real tokens per second of the whole
step. Every kernel launch inside the timed region is bracketed by HIP events
(pe_timing_enable), which gives each kernel's average duration; the roofline
entry is for the kernel with the largest time per step, priced at its
algorithmic work (algo_work below). The CPU baseline times the fp64 oracle on a
bounded sample of the same batch.

Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed varlen attn fwd real tokens/s + TFLOP/s, % of MI355X MFMA/HBM roofline"
PEAK = {"bf16": 2500.0, "fp32": 157.3}   # dense MFMA TFLOP/s
HBM_PEAK = 8000.0                        # GB/s


def band_pairs(lengths, window):
    """Query-key pairs a sequence keeps: L^2 (global), or those with |i - j| <= window."""
    import numpy as np
    L = np.asarray(lengths, dtype=np.float64)
    if window is None:
        return float((L * L).sum())
    m = np.minimum(float(window), L - 1)
    return float((L + 2.0 * (m * L - m * (m + 1) / 2.0)).sum())


def algo_work(kernel, w, N, L2, e, with_lse, with_grid=True):
    """Algorithmic work of one launch: {'flop': count, 'byte': count} (attention kernels
    carry both). L2 is the number of attended (query, key) pairs: sum L^2, or the
    band's for local attention."""
    B, S, H, d = w.num_seqs, w.max_seq_len, w.num_heads, w.head_dim
    D = H * d
    T = (N + 127) // 128
    lse_b = 4.0 * N * H if with_lse else 0.0
    wave_dq = e == 4 and d in (32, 64)
    return {
        # forward: 4 L2 H d flops (QK^T and PV); read Q, K, V, write O (+ LSE)
        "attn_fwd": {"flop": 4.0 * L2 * H * d, "byte": 4.0 * N * D * e + lse_b},
        # backward split by kernel: dK/dV performs S, dP, dV and dK (8 L2 H d) and moves
        # Q, K, V, dO, LSE, D in and dK, dV out; dQ is credited with dQ alone (2 L2 H d),
        # its recomputation of S and dP is not counted
        "bwd_dkdv": {"flop": 8.0 * L2 * H * d, "byte": 6.0 * N * D * e + 8.0 * N * H},
        # (the fp32 one-wave dQ also reads O and writes D, the delta pass it replaces)
        "bwd_dq": {"flop": 2.0 * L2 * H * d, "byte": (6.0 if wave_dq else 5.0) * N * D * e + 8.0 * N * H},
        # first token: read K and V once, the B queries, write B outputs (+ LSE)
        "attn_fwd_first": {"byte": 2.0 * N * D * e + 2.0 * B * D * e + (4.0 * B * H if with_lse else 0.0)},
        # first-token backward: read K, V and the B rows of q, dO, O (+ LSE), write dK, dV and dq_first
        "attn_bwd_first": {"byte": 4.0 * N * D * e + 4.0 * B * D * e + 4.0 * B * H},
        "bwd_delta": {"byte": 2.0 * N * D * e + 4.0 * N * H},
        # pack: read and write the real rows, write flat_index (only flat_index without a grid)
        "pack_rows": {"byte": (2.0 * N * D * e if with_grid else 0.0) + 8.0 * N},
        # unpack: read the real rows, write the whole grid
        "unpack_rows": {"byte": 1.0 * N * D * e + 1.0 * B * S * D * e},
        "scan": {"byte": 4.0 * B + 4.0 * (B + 1)},
        # NeMo rows: the mask is read by both passes; flat index and cu written once
        "flatten_count": {"byte": 4.0 * w.extra.get("grid_rows", 0) + 8.0 * w.extra.get("rows", 0)},
        "flatten_write": {"byte": 4.0 * w.extra.get("grid_rows", 0) + 8.0 * N + 4.0 * (B + 1)},
        # gather: read and write the real rows (+ the flat index); scatter: read the real rows, write the grid
        "gather_rows": {"byte": 2.0 * N * D * e + 8.0 * N},
        "scatter_rows": {"byte": 1.0 * N * D * e + 1.0 * w.extra.get("grid_rows", 0) * D * e + 8.0 * N},
        "worklist": {"byte": 4.0 * (B + 1) + 4.0 * (T + 1)},
    }.get(kernel)


def rate(work, ms, dtype):
    """Roofline entry of one launch: bound by arithmetic intensity (flops per algorithmic
    byte) against the ridge point peak / 8 TB/s; HBM-bound work is priced in bytes."""
    peak = PEAK[dtype]
    ridge = peak * 1e12 / (HBM_PEAK * 1e9)
    if "flop" in work and work["flop"] >= ridge * work["byte"]:
        a = work["flop"] / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": a, "peak": peak, "unit": "TFLOP/s", "frac": a / peak,
                "intensity": work["flop"] / work["byte"]}
    a = work["byte"] / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK, "unit": "GB/s", "frac": a / HBM_PEAK}
    if "flop" in work:
        r["intensity"] = work["flop"] / work["byte"]
    return r


def load_traffic(kernel, workload):
    from padding_free_packed_amd.profiling import source_hash

    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this source."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel):
        return None
    return t.get("bytes_per_launch")


def graph_bench(args):
    """The short_batch workload: one step is one replay of the captured bucket forward
    (the work of pe_pack_async of the fused Q/K/V grid, pe_varlen_attn_fwd_qkv over the
    bucket's capacity and pe_unpack, with the scan and work lists fused into one plan
    kernel) for a batch of 64 short sequences in a (64, 48) bucket. The same forward by
    the eager calls (pe_pack with its host read, then the same two calls) is timed beside
    it; per-kernel times come from the eager pass (launches inside a graph carry no
    events), and the graph replays the same copy and attention kernels."""
    import numpy as np
    import torch

    from padding_free_packed_amd import graphs, pe
    from padding_free_packed_amd import workloads as W

    w = W.short_batch(args.num_seqs)
    dev = "cuda:0"
    B, S, H, d = w.num_seqs, w.max_seq_len, w.num_heads, w.head_dim
    D, N, e = H * d, w.total_tokens, 2
    cu_h = np.concatenate([[0], np.cumsum(w.lengths.astype(np.int64))])
    # the fused grid [B, S, 3, H, d] holding each sequence's q, k, v rows; padding NaN
    fused = np.full((B, S, 3, H, d), W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0], dtype=np.uint16)
    for b in range(B):
        for j, x in enumerate((w.q, w.k, w.v)):
            fused[b, :w.lengths[b], j] = x[cu_h[b]:cu_h[b + 1]]
    w.grid = fused.reshape(B, S, 3 * D)
    bucket = graphs.ForwardBucket(B, S, H, d, torch.bfloat16, w.scale, -1, with_lse=False, device=dev)
    bucket.lengths.copy_(torch.from_numpy(w.lengths.astype(np.int32)))
    bucket.qkv_grid.copy_(torch.from_numpy(fused.view(np.int16)).view(torch.bfloat16))
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    packed = torch.empty(N, 3, H, d, dtype=torch.bfloat16, device=dev)
    out = torch.empty(N, H, d, dtype=torch.bfloat16, device=dev)
    grid_out = torch.empty_like(bucket.out_grid)
    ws_pack = pe.workspace(pe.pe_pack_workspace_size(B, S, 3 * D, pe.PE_BF16), dev)
    ws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, d, pe.PE_BF16, False), dev)
    grid_in = bucket.qkv_grid.view(B, S, 3 * D)

    def eager():
        n = pe.pe_pack(bucket.lengths, S, grid_in, cu, None, packed.view(N, 3 * D), N, ws_pack, pe.PE_BF16)
        pe.pe_varlen_attn_fwd_qkv(packed, cu, B, n, S, w.scale, -1, out, None, ws)
        pe.pe_unpack(out, cu, B, S, n, grid_out)

    def timed(fn, steps):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps, time.perf_counter() - wall0

    for _ in range(args.warmup):
        bucket.replay()
        eager()
    torch.cuda.synchronize()
    assert bucket.status.tolist() == [N, pe.PACK_OK]
    assert torch.equal(bucket.out_grid.view(torch.int16), grid_out.view(torch.int16))
    ms_step, wall = timed(bucket.replay, args.steps)
    ms_eager, _ = timed(eager, args.steps)
    pe.pe_timing_enable(True)
    pe.pe_timing_read()
    eager()
    torch.cuda.synchronize()
    recs = pe.pe_timing_read()
    pe.pe_timing_enable(False)
    breakdown = {}
    L2 = band_pairs(w.lengths, None)
    for name, ms in recs:
        ent = breakdown.setdefault(name, {"avg_ms": 0.0, "launches_per_step": 0})
        ent["avg_ms"] += ms
        ent["launches_per_step"] += 1
    for name, ent in breakdown.items():
        ent["avg_ms"] /= ent["launches_per_step"]
        ent["ms_per_step"] = ent["avg_ms"] * ent["launches_per_step"]
        aw = algo_work(name, w, N, L2, e, False, True)
        if name == "pack_rows":
            aw = {"byte": 2.0 * N * 3 * D * e}          # rows of the fused grid; no flat_index written
        if aw is not None and ent["avg_ms"] > 0:
            ent.update(rate(aw, ent["avg_ms"], "bf16"))
    dom = max(breakdown, key=lambda k_: breakdown[k_]["ms_per_step"])
    work = algo_work(dom, w, N, L2, e, False, True)
    if dom == "pack_rows":
        work = {"byte": 2.0 * N * 3 * D * e}
    roof = rate(work, breakdown[dom]["avg_ms"], "bf16")
    roof.update({"traffic": None, "kernel": dom,
                 "algorithmic_per_launch": work["flop"] if roof["bound"] == "mfma" else work["byte"]})
    result = {
        "metric": METRIC, "value": N / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "short_batch", "num_seqs": B, "max_seq_len": S, "total_tokens": N, "num_heads": H,
                   "head_dim": d, "grid": [B, S, 3, H, d], "window": None,
                   "step": "graph replay: plan(scan+work lists)+pack(fused qkv grid)+fwd_qkv(capacity rows)+unpack"},
        "eager_ms_per_step": ms_eager,
        "kernel_ms_sum": sum(v_["ms_per_step"] for v_ in breakdown.values()),
        "roofline": roof, "breakdown": breakdown, "wall_s_timed_region": wall,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, first_token=False)
    bucket.close()
    print(json.dumps(result))


def cpu_baseline(w, budget_s, window=None, nemo_mask=None, first_token=True):
    """The fp64 oracle on the first m sequences of the batch (a valid packed batch itself),
    with m sized for about `budget_s` seconds, BLAS limited to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from padding_free_packed_amd import workloads as W

    cu_all = np.concatenate([[0], np.cumsum(w.lengths.astype(np.int64))])

    def run(m):
        n = int(cu_all[m])
        L = w.lengths[:m]
        grid = w.grid[:m] if w.grid is not None else None
        q, k, v = (W.to_f64(x[:n], w.dtype) for x in (w.q, w.k, w.v))
        do = W.to_f64(w.dout[:n], w.dtype) if w.dout is not None else None
        t0 = time.perf_counter()
        if nemo_mask is not None:  # the rows holding these documents: flatten, gather q, k, v
            rows = int(np.count_nonzero(nemo_mask.max(axis=1) > 0)) if m == w.num_seqs else \
                min(nemo_mask.shape[0], 1 + int(np.searchsorted(np.cumsum((nemo_mask > 0).sum(1)), n)))
            fl, _ = oracle.flatten_document_mask(nemo_mask[:rows])
            for x in (w.q, w.k, w.v):
                oracle.gather_rows(np.zeros((rows * nemo_mask.shape[1],) + x.shape[1:], dtype=x.dtype), fl)
        cu, flat, N = oracle.layout(L, w.max_seq_len)
        if grid is not None:
            oracle.pack(grid, flat)
        o, _ = oracle.attention(q, k, v, cu, w.scale, window=window)
        if nemo_mask is None and first_token:
            oracle.attention_first_token(q[cu[:-1]], k, v, cu, w.scale)
        if do is not None:
            oracle.attention_backward(do, q, k, v, cu, w.scale, window=window)
            oracle.attention_first_token_backward(do[cu[:-1]], q[cu[:-1]], k, v, cu, w.scale)
        if grid is not None:
            oracle.unpack(o.reshape(N, -1), cu, w.max_seq_len)
        return time.perf_counter() - t0, n

    with threadpool_limits(limits=1):
        m = min(64, w.num_seqs)
        t, n = run(m)
        m = int(min(w.num_seqs, max(m, m * budget_s / max(t, 1e-3))))
        t, n = run(m)
    return {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {m} of {w.num_seqs} sequences ({n} tokens): "
                      + ("flatten of their rows, gather, layout, forward," if nemo_mask is not None else
                         "layout, pack, forward," + (" first-token," if first_token else ""))
                      + (" backward, first-token backward," if w.dout is not None else "")
                      + (" unpack" if w.grid is not None else "") + f" in float64, {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="graph_transformer",
                    choices=["graph_transformer", "short_query", "long_document", "mixed_training", "tiny",
                             "nemo_packed", "short_batch"])
    ap.add_argument("--num-seqs", type=int, default=64,
                    help="short_batch only: sequences in the batch (and slots of its captured bucket)")
    ap.add_argument("--window", type=int, default=None,
                    help="local attention: each query sees the keys within this distance in its sequence "
                         "(pe_varlen_attn_fwd_local / _bwd_local); default global attention")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, copy a buffer of this many MiB three times (a plain copy kernel "
                         "of known size, for scaling HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): it measures "
              "one GPU's share of the batch. The path shards by sequence (no exchange inside attention), "
              "which is not run here.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "short_batch":
        return graph_bench(args)

    import numpy as np
    import torch

    from padding_free_packed_amd import pe
    from padding_free_packed_amd import workloads as W

    gen = {
        "graph_transformer": lambda: W.graph_transformer(grid=True, with_grad=True),
        "short_query": lambda: W.short_query(grid=True),
        "long_document": W.long_document,
        "mixed_training": W.mixed_training,
        "tiny": lambda: W.tiny(with_grad=True),
        # the mixed-training documents packed NeMo-style into rows of 8192 tokens (forward only)
        "nemo_packed": W.mixed_training,
    }[args.workload]
    w = gen()
    nemo = args.workload == "nemo_packed"
    if nemo:
        nemo_mask, nemo_grids = W.nemo_rows(w, w.max_seq_len)
        w.dout = None
        w.extra["rows"] = nemo_mask.shape[0]
        w.extra["grid_rows"] = nemo_mask.size
    dev = "cuda:0"
    B, S, H, d = w.num_seqs, w.max_seq_len, w.num_heads, w.head_dim
    D = H * d
    N = w.total_tokens
    L2 = band_pairs(w.lengths, args.window)
    bf = w.dtype == W.BF16
    e = 2 if bf else 4
    code = pe.PE_BF16 if bf else pe.PE_FP32

    def up(x):
        if x is None:
            return None
        if bf:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    lengths = torch.from_numpy(w.lengths.astype(np.int32)).to(dev)
    q, k, v, dout = up(w.q), up(w.k), up(w.v), up(w.dout)
    # workloads without a padded grid of their own pack the layout only (cu_seqlens, flat_index)
    grid = up(w.grid)
    cu_h = np.concatenate([[0], np.cumsum(w.lengths.astype(np.int64))])
    q_first = q[torch.from_numpy(cu_h[:-1]).to(dev)].contiguous()

    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    flat = torch.empty(N, dtype=torch.int64, device=dev)
    packed = torch.empty(N, D, dtype=q.dtype, device=dev) if grid is not None else None
    out = torch.empty_like(q)
    lse = torch.empty(H, N, device=dev)
    out_first = torch.empty_like(q_first)
    lse_first = torch.empty(H, B, device=dev)
    grid_out = torch.empty_like(grid) if grid is not None else None
    with_bwd = dout is not None
    dq, dk, dv = ((torch.empty_like(q) for _ in range(3)) if with_bwd else (None, None, None))
    # the first-token readout is trained through as well: its gradient is dO at the first rows
    first_rows = torch.from_numpy(cu_h[:-1]).to(dev)
    dout_first = dout[first_rows].contiguous() if with_bwd else None
    dq_first = torch.empty_like(q_first) if with_bwd else None
    dk_first, dv_first = ((torch.empty_like(k), torch.empty_like(v)) if with_bwd else (None, None))
    ws_pack = pe.workspace(pe.pe_pack_workspace_size(B, S, D, code), dev)
    ws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, d, code, with_bwd), dev)
    scale = w.scale

    if nemo:
        # flatten the indexed document mask, gather Q, K, V from the padded row grids, attend,
        # scatter the output back to the row grid
        mask_d = torch.from_numpy(nemo_mask).to(dev)
        ws_flat = pe.workspace(pe.pe_flatten_workspace_size(nemo_mask.shape[0]), dev)
        grids_d = [up(nemo_grids[nm]) for nm in ("q", "k", "v")]
        del nemo_grids
        grid_rows_out = torch.empty_like(grids_d[0])

    def step():
        if nemo:
            n, docs = pe.pe_flatten_document_mask(mask_d, flat, cu, ws_flat)
            assert (n, docs) == (N, B)
            for src, dst in zip(grids_d, (q, k, v)):
                pe.pe_gather_rows(src, flat, dst)
            pe.pe_varlen_attn_fwd(q, k, v, cu, B, N, S, scale, out, lse, ws)
            pe.pe_scatter_rows(out, flat, grid_rows_out)
            return
        n = pe.pe_pack(lengths, S, grid, cu, flat, packed, N, ws_pack, code)
        assert n == N
        if args.window is None:
            pe.pe_varlen_attn_fwd(q, k, v, cu, B, N, S, scale, out, lse, ws)
        else:
            pe.pe_varlen_attn_fwd_local(q, k, v, cu, B, N, S, scale, args.window, out, lse, ws)
        pe.pe_varlen_attn_fwd_first_token(q_first, k, v, cu, B, N, S, scale, out_first, lse_first)
        if with_bwd and args.window is None:
            pe.pe_varlen_attn_bwd(dout, q, k, v, out, lse, cu, B, N, S, scale, dq, dk, dv, ws)
        elif with_bwd:
            pe.pe_varlen_attn_bwd_local(dout, q, k, v, out, lse, cu, B, N, S, scale, args.window, dq, dk, dv, ws)
        if with_bwd:
            pe.pe_varlen_attn_bwd_first_token(dout_first, q_first, k, v, out_first, lse_first, cu, B, N, S, scale,
                                              dq_first, dk_first, dv_first)
        if grid is not None:
            pe.pe_unpack(out.view(N, D), cu, B, S, N, grid_out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    pe.pe_timing_enable(True)
    pe.pe_timing_read()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    recs = pe.pe_timing_read()
    pe.pe_timing_enable(False)
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps

    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    breakdown = {}
    for name, lst in per.items():
        launches_per_step = len(lst) / args.steps
        avg = float(np.mean(lst))
        ent = {"avg_ms": avg, "launches_per_step": launches_per_step, "ms_per_step": avg * launches_per_step}
        aw = algo_work(name, w, N, L2, e, True, grid is not None)
        if aw is not None and avg > 0:
            ent.update(rate(aw, avg, "bf16" if bf else "fp32"))
        breakdown[name] = ent
    dom = max(breakdown, key=lambda k_: breakdown[k_]["ms_per_step"])
    work = algo_work(dom, w, N, L2, e, True, grid is not None)
    roof = rate(work, breakdown[dom]["avg_ms"], "bf16" if bf else "fp32")
    roof["traffic"] = load_traffic(dom, args.workload if args.window is None else f"{args.workload}_w{args.window}")
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = work["flop"] if roof["bound"] == "mfma" else work["byte"]

    fwd_ms = breakdown["attn_fwd"]["avg_ms"]
    result = {
        "metric": METRIC,
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "num_seqs": B, "max_seq_len": S, "total_tokens": N, "num_heads": H,
            "head_dim": d, "grid": [B, S, D] if grid is not None else None, "window": args.window,
            "step": ("flatten(mask)+gather(q,k,v)+fwd(lse)+scatter" if nemo else
                     ("pack" if grid is not None else "pack(layout only)") + "+fwd(lse)+first_token"
                     + ("+bwd+first_token_bwd" if with_bwd else "") + ("+unpack" if grid is not None else "")),
            "rows": [int(w.extra["rows"]), int(S)] if nemo else None,
        },
        "fwd": {"ms": fwd_ms, "tokens_per_s": N / (fwd_ms * 1e-3),
                "tflops": 4.0 * L2 * H * d / (fwd_ms * 1e-3) / 1e12},
        "roofline": roof,
        "breakdown": breakdown,
        "wall_s_timed_region": wall,
    }
    if args.copy_probe_mib > 0:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = nbytes
        del src, dst
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, args.window, nemo_mask if nemo else None)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
