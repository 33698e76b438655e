#!/usr/bin/env python3
"""Benchmark of the packed-attention path on one MI355X.

Default workload: the long-document encoding batch, 1024 documents with lengths
round(lognormal(ln 512, 0.8)) clipped to [64, 8192] (740,881 real tokens),
12 heads x 64, bf16 with fp32 accumulation. One step is the forward as a caller
runs it over the batch resident in HBM:

    pe_pack (lengths -> cu_seqlens and flat_index; its one host read included)
    pe_varlen_attn_fwd (work list + forward, with the log-sum-exp)

`value` is real tokens per second of that step (ms_per_step is the mean of the
K timed steps; median and min are reported too). Each timed step is preceded by
a read of a 1 GiB buffer, so no input is served from the 256 MB last-level
cache, and is bracketed by two events on the stream the library launches on;
per-kernel events are off while the steps are timed. A second pass over the
same steps with the library's per-kernel HIP events on gives each kernel's
launch durations (`breakdown`); `roofline` is the forward kernel priced at its
algorithmic work (4 sum(L^2) H d flops) against the bf16 MFMA peak.

`configs` holds the same measurements for every standing workload (tiny,
graph_transformer, short_query, long_document, mixed_training): for each call
of its path (pack, forward, first-token forward, backward, first-token
backward, unpack) the median, min and mean time over timed launches with a
flush before each, and for each kernel its rate against the roofline that bounds
it (bf16 or fp32 MFMA for attention on long sequences, 8 TB/s HBM for copies,
the first-token calls and the short-query forward).

Inputs: the lengths are the seeded recipe of each workload (numpy); Q, K, V,
dO and the padded grids are N(0, 1) draws of torch's seeded generator on the
device, rounded to the workload's dtype (workloads.device_inputs).

The CPU baseline runs first, before the GPU is touched: the fp64 oracle on the
first m sequences of the default workload (m sized for about --cpu-budget
seconds), split across host processes (one BLAS thread each), and reports real
tokens per second of the same step.

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
CONFIGS = ("tiny", "graph_transformer", "short_query", "long_document", "mixed_training")
# calls of each standing workload's path, in path order, and those its step runs
OPS = {
    "tiny": ("pack", "fwd", "first_token", "bwd", "first_token_bwd", "unpack"),
    "graph_transformer": ("pack", "fwd", "first_token", "bwd", "first_token_bwd", "unpack"),
    "short_query": ("pack", "fwd", "first_token", "unpack"),
    "long_document": ("pack", "fwd", "first_token"),
    "mixed_training": ("pack", "fwd", "first_token", "bwd", "first_token_bwd"),
}
STEP = {
    "tiny": OPS["tiny"],
    "graph_transformer": OPS["graph_transformer"],
    "short_query": ("pack", "fwd", "unpack"),
    "long_document": ("pack", "fwd"),
    "mixed_training": ("pack", "fwd", "bwd"),
}
WITH_LSE = {"tiny": True, "graph_transformer": True, "short_query": False, "long_document": True,
            "mixed_training": True}


def band_pairs(lengths, window):
    """Query-key pairs a sequence keeps: L^2 (global), or those with |i - j| <= window."""
    import numpy as np
    L = np.asarray(lengths, dtype=np.float64)
    if window is None:
        return float((L * L).sum())
    m = np.minimum(float(window), L - 1)
    return float((L + 2.0 * (m * L - m * (m + 1) / 2.0)).sum())


def algo_work(kernel, w, N, L2, e, with_lse, with_grid=True, window=None):
    """Algorithmic work of one launch: {'flop': count, 'byte': count} (attention kernels
    carry both). L2 is the number of attended (query, key) pairs: sum L^2, or the
    band's for local attention (window not None)."""
    B, S, H, d = w.num_seqs, w.max_seq_len, w.num_heads, w.head_dim
    D = H * d
    T = (N + 127) // 128
    lse_b = 4.0 * N * H if with_lse else 0.0
    # fp32 at d 32/64: with a window the one-wave dQ recomputes S and dP and forms D itself;
    # for global attention it takes the dS blocks the dK/dV pass stored and reads only K
    # (dS is an intermediate of the method, not one of its inputs: not credited)
    wave_dq = e == 4 and d in (32, 64) and window is not None
    ds_dq = e == 4 and d in (32, 64) and window is None
    return {
        # forward: 4 L2 H d flops (QK^T and PV); read Q, K, V, write O (+ LSE)
        "attn_fwd": {"flop": 4.0 * L2 * H * d, "byte": 4.0 * N * D * e + lse_b},
        # backward split by kernel: dK/dV performs S, dP, dV and dK (8 L2 H d) and moves
        # Q, K, V, dO, LSE, D in and dK, dV out; dQ is credited with dQ alone (2 L2 H d),
        # its recomputation of S and dP is not counted
        "bwd_dkdv": {"flop": 8.0 * L2 * H * d, "byte": 6.0 * N * D * e + 8.0 * N * H},
        # (the fp32 one-wave dQ also reads O and writes D, the delta pass it replaces; the fp32
        # dQ from stored dS reads K and writes dQ)
        "bwd_dq": {"flop": 2.0 * L2 * H * d,
                   "byte": 2.0 * N * D * e if ds_dq else (6.0 if wave_dq else 5.0) * N * D * e + 8.0 * N * H},
        # the whole backward in one pass (short sequences): 10 L2 H d; reads Q, K, V, O, dO, LSE,
        # writes dQ, dK, dV
        "bwd_short": {"flop": 10.0 * L2 * H * d, "byte": 8.0 * N * D * e + 4.0 * N * H},
        # first token: read K and V once, the B queries, write B outputs (+ LSE)
        "attn_fwd_first": {"byte": 2.0 * N * D * e + 2.0 * B * D * e + (4.0 * B * H if with_lse else 0.0)},
        # first-token backward: read K, V and the B rows of q, dO, O (+ LSE), write dK, dV and dq_first
        "attn_bwd_first": {"byte": 4.0 * N * D * e + 4.0 * B * D * e + 4.0 * B * H},
        # D = rowsum(dO * O): read dO and O, write D; the 16-bit pass at head dims 32 and 64 also
        # reads the LSE and writes its scaled copy
        "bwd_delta": {"byte": 2.0 * N * D * e + (12.0 if e == 2 and d in (32, 64) else 4.0) * N * H},
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
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this source."""
    from padding_free_packed_amd.profiling import source_hash

    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel):
        return None
    return t.get("bytes_per_launch")


def stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "min_ms": float(a.min()), "mean_ms": float(a.mean()),
            "launches": int(a.size)}


# ---------------------------------------------------------------- CPU baseline (the oracle)

def _host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count(), len(os.sched_getaffinity(0))


def _oracle_step(name, lengths, S, H, d, scale, dtype, ops, seed):
    """Draws a batch of the given lengths (seeded, host) and runs the oracle over the calls
    `ops` of its path; returns (seconds of oracle work, tokens)."""
    import numpy as np

    import oracle
    from padding_free_packed_amd import workloads as W

    rng = np.random.default_rng(seed)
    L = np.asarray(lengths, dtype=np.int64)
    N = int(L.sum())

    def draw(shape):
        return W.to_f64(W.to_bits(rng.standard_normal(shape, dtype=np.float32), dtype), dtype)

    q, k, v = draw((N, H, d)), draw((N, H, d)), draw((N, H, d))
    do = draw((N, H, d)) if ("bwd" in ops) else None
    grid = None
    if "unpack" in ops:  # workloads with a padded grid pack it (NaN padding)
        grid = rng.standard_normal((L.size, S, H * d), dtype=np.float32)
        grid[np.arange(S)[None, :] >= L[:, None]] = np.nan
    t0 = time.perf_counter()
    cu, flat, n = oracle.layout(L, S)
    if grid is not None:
        oracle.pack(grid, flat)
    o, lse = oracle.attention(q, k, v, cu, scale)
    if "first_token" in ops:
        oracle.attention_first_token(q[cu[:-1]], k, v, cu, scale)
    if "bwd" in ops:
        oracle.attention_backward(do, q, k, v, cu, scale)
    if "first_token_bwd" in ops:
        oracle.attention_first_token_backward(do[cu[:-1]], q[cu[:-1]], k, v, cu, scale)
    if grid is not None:
        oracle.unpack(o.reshape(n, -1), cu, S)
    return time.perf_counter() - t0, n


def _cpu_worker(args, barrier, results, idx):
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        barrier.wait()
        t = time.time()
        secs, n = _oracle_step(*args)
        results.put((idx, t, time.time(), secs, n))


def cpu_baseline(name, budget_s, max_procs=16):
    """The fp64 oracle over the step of workload `name` on the first m sequences of its
    batch, m sized for about budget_s seconds of wall time on P host processes (one BLAS
    thread each; sequences dealt to the processes longest first, balanced by sum L^2).
    Runs before the GPU is touched."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    from padding_free_packed_amd import workloads as W

    w = W.standing_lengths(name)
    ops = STEP[name]
    L = w.lengths.astype(np.int64)
    model, ncpu, avail = _host_info()
    P = max(1, min(max_procs, avail))
    cost = L.astype(np.float64) ** 2 + 64.0 * L
    # calibrate on one process: the first sequences, about 1 s of work
    m0 = 1
    while m0 < L.size and cost[:m0].sum() < 2e6:
        m0 += 1
    with threadpool_limits(limits=1):
        t0, _ = _oracle_step(name, L[:m0], w.max_seq_len, w.num_heads, w.head_dim, w.scale, w.dtype, ops, 99)
    per_cost = t0 / cost[:m0].sum()
    target = budget_s * P / max(per_cost, 1e-12)
    m = int(min(L.size, max(m0, np.searchsorted(np.cumsum(cost), target))))
    # longest first, each to the least loaded process
    order = np.argsort(-cost[:m], kind="stable")
    load = np.zeros(P)
    parts = [[] for _ in range(P)]
    for i in order:
        j = int(np.argmin(load))
        parts[j].append(int(i))
        load[j] += cost[i]
    parts = [sorted(p) for p in parts if p]
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(len(parts))
    results = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker,
                         args=((name, L[p], w.max_seq_len, w.num_heads, w.head_dim, w.scale, w.dtype, ops, 1000 + j),
                               barrier, results, j))
             for j, p in enumerate(parts)]
    for p in procs:
        p.start()
    got = [results.get() for _ in procs]
    for p in procs:
        p.join()
    start = min(g[1] for g in got)
    end = max(g[2] for g in got)
    n = sum(g[4] for g in got)
    wall = end - start
    return {"value": n / wall, "unit": "tokens/s", "cores": len(parts), "kind": "oracle",
            "nproc": ncpu, "cpus_available": avail, "cpu_model": model,
            "sample": f"{name}: first {m} of {L.size} sequences ({n} tokens), step {'+'.join(ops)} in float64, "
                      f"{len(parts)} processes x 1 BLAS thread, {wall:.1f} s wall "
                      f"(sum of per-process oracle time {sum(g[3] for g in got):.1f} s)"}


def cpu_baseline_single(w, budget_s, window=None, nemo_mask=None, first_token=True):
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
    model, ncpu, avail = _host_info()
    return {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle", "nproc": ncpu,
            "cpus_available": avail, "cpu_model": model,
            "sample": f"first {m} of {w.num_seqs} sequences ({n} tokens): "
                      + ("flatten of their rows, gather, layout, forward," if nemo_mask is not None else
                         "layout, pack, forward," + (" first-token," if first_token else ""))
                      + (" backward, first-token backward," if w.dout is not None else "")
                      + (" unpack" if w.grid is not None else "") + f" in float64, {t:.1f} s"}


# ---------------------------------------------------------------- GPU side

class Case:
    """Device buffers and the calls of one workload's path."""

    def __init__(self, name, dev, window=None):
        import numpy as np
        import torch

        from padding_free_packed_amd import pe
        from padding_free_packed_amd import workloads as W

        self.name, self.window = name, window
        self.w = w = W.standing_lengths(name)
        self.ops = OPS[name]
        B, S, H, d = w.num_seqs, w.max_seq_len, w.num_heads, w.head_dim
        self.N = N = w.total_tokens
        D = H * d
        self.bf = bf = w.dtype == W.BF16
        self.e = 2 if bf else 4
        self.code = pe.PE_BF16 if bf else pe.PE_FP32
        self.dt = "bf16" if bf else "fp32"
        self.L2 = band_pairs(w.lengths, window)
        self.with_lse = WITH_LSE[name]
        with_grid = "unpack" in self.ops
        with_bwd = "bwd" in self.ops
        x = W.device_inputs(w, dev, seed=1000 + CONFIGS.index(name), grid=with_grid, with_grad=with_bwd)
        self.lengths = torch.from_numpy(w.lengths.astype(np.int32)).to(dev)
        self.q, self.k, self.v = x["q"], x["k"], x["v"]
        self.dout = x.get("dout")
        self.grid = x.get("grid")
        cu_h = np.concatenate([[0], np.cumsum(w.lengths.astype(np.int64))])
        first = torch.from_numpy(cu_h[:-1]).to(dev)
        self.q_first = self.q[first].contiguous()
        self.cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.flat = torch.empty(N, dtype=torch.int64, device=dev)
        self.packed = torch.empty(N, D, dtype=self.q.dtype, device=dev) if with_grid else None
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(H, N, device=dev)
        self.out_first = torch.empty_like(self.q_first)
        self.lse_first = torch.empty(H, B, device=dev)
        self.grid_out = torch.empty_like(self.grid) if with_grid else None
        if with_bwd:
            self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
            self.dout_first = self.dout[first].contiguous()
            self.dq_first = torch.empty_like(self.q_first)
            self.dk_first, self.dv_first = torch.empty_like(self.k), torch.empty_like(self.v)
        self.ws_pack = pe.workspace(pe.pe_pack_workspace_size(B, S, D, self.code), dev)
        # a backward case takes the workspace of the fastest backward path
        self.ws = pe.workspace(pe.pe_attn_bwd_workspace_size(B, N, S, H, d, self.code) if with_bwd
                               else pe.pe_attn_workspace_size(B, N, H, d, self.code, False), dev)
        self.pe = pe
        self.call("pack")  # cu_seqlens for every later call

    def call(self, op):
        pe, w, N = self.pe, self.w, self.N
        B, S, sc, win = w.num_seqs, w.max_seq_len, w.scale, self.window
        lse = self.lse if self.with_lse else None
        if op == "pack":
            n = pe.pe_pack(self.lengths, S, self.grid, self.cu, self.flat, self.packed, N, self.ws_pack, self.code)
            assert n == N
        elif op == "fwd":
            if win is None:
                pe.pe_varlen_attn_fwd(self.q, self.k, self.v, self.cu, B, N, S, sc, self.out, lse, self.ws)
            else:
                pe.pe_varlen_attn_fwd_local(self.q, self.k, self.v, self.cu, B, N, S, sc, win, self.out, lse, self.ws)
        elif op == "first_token":
            pe.pe_varlen_attn_fwd_first_token(self.q_first, self.k, self.v, self.cu, B, N, S, sc, self.out_first,
                                              self.lse_first)
        elif op == "bwd":
            if win is None:
                pe.pe_varlen_attn_bwd(self.dout, self.q, self.k, self.v, self.out, self.lse, self.cu, B, N, S, sc,
                                      self.dq, self.dk, self.dv, self.ws)
            else:
                pe.pe_varlen_attn_bwd_local(self.dout, self.q, self.k, self.v, self.out, self.lse, self.cu, B, N, S,
                                            sc, win, self.dq, self.dk, self.dv, self.ws)
        elif op == "first_token_bwd":
            pe.pe_varlen_attn_bwd_first_token(self.dout_first, self.q_first, self.k, self.v, self.out_first,
                                              self.lse_first, self.cu, B, N, S, sc, self.dq_first, self.dk_first,
                                              self.dv_first)
        elif op == "unpack":
            pe.pe_unpack(self.out.view(N, -1), self.cu, B, S, N, self.grid_out)
        else:
            raise ValueError(op)

    def kernel_rate(self, kernel, ms):
        aw = algo_work(kernel, self.w, self.N, self.L2, self.e, self.with_lse, self.grid is not None, self.window)
        if aw is None or ms <= 0:
            return {}
        return rate(aw, ms, self.dt)


class Flush:
    """A 1 GiB buffer read (summed) before each timed launch: nothing the launch reads is
    then still in the 256 MB last-level cache or the L2s. Reading only leaves clean lines,
    so the timed launch pays no write-back of the flush itself."""

    def __init__(self, dev, mib=1024):
        import torch
        self.buf = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev) if mib > 0 else None

    def __call__(self):
        if self.buf is not None:
            self.buf.sum()


def timed(fn, iters, flush, kernels):
    """Runs fn `iters` times, each after a flush, bracketed by events on the current stream.
    Returns (per-iteration ms, {kernel: [launch ms]}) with the library's per-kernel events
    on when `kernels`, else off."""
    import torch

    pe = sys.modules["padding_free_packed_amd.pe"]
    if kernels:
        pe.pe_timing_enable(True)
        pe.pe_timing_read()
    evs = []
    for _ in range(iters):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    per = {}
    if kernels:
        for name, t in pe.pe_timing_read():
            per.setdefault(name, []).append(t)
        pe.pe_timing_enable(False)
    return ms, per


def measure_case(case, iters, flush):
    """Per-call timing of one workload: each call alone, warm, with a flush before each launch."""
    import torch

    entry = {"num_seqs": case.w.num_seqs, "total_tokens": case.N, "sum_L2": case.L2, "max_seq_len": case.w.max_seq_len,
             "num_heads": case.w.num_heads, "head_dim": case.w.head_dim, "dtype": case.dt, "lse": case.with_lse,
             "grid": case.grid is not None, "ops": {}}
    for op in case.ops:
        for _ in range(2):
            case.call(op)
        torch.cuda.synchronize()
        ms, per = timed(lambda: case.call(op), iters, flush, True)
        ent = stats(ms)
        ent["tokens_per_s"] = case.N / (ent["median_ms"] * 1e-3)
        if op == "fwd":
            ent["tflops"] = 4.0 * case.L2 * case.w.num_heads * case.w.head_dim / (ent["median_ms"] * 1e-3) / 1e12
        ks = {}
        for name, lst in per.items():
            k = stats(lst)
            k["launches"] = len(lst) // iters
            k.update(case.kernel_rate(name, k["median_ms"]))
            ks[name] = k
        ent["kernels"] = ks
        entry["ops"][op] = ent
    return entry


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
        result["cpu_baseline"] = cpu_baseline_single(w, args.cpu_budget, first_token=False)
    bucket.close()
    print(json.dumps(result))


def nemo_bench(args):
    """The mixed-training documents packed NeMo-style into rows of 8192 tokens: one step
    flattens the indexed document mask (pe_flatten_document_mask, its host read included),
    gathers Q, K and V from the padded row grids, runs the forward with the log-sum-exp and
    scatters the output back to the row grid."""
    import numpy as np
    import torch

    from padding_free_packed_amd import pe
    from padding_free_packed_amd import workloads as W

    w = W.mixed_training()
    nemo_mask, nemo_grids = W.nemo_rows(w, w.max_seq_len)
    w.dout = None
    w.extra["rows"] = nemo_mask.shape[0]
    w.extra["grid_rows"] = nemo_mask.size
    cpu = None if args.no_cpu_baseline else cpu_baseline_single(w, args.cpu_budget, nemo_mask=nemo_mask)
    dev = "cuda:0"
    B, S, H, d = w.num_seqs, w.max_seq_len, w.num_heads, w.head_dim
    N, e = w.total_tokens, 2
    L2 = band_pairs(w.lengths, None)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = (torch.empty(N, H, d, dtype=torch.bfloat16, device=dev) for _ in range(3))
    out = torch.empty_like(q)
    lse = torch.empty(H, N, device=dev)
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    flat = torch.empty(N, dtype=torch.int64, device=dev)
    ws = pe.workspace(pe.pe_attn_workspace_size(B, N, H, d, pe.PE_BF16, False), dev)
    mask_d = torch.from_numpy(nemo_mask).to(dev)
    ws_flat = pe.workspace(pe.pe_flatten_workspace_size(nemo_mask.shape[0]), dev)
    grids_d = [up(nemo_grids[nm]) for nm in ("q", "k", "v")]
    del nemo_grids
    grid_rows_out = torch.empty_like(grids_d[0])
    flush = Flush(dev, args.flush_mib)

    def step():
        n, docs = pe.pe_flatten_document_mask(mask_d, flat, cu, ws_flat)
        assert (n, docs) == (N, B)
        for src, dst in zip(grids_d, (q, k, v)):
            pe.pe_gather_rows(src, flat, dst)
        pe.pe_varlen_attn_fwd(q, k, v, cu, B, N, S, w.scale, out, lse, ws)
        pe.pe_scatter_rows(out, flat, grid_rows_out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms, _ = timed(step, args.steps, flush, False)
    wall = time.perf_counter() - wall0
    _, per = timed(step, args.steps, flush, True)
    breakdown = {}
    for name, lst in per.items():
        ent = stats(lst)
        ent["launches_per_step"] = len(lst) / args.steps
        ent["ms_per_step"] = ent["mean_ms"] * ent["launches_per_step"]
        aw = algo_work(name, w, N, L2, e, True, False)
        if aw is not None:
            ent.update(rate(aw, ent["mean_ms"], "bf16"))
        breakdown[name] = ent
    work = algo_work("attn_fwd", w, N, L2, e, True, False)
    roof = rate(work, breakdown["attn_fwd"]["mean_ms"], "bf16")
    roof.update({"traffic": None, "kernel": "attn_fwd", "algorithmic_per_launch": work["flop"],
                 "avg_launch_ms": breakdown["attn_fwd"]["mean_ms"]})
    ms_step = float(np.mean(ms))
    result = {
        "metric": METRIC, "value": N / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "ms_per_step_median": float(np.median(ms)),
        "ms_per_step_min": float(np.min(ms)), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "nemo_packed", "num_seqs": B, "max_seq_len": S, "total_tokens": N, "num_heads": H,
                   "head_dim": d, "rows": [int(w.extra["rows"]), int(S)],
                   "step": "flatten(mask)+gather(q,k,v)+fwd(lse)+scatter"},
        "roofline": roof, "breakdown": breakdown, "wall_s_timed_region": wall,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_document", choices=list(CONFIGS) + ["nemo_packed", "short_batch"])
    ap.add_argument("--num-seqs", type=int, default=64,
                    help="short_batch only: sequences in the batch (and slots of its captured bucket)")
    ap.add_argument("--window", type=int, default=None,
                    help="local attention: each query sees the keys within this distance in its sequence "
                         "(pe_varlen_attn_fwd_local / _bwd_local); default global attention")
    ap.add_argument("--configs", default="all",
                    help="standing workloads measured per call into `configs` (comma list, 'all' or 'none')")
    ap.add_argument("--config-iters", type=int, default=10)
    ap.add_argument("--flush-mib", type=int, default=1024)
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
    if args.workload == "nemo_packed":
        return nemo_bench(args)

    # the oracle first: no GPU state exists yet when its processes start
    cpu = None
    if not args.no_cpu_baseline and args.window is None:
        cpu = cpu_baseline(args.workload, args.cpu_budget)

    import numpy as np
    import torch

    from padding_free_packed_amd import pe  # noqa: F401  (fails loudly without the library)

    dev = "cuda:0"
    flush = Flush(dev, args.flush_mib)
    case = Case(args.workload, dev, args.window)
    step_ops = STEP[args.workload]

    def step():
        for op in step_ops:
            case.call(op)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms, _ = timed(step, args.steps, flush, False)
    wall = time.perf_counter() - wall0
    # the same steps again with the per-kernel events on
    ms_k, per = timed(step, args.steps, flush, True)

    w = case.w
    N = case.N
    breakdown = {}
    for name, lst in per.items():
        ent = stats(lst)
        ent["launches_per_step"] = len(lst) / args.steps
        ent["ms_per_step"] = ent["mean_ms"] * ent["launches_per_step"]
        ent.update(case.kernel_rate(name, ent["mean_ms"]))
        breakdown[name] = ent
    dom = "attn_fwd" if "attn_fwd" in breakdown else max(breakdown, key=lambda k_: breakdown[k_]["ms_per_step"])
    work = algo_work(dom, w, N, case.L2, case.e, case.with_lse, case.grid is not None, case.window)
    roof = rate(work, breakdown[dom]["mean_ms"], case.dt)
    roof["traffic"] = load_traffic(dom, args.workload if args.window is None else f"{args.workload}_w{args.window}")
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = work["flop"] if roof["bound"] == "mfma" else work["byte"]
    roof["avg_launch_ms"] = breakdown[dom]["mean_ms"]
    ms_step = float(np.mean(ms))
    fwd_ms = breakdown["attn_fwd"]["mean_ms"]
    result = {
        "metric": METRIC,
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": float(np.median(ms)),
        "ms_per_step_min": float(np.min(ms)),
        "ms_per_step_with_kernel_events": float(np.mean(ms_k)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dt,
        "data": "synthetic",
        "config": {
            "workload": args.workload, "num_seqs": w.num_seqs, "max_seq_len": w.max_seq_len, "total_tokens": N,
            "sum_L2": case.L2, "num_heads": w.num_heads, "head_dim": w.head_dim,
            "grid": [w.num_seqs, w.max_seq_len, w.num_heads * w.head_dim] if case.grid is not None else None,
            "window": args.window, "lse": case.with_lse,
            "step": "+".join(("pack(layout only)" if op == "pack" and case.grid is None else op) for op in step_ops),
            "flush_mib_between_steps": args.flush_mib,
        },
        "fwd": {"ms": fwd_ms, "tokens_per_s": N / (fwd_ms * 1e-3),
                "tflops": 4.0 * case.L2 * w.num_heads * w.head_dim / (fwd_ms * 1e-3) / 1e12},
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
    names = CONFIGS if args.configs == "all" else (() if args.configs == "none" else args.configs.split(","))
    if names and args.window is None:
        cfg = {}
        for nm in names:
            c = case if nm == args.workload else Case(nm, dev)
            cfg[nm] = measure_case(c, args.config_iters, flush)
            if c is not case:
                del c
                torch.cuda.empty_cache()
        result["configs"] = cfg
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()
