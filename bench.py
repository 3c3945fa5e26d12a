"""Benchmark of one tensor-parallel rank's hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs:
  1. tp_mlp_fwd_bwd: one TP=8 rank's share of a Llama-3-70B-shaped GELU MLP,
     forward + backward (T=8192, d=8192, f=3584, bf16 in, fp32 accumulate),
     six MFMA GEMMs with the GELU / GELU' epilogues fused;
  2. sharded_matmul_fwd_bwd: the same rank's inner-axis GEMM shard,
     forward + backward (M=8192, K_r=1024, N=8192, bf16);
  3. vocab_parallel_ce_fwd_bwd: 4096 positions x vocab 128256 split into 8
     shards, bf16 logits, mean loss and dlogits.
Inputs are resident in HBM before timing starts.  ``value`` is the MLP's
fwd+bwd TFLOP/s (12*T*d*f algorithmic FLOP per call); the CE's algorithmic
GB/s (2 bytes read + 2 bytes written per logit) and the inner GEMM's TFLOP/s
are reported beside it.  Each call is timed with HIP events on the stream the
library launches on.  After the timed steps, torch's copy_ of the logits (the
CE's bytes, read once and written once) is timed as the copy-rate context of
the CE figure (``roofline_ce.copy_same_bytes_gbs``), and the MLP's six
products through torch.mm (hipBLASLt) as library context
(``mlp_gemms_via_torch_mm``).  The cross-rank partial sum is timed on its own
through tprank_partial_sum (``roofline_reduce``: 8 fp32 partials of the
inner split's 8192 x 8192 Y, (8 + 1) * 4 bytes per output element).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-runs N] [--blas-runs N]
                       [--copy-bytes N]
       python bench.py --traffic-from FETCH_CSV WRITE_CSV COPY_BYTES
The second form turns two rocprofv3 counter runs of the first form (one with
--pmc FETCH_SIZE, one with --pmc WRITE_SIZE, both with --copy-bytes) into
profiles/traffic.json; it needs no GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "TP-rank MLP fwd+bwd TFLOP/s (% bf16 MFMA peak); vocab-CE HBM GB/s"

MLP = dict(T=8192, d=8192, f=3584)
INNER = dict(M=8192, K=1024, N=8192)
CE = dict(T=4096, V=128256, parts=8)
HEAD = dict(T=4096, d=4096, V=128256, parts=8)
MLP_8B = dict(T=4096, d=4096, f=1792)
ATTN = dict(T=8192, d=8192, n_q_heads=8, n_kv_heads=1, head_dim=128)
GATED = dict(T=8192, d=8192, f=3584, act="silu")
CE_OPTS = dict(T=4096, V=128256, v_valid=128000, parts=8, label_smoothing=0.1, ignore_frac=0.125)
REDUCE = dict(slots=8, M=8192, N=8192)


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "megatron_mlp_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def stored_traffic(kernel, path=TRAFFIC_JSON):
    """HBM bytes per launch measured with rocprofv3 counters for the current
    kernel sources, or None when the sources changed since."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    v = t.get(kernel)
    return None if v is None else float(v)


GEMM_KERNEL = "gemm_bf16_dma_kernel"
CE_KERNEL = "ce_pair_kernel"
REDUCE_KERNEL = "reduce_vec4_kernel"
COPY_KERNEL = "neg_kernel"
# Kernel-name patterns for the counter rows: every launch of the GEMM kernel,
# and the CE kernel's plain instance (the one the bench's CE call runs; the
# per-shard-statistics instance ce_pair_kernel<3> is another workload).
TRAFFIC_MATCH = {GEMM_KERNEL: GEMM_KERNEL, CE_KERNEL: CE_KERNEL + "<0>", REDUCE_KERNEL: REDUCE_KERNEL + "<8>"}


def traffic_from(fetch_csv, write_csv, copy_bytes, out_path=TRAFFIC_JSON):
    """HBM bytes per launch from rocprofv3 counter_collection CSVs.

    FETCH_SIZE / WRITE_SIZE are reported in KiB per dispatch; each is scaled
    by copy_bytes / (what the same counter reads for the plain copy kernel of
    copy_bytes read + copy_bytes written), so the figures are in true bytes.
    """
    import csv

    def per_dispatch(path, counter):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    key = int(r["Dispatch_Id"])
                    rows[key] = (r["Kernel_Name"], rows.get(key, ("", 0.0))[1] + float(r["Counter_Value"]))
        return [rows[k] for k in sorted(rows)]

    out = {"kernel_source_digest": kernel_source_digest(), "copy_bytes": copy_bytes}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = per_dispatch(path, counter)
        copy = [v for n, v in rows if COPY_KERNEL in n]
        if len(copy) != 1:
            raise SystemExit(f"{path}: expected one {COPY_KERNEL} dispatch, found {len(copy)}")
        scale = copy_bytes / (copy[0] * 1024.0)
        out[counter] = {"copy_kib": copy[0], "scale": scale}
        for kernel in (GEMM_KERNEL, CE_KERNEL, REDUCE_KERNEL):
            vals = [v * 1024.0 * scale for n, v in rows if TRAFFIC_MATCH[kernel] in n]
            out[counter][kernel] = {"launches": len(vals), "avg_bytes": sum(vals) / max(len(vals), 1)}
    for kernel in (GEMM_KERNEL, CE_KERNEL, REDUCE_KERNEL):
        if out["FETCH_SIZE"][kernel]["launches"] == 0:
            continue
        out[kernel + "_bytes_per_launch"] = (out["FETCH_SIZE"][kernel]["avg_bytes"] +
                                             out["WRITE_SIZE"][kernel]["avg_bytes"])
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return out


def cpu_baseline(budget_s=10.0, max_reps=4):
    """Time the fp64 oracle on the full 70B-rank MLP workload (all T tokens at
    the same d and f), repeated until about budget_s seconds have passed."""
    import numpy as np
    import threadpoolctl

    import oracle
    import workloads

    T, d, f = MLP["T"], MLP["d"], MLP["f"]
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=11, device="cpu")
    xs = [t.float().numpy().astype(np.float64) for t in (x, w1, w2, gy)]
    times = []
    while len(times) < max_reps and sum(times) < budget_s:
        t0 = time.perf_counter()
        oracle.mlp_fwd_bwd(*xs, "math")
        times.append(time.perf_counter() - t0)
    dt = sum(times) / len(times)
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    return {"value": 12.0 * T * d * f / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle.mlp_fwd_bwd (NumPy fp64) on the full T={T}, d={d}, f={f} MLP, "
                      f"{len(times)} runs of {dt:.2f} s on average, {os.cpu_count()} host CPUs visible"}


def bench_head(tpr, workloads, dev, steps):
    """The vocabulary-parallel output head + CE (Llama-3-8B hidden size and
    vocabulary, 8 shards, bf16), timed on its own after the step: three GEMMs
    of 2*T*d*V FLOP each plus the CE and the dh reduction per call."""
    import torch

    T, d, V, P = HEAD["T"], HEAD["d"], HEAD["V"], HEAD["parts"]
    h, w, y = workloads.vocab_head(T, d, V, seed=5, device=dev, w_std=2.0 / d ** 0.5)
    out = (torch.empty((), device=dev), torch.empty(T, d, device=dev), torch.empty(d, V, device=dev))
    ws = torch.empty(tpr.vocab_parallel_head_ce_workspace_bytes(P, torch.bfloat16, T, d, V), dtype=torch.uint8,
                     device=dev)
    tpr.vocab_parallel_head_ce_fwd_bwd(P, h, w, y, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        tpr.vocab_parallel_head_ce_fwd_bwd(P, h, w, y, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = 6.0 * T * d * V
    tflops = flop / (ms * 1e-3) / 1e12
    return {"config": dict(HEAD, dtype="bf16", w_layout="math"), "steps": steps, "ms": round(ms, 3),
            "tflops": round(tflops, 1), "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
            "flop_per_call": flop}


def bench_mlp_8b(tpr, workloads, dev, steps):
    """The Llama-3-8B tensor-parallel-8 rank MLP fwd+bwd (T=4096, d=4096,
    f=1792, bf16), timed on its own after the step and reported beside it."""
    import torch

    T, d, f = MLP_8B["T"], MLP_8B["d"], MLP_8B["f"]
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=3, device=dev)
    out = (torch.empty(T, d, device=dev), torch.empty(T, d, device=dev),
           torch.empty(d, f, device=dev), torch.empty(f, d, device=dev))
    ws = torch.empty(tpr.tp_mlp_workspace_bytes(1, torch.bfloat16, T, d, f), dtype=torch.uint8, device=dev)
    for _ in range(2):
        tpr.tp_mlp_fwd_bwd(1, x, w1, w2, gy, "math", out=out, workspace=ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        tpr.tp_mlp_fwd_bwd(1, x, w1, w2, gy, "math", out=out, workspace=ws)
        e[1].record()
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    flop = 12.0 * T * d * f
    mean = sum(ms) / len(ms)
    tflops = flop / (mean * 1e-3) / 1e12
    return {"config": dict(MLP_8B, dtype="bf16", w_layout="math"), "steps": steps, "ms": round(mean, 4),
            "ms_median": round(ms[len(ms) // 2], 4), "ms_min": round(ms[0], 4), "tflops": round(tflops, 1),
            "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2), "flop_per_call": flop}


def bench_gated_mlp(tpr, dev, steps):
    """The gated SiLU MLP (gate / up / down) of a Llama-3-70B rank at TP = 8
    (T=8192, d=8192, f=3584, bf16): nine GEMMs of 2*T*d*f FLOP per call."""
    import torch

    T, d, f = GATED["T"], GATED["d"], GATED["f"]
    g = torch.Generator(device=dev)
    g.manual_seed(12)
    mk = lambda shape, std: (torch.randn(shape, generator=g, device=dev) * std).bfloat16()
    x, gy = mk((T, d), 1.0), mk((T, d), 1.0)
    w1, w3, w2 = mk((d, f), 0.02), mk((d, f), 0.02), mk((f, d), 0.02)
    out = (torch.empty(T, d, device=dev), torch.empty(T, d, device=dev), torch.empty(d, f, device=dev),
           torch.empty(f, d, device=dev), torch.empty(d, f, device=dev))
    ws = torch.empty(tpr.tp_mlp_act_workspace_bytes(1, torch.bfloat16, True, T, d, f), dtype=torch.uint8,
                     device=dev)
    call = lambda: tpr.tp_mlp_act_fwd_bwd(1, x, w1, w2, gy, act=GATED["act"], w3=w3, out=out, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    flop = 18.0 * T * d * f
    mean = sum(ms) / len(ms)
    tflops = flop / (mean * 1e-3) / 1e12
    return {"config": dict(GATED, dtype="bf16", w_layout="math", gated=True), "steps": steps, "ms": round(mean, 4),
            "ms_min": round(ms[0], 4), "tflops": round(tflops, 1),
            "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2), "flop_per_call": flop}


def _time_calls(call, runs, warmup=5):
    """Median and minimum (µs) of `runs` calls, each bracketed by HIP events
    on the current stream, after `warmup` untimed calls."""
    import torch

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(runs)]
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    us = sorted(1e3 * e[0].elapsed_time(e[1]) for e in ev)
    return {"median_us": round(us[len(us) // 2], 2), "min_us": round(us[0], 2), "runs": runs}


def bench_small_configs(tpr, workloads, dev, runs):
    """Latency of the fp32 walk-through configurations (launch-bound: reported
    in µs, no roofline): the 3x5x4 sharded GEMM on each axis at 2 and 7
    parts, and the tp=4 MLP of (2, 8, 64) tokens with f=256 in the torch
    layout; plus the vocab CE of the step timed over `runs` calls."""
    out = {}
    a, b, g = workloads.sharded_gemm_tiny(seed=0, device=dev)
    for axis in ("rows", "columns", "inner"):
        for parts in (2, 7):
            out[f"sharded_gemm_m3k5n4_{axis}_p{parts}"] = _time_calls(
                lambda: tpr.sharded_matmul_fwd_bwd(axis, parts, a, b, g), runs)
    x, w1, w2, gy = workloads.tp_mlp_tiny(seed=0, device=dev)
    out["tp_mlp_tp4_x2x8x64_f256_fp32"] = _time_calls(lambda: tpr.tp_mlp_fwd_bwd(4, x, w1, w2, gy, "torch"), runs)
    logits, labels = workloads.vocab_ce(T=CE["T"], V=CE["V"], seed=2, device=dev)
    import torch
    ce_out = (torch.empty((), device=dev), torch.empty_like(logits), None)
    ws = torch.empty(tpr.vocab_parallel_ce_workspace_bytes(CE["parts"], CE["T"], CE["V"]), dtype=torch.uint8,
                     device=dev)
    r = _time_calls(lambda: tpr.vocab_parallel_ce_fwd_bwd(CE["parts"], logits, labels, out=ce_out, workspace=ws), runs)
    r["gbs_at_median"] = round(4.0 * CE["T"] * CE["V"] / (r["median_us"] * 1e-6) / 1e9, 1)
    out["vocab_ce_t4096_v128256_p8"] = r
    return out


def bench_attn_proj(tpr, dev, steps):
    """The attention-block projections of a Llama-3-70B rank at TP = 8 (8
    query heads and 1 KV head of 128, d = 8192, T = 8192 tokens, bf16): the
    fused QKV projection and the output projection, forward and backward,
    one grouped launch of six GEMMs (6*T*d*(nqkv + nq) FLOP)."""
    import torch

    a = ATTN
    T, d, dh = a["T"], a["d"], a["head_dim"]
    nq, nkv = a["n_q_heads"] * dh, a["n_kv_heads"] * dh
    nqkv = nq + 2 * nkv
    g = torch.Generator(device=dev)
    g.manual_seed(13)
    mk = lambda shape, std: (torch.randn(shape, generator=g, device=dev) * std).bfloat16()
    x, gy, ctx, dqkv = mk((T, d), 1.0), mk((T, d), 1.0), mk((T, nq), 1.0), mk((T, nqkv), 1.0)
    w_qkv, w_o = mk((d, nqkv), 0.02), mk((nq, d), 0.02)
    out = (torch.empty(T, nqkv, dtype=torch.bfloat16, device=dev), torch.empty(T, d, device=dev),
           torch.empty(T, nq, dtype=torch.bfloat16, device=dev), torch.empty(T, d, device=dev),
           torch.empty(d, nqkv, device=dev), torch.empty(nq, d, device=dev))
    call = lambda: tpr.tp_attn_proj_fwd_bwd(1, x, w_qkv, w_o, ctx, gy, dqkv, a["n_q_heads"], a["n_kv_heads"], dh,
                                            out=out)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    flop = 6.0 * T * d * (nqkv + nq)
    mean = sum(ms) / len(ms)
    tflops = flop / (mean * 1e-3) / 1e12
    return {"config": dict(a, dtype="bf16", w_layout="math", tp_simulated=1), "steps": steps, "ms": round(mean, 4),
            "ms_min": round(ms[0], 4), "tflops": round(tflops, 1),
            "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2), "flop_per_call": flop}


def bench_ce_stats(tpr, workloads, dev, steps):
    """The vocabulary-parallel CE of the main step with the per-shard
    statistics (m_r, s_r, t_r for every row and shard, the simulated ranks'
    partial results) also written out.  Algorithmic bytes: the CE's 2 read +
    2 written per logit, plus 12 per row and shard."""
    import torch

    logits, labels = workloads.vocab_ce(T=CE["T"], V=CE["V"], seed=2, device=dev)
    out = (torch.empty((), device=dev), torch.empty_like(logits),
           torch.empty(CE["T"], CE["parts"], 3, device=dev))
    ws = torch.empty(tpr.vocab_parallel_ce_workspace_bytes(CE["parts"], CE["T"], CE["V"]), dtype=torch.uint8,
                     device=dev)
    call = lambda: tpr.vocab_parallel_ce_fwd_bwd(CE["parts"], logits, labels, shard_stats=True, out=out,
                                                 workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    nbytes = 4.0 * CE["T"] * CE["V"] + 12.0 * CE["T"] * CE["parts"]
    mean = sum(ms) / len(ms)
    gbs = nbytes / (mean * 1e-3) / 1e9
    return {"config": dict(CE, dtype="bf16", shard_stats=True), "steps": steps, "ms": round(mean, 4),
            "ms_min": round(ms[0], 4), "gbs": round(gbs, 1), "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
            "bytes_per_call": nbytes}


def bench_ce_opts(tpr, workloads, dev, steps):
    """The cross-entropy with options: a 128000-entry vocabulary padded to
    128256 columns, 8 shards, label smoothing 0.1, about one position in
    eight ignored.  Algorithmic bytes: 2 per vocabulary logit of a counted
    row read, 2 per column of every row written."""
    import torch

    c = CE_OPTS
    logits, labels = workloads.vocab_ce_opts(c["T"], c["V"], c["v_valid"], seed=6, device=dev,
                                             ignore_frac=c["ignore_frac"])
    out = (torch.empty((), device=dev), torch.empty_like(logits), None)
    ws = torch.empty(tpr.vocab_parallel_ce_opts_workspace_bytes(c["parts"], c["T"], c["V"]), dtype=torch.uint8,
                     device=dev)
    call = lambda: tpr.vocab_parallel_ce_opts_fwd_bwd(c["parts"], logits, labels, v_valid=c["v_valid"],
                                                      ignore_index=-100, label_smoothing=c["label_smoothing"],
                                                      out=out, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    n = int((labels != -100).sum().item())
    nbytes = 2.0 * n * c["v_valid"] + 2.0 * c["T"] * c["V"]
    mean = sum(ms) / len(ms)
    gbs = nbytes / (mean * 1e-3) / 1e9
    return {"config": dict(c, dtype="bf16", counted_rows=n), "steps": steps, "ms": round(mean, 4),
            "ms_min": round(ms[0], 4), "gbs": round(gbs, 1), "pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
            "bytes_per_call": nbytes}


def bench_reduce(tpr, dev, steps):
    """The cross-rank partial sum on its own (tprank_partial_sum): the
    70B rank's inner-axis split over 8 ranks leaves 8 fp32 partials of
    Y (8192 x 8192) to be summed.  Algorithmic bytes: (8 + 1) * 4 per output
    element (each partial read once, the sum written once)."""
    import torch

    P, n = REDUCE["slots"], REDUCE["M"] * REDUCE["N"]
    g = torch.Generator(device=dev)
    g.manual_seed(14)
    parts = torch.randn(P, n, generator=g, device=dev)
    out = torch.empty(n, device=dev)
    for _ in range(2):
        tpr.partial_sum(parts, out=out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        tpr.partial_sum(parts, out=out)
        e[1].record()
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    nbytes = (P + 1) * 4.0 * n
    mean = sum(ms) / len(ms)
    gbs = nbytes / (mean * 1e-3) / 1e9
    del parts, out
    torch.cuda.empty_cache()
    return {"kernel": f"reduce_vec4_kernel<{P}> (one launch per call)", "bound": "hbm",
            "workload": f"{P} fp32 partials of the inner-split Y, {REDUCE['M']} x {REDUCE['N']}",
            "steps": steps, "bytes_per_launch": nbytes, "avg_launch_us": round(mean * 1e3, 2),
            "min_launch_us": round(ms[0] * 1e3, 2), "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": stored_traffic(REDUCE_KERNEL + "_bytes_per_launch")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--head-steps", type=int, default=3,
                    help="timed calls of the vocabulary-parallel output head + CE (reported beside the step; 0 = skip)")
    ap.add_argument("--mlp-8b-steps", type=int, default=10,
                    help="timed calls of the 8B-rank MLP fwd+bwd (reported beside the step; 0 = skip)")
    ap.add_argument("--ce-stats-steps", type=int, default=10,
                    help="timed calls of the CE with per-shard statistics written out (0 skips)")
    ap.add_argument("--ce-opts-steps", type=int, default=10,
                    help="timed calls of the cross-entropy with options (reported beside the step; 0 = skip)")
    ap.add_argument("--gated-steps", type=int, default=5,
                    help="timed calls of the gated SiLU MLP at the 70B rank size (reported beside the step; 0 = skip)")
    ap.add_argument("--attn-steps", type=int, default=10,
                    help="timed calls of the 70B-rank attention projections (reported beside the step; 0 = skip)")
    ap.add_argument("--reduce-steps", type=int, default=20,
                    help="timed calls of the cross-rank partial sum (8 x 8192 x 8192 fp32; 0 = skip)")
    ap.add_argument("--small-runs", type=int, default=100,
                    help="timed calls per small (latency-bound) configuration and of the CE (0 = skip)")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_BYTES"))
    ap.add_argument("--blas-runs", type=int, default=5,
                    help="time the MLP's six products through torch.mm this many times (median) as library "
                         "context; 0 skips")
    ap.add_argument("--copy-runs", type=int, default=20,
                    help="time this many torch copy_ calls of the CE's logits (median) as the copy-rate context "
                         "of the CE figure; 0 skips")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run one plain copy kernel (torch.neg on fp32) of this many bytes before timing, "
                         "so that profiler byte counters can be calibrated against a known size")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], int(args.traffic_from[2]))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every simulated tensor-parallel rank runs on that device. "
              "Runs on more than one GPU are not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    import megatron_mlp_fwd_amd as tpr
    import workloads

    tpr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x, w1, w2, gy = workloads.rank_mlp(MLP["T"], MLP["d"], MLP["f"], seed=0, device=dev)
    a, b, g = workloads.inner_gemm(INNER["M"], INNER["K"], INNER["N"], seed=1, device=dev)
    logits, labels = workloads.vocab_ce(T=CE["T"], V=CE["V"], seed=2, device=dev)
    T, d, f = MLP["T"], MLP["d"], MLP["f"]
    mlp_out = (torch.empty(T, d, device=dev), torch.empty(T, d, device=dev),
               torch.empty(d, f, device=dev), torch.empty(f, d, device=dev))
    mlp_ws = torch.empty(tpr.tp_mlp_workspace_bytes(1, torch.bfloat16, T, d, f), dtype=torch.uint8, device=dev)
    M, K, N = INNER["M"], INNER["K"], INNER["N"]
    inner_out = (torch.empty(M, N, device=dev), torch.empty(M, K, device=dev), torch.empty(K, N, device=dev))
    ce_out = (torch.empty((), device=dev), torch.empty_like(logits), None)
    ce_ws = torch.empty(tpr.vocab_parallel_ce_workspace_bytes(CE["parts"], CE["T"], CE["V"]), dtype=torch.uint8,
                        device=dev)

    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes // 4, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step(ev):
        ev[0].record()
        tpr.tp_mlp_fwd_bwd(1, x, w1, w2, gy, "math", out=mlp_out, workspace=mlp_ws)
        ev[1].record()
        tpr.sharded_matmul_fwd_bwd("inner", 1, a, b, g, out=inner_out)
        ev[2].record()
        tpr.vocab_parallel_ce_fwd_bwd(CE["parts"], logits, labels, out=ce_out, workspace=ce_ws)
        ev[3].record()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(max(args.steps, args.warmup))]
    for i in range(args.warmup):
        step(events[i])
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        step(events[i])
    t_end.record()
    torch.cuda.synchronize()

    total_ms = t_start.elapsed_time(t_end)
    mlp_ms = [e[0].elapsed_time(e[1]) for e in events[:args.steps]]
    inner_ms = [e[1].elapsed_time(e[2]) for e in events[:args.steps]]
    ce_ms = [e[2].elapsed_time(e[3]) for e in events[:args.steps]]
    avg = lambda v: sum(v) / len(v)

    mlp_flop = 12.0 * T * d * f
    inner_flop = 6.0 * M * K * N
    ce_bytes = 4.0 * CE["T"] * CE["V"]
    mlp_tflops = mlp_flop / (avg(mlp_ms) * 1e-3) / 1e12
    inner_tflops = inner_flop / (avg(inner_ms) * 1e-3) / 1e12
    ce_gbs = ce_bytes / (avg(ce_ms) * 1e-3) / 1e9

    # Dominant kernel: the bf16 MFMA GEMM.  Per step it is launched four times
    # and nothing else runs in those two calls: the tp=1 MLP call makes three
    # grouped launches ({fc1}, {fc2, dW2, dH}, {dW1, dx}) and the inner-axis
    # call one ({Y, dA, dB}).  Average FLOP per launch / average launch time.
    gemm_launches = 4
    gemm_launch_ms = (avg(mlp_ms) + avg(inner_ms)) / gemm_launches
    gemm_flop_per_launch = (mlp_flop + inner_flop) / gemm_launches
    gemm_achieved = gemm_flop_per_launch / (gemm_launch_ms * 1e-3) / 1e12
    gemm_traffic = stored_traffic(GEMM_KERNEL + "_bytes_per_launch")
    ce_traffic = stored_traffic(CE_KERNEL + "_bytes_per_launch")

    # Context for the CE's HBM figure: a plain copy of the same bytes (torch's
    # copy_ of the logits into the dlogits buffer), timed after the step loop
    # on the same device.  The CE cannot beat what the HBM gives a copy.
    copy_gbs = None
    if args.copy_runs > 0:
        src, dst = logits, ce_out[1]
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        cms = []
        for _ in range(args.copy_runs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            e1.synchronize()
            cms.append(e0.elapsed_time(e1))
        copy_gbs = ce_bytes / (sorted(cms)[len(cms) // 2] * 1e-3) / 1e9

    # Context for the GEMM figure: the MLP's six products through torch.mm
    # (hipBLASLt, bf16 results, so less output traffic than the fp32 results
    # of the library's call) at the same shapes and layouts, on the same
    # device after the timed steps.  A library measurement, not the product.
    blas = None
    if args.blas_runs > 0:
        Hb = torch.randn(T, f, device=dev).bfloat16()
        def blas_call():
            torch.mm(x, w1)                # P = x W1
            torch.mm(Hb, w2)               # y = H W2
            torch.mm(Hb.t(), gy)           # dW2 = H^T G
            torch.mm(gy, w2.t())           # dH = G W2^T
            torch.mm(x.t(), Hb)            # dW1 = x^T dZ
            torch.mm(Hb, w1.t())           # dx = dZ W1^T
        for _ in range(2):
            blas_call()
        torch.cuda.synchronize()
        bms = []
        for _ in range(args.blas_runs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            blas_call()
            e1.record()
            e1.synchronize()
            bms.append(e0.elapsed_time(e1))
        bmed = sorted(bms)[len(bms) // 2]
        blas = {"op": "torch.mm x 6 (hipBLASLt), bf16 results, the MLP's shapes and layouts",
                "ms_median": round(bmed, 4), "tflops": round(mlp_flop / (bmed * 1e-3) / 1e12, 2)}
        del Hb

    head = None
    if args.head_steps > 0:
        head = bench_head(tpr, workloads, dev, args.head_steps)
    mlp_8b = None
    if args.mlp_8b_steps > 0:
        mlp_8b = bench_mlp_8b(tpr, workloads, dev, args.mlp_8b_steps)
    small = None
    if args.small_runs > 0:
        small = bench_small_configs(tpr, workloads, dev, args.small_runs)
    attn = None
    if args.attn_steps > 0:
        attn = bench_attn_proj(tpr, dev, args.attn_steps)
    gated = None
    if args.gated_steps > 0:
        gated = bench_gated_mlp(tpr, dev, args.gated_steps)
    ce_stats = None
    if args.ce_stats_steps > 0:
        ce_stats = bench_ce_stats(tpr, workloads, dev, args.ce_stats_steps)
    reduce = None
    if args.reduce_steps > 0:
        reduce = bench_reduce(tpr, dev, args.reduce_steps)
    ce_opts = None
    if args.ce_opts_steps > 0:
        ce_opts = bench_ce_opts(tpr, workloads, dev, args.ce_opts_steps)
    med = lambda v: sorted(v)[len(v) // 2]

    line = {
        "metric": METRIC,
        "value": round(mlp_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_70b_tp8_rank_mlp_fwd_bwd + llama3_70b_tp8_inner_gemm_fwd_bwd + "
                        "vocab_ce_t4096_v128256_p8",
            "mlp": dict(MLP, tp_simulated=1, w_layout="math"),
            "inner_gemm": INNER,
            "vocab_ce": CE,
            "parallelism": "tp8 rank share on 1 GPU",
        },
        "mlp_pct_of_bf16_peak": round(100.0 * mlp_tflops / PEAK_BF16_TFLOPS, 2),
        "mlp_ms": round(avg(mlp_ms), 4),
        "mlp_ms_median": round(med(mlp_ms), 4),
        "mlp_ms_min": round(min(mlp_ms), 4),
        "inner_gemm_tflops": round(inner_tflops, 2),
        "inner_gemm_ms": round(avg(inner_ms), 4),
        "inner_gemm_ms_min": round(min(inner_ms), 4),
        "mlp_gemms_via_torch_mm": blas,
        "vocab_ce_gbs": round(ce_gbs, 1),
        "vocab_ce_pct_of_hbm_peak": round(100.0 * ce_gbs / PEAK_HBM_GBS, 2),
        "vocab_ce_ms": round(avg(ce_ms), 4),
        "vocab_ce_ms_median": round(med(ce_ms), 4),
        "vocab_ce_ms_min": round(min(ce_ms), 4),
        "roofline": {
            "kernel": GEMM_KERNEL + " (4 grouped launches per step: 3 of the MLP call, 1 of the inner GEMM)",
            "bound": "mfma",
            "flop_per_launch": gemm_flop_per_launch,
            "avg_launch_us": round(gemm_launch_ms * 1e3, 2),
            "achieved": round(gemm_achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": gemm_traffic,
        },
        "roofline_ce": {
            "kernel": CE_KERNEL + " + loss_mean_kernel (one call)",
            "bound": "hbm",
            "bytes_per_launch": ce_bytes,
            "avg_call_us": round(avg(ce_ms) * 1e3, 2),
            "achieved": round(ce_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(ce_gbs / PEAK_HBM_GBS, 4),
            "traffic": ce_traffic,
            "copy_same_bytes_gbs": None if copy_gbs is None else round(copy_gbs, 1),
            "frac_of_copy": None if copy_gbs is None else round(ce_gbs / copy_gbs, 4),
        },
        "roofline_reduce": reduce,
        "kernel_source_digest": kernel_source_digest(),
    }
    if head is not None:
        line["vocab_head_ce"] = head
    if mlp_8b is not None:
        line["mlp_8b_rank"] = mlp_8b
    if ce_stats is not None:
        line["vocab_ce_shard_stats"] = ce_stats
    if ce_opts is not None:
        line["vocab_ce_opts"] = ce_opts
    if gated is not None:
        line["gated_silu_mlp_70b_rank"] = gated
    if attn is not None:
        line["attn_proj_70b_rank"] = attn
    if small is not None:
        line["latency"] = small
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
