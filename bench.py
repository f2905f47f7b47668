#!/usr/bin/env python3
"""Throughput of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--splits S] [--no-cpu-baseline] [--graph]

One step is one fa_fwd call (the whole forward: QK^T, online softmax, PV,
normalisation, O and L written) over one batch of seeded synthetic inputs
already resident in device memory (200 untimed warm-up steps, then 100 timed
steps, by default).  The default workload is the causal bf16
case B=2, H=32, N=4096, d=128, on which the MFMA-peak target is stated.

For the block-sparse workload a step is one fa_fwd_blocksparse call with its
local-global block mask (64 x 64 blocks); `value` then counts 4*d flops per
visible (query, key) pair of the mask, and the line also carries fa_fwd on the
same inputs (all pairs) under `dense`.

For the backward workload a step is one fa_bwd call (the row sums D, then the
dK/dV and dQ kernels) on the forward's O and L computed before the timed
region; `value` counts the conventional 10*B*H*N^2*d flops (two and a half
forward passes: the recomputed S and four products), halved for causal.

For the key-range split workloads (few query tiles per head) a step is one
fa_fwd_splitkv call instead: the split kernel and the merge kernel, with the
workspace allocated before the timed region.  The line then also carries the
unsplit fa_fwd time on the same inputs for comparison (`unsplit`).

With --graph the K timed steps are captured into one HIP graph and the
timed region is one replay of it (launch overhead between steps removed);
the default is K eager calls.

Prints ONE JSON line.  `value` is attention TFLOP/s with the conventional
count 4*B*H*N^2*d (halved for causal) over the timed steps' wall time.
`roofline` relates the kernel's average launch duration (HIP events on the
launch stream) to the dense bf16 MFMA peak, with the MFMA-busy fraction and
HBM bytes of the committed counter summaries (null once the kernel sources
have changed since they were taken) and, for d <= 64, the VALU bound.
`steady` times the same step again after the timed window, once at least 300
launches and 0.1 s of back-to-back launches have run: with a short --warmup the
timed window falls in the GPU's slower first ~30 ms, and the two figures then
differ.  `cpu_baseline` times the float64
CPU oracle on a bounded sample of the same workload (whole heads, ~10 s).
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) + % of bf16 MFMA peak, 1×MI355X"
# Dense bf16 MFMA peak of MI355X: 256 CUs x 4096 flop/clk/CU x 2.4 GHz.
PEAK_BF16_TFLOPS = 2516.6
PEAK_F32_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")
# Load after which the GPU clock has settled: the slow start lasts about 100
# launches (~30 ms) of the causal N=4096 workload; short kernels need more
# launches for the same time (the N=1024 d=64 workload: ~2000, ~50 ms).
STEADY_AFTER_LAUNCHES = 300
STEADY_AFTER_SECONDS = 0.1
CSRC = os.path.join(ROOT, "io_aware_softmax_06_amd", "csrc")


def attention_flops(w):
    f = 4.0 * w.B * w.H * w.N * w.N * w.d
    return f / 2.0 if w.causal else f


def visible_pairs(mask, N, causal, block=64):
    """(query, key) pairs a [nb, nb] block mask (shared by all heads) leaves
    visible: the flop count of the block-sparse workload is 4 d per pair."""
    import torch
    idx = torch.arange(N) // block
    vis = mask.cpu().bool()[idx][:, idx]
    if causal:
        vis &= torch.ones((N, N), dtype=torch.bool).tril()
    return int(vis.sum())


# The sources the forward kernels and their launches are built from; a
# change to any of them makes a recorded traffic figure stale.
FORWARD_SOURCES = ("fa355.hip", "fa355_w4.hip", "fa_common.hpp", "fa_fwd_bf16.hpp",
                   "fa_fwd_f32.hpp", "fa_merge.hpp")


def kernel_source_digest():
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def committed_fields(kind, workload_name):
    """The `name: value` fields of profiles/<kind>_<workload>.txt, or None when
    the file is missing or was taken with other kernel sources (its
    source_digest differs from the current one)."""
    path = os.path.join(PROFILES, f"{kind}_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", line)
        if m:
            fields[m.group(1)] = m.group(2)
    if fields.get("source_digest") != kernel_source_digest():
        return None
    return fields


def measured_mfma_busy(workload_name):
    """MFMA-busy fraction of the committed counter summary (None if stale):
    SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles of the dispatch
    (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)."""
    f = committed_fields("mfma_busy", workload_name)
    try:
        return None if f is None else float(f["mfma_busy"])
    except (KeyError, ValueError):
        return None


def valu_bound(workload_name, flops, peak):
    """The VALU bound of one launch from the committed counters (None if
    stale).  The non-MFMA VALU instructions of the dispatch, spread evenly
    over the 1024 SIMDs at the throughputs measured with two waves per SIMD
    and one workgroup per CU (9.8 SIMD cycles per exponential, 2.9 per other
    wave64 instruction: the cheapest, fma/add/mul, so that this is a lower
    bound), give `valu_us` at the 2.4 GHz peak clock; the MFMA work gives
    `mfma_us`.  A SIMD issues VALU work of one wave while another wave's
    MFMA runs, so the launch can reach at most flops / max(valu_us, mfma_us)
    (fully overlapped) and, with no overlap at all, flops / (valu_us +
    mfma_us)."""
    f = committed_fields("mfma_busy", workload_name)
    try:
        valu_us = float(f["valu_bound_us_at_2400mhz"])
        mfma_us = float(f["mfma_bound_us_at_2400mhz"])
        insts = int(float(f["valu_non_mfma_insts"]))
    except (TypeError, KeyError, ValueError):
        return None
    tf = flops / 1e12 / 1e-6
    return {"valu_insts_per_launch": insts,
            "valu_us_at_2400mhz": round(valu_us, 2),
            "mfma_us_at_2400mhz": round(mfma_us, 2),
            "frac_ceiling_overlapped": round(tf / max(valu_us, mfma_us) / peak, 4),
            "frac_ceiling_serial": round(tf / (valu_us + mfma_us) / peak, 4)}


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed PMC summary, if it is current.

    The summary records FETCH_SIZE and WRITE_SIZE (KiB per dispatch, each
    scaled by the copy-kernel calibration factor) and the digest of the kernel
    sources it was taken with; a changed kernel makes the figure stale (None).
    """
    f = committed_fields("hbm_traffic", workload_name)
    try:
        return None if f is None else float(f["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_description():
    """The host CPU the oracle runs on: lscpu's model name, the logical CPUs
    this process may run on, and the BLAS threads NumPy uses."""
    model = None
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:
        model = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads": blas}


def cpu_baseline(w, seed, budget_s=10.0, block_mask=None, flops=None):
    """The float64 oracle on whole heads of the same inputs, ~budget_s seconds.

    With a block mask (shared by all heads) the oracle is the block-sparse
    definition and ``flops`` the workload's count of useful flops."""
    import numpy as np
    import oracle
    from workloads import make_inputs, to_f64_numpy
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    q, k, v = make_inputs(w, seed)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        if block_mask is None:
            oracle.attention(to_f64_numpy(q[sl]), to_f64_numpy(k[sl]), to_f64_numpy(v[sl]),
                             w.scale, w.causal)
        else:
            oracle.attention_block_sparse(to_f64_numpy(q[sl]), to_f64_numpy(k[sl]),
                                          to_f64_numpy(v[sl]), w.scale, w.causal, block_mask)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_head = (flops if flops is not None else attention_flops(w)) / (w.B * w.H)
    del np
    return {
        "value": round(per_head * done / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} (batch, head) slices of {w.name}, seed {seed}, "
                  f"float64 NumPy oracle with materialised S, {dt:.1f} s",
        "host": host_description(),
    }


def cpu_baseline_backward(w, seed, budget_s=10.0):
    """The float64 backward oracle on whole heads of the same inputs."""
    import oracle
    from workloads import make_grad, make_inputs, to_f64_numpy
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    q, k, v = make_inputs(w, seed)
    do = make_grad(w.B, w.H, w.N, w.d, w.torch_dtype, seed)
    done, t0 = 0, time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            oracle.attention_backward(to_f64_numpy(q[sl]), to_f64_numpy(k[sl]),
                                      to_f64_numpy(v[sl]), to_f64_numpy(do[sl]), w.scale, w.causal)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_head = 2.5 * attention_flops(w) / (w.B * w.H)
    return {"value": round(per_head * done / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} (batch, head) slices of {w.name}, seed {seed}, "
                      f"float64 NumPy backward oracle with materialised S and P, {dt:.1f} s",
            "host": host_description()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The GPU's clocks take about 30 ms of back-to-back launches to settle
    # (about 100 launches of the causal 4096 workload); by default 200 warm-up
    # steps put every timed step in the steady state.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="causal_bf16_b2h32n4096d128")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--splits", type=int, default=None,
                    help="key ranges of the split path (default: the workload's own, if it "
                         "has one; 0 runs fa_fwd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps into one HIP graph (torch.cuda.graph) "
                         "and time one replay of it instead of K eager calls")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one elementwise copy of this many MiB "
                         "(read once, written once) so that a counter run can scale its HBM "
                         "byte counters against a kernel of known traffic")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward pass is benchmarked on a single "
              "MI355X (no multi-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import io_aware_softmax_06_amd as fa
    import workloads

    fa.load()
    w = workloads.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_inputs(w, args.seed, device=dev)
    O = torch.empty_like(q)
    L = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # The library launches on the stream it is given; under graph capture that
    # must be the capture stream, which the binding picks when given None.
    call_stream = None if args.graph else stream
    sparse_mask = None
    flops = attention_flops(w)
    if w.name == workloads.SPARSE_4K.name:
        sparse_mask = workloads.local_global_block_mask(
            (w.N + 63) // 64, workloads.SPARSE_4K_WINDOW, workloads.SPARSE_4K_GLOBAL).to(dev)
        flops = 4.0 * w.d * w.B * w.H * visible_pairs(sparse_mask, w.N, w.causal)
    backward = w.name == workloads.BWD_CAUSAL_4K.name
    if backward:
        flops = 2.5 * attention_flops(w)
        do = workloads.make_grad(w.B, w.H, w.N, w.d, w.torch_dtype, args.seed, device=dev)
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=O, lse=L, stream=stream)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        bwd_ws = torch.empty(fa.fa_bwd_workspace(w.B, w.H, w.N, w.d), dtype=torch.uint8,
                             device=dev)
    splits = workloads.SPLITS_OF.get(w.name, 0) if args.splits is None else args.splits
    ws = None
    if splits:
        need = fa.fa_fwd_splitkv_workspace(w.B, w.H, w.N, w.d, splits)
        if need < 0:
            raise fa.FaError(need)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def unsplit_step():
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=O, lse=L, stream=call_stream)

    def split_step():
        fa.fwd_splitkv(q, k, v, splits, scale=w.scale, causal=w.causal, out=O, lse=L,
                       workspace=ws, stream=call_stream)

    def sparse_step():
        fa.fwd_blocksparse(q, k, v, sparse_mask, scale=w.scale, causal=w.causal, out=O, lse=L,
                           stream=call_stream)

    def backward_step():
        fa.bwd(q, k, v, O, do, L, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dv,
               workspace=bwd_ws, stream=call_stream)

    step = (backward_step if backward else sparse_step if sparse_mask is not None
            else split_step if splits else unsplit_step)

    def timed(fn, n):
        """(wall seconds, average GPU seconds per call) of n back-to-back calls.

        One pair of HIP events on `stream` brackets the n launches.  Events
        recorded between consecutive launches would sit in the queue as
        markers of their own and slow the launches they separate (measured on
        the causal workload: 278 us per launch with an event pair around each,
        274 us without), so the average duration comes from the pair around
        the whole region; it includes the short gaps between launches."""
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(n):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        return wall_s, start.elapsed_time(end) / 1e3 / n

    def timed_graph(fn, n):
        """As timed(), for one replay of a graph that holds n calls."""
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for _ in range(n):
                fn()
        torch.cuda.synchronize()
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        return wall_s, start.elapsed_time(end) / 1e3 / n

    t_load = time.perf_counter()  # start of back-to-back launches (for `steady`)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    wall, avg_launch_s = (timed_graph if args.graph else timed)(step, args.steps)
    call_stream = stream  # the runs below are eager

    # After the timed window: the same step once the clocks have settled.  The
    # first ~100 launches of a cold GPU run at a lower clock (the cycle counts
    # per launch stay flat), so a short warm-up puts the timed window inside
    # that phase; this figure is reported beside `value`, never in its place.
    before = args.warmup + args.steps
    settle = 0
    while before + settle < STEADY_AFTER_LAUNCHES or time.perf_counter() - t_load < STEADY_AFTER_SECONDS:
        for _ in range(50):
            step()
        settle += 50
        torch.cuda.synchronize()
    _, steady_s = timed(step, max(args.steps, 50))
    steady = {"kernel_us": round(steady_s * 1e6, 2),
              "tflops": round(flops / steady_s / 1e12, 3),
              "launches_before": before + settle}

    dense = None
    if sparse_mask is not None:  # after the timed region: every pair, on the same inputs
        for _ in range(max(1, args.warmup // 2)):
            unsplit_step()
        _, avg = timed(unsplit_step, args.steps)
        dense = {"kernel_us": round(avg * 1e6, 2),
                 "tflops_all_pairs": round(attention_flops(w) / avg / 1e12, 3),
                 "sparse_speedup": round(avg / avg_launch_s, 3),
                 "mask_density": round(flops / attention_flops(w), 4)}

    unsplit = None
    if splits:  # after the timed region: the single-pass kernel on the same inputs
        for _ in range(max(1, args.warmup // 2)):
            unsplit_step()
        _, avg = timed(unsplit_step, args.steps)
        unsplit = {"kernel_us": round(avg * 1e6, 2),
                   "tflops": round(attention_flops(w) / avg / 1e12, 3),
                   "split_speedup": round(avg / avg_launch_s, 3)}

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # one streaming kernel: n*4 bytes read, n*4 written
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = wall / args.steps * 1e3
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / avg_launch_s / 1e12
    peak = PEAK_F32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS  # fp16 MFMA: same peak
    props = torch.cuda.get_device_properties(dev)
    print(f"device: {props.name}, {props.multi_processor_count} CUs; kernel avg "
          f"{avg_launch_s * 1e6:.1f} us, "
          f"{achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% of {peak} TFLOP/s",
          file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q, K, V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "dtype": w.dtype, "layout": "[B,H,N,d]",
                   "parallelism": "single GPU",
                   "launch": "one HIP graph of the K steps" if args.graph else "eager",
                   "entry_point": ("fa_bwd" if backward else
                                   "fa_fwd_blocksparse" if sparse_mask is not None
                                   else "fa_fwd_splitkv" if splits else "fa_fwd"),
                   **({"block_mask": f"local-global, band {workloads.SPARSE_4K_WINDOW}, "
                                     f"{workloads.SPARSE_4K_GLOBAL} global blocks, 64x64; "
                                     "flops over visible pairs"}
                      if sparse_mask is not None else {}),
                   **({"num_splits": splits} if splits else {})},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        # the peak assumes 256 CUs at 2.4 GHz (the clock under load is in the
        # committed counter summaries: GRBM_GUI_ACTIVE cycles over time)
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "roofline": {
            "bound": "alu" if w.dtype == "fp32" else "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.name),
            "mfma_busy": measured_mfma_busy(w.name),
            **({"valu_bound": valu_bound(w.name, flops, peak)} if w.d <= 64 else {}),
            **({"kernels": "split forward + merge (one step, both launches)"}
               if splits else {}),
            **({"kernels": "row sums D + dK/dV + dQ (one step, three launches)"}
               if backward else {}),
        },
        "steady": {**steady, "frac": round(flops / steady_s / 1e12 / peak, 4)},
        "cpu_baseline": None,
        **({"unsplit": unsplit} if splits else {}),
        **({"dense": dense} if sparse_mask is not None else {}),
    }
    if not args.no_cpu_baseline and backward:
        result["cpu_baseline"] = cpu_baseline_backward(w, args.seed)
    elif not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(
            w, args.seed, block_mask=None if sparse_mask is None else sparse_mask.cpu().numpy(),
            flops=flops)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
