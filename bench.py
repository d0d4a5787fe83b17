"""Benchmark of the chunkwise gated-delta-rule forward on one MI355X.

One step = one gdn_chunk_fwd call over the training-shape workload
(B=8, T=4096, H=6, K=V=128, chunk 64, bf16 q/k/v/o, fp32 gates and state),
inputs already resident in HBM.  Three input sets are rotated so that the
256 MB Infinity Cache cannot serve a repeat of the previous step's inputs.

Prints ONE JSON line (rank 0) with throughput in tokens/s, the roofline of the
kernel, and the fp64 CPU oracle timed on the host as a reported baseline.
The run is correctness-gated: the GPU output of input set 0 must match the
oracle (relative L2 <= 2e-2) before any number is printed.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3        # MI355X fp32 (matrix and vector), published
METRIC = "GDN chunk fwd tokens/s + % bf16 MFMA peak at B8·T4096·H6·d128"

# Sources of the timed kernel (its body and the device helpers it includes): a
# traffic record measured on other sources is stale.
KERNEL_SOURCES = ["linear_attention_sequence_chunked_amd/csrc/fwd_bf16.hip",
                  "linear_attention_sequence_chunked_amd/csrc/fwd_bf16_kernel.h",
                  "linear_attention_sequence_chunked_amd/csrc/mfma_common.h"]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "fwd_bf16_train_B8T4096H6_hbm_traffic.md")
COPY_BYTES = 1 << 30           # calibration copy: 1 GiB read, 1 GiB written


def pick_roof(flops, nbytes, kern_ms, peak_tflops):
    """Roofline object for one launch of kern_ms: the roof the arithmetic
    intensity (flops / nbytes) reaches first, HBM below the ridge
    peak_tflops / HBM peak, the matrix cores above it (then with the HBM
    figures under "hbm")."""
    gbs = nbytes / (kern_ms / 1e3) / 1e9
    hbm = {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    if flops / nbytes > peak_tflops * 1e12 / (HBM_PEAK_GBS * 1e9):
        tf = flops / (kern_ms / 1e3) / 1e12
        return {"bound": "mfma", "achieved": tf, "peak": peak_tflops, "unit": "TFLOP/s",
                "frac": tf / peak_tflops, "hbm": hbm}
    return dict(bound="hbm", **hbm)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# The timed region is K calls back to back between one pair of events; its mean
# (launch gaps included) is also the kernel time the roofline uses, since the
# stream holds nothing else.  Events around single launches add two packets each
# (about 5 us per call at the training shape, 2-8% of a call), so the per-launch
# spread is taken from a separate pass after the timed region.
SPREAD_LAUNCHES = 25


def time_steps(step, steps, stream):
    """Time `steps` calls of step(i) on `stream`: (total ms between events recorded
    before the first and after the last call, per-launch ms of SPREAD_LAUNCHES
    further calls, each between its own pair of events, after the timed region)."""
    import numpy as np
    import torch

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total = t_start.elapsed_time(t_end)
    pairs = []
    for i in range(SPREAD_LAUNCHES):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(steps + i)
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return total, np.array([a.elapsed_time(b) for a, b in pairs])


def replay_check(step, outputs, min_seconds=0.3, min_reps=16):
    """Part of the correctness gate: replays step() (which rewrites `outputs`)
    for at least min_seconds and min_reps calls and checks every replay bitwise
    against the first result (the kernels sum in a fixed order, so the results
    must not vary between launches).  Returns (replays, reproducible).

    The replays also take the GPU out of its idle clock state before the
    warm-up: a few warm-up steps of 0.13 ms after the seconds of CPU work of the
    oracle gate otherwise leave the first timed launches ~8% slower."""
    import torch

    ref = [t.clone() for t in outputs]
    bad = torch.zeros((), dtype=torch.bool, device=ref[0].device)
    n = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while n < min_reps or time.perf_counter() - t0 < min_seconds:
        step()
        for r, t in zip(ref, outputs):
            bad |= torch.ne(t, r).any()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()   # keep the host within a few calls of the GPU
    torch.cuda.synchronize()
    return n, not bool(bad)


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter record, or None
    when there is none or it was taken on different kernel sources.

    The record holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the forward
    kernel and of a calibration copy of COPY_BYTES; each kernel counter is divided
    by the copy's reading per byte copied."""
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    rec = None
    for line in open(TRAFFIC_RECORD):
        if line.startswith("TRAFFIC_JSON "):
            rec = json.loads(line[len("TRAFFIC_JSON "):])
    if rec is None or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    f_fetch = rec["copy_fetch_kib"] * 1024.0 / COPY_BYTES
    f_write = rec["copy_write_kib"] * 1024.0 / COPY_BYTES
    return rec["fwd_fetch_kib"] * 1024.0 / f_fetch + rec["fwd_write_kib"] * 1024.0 / f_write


def copy_calibration():
    """A plain device-to-device copy of known size, for counter calibration:
    rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) on this run gives the counter's
    reading for COPY_BYTES read and COPY_BYTES written."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "kernel_source_sha256": kernel_source_hash()}),
          flush=True)


def algorithmic_bytes(B, T, H, K, V, esz=2, with_s0=False):
    """HBM bytes one forward must move: q, k, v read, o written, gates read, final state written."""
    tok = B * T * H
    by = tok * (2 * K + 2 * V) * esz + tok * 2 * 4 + B * H * V * K * 4
    if with_s0:
        by += B * H * V * K * 4
    return by


def executed_mfma_flops(B, T, H, K, V, C, vs):
    """Dense MFMA FLOPs the bf16 forward kernel issues (16x16x32 instructions x
    16384): per (stream, chunk) and workgroup of vs value rows, the Gram tiles
    (10 of A and 10 of P, K/32 k-steps each), the two levels of the block solve
    (16 instructions) and, per 16 value rows, the chain (Y, Z: C/16 token blocks
    x K/32; S: K/16 x C/32; U and O: 6 (C = 64) or 2 (C = 32) lower-triangular
    block products each).  Gram and solve are repeated by every value slice of a
    stream.  (A states-only call skips O; rocprofv3's SQ_INSTS_MFMA matched this
    count per launch.)"""
    ntb = C // 16
    tri = ntb * (ntb + 1) // 2              # lower token-block pairs
    gram = 2 * tri * (K // 32)
    levels = 16 if ntb == 4 else 2
    chain = 2 * ntb * (K // 32) + (K // 16) * (C // 32) + 2 * (6 if ntb == 4 else 2)
    per_wg = gram + levels + (vs // 16) * chain
    nchunks = (T + C - 1) // C
    return B * H * (V // vs) * nchunks * per_wg * 16384.0


def copy_bandwidth_gbs(nbytes=1 << 30, reps=5):
    """Achievable HBM bandwidth of a plain device copy (bytes read + written per
    second), the practical reference beside the published peak."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_baseline(call, tokens, streams, sample, repeats=1):
    """The fp64 CPU oracle timed on the host: call(nthreads) runs it once over the
    sample (threads over the streams); tokens/s over `repeats` calls."""
    import oracle
    used = max(1, min(oracle.default_threads(), streams))
    t0 = time.perf_counter()
    for _ in range(repeats):
        call(used)
    dt = (time.perf_counter() - t0) / repeats
    return {"value": tokens / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": sample % dt, "cpu_model": cpu_model()}


def algorithmic_flops(B, T, H, K, V, C):
    """Structural FLOPs per token-head of the chunk algorithm (triangular products at
    their structural size, the inverse as C^3/3 per chunk):
    (3C-1)K + 2CV + 6KV + C^2/3."""
    per = (3 * C - 1) * K + 2 * C * V + 6 * K * V + C * C / 3.0
    return per * B * T * H


def tile_flops(B, T, H, K, V, C):
    """FLOPs of the same products counted as dense tiles (every C x C product in
    full, the inverse as C^3/3 per chunk): per token-head 6CK + 4CV + 6KV + C^2/3
    (10Cd + 6d^2 + C^2/3 when K = V = d)."""
    per = 6 * C * K + 4 * C * V + 6 * K * V + C * C / 3.0
    return per * B * T * H


def backward_flops(B, T, H, K, V, C):
    """Structural FLOPs per call of the backward as built (backward chunk C):
    per token-head 22KV + 8CV + 9CK + C^2 (state recompute 4KV + CV + CK; reverse
    state-gradient walk 6KV + 2CV + 2CK; token gradients 12KV + 5CV + 6CK; three
    triangular solves)."""
    return (22 * K * V + 8 * C * V + 9 * C * K + C * C) * B * T * H


def bench_backward(args):
    """One step = one gdn_chunk_bwd call (state recompute, reverse walk, token
    gradients) on the forward+backward workload, inputs resident in HBM."""
    import numpy as np
    import torch

    from linear_attention_sequence_chunked_amd import bwd_workspace_size, chunk_bwd
    from linear_attention_sequence_chunked_amd.workloads import WORKLOADS, workload_inputs

    # --workload names a forward+backward workload (one that draws d_o); the
    # default forward workload maps to the bf16 one
    w = WORKLOADS[args.workload if WORKLOADS[args.workload].with_do else "fwdbwd_bf16"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, H, K, V, C = w.B, w.T, w.H, w.K, w.V, w.chunk
    cpu = workload_inputs(w)
    g = {n: (t.to(dev) if t is not None else None) for n, t in cpu.items()}
    ws = torch.empty(bwd_workspace_size(B, T, H, K, V, C, dtype=w.dtype), dtype=torch.uint8, device=dev)
    res = (torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"]),
           torch.empty_like(g["alpha"]), torch.empty_like(g["beta"]),
           torch.empty(B, H, V, K, dtype=torch.float32, device=dev))

    def step():
        return chunk_bwd(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["d_o"],
                         g["initial_state"], chunk=C, workspace=ws, out=res)

    gate = None
    if not args.no_gate:
        import oracle
        got = step()
        torch.cuda.synchronize()
        ref = oracle.bwd(cpu["q"], cpu["k"], cpu["v"], cpu["alpha"], cpu["beta"], cpu["d_o"])
        names = ("dq", "dk", "dv", "dalpha", "dbeta", "d_initial_state")
        gate = {n: float(np.linalg.norm(x.double().cpu().numpy() - ref[n]) / np.linalg.norm(ref[n]))
                for n, x in zip(names, got)}
        tol = 1e-5 if w.dtype == torch.float32 else 2e-2
        ok = all(e <= tol for e in gate.values())
        reps, same = replay_check(step, list(res))
        gate.update(replays_bitwise_equal=same, replays=reps)
        if not (ok and same):
            print("correctness gate failed: %s" % json.dumps(gate), file=sys.stderr)
            sys.exit(1)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one event pair around the K calls (a call is three launches; events
    # between the calls would add their own packets to every call's critical
    # path)
    stream = torch.cuda.current_stream(dev)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    # bf16 inputs with K, V >= 32 take the bf16 MFMA path (64-token chunks, bf16
    # operands, fp32 accumulation); float32 inputs take 32-token chunks with the
    # state recompute, reverse walk and token gradients on v_mfma_f32_16x16x4_f32
    mfma = w.dtype == torch.bfloat16 and K >= 32 and V >= 32
    f32_mfma = w.dtype == torch.float32
    bwd_c = 64 if mfma else min(C, 32)
    flops = backward_flops(B, T, H, K, V, bwd_c)
    peak = 2500.0 if mfma else F32_PEAK_TFLOPS
    tok = B * T * H
    esz = 2 if w.dtype == torch.bfloat16 else 4
    abytes = tok * (4 * K * esz + 3 * K * esz + 2 * 4 + 2 * 4) + B * H * V * K * 4  # q,k,v,dO,gates in; dq,dk,dv,dgates out; dS0
    cpub = None
    if not args.no_cpu_baseline:
        import oracle
        cpub = oracle_baseline(
            lambda n: oracle.bwd(cpu["q"], cpu["k"], cpu["v"], cpu["alpha"], cpu["beta"], cpu["d_o"],
                                 cpu["initial_state"], nthreads=n),
            B * T, B * H, "whole workload (%d streams x %d tokens), fp64 reverse mode with fp64 "
                          "checkpoints every 64 tokens, %%.2f s" % (B * H, T))
    print(json.dumps({
        "metric": "GDN chunk bwd tokens/s at B%d\u00b7T%d\u00b7H%d\u00b7d%d" % (B, T, H, K),
        "value": B * T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if mfma else "f32", "data": "synthetic",
        "config": {"workload": "%s: B=%d T=%d H=%d K=%d V=%d chunk=%d (backward chunk %d)"
                               % (w.name, B, T, H, K, V, C, bwd_c)},
        "roofline": {"bound": "mfma" if mfma or f32_mfma else "alu", "achieved": flops / (ms / 1e3) / 1e12,
                     "peak": peak, "unit": "TFLOP/s", "frac": flops / (ms / 1e3) / 1e12 / peak,
                     "traffic": None, "algorithmic_flops": flops,
                     "hbm_gbs_algorithmic": abytes / (ms / 1e3) / 1e9},
        "cpu_baseline": cpub,
        "gate": gate,
    }), flush=True)


def oracle_timing(args):
    """The fp64 CPU oracle timed on the host over the forward configurations
    (mid, training shape, long context) and, in reverse mode, the forward+backward
    one: every (batch, head) stream on all host cores, and the same on one core.
    Prints one JSON line; the GPU is not used."""
    import oracle
    from linear_attention_sequence_chunked_amd.workloads import WORKLOADS, workload_inputs
    cores = oracle.default_threads()
    res = {"kind": "oracle", "cpu_model": cpu_model(), "cores": cores, "configs": []}
    for name, mode in (("mid_bf16", "fwd"), ("train_bf16", "fwd"), ("fwdbwd_bf16", "bwd"),
                       ("long_bf16", "fwd")):
        w = WORKLOADS[name]
        c = workload_inputs(w)
        row = {"workload": name, "mode": mode, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "V": w.V}
        for nth in (cores, 1):
            t0 = time.perf_counter()
            if mode == "fwd":
                oracle.fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["initial_state"], nthreads=nth)
            else:
                oracle.bwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["d_o"], c["initial_state"],
                           nthreads=nth)
            dt = time.perf_counter() - t0
            row["seconds_%d_cores" % nth] = dt
            row["tokens_per_s_%d_cores" % nth] = w.B * w.T / dt
        if mode == "fwd":
            row["gflops_fp64_all_cores"] = 8.0 * w.K * w.V * w.B * w.T * w.H / row["seconds_%d_cores" % cores] / 1e9
        res["configs"].append(row)
        print("  %s %s: %.2f s on %d cores, %.2f s on 1" % (name, mode, row["seconds_%d_cores" % cores], cores,
                                                           row["seconds_1_cores"]), file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def bench_decode(args):
    """One step = one gdn_decode_step call (one token for 64 streams x 16 heads,
    K = V = 128).  Five state buffers (5 x 64 MiB) rotate so the Infinity Cache
    cannot hold the state between steps; the state is read and written once per
    step, so the bound is HBM."""
    import numpy as np
    import torch

    from linear_attention_sequence_chunked_amd import decode_step
    from linear_attention_sequence_chunked_amd.workloads import WORKLOADS, workload_inputs

    w = WORKLOADS["decode_bf16"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, K, V = w.B, w.H, w.K, w.V
    cpu = workload_inputs(w)
    g = {n: (t[:, 0].contiguous().to(dev) if t is not None and n != "initial_state" else None)
         for n, t in cpu.items()}
    nsets = 5
    states = [cpu["initial_state"].to(dev) for _ in range(nsets)]
    out = torch.empty(B, H, V, dtype=w.dtype, device=dev)

    def step(i):
        decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], states[i % nsets], out=out)

    gate = None
    if not args.no_gate:
        import oracle
        step(0)
        torch.cuda.synchronize()
        ro, rs = oracle.fwd(cpu["q"], cpu["k"], cpu["v"], cpu["alpha"], cpu["beta"],
                            cpu["initial_state"])
        gate = {"rel_l2_o": float(np.linalg.norm(out.double().cpu().numpy() - ro[:, 0]) / np.linalg.norm(ro)),
                "rel_l2_state": float(np.linalg.norm(states[0].double().cpu().numpy() - rs) / np.linalg.norm(rs))}
        if not (gate["rel_l2_o"] <= 2e-2 and gate["rel_l2_state"] <= 1e-5):
            print("correctness gate failed: %s" % json.dumps(gate), file=sys.stderr)
            sys.exit(1)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    total_ms, per_launch = time_steps(step, args.steps, stream)
    ms = total_ms / args.steps
    kern_ms = ms
    abytes = B * H * (2 * V * K * 4 + (2 * K + 2 * V) * 2 + 8)
    gbs = abytes / (kern_ms / 1e3) / 1e9
    cpub = None
    if not args.no_cpu_baseline:
        import oracle
        reps = 5
        cpub = oracle_baseline(
            lambda n: oracle.fwd(cpu["q"], cpu["k"], cpu["v"], cpu["alpha"], cpu["beta"],
                                 cpu["initial_state"], nthreads=n),
            B, B * H, "one token for all %d streams (the same step), fp64, %d calls of %%.4f s" % (B * H, reps),
            repeats=reps)
    print(json.dumps({
        "metric": "GDN decode step tokens/s at B64\u00b7H16\u00b7d128",
        "value": B / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in/out, f32 state", "data": "synthetic",
        "config": {"workload": "%s: B=%d H=%d K=%d V=%d, one token per call, 5 rotating states"
                               % (w.name, B, H, K, V)},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel_ms": kern_ms,
                     "kernel_ms_source": "mean over the timed region (calls back to back)",
                     "kernel_ms_pct": {"p10": float(np.percentile(per_launch, 10)),
                                       "p50": float(np.percentile(per_launch, 50)),
                                       "p90": float(np.percentile(per_launch, 90))},
                     "kernel_ms_pct_launches": int(per_launch.size),
                     "algorithmic_bytes": abytes},
        "cpu_baseline": cpub,
        "gate": gate,
    }), flush=True)


def varlen_lengths(n=24, lo=128, hi=8192, seed=7):
    """Seeded ragged length mix: n lengths log-uniform in [lo, hi]."""
    import numpy as np
    rng = np.random.default_rng(seed)
    return [int(x) for x in np.exp(rng.uniform(np.log(lo), np.log(hi), n))]


def bench_varlen(args):
    """One step = one gdn_chunk_fwd_varlen call over a packed batch of 24 sequences
    (lengths log-uniform in [128, 8192], seeded), H = 6, K = V = 128, bf16, chunk 64.
    The call's time is set by the longest sequence (each (sequence, head, value
    slice) is one workgroup walking its chunks in order)."""
    import numpy as np
    import torch

    from linear_attention_sequence_chunked_amd import chunk_fwd_varlen
    from linear_attention_sequence_chunked_amd.workloads import make_inputs

    lengths = varlen_lengths()
    N, T, H, K, V, C = len(lengths), int(sum(lengths)), 6, 128, 128, 64
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(1, T, H, K, V, dtype=torch.bfloat16, seed=8, gate="decay")
    g = {n: (t.to(dev) if t is not None else None) for n, t in inp.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    out = torch.empty(1, T, H, V, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(N, H, V, K, dtype=torch.float32, device=dev)

    def step():
        chunk_fwd_varlen(g["q"], g["k"], g["v"], g["alpha"], g["beta"], cu, None, chunk=C,
                         out=out, final_state=sf)

    gate = None
    if not args.no_gate:
        import oracle
        step()
        torch.cuda.synchronize()
        i = int(np.argmax(lengths))
        a, b = int(cu[i]), int(cu[i + 1])
        ro, rs = oracle.fwd(*(inp[n][:, a:b].contiguous() for n in ("q", "k", "v", "alpha", "beta")))
        gate = {"longest_sequence": lengths[i],
                "rel_l2_o": float(np.linalg.norm(out[:, a:b].double().cpu().numpy() - ro) / np.linalg.norm(ro)),
                "rel_l2_state": float(np.linalg.norm(sf[i].double().cpu().numpy() - rs[0]) / np.linalg.norm(rs))}
        gate["replays"], gate["replays_bitwise_equal"] = replay_check(step, [out, sf])
        if not (gate["rel_l2_o"] <= 2e-2 and gate["rel_l2_state"] <= 2e-2 and gate["replays_bitwise_equal"]):
            print("correctness gate failed: %s" % json.dumps(gate), file=sys.stderr)
            sys.exit(1)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    total_ms, per_launch = time_steps(lambda i: step(), args.steps, stream)
    ms = total_ms / args.steps
    abytes = T * H * 1032 + N * H * V * K * 4
    longest_chunks = -(-max(lengths) // C)
    cpub = None
    if not args.no_cpu_baseline:
        import oracle
        bounds = np.concatenate([[0], np.cumsum(lengths)])

        def every_sequence(n):
            for i in range(N):
                a, b = int(bounds[i]), int(bounds[i + 1])
                oracle.fwd(*(inp[nm][:, a:b].contiguous() for nm in ("q", "k", "v", "alpha", "beta")),
                           nthreads=n)
        cpub = oracle_baseline(every_sequence, T, H,
                               "whole workload (%d sequences one after another, threads over the %d "
                               "heads), fp64 token loop, %%.2f s" % (N, H))
    print(json.dumps({
        "metric": "GDN chunk fwd (packed ragged batch) tokens/s",
        "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "varlen_bf16: %d sequences, %d tokens, lengths log-uniform in "
                               "[128, 8192] (longest %d), H=%d K=V=%d chunk=%d"
                               % (N, T, max(lengths), H, K, C)},
        "roofline": {"bound": "hbm", "achieved": abytes / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": abytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes": abytes},
        "us_per_chunk_of_longest": ms * 1e3 / longest_chunks,
        "cpu_baseline": cpub,
        "gate": gate,
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gate", action="store_true", help="skip the oracle correctness gate")
    ap.add_argument("--workload", default="train_bf16")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the known-size copy used to calibrate HBM counters")
    ap.add_argument("--backward", action="store_true",
                    help="time gdn_chunk_bwd on the forward+backward workload instead")
    ap.add_argument("--decode", action="store_true",
                    help="time gdn_decode_step on the decode workload instead")
    ap.add_argument("--segments", type=int, default=1,
                    help="run the forward segment-parallel with this many segments per sequence")
    ap.add_argument("--varlen", action="store_true",
                    help="time gdn_chunk_fwd_varlen on a packed ragged batch instead")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="only time the fp64 CPU oracle on the configurations (no GPU)")
    args = ap.parse_args()
    if args.oracle_timing:
        oracle_timing(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.varlen:
        if args.gpus != 1:
            print("bench.py measures one GPU only; run with --gpus 1", file=sys.stderr)
            sys.exit(2)
        bench_varlen(args)
        return
    if args.decode:
        if args.gpus != 1:
            print("bench.py measures one GPU only; run with --gpus 1", file=sys.stderr)
            sys.exit(2)
        bench_decode(args)
        return
    if args.backward:
        if args.gpus != 1:
            print("bench.py measures one GPU only; run with --gpus 1", file=sys.stderr)
            sys.exit(2)
        bench_backward(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the (batch, head) streams are independent, so "
              "a multi-GPU run is one of these per GPU with no communication; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_sequence_chunked_amd import chunk_fwd, chunk_fwd_segmented, segmented_workspace_size
    from linear_attention_sequence_chunked_amd.workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, H, K, V, C = w.B, w.T, w.H, w.K, w.V, w.chunk
    nsets = 3
    cpu_sets = [workload_inputs(w, seed=w.seed + 1000 * i) for i in range(nsets)]
    sets = [{n: (t.to(dev) if t is not None else None) for n, t in s.items()} for s in cpu_sets]
    outs = [torch.empty(B, T, H, V, dtype=w.dtype, device=dev) for _ in range(nsets)]
    states = [torch.empty(B, H, V, K, dtype=torch.float32, device=dev) for _ in range(nsets)]

    seg_ws = None
    if args.segments > 1:
        seg_ws = torch.empty(segmented_workspace_size(B, T, H, K, V, C, args.segments),
                             dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % nsets]
        if seg_ws is None:
            chunk_fwd(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["initial_state"], chunk=C,
                      out=outs[i % nsets], final_state=states[i % nsets])
        else:
            chunk_fwd_segmented(s["q"], s["k"], s["v"], s["alpha"], s["beta"], s["initial_state"],
                                chunk=C, segments=args.segments, out=outs[i % nsets],
                                final_state=states[i % nsets], workspace=seg_ws)

    # correctness gate on input set 0
    gate = None
    if not args.no_gate:
        import oracle
        step(0)
        torch.cuda.synchronize()
        c = cpu_sets[0]
        ro, rs = oracle.fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["initial_state"])
        eo = float(np.linalg.norm(outs[0].double().cpu().numpy() - ro) / np.linalg.norm(ro))
        es = float(np.linalg.norm(states[0].double().cpu().numpy() - rs) / np.linalg.norm(rs))
        tol = 2e-2 if w.dtype == torch.bfloat16 else 1e-5
        reps, same = replay_check(lambda: step(0), [outs[0], states[0]])
        gate = {"rel_l2_o": eo, "rel_l2_final_state": es, "tol": tol, "replays_bitwise_equal": same,
                "replays": reps}
        if not (eo <= tol and es <= tol and same):
            print("correctness gate failed: %s" % json.dumps(gate), file=sys.stderr)
            sys.exit(1)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)   # the stream the kernel is launched on
    total_ms, per_launch = time_steps(step, args.steps, stream)
    ms_per_step = total_ms / args.steps
    kern_ms = ms_per_step
    pcts = {"p10": float(np.percentile(per_launch, 10)), "p50": float(np.percentile(per_launch, 50)),
            "p90": float(np.percentile(per_launch, 90))}

    tokens = B * T
    value = tokens / (ms_per_step / 1e3)
    abytes = algorithmic_bytes(B, T, H, K, V, esz=2 if w.dtype == torch.bfloat16 else 4,
                               with_s0=w.s0_std is not None)
    aflops = algorithmic_flops(B, T, H, K, V, C)
    tflops_tile = tile_flops(B, T, H, K, V, C)
    peak = BF16_PEAK_TFLOPS if w.dtype == torch.bfloat16 else F32_PEAK_TFLOPS
    achieved_gbs = abytes / (kern_ms / 1e3) / 1e9
    traffic = measured_traffic() if args.workload == "train_bf16" else None
    tflops = aflops / (kern_ms / 1e3) / 1e12
    xflops = None
    if w.dtype == torch.bfloat16 and args.segments == 1 and K in (32, 64, 128) and C in (32, 64):
        vs = 32 if (V >= 32 and B * H * (V // 32) >= 192) else 16
        xflops = executed_mfma_flops(B, T, H, K, V, C, vs)
    copy_gbs = copy_bandwidth_gbs()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        c = cpu_sets[0]
        threads = oracle.default_threads()
        used = min(threads, B * H)
        # the whole workload: every (b, h) stream over all T tokens
        t0 = time.perf_counter()
        oracle.fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["initial_state"], nthreads=used)
        dt = time.perf_counter() - t0
        # one core on a sample of the streams, for a per-core rate
        ns1 = min(4, B * H) if B * H >= 4 else B * H
        sl = lambda x: None if x is None else x.reshape(1, T, B * H, *x.shape[3:])[:, :, :ns1].contiguous() \
            if x.dim() == 4 else x.reshape(1, T, B * H)[:, :, :ns1].contiguous()
        q1 = c["q"].permute(1, 0, 2, 3).reshape(T, B * H, K)[:, :ns1].reshape(1, T, ns1, K)
        k1 = c["k"].permute(1, 0, 2, 3).reshape(T, B * H, K)[:, :ns1].reshape(1, T, ns1, K)
        v1 = c["v"].permute(1, 0, 2, 3).reshape(T, B * H, V)[:, :ns1].reshape(1, T, ns1, V)
        a1 = c["alpha"].permute(1, 0, 2).reshape(T, B * H)[:, :ns1].reshape(1, T, ns1)
        b1 = c["beta"].permute(1, 0, 2).reshape(T, B * H)[:, :ns1].reshape(1, T, ns1)
        t1 = time.perf_counter()
        oracle.fwd(q1, k1, v1, a1, b1, None, nthreads=1)
        dt1 = time.perf_counter() - t1
        flop_tok = 8.0 * K * V     # fp64 FLOPs per token-head of the token loop
        cpu = {"value": tokens / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
               "sample": "whole workload (all %d streams x %d tokens), fp64 token loop, %.2f s"
                         % (B * H, T, dt),
               "gflops_fp64": flop_tok * B * T * H / dt / 1e9,
               "one_core": {"streams": ns1, "seconds": dt1,
                            "token_heads_per_s": ns1 * T / dt1},
               "cpu_model": cpu_model()}

    # The bound is the roof the arithmetic intensity reaches first: bf16 inputs
    # (134 FLOP/B at d = 128) sit below the bf16 ridge (2.5 PFLOP/s / 8 TB/s =
    # 312 FLOP/B) and are HBM-bound; float32 inputs move twice the bytes but run
    # on the fp32 matrix cores, whose ridge (157.3 TFLOP/s / 8 TB/s = 19.7 FLOP/B)
    # they exceed, so their roof is the fp32 MFMA peak.
    roof = pick_roof(aflops, abytes, kern_ms, peak)
    roof.update({"traffic": traffic, "kernel_ms": kern_ms,
                 "kernel_ms_source": "mean over the timed region (calls back to back)",
                 "kernel_ms_pct": pcts, "kernel_ms_pct_launches": int(per_launch.size),
                 "algorithmic_bytes": abytes,
                 "arithmetic_intensity": aflops / abytes,
                 "copy_gbs": copy_gbs, "frac_of_copy": achieved_gbs / copy_gbs})

    # the headline metric names the training shape; other workloads and the
    # segment-parallel call get a metric that names what was timed
    if w.name == "train_bf16" and args.segments == 1:
        metric = METRIC
    else:
        metric = "GDN chunk fwd%s tokens/s at B%d\u00b7T%d\u00b7H%d\u00b7d%d" % (
            " (segment-parallel, P = %d)" % args.segments if args.segments > 1 else "", B, T, H, K)
    line = {
        "metric": metric,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d T=%d H=%d K=%d V=%d chunk=%d, inputs resident in HBM, "
                               "3 rotating input sets%s" % (w.name, B, T, H, K, V, C,
                                                            ", %d segments per sequence" % args.segments
                                                            if args.segments > 1 else ""),
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": K,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "mfma": {"tflops_algorithmic": tflops, "peak_tflops": peak,
                 "peak_dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
                 "frac": tflops / peak, "algorithmic_flops": aflops,
                 "tile_flops": tflops_tile,
                 "tflops_tile": tflops_tile / (kern_ms / 1e3) / 1e12,
                 "frac_tile": tflops_tile / (kern_ms / 1e3) / 1e12 / peak,
                 "executed_flops": xflops,
                 "tflops_executed": xflops / (kern_ms / 1e3) / 1e12 if xflops else None,
                 "frac_executed": xflops / (kern_ms / 1e3) / 1e12 / peak if xflops else None},
        "cpu_baseline": cpu,
        "gate": gate,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
