#!/usr/bin/env python3
"""Throughput of one GPU's share of a tensor-parallel FFN sub-layer on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--headline-only] [--reduce-only] [--copy-calibration]
    python bench.py --summarize-{profiles,reduce-traffic,attn-profile,sweep,tile-sweep} ...
                    (write profiles/*.md from rocprofv3 output)

Headline workload (one "step"): the FFN shard of the hidden-size sweep's
largest point, t=1 (the TP:1 end of the throughput-vs-hidden-size chart):
hidden 22528, ffn 90112, 2048 tokens, shard 0 of 1, bf16 inputs from the
seeded generator (seed 311: X ~ N(0,1), W1, W2 ~ N(0, 0.02^2)), fp32
accumulation, fp32 output:
    tp_ffn_shard: Z = X W1, GeLU in the epilogue, Y = GeLU(Z) W2.
value = algorithmic FFN FLOPs of the shard (4*M*h*f/t) / median time of one
call (HIP events on the stream the call is launched on).  Every timed row
starts after about 0.1 s of the same work, untimed, so that the GPU has left
its idle clock state, then W warmup calls.

The same run times, under "rows":
  * sweep: all 44 points of hidden 2048..22528 x t in {1,2,4,8} (2048
    tokens, shard 0, device-seeded inputs), each next to the same shard
    through torch (hipBLASLt GEMMs and a separate exact-erf GeLU kernel);
  * ffn_step_h4096_t8: the FFN sub-layer of shard 3 of 8 at hidden 4096,
    ffn 16384, 4096 tokens, bf16 partial, then the reduce of the 8 partials
    plus the residual (fp32 out); the other seven partials are computed once
    before timing and stand for what the peers would contribute;
  * partial_reduce_t8_h4096 / partial_reduce_t4_h12288: the reduce alone at
    those two shapes with the calls rotating over 3 buffer sets of 369 MB /
    1.41 GB each (more than the 256 MB Infinity Cache), so it reads HBM;
    per-call event times (median, min) and, for "gbs", the time per call of
    back-to-back calls between one pair of events (a 60 us kernel between
    its own events also carries the events' overhead);
  * partial_reduce_slice: one row block of the t=8 reduce (the
    reduce-scatter half), blocks rotating;
  * sp_reduce_layernorm_t4_h12288: the sequence-parallel sum + LayerNorm
    (4 bf16 partials + residual, fp32 x, bf16 LayerNorm out) over all rows
    of [8192, 12288], rotating over 3 buffer sets, timed like the reduce;
  * ffn_shard_reduce_fused: the t=8 step with the sum fused into the second
    GEMM's epilogue, and the same comparison at the t=4 hidden-12288 shape;
  * attn_shard: the attention shard (t=8, 8 of 64 heads of 128, hidden
    8192, 2048 tokens, causal);
  * layer: a whole layer of four shards on this GPU (hidden 12288, 96 heads,
    8192 tokens).
On rank 0 at N=1 it also times the fp64 CPU oracle on a bounded sample of the
headline workload ("cpu_baseline").  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "TP-shard FFN TFLOP/s vs hidden size (bf16, 1 GPU); % of MFMA peak"

HEADLINE = dict(tokens=2048, hidden=22528, ffn=4 * 22528, t=1, i=0, seed=300 + 22528 // 2048)
FFN = dict(tokens=4096, hidden=4096, ffn=16384, t=8, i=3, seed=2)
ATTN = dict(batch=1, seq=2048, hidden=8192, n_heads=64, head_dim=128, t=8, i=0, seed=4)
SWEEP_HIDDEN = list(range(2048, 22528 + 1, 2048))
SWEEP_T = (1, 2, 4, 8)


def _tag(p):
    return f"h{p['hidden']}_t{p['t']}"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", f"traffic_ffn_shard_{_tag(HEADLINE)}.json")


def ffn_flops(M, h, f, t):
    return 4.0 * M * h * f / t


def attn_flops(batch, seq, hidden, n_heads, head_dim, t):
    nl = n_heads // t
    S = seq
    qkv = 2.0 * batch * S * hidden * 3 * nl * head_dim
    core = 4.0 * head_dim * (S * (S + 1) / 2) * nl * batch      # causal pairs only
    out = 2.0 * batch * S * nl * head_dim * hidden
    return qkv + core + out


def reduce_bytes(t, rows, cols, pb=2, rb=2, ob=4):
    return (t * pb + rb + ob) * rows * cols


def src_hash(*names):
    """Hash of the code in csrc/ files: `//` comments, blank lines and
    surrounding whitespace are dropped, so editing comments keeps the hash."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_shards_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per headline FFN-shard call from the committed rocprofv3
    counter runs, or None when the kernels changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != src_hash("gemm.hip"):
        return None
    return rec.get("traffic_bytes")


def dev_tensor(np_arr, dtype):
    import numpy as np
    import torch
    from attention_shards_amd import synthetic as syn
    if dtype == syn.BF16:
        return torch.from_numpy(np.ascontiguousarray(np_arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(np_arr)).cuda()


def settle(fn, seconds=0.1):
    """Run fn untimed for about `seconds` of wall time.  An idle MI355X needs
    about 10 ms of sustained work to leave its low clock state (the first 50
    FFN steps after an idle second run ~35% slower than the rest), so every
    timed row starts from a settled clock; W warmup calls follow."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def time_calls(fn, steps, warmup):
    """Per-call durations in ms: HIP events recorded on the current stream
    (the stream the binding launches on) around each of `steps` calls."""
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def stats(ms):
    return {"median_ms": round(statistics.median(ms), 5), "min_ms": round(min(ms), 5),
            "mean_ms": round(statistics.mean(ms), 5)}


def time_batched(fn, steps, warmup):
    """Milliseconds per call of `steps` back-to-back calls between one pair of
    events, for calls shorter than the host's time to issue them: a GPU spin
    of about 10 ms holds the stream while the host enqueues all of them, so
    the events time the kernels, not the Python binding."""
    import torch
    settle(fn)
    for _ in range(warmup):
        fn()
    steps = min(steps, 200)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def device_info():
    """Name, compute units, the maximum shader and memory clocks the device
    reports, and the HIP / ROCm versions (the clock the GEMMs run at under
    load is measured with counters: profiles/counters_mfma_clock.md)."""
    import ctypes
    import torch
    prop = torch.cuda.get_device_properties(0)
    info = {"name": torch.cuda.get_device_name(0), "compute_units": prop.multi_processor_count,
            "hip": torch.version.hip}
    try:   # hipDeviceGetAttribute: hipDeviceAttributeClockRate = 5, MemoryClockRate = 60 (kHz)
        hip = ctypes.CDLL("libamdhip64.so")
        for key, attr in (("max_sclk_mhz", 5), ("max_mclk_mhz", 60)):
            v = ctypes.c_int(0)
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, torch.cuda.current_device()) == 0:
                info[key] = round(v.value / 1000)
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    return info


def host_info():
    """CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def headline_inputs():
    """The headline shard's inputs from the seeded generator (the same bytes
    the sweep parity test checks at this point)."""
    from attention_shards_amd import synthetic as syn
    p = HEADLINE
    return syn.make_ffn_inputs(p["seed"], p["tokens"], p["hidden"], p["ffn"], syn.BF16)


def cpu_baseline(d, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the headline
    shard: blocks of 256 token rows times the first of eight column blocks
    of W1 (and the matching rows of W2), repeated for about `budget_s`."""
    import numpy as np
    import oracle
    from attention_shards_amd import synthetic as syn
    model, cores = host_info()
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        blas = None
    p = HEADLINE
    cols = syn.column_slice(p["ffn"], 0, 8)
    W1b = syn.to_f64(d["W1"][:, cols], syn.BF16)
    W2b = syn.to_f64(d["W2"][cols, :], syn.BF16)
    rows_done, block = 0, 256
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        r0 = rows_done % p["tokens"]
        Xb = syn.to_f64(d["X"][r0:r0 + block], syn.BF16)
        oracle.ffn_shard(Xb, W1b, W2b)
        rows_done += Xb.shape[0]
    dt = time.perf_counter() - t0
    fl = 4.0 * rows_done * p["hidden"] * (cols.stop - cols.start)
    used = blas if blas else cores
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(used),
            "kind": "oracle", "cpu_model": model, "cores_available": cores,
            "sample": f"{rows_done} token rows (256-row blocks over the {p['tokens']}) x ffn "
                      f"columns {cols.start}..{cols.stop - 1} of {p['ffn']} (1/8 of the shard) "
                      f"of the hidden-{p['hidden']} t=1 FFN shard, fp64 numpy "
                      f"({used} BLAS threads), {dt:.1f} s; extrapolated full shard "
                      f"{ffn_flops(p['tokens'], p['hidden'], p['ffn'], 1) / (fl / dt):.0f} s"}


def sweep_rows(steps, warmup, with_torch=True, log=None):
    """All 44 sweep points, timing only (device-seeded inputs; parity of
    every point is in the tests)."""
    import torch
    from attention_shards_amd import binding as B
    g = torch.Generator(device="cuda")
    out = []
    for h in SWEEP_HIDDEN:
        g.manual_seed(300 + h // 2048)
        f = 4 * h
        X = torch.randn(2048, h, device="cuda", generator=g).to(torch.bfloat16)
        W1 = (torch.randn(h, f, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        W2 = (torch.randn(f, h, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        Y = torch.empty(2048, h, device="cuda")
        for t in SWEEP_T:
            fs = f // t
            W1_0, W2_0 = W1[:, :fs], W2[:fs]
            ws = torch.empty(B.tp_ffn_shard_workspace_bytes(2048, h, f, t, B.TP_BF16),
                             dtype=torch.uint8, device="cuda")
            ms = time_calls(lambda: B.tp_ffn_shard(X, W1_0, W2_0, Y, 0, t, workspace=ws),
                            steps, warmup)
            fl = ffn_flops(2048, h, f, t)
            med = statistics.median(ms)
            rec = {"hidden": h, "t": t, **stats(ms),
                   "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                   "frac_peak": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
            if with_torch:
                W1c = W1_0.contiguous()
                tms = statistics.median(time_calls(
                    lambda: torch.nn.functional.gelu(X @ W1c) @ W2_0, steps, warmup))
                rec["torch_median_ms"] = round(tms, 5)
                rec["torch_tflops"] = round(fl / (tms * 1e-3) / 1e12, 1)
                del W1c
            out.append(rec)
            if log:
                log(json.dumps(rec))
            del ws
        del X, W1, W2, Y
        torch.cuda.empty_cache()
    return out


def reduce_rotated(t, rows, cols, steps, warmup, nsets=3):
    """tp_partial_reduce of t bf16 partials plus a bf16 residual into an fp32
    output, the calls rotating over `nsets` buffer sets (device-generated
    values), so every call reads its inputs from HBM, not the cache."""
    import torch
    from attention_shards_amd import binding as B
    g = torch.Generator(device="cuda").manual_seed(7 + t)
    sets = []
    for _ in range(nsets):
        parts = [torch.randn(rows, cols, device="cuda", generator=g).to(torch.bfloat16)
                 for _ in range(t)]
        R = torch.randn(rows, cols, device="cuda", generator=g).to(torch.bfloat16)
        out = torch.empty(rows, cols, device="cuda")
        sets.append((parts, R, out))
    nxt = [0]

    def call():
        parts, R, out = sets[nxt[0] % nsets]
        nxt[0] += 1
        B.tp_partial_reduce(parts, R, out)

    ms = time_calls(call, steps, warmup)
    batched = time_batched(call, steps, warmup)
    by = reduce_bytes(t, rows, cols)
    med = statistics.median(ms)
    del sets
    torch.cuda.empty_cache()
    return {"t": t, "rows": rows, "cols": cols, "dtypes": "bf16 partials, bf16 residual, fp32 out",
            "buffer_sets": nsets, "bytes_per_set": by, **stats(ms), "bytes": by,
            "batched_ms": round(batched, 5),
            "gbs": round(by / (batched * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(by / (batched * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "gbs_per_call_events": round(by / (med * 1e-3) / 1e9, 1), "bound": "hbm"}


def sp_layernorm_rotated(t, rows, cols, steps, warmup, nsets=3):
    """tp_sp_reduce_layernorm over all rows (one call = every row block):
    t bf16 partials + bf16 residual in, fp32 x and bf16 LayerNorm out, the
    calls rotating over `nsets` buffer sets (device-generated values)."""
    import torch
    from attention_shards_amd import binding as B
    g = torch.Generator(device="cuda").manual_seed(11 + t)
    sets = []
    for _ in range(nsets):
        parts = [torch.randn(rows, cols, device="cuda", generator=g).to(torch.bfloat16)
                 for _ in range(t)]
        R = torch.randn(rows, cols, device="cuda", generator=g).to(torch.bfloat16)
        sets.append((parts, R, torch.empty(rows, cols, device="cuda"),
                     torch.empty(rows, cols, device="cuda", dtype=torch.bfloat16)))
    gamma = torch.ones(cols, device="cuda")
    beta = torch.zeros(cols, device="cuda")
    nxt = [0]

    def call():
        parts, R, x, y = sets[nxt[0] % nsets]
        nxt[0] += 1
        B.tp_sp_reduce_layernorm(parts, R, x, y, gamma, beta, 1e-5)

    ms = time_calls(call, steps, warmup)
    batched = time_batched(call, steps, warmup)
    by = (t * 2 + 2 + 4 + 2) * rows * cols
    med = statistics.median(ms)
    del sets
    torch.cuda.empty_cache()
    return {"t": t, "rows": rows, "cols": cols,
            "dtypes": "bf16 partials, bf16 residual, fp32 x, bf16 LayerNorm out",
            "buffer_sets": nsets, **stats(ms), "bytes": by, "batched_ms": round(batched, 5),
            "gbs": round(by / (batched * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(by / (batched * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "gbs_per_call_events": round(by / (med * 1e-3) / 1e9, 1), "bound": "hbm"}


def ffn_step_row(steps, warmup, fused=True):
    """FFN shard 3 of 8 at hidden 4096 (bf16 partial) + reduce of the 8
    partials and the residual; the fused variant; the reduce-scatter block."""
    import torch
    from attention_shards_amd import binding as B
    from attention_shards_amd import synthetic as syn
    p = FFN
    M, h, f, t, i = p["tokens"], p["hidden"], p["ffn"], p["t"], p["i"]
    fs = f // t
    d = syn.make_ffn_inputs(p["seed"], M, h, f, syn.BF16, residual=True)
    X, W1, W2, R = (dev_tensor(d[k], syn.BF16) for k in ("X", "W1", "W2", "R"))
    del d
    parts = [torch.empty(M, h, dtype=torch.bfloat16, device="cuda") for _ in range(t)]
    ws = torch.empty(B.tp_ffn_shard_workspace_bytes(M, h, f, t, B.TP_BF16),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(M, h, dtype=torch.float32, device="cuda")
    W1v = [W1[:, j * fs:(j + 1) * fs] for j in range(t)]
    W2v = [W2[j * fs:(j + 1) * fs] for j in range(t)]
    for j in range(t):                      # the peers' partials, once
        B.tp_ffn_shard(X, W1v[j], W2v[j], parts[j], j, t, workspace=ws)
    torch.cuda.synchronize()

    def ffn():
        B.tp_ffn_shard(X, W1v[i], W2v[i], parts[i], i, t, workspace=ws)

    def red():
        B.tp_partial_reduce(parts, R, out)

    ffn_ms = time_calls(ffn, steps, warmup)
    step_ms = time_calls(lambda: (ffn(), red()), steps, warmup)
    fl = ffn_flops(M, h, f, t)
    row = {"workload": "ffn_shard_t8_i3_h4096_f16384_tokens4096_plus_reduce8",
           "ffn": {**stats(ffn_ms),
                   "tflops": round(fl / (statistics.median(ffn_ms) * 1e-3) / 1e12, 1),
                   "frac_peak": round(fl / (statistics.median(ffn_ms) * 1e-3) / 1e12
                                      / PEAK_BF16_TFLOPS, 4)},
           "step_ffn_plus_reduce": {**stats(step_ms),
                                    "tflops": round(fl / (statistics.median(step_ms) * 1e-3)
                                                    / 1e12, 1)}}
    # The reduce-scatter half of the all-reduce on this GPU: one row block
    # (rows [j*M/t, (j+1)*M/t) of every partial) per call, j rotating over the
    # t blocks so that successive calls do not find their inputs in the
    # Infinity Cache (one block is 46 MB; all t together 369 MB).
    nxt = [0]

    def one_slice():
        B.tp_partial_reduce_slice(parts, R, out, nxt[0] % t, t)
        nxt[0] += 1

    slice_ms = time_batched(one_slice, steps, warmup)
    sb = reduce_bytes(t, M // t, h)
    row_slice = {"slices": "rotating 0..t-1", "nslices": t, "ms": round(slice_ms, 5),
                 "bytes": sb, "gbs": round(sb / (slice_ms * 1e-3) / 1e9, 1),
                 "frac_hbm_peak": round(sb / (slice_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    fused_row = None
    if fused:
        peers = [None if j == i else parts[j] for j in range(t)]
        wsf = torch.empty(B.tp_ffn_shard_reduce_workspace_bytes(M, h, f, t, B.TP_BF16),
                          dtype=torch.uint8, device="cuda")
        fu = time_calls(lambda: B.tp_ffn_shard_reduce(X, W1v[i], W2v[i], peers, R, out, i,
                                                      workspace=wsf), steps, warmup)
        fused_row = {**stats(fu), "unfused_median_ms": row["step_ffn_plus_reduce"]["median_ms"],
                     "hbm_bytes_saved": 2 * 2 * M * h}
        del peers, wsf
    del parts, W1v, W2v, W1, W2, ws, out, X, R
    torch.cuda.empty_cache()
    return row, row_slice, fused_row


def fused_vs_unfused_large(steps, warmup):
    """Timing only (device-generated inputs): the FFN step of the four-way
    layer shape (8192 tokens, hidden 12288, ffn 49152, shard 0 of 4, bf16
    partials and residual, fp32 out), unfused (tp_ffn_shard + reduce) and
    fused (tp_ffn_shard_reduce)."""
    import torch
    from attention_shards_amd import binding as B
    M, h, f, t, i = 8192, 12288, 49152, 4, 0
    fs = f // t
    g = torch.Generator(device="cuda").manual_seed(5)
    X = torch.randn(M, h, device="cuda", generator=g).to(torch.bfloat16)
    W1 = (torch.randn(h, fs, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    W2 = (torch.randn(fs, h, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    R = torch.randn(M, h, device="cuda", generator=g).to(torch.bfloat16)
    parts = [torch.randn(M, h, device="cuda", generator=g).to(torch.bfloat16) for _ in range(t)]
    out = torch.empty(M, h, device="cuda")
    ws = torch.empty(B.tp_ffn_shard_reduce_workspace_bytes(M, h, f, t, B.TP_BF16),
                     dtype=torch.uint8, device="cuda")

    def unfused():
        B.tp_ffn_shard(X, W1, W2, parts[i], i, t, workspace=ws)
        B.tp_partial_reduce(parts, R, out)

    peers = [None if j == i else parts[j] for j in range(t)]
    un = statistics.median(time_calls(unfused, steps, warmup))
    fu = statistics.median(time_calls(
        lambda: B.tp_ffn_shard_reduce(X, W1, W2, peers, R, out, i, workspace=ws), steps, warmup))
    fl = ffn_flops(M, h, f, t)
    del X, W1, W2, R, parts, peers, out, ws
    torch.cuda.empty_cache()
    return {"workload": "t4_i0_h12288_f49152_tokens8192", "unfused_median_ms": round(un, 4),
            "fused_median_ms": round(fu, 4), "unfused_tflops": round(fl / (un * 1e-3) / 1e12, 1),
            "fused_tflops": round(fl / (fu * 1e-3) / 1e12, 1)}


def attn_row(steps, warmup):
    import numpy as np
    import torch
    from attention_shards_amd import binding as B
    from attention_shards_amd import synthetic as syn
    a = ATTN
    ad = syn.make_attn_inputs(a["seed"], a["batch"], a["seq"], a["hidden"], a["n_heads"],
                              a["head_dim"])
    Xa = dev_tensor(ad["X"], syn.BF16)
    Wqkv = dev_tensor(syn.qkv_held_shard(ad["WQ"], ad["WK"], ad["WV"], a["n_heads"],
                                         a["head_dim"], a["i"], a["t"]), syn.BF16)
    Wo = dev_tensor(np.ascontiguousarray(
        ad["WO"][syn.head_slice(a["n_heads"], a["head_dim"], a["i"], a["t"]), :]), syn.BF16)
    del ad
    Ya = torch.empty(a["batch"] * a["seq"], a["hidden"], dtype=torch.float32, device="cuda")
    wsa = torch.empty(B.tp_attn_shard_workspace_bytes(a["batch"], a["seq"], a["n_heads"],
                                                      a["head_dim"], a["t"]),
                      dtype=torch.uint8, device="cuda")
    ms = time_calls(lambda: B.tp_attn_shard(Xa, Wqkv, Wo, Ya, a["batch"], a["seq"],
                                            a["n_heads"], a["head_dim"], a["i"], a["t"],
                                            True, workspace=wsa), steps, warmup)
    afl = attn_flops(a["batch"], a["seq"], a["hidden"], a["n_heads"], a["head_dim"], a["t"])
    med = statistics.median(ms)
    del Xa, Wqkv, Wo, Ya, wsa
    torch.cuda.empty_cache()
    return {"workload": "t8_i0_h8192_64x128heads_seq2048_causal", **stats(ms), "flop": afl,
            "tflops": round(afl / (med * 1e-3) / 1e12, 1),
            "frac_peak": round(afl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def layer_row(steps, warmup):
    """Timing only (device-generated inputs): a whole layer on one GPU
    (attention_shards_amd.layer.layer_forward) at the four-way layer shape:
    hidden 12288, 96 heads of 128, ffn 49152, 4 sequences of 2048 tokens,
    causal, t = 4; all four attention shards, their sum + residual, all four
    FFN shards (bf16 partials), their sum + residual."""
    import torch
    from attention_shards_amd.layer import layer_forward
    batch, seq, h, nh, d, f, t = 4, 2048, 12288, 96, 128, 49152, 4
    M, nl, fs = batch * seq, nh // t, f // t
    g = torch.Generator(device="cuda").manual_seed(6)

    def w(*shape):
        return (torch.randn(*shape, device="cuda", generator=g) * 0.02).to(torch.bfloat16)

    X = torch.randn(M, h, device="cuda", generator=g).to(torch.bfloat16)
    Wqkv = [w(h, 3 * nl * d) for _ in range(t)]
    Wo = [w(nl * d, h) for _ in range(t)]
    W1 = w(h, f)
    W1v = [W1[:, j * fs:(j + 1) * fs] for j in range(t)]
    W2v = [w(fs, h) for _ in range(t)]

    def step():
        layer_forward(X, Wqkv, Wo, W1v, W2v, batch, seq, nh, d, True,
                      ffn_partial_dtype=torch.bfloat16)

    ms = time_calls(step, steps, warmup)
    fl = t * attn_flops(batch, seq, h, nh, d, t) + t * ffn_flops(M, h, f, t)
    med = statistics.median(ms)
    del X, Wqkv, Wo, W1, W1v, W2v
    torch.cuda.empty_cache()
    return {"workload": "layer_t4_h12288_96x128heads_f49152_b4x2048_causal", **stats(ms),
            "flop": fl, "tflops": round(fl / (med * 1e-3) / 1e12, 1),
            "frac_peak": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


COPY_BYTES = 1 << 30


def copy_calibration():
    """One plain device-to-device copy of COPY_BYTES: the reference reading of
    the FETCH_SIZE / WRITE_SIZE counters for a kernel of known traffic."""
    import torch
    a = torch.ones(COPY_BYTES // 2, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def _read_counters(path):
    """{kernel: {counter: [per-dispatch values]}} and {dispatch: grid} from a
    rocprofv3 counter CSV."""
    import collections
    import csv
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names, grids = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[key[0]][key[1]] += float(r["Counter_Value"])
            names[key[0]] = r["Kernel_Name"]
            grids[key[0]] = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
    return per, names, grids


def _short(name):
    n = name.replace("tp::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0] if "<" not in n.split("(")[0] else n[:n.index(">(") + 1]


def _trace_groups(trace_csv):
    import csv
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return groups


def _copy_factors(per, names):
    def mean(counter):
        vals = [c[counter] for d, c in per.items() if "copyBuffer" in names[d] and counter in c]
        return sum(vals) / len(vals) if vals else None
    return mean


def summarize_profiles(trace_csv, fetch_csv, write_csv, cmd_stats, cmd_pmc):
    """Write profiles/kernel_stats_ffn_shard_<tag>.md, traffic_ffn_shard_<tag>.md
    and the traffic record bench.py reads, for the headline FFN shard."""
    p = HEADLINE
    tag = _tag(p)
    M, h, fs = p["tokens"], p["hidden"], p["ffn"] // p["t"]
    gemm_src = src_hash("gemm.hip")
    groups = {k: v for k, v in _trace_groups(trace_csv).items()
              if not k[0].startswith("at::") and "copyBuffer" not in k[0]}
    total_us = sum(sum(v) for v in groups.values())
    fl = ffn_flops(M, h, p["ffn"], p["t"])
    lines = [f"# Kernel durations: FFN shard t={p['t']} i={p['i']}, hidden {h}, ffn {p['ffn']}, "
             f"{M} tokens (bf16 in, fp32 out)",
             "", "Command (from the repository root, on one MI355X):", "",
             "```", cmd_stats, "```", "",
             "Per-dispatch durations from the kernel trace of the same run, grouped by kernel",
             "and number of workgroups.", "",
             "| kernel | workgroups | calls | avg us | min us | max us | share |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    avg_call = 0.0
    for (name, wgs), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {wgs} | {len(v)} | {sum(v)/len(v):.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} | {100*sum(v)/total_us:.1f}% |")
        avg_call += sum(v) / len(v)
    lines += ["", f"One tp_ffn_shard call = one dispatch of each kernel above (the K-blocking copy "
              f"of X, GEMM1 with the GeLU epilogue, GEMM2 over its tile plan): {avg_call:.1f} us "
              f"on average, {fl/1e12:.2f} TFLOP algorithmic, {fl/(avg_call*1e-6)/1e12:.0f} TFLOP/s = "
              f"{fl/(avg_call*1e-6)/1e12/PEAK_BF16_TFLOPS:.1%} of the {PEAK_BF16_TFLOPS} TFLOP/s "
              "bf16 peak.", "", f"GEMM source hash: `{gemm_src}`"]
    with open(os.path.join(ROOT, "profiles", f"kernel_stats_ffn_shard_{tag}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fe, fe_names, fe_grid = _read_counters(fetch_csv)
    wr, wr_names, wr_grid = _read_counters(write_csv)
    copy_fetch = _copy_factors(fe, fe_names)("FETCH_SIZE")
    copy_write = _copy_factors(wr, wr_names)("WRITE_SIZE")
    f_fac = (COPY_BYTES / 1024) / copy_fetch
    w_fac = (COPY_BYTES / 1024) / copy_write

    def by_kernel(per, names, grid, counter):
        out = {}
        for d, c in per.items():
            n = _short(names[d])
            if n.startswith("at::") or "copyBuffer" in n or "fillBuffer" in n or counter not in c:
                continue
            out.setdefault((n, grid[d]), []).append(c[counter])
        return {k: sum(v) / len(v) for k, v in out.items()}
    fk, wk = by_kernel(fe, fe_names, fe_grid, "FETCH_SIZE"), by_kernel(wr, wr_names, wr_grid, "WRITE_SIZE")
    table = [f"# HBM traffic per launch: FFN shard t={p['t']} i={p['i']}, hidden {h}, ffn "
             f"{p['ffn']}, {M} tokens", "",
             "Commands (from the repository root, one MI355X, one counter per run):", "",
             "```", cmd_pmc.replace("COUNTER", "FETCH_SIZE"),
             cmd_pmc.replace("COUNTER", "WRITE_SIZE"), "```", "",
             f"Calibration: a {COPY_BYTES >> 20} MiB device copy read FETCH_SIZE {copy_fetch:.0f} KiB "
             f"and WRITE_SIZE {copy_write:.0f} KiB, so the counters are scaled by "
             f"{f_fac:.3f} (fetch) and {w_fac:.3f} (write).", "",
             "| kernel | workgroups | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB read | scaled MB written |",
             "|---|---:|---:|---:|---:|---:|"]
    total = 0.0
    for key in sorted(fk, key=lambda k: -fk[k]):
        f_, w_ = fk[key], wk.get(key, 0.0)
        rb_, wb_ = f_ * 1024 * f_fac, w_ * 1024 * w_fac
        total += rb_ + wb_
        table.append(f"| `{key[0]}` | {key[1]} | {f_:.0f} | {w_:.0f} | {rb_/1e6:.1f} | {wb_/1e6:.1f} |")
    alg = 2 * (M * h + h * fs + M * fs) + 2 * (M * fs + fs * h) + 4 * M * h
    table += ["", f"Sum for one tp_ffn_shard call (one dispatch of each kernel): {total/1e6:.1f} MB "
              f"of HBM traffic; the algorithmic minimum (X, W1, GeLU(Z) written and re-read, W2, "
              f"fp32 Y) is {alg/1e6:.1f} MB ({total/alg:.2f}x).", "", f"GEMM source hash: `{gemm_src}`"]
    with open(os.path.join(ROOT, "profiles", f"traffic_ffn_shard_{tag}.md"), "w") as f:
        f.write("\n".join(table) + "\n")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"kernel_source_sha": gemm_src, "traffic_bytes": round(total),
                   "fetch_factor": f_fac, "write_factor": w_fac, "algorithmic_bytes": alg,
                   "avg_call_us_trace": round(avg_call, 2)}, f, indent=1)
    print(f"wrote profiles for {tag} (call {avg_call:.1f} us; traffic {total/1e6:.1f} MB, "
          f"algorithmic {alg/1e6:.1f} MB)")


REDUCE_SHAPES = ((8, 4096, 4096), (4, 8192, 12288))


def summarize_reduce_traffic(trace_csv, fetch_csv, write_csv, cmd_stats, cmd_pmc):
    """profiles/reduce_rotated.md: per-launch durations and HBM bytes of
    reduce_kernel at the two rotated reduce shapes (told apart by grid size)."""
    groups = _trace_groups(trace_csv)
    fe, fe_names, fe_grid = _read_counters(fetch_csv)
    wr, wr_names, wr_grid = _read_counters(write_csv)
    copy_fetch = _copy_factors(fe, fe_names)("FETCH_SIZE")
    copy_write = _copy_factors(wr, wr_names)("WRITE_SIZE")
    f_fac = (COPY_BYTES / 1024) / copy_fetch
    w_fac = (COPY_BYTES / 1024) / copy_write
    lines = ["# Partial reduce with inputs rotated over 3 buffer sets (HBM, not cache)", "",
             "Commands (from the repository root, one MI355X):", "", "```", cmd_stats,
             cmd_pmc.replace("COUNTER", "FETCH_SIZE"), cmd_pmc.replace("COUNTER", "WRITE_SIZE"),
             "```", "",
             f"Counters scaled by a {COPY_BYTES >> 20} MiB device copy: FETCH x {f_fac:.3f}, "
             f"WRITE x {w_fac:.3f}. Algorithmic bytes: t bf16 partials + bf16 residual read, "
             "fp32 output written.", "",
             "| shape | workgroups | launches | avg us | min us | algorithmic MB | TB/s (avg) | "
             "scaled MB read | scaled MB written | counted / algorithmic |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for t, rows, cols in REDUCE_SHAPES:
        wgs = (rows * cols // 8 + 255) // 256
        durs = [v for (n, g), vs in groups.items() if "reduce_kernel" in n and g == wgs for v in vs]
        fvals = [c["FETCH_SIZE"] for d, c in fe.items()
                 if "reduce_kernel" in fe_names[d] and fe_grid[d] == wgs]
        wvals = [c["WRITE_SIZE"] for d, c in wr.items()
                 if "reduce_kernel" in wr_names[d] and wr_grid[d] == wgs]
        alg = reduce_bytes(t, rows, cols)
        avg = sum(durs) / len(durs)
        rd = sum(fvals) / len(fvals) * 1024 * f_fac
        wt = sum(wvals) / len(wvals) * 1024 * w_fac
        lines.append(f"| t={t} [{rows},{cols}] | {wgs} | {len(durs)} | {avg:.1f} | {min(durs):.1f} "
                     f"| {alg/1e6:.1f} | {alg/(avg*1e-6)/1e12:.2f} | {rd/1e6:.1f} | {wt/1e6:.1f} | "
                     f"{(rd + wt)/alg:.3f} |")
    lines += ["", f"Reduce source hash: `{src_hash('reduce.hip')}`"]
    with open(os.path.join(ROOT, "profiles", "reduce_rotated_t8_h4096_t4_h12288.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/reduce_rotated_t8_h4096_t4_h12288.md")


def summarize_attn_profile(trace_csv, cmd):
    """Write profiles/kernel_stats_attn_shard_h8192_t8.md from a rocprofv3
    kernel trace of a bench run: the kernels of each tp_attn_shard call at the
    attention configuration (QKV projection, attention, merge, output
    projection), told apart from the layer row's larger calls by grid size."""
    import csv
    import statistics
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    wg = lambda r: int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    a = ATTN
    S, h, nl, d = a["batch"] * a["seq"], a["hidden"], a["n_heads"] // a["t"], a["head_dim"]
    qkv_tiles = None
    per, grids, calls = {}, {}, []
    for k in range(len(rows) - 3):
        seq = rows[k:k + 4]
        if "EpiQkv" not in seq[0]["Kernel_Name"] or "attn_fwd" not in seq[1]["Kernel_Name"]:
            continue
        if "attn_combine" not in seq[2]["Kernel_Name"] or "EpiStore" not in seq[3]["Kernel_Name"]:
            continue
        if qkv_tiles is None:
            qkv_tiles = wg(seq[0])
        if wg(seq[0]) != qkv_tiles:
            continue
        for x in seq:
            per.setdefault(_short(x["Kernel_Name"]), []).append(dur(x))
            grids[_short(x["Kernel_Name"])] = wg(x)
        calls.append((int(seq[3]["End_Timestamp"]) - int(seq[0]["Start_Timestamp"])) / 1e3)
    role = {"EpiQkv": f"QKV projection [{S} x {h}] x [{h} x {3 * nl * d}], Q and K fp16 rows, "
                      "V^T as an fp16 hi/lo pair in 16-byte runs along the sequence",
            "attn_fwd": "causal attention (query blocks of 128 or 256 x up to a chunk of 64-key tiles each)",
            "attn_combine": "merge of the split query blocks",
            "EpiStore": f"output projection [{S} x {nl * d}] x [{nl * d} x {h}] with O as "
                        "fp16 + bf8 residual (an fp16 pass and a 32x32x64 bf8 pass over W_o converted in registers), fp32 partial"}
    flop = 2 * S * h * 3 * nl * d + 4 * d * S * (S + 1) // 2 * nl + 2 * S * nl * d * h
    med = statistics.median(calls)
    lines = [f"# Kernel durations: attention shard t={a['t']} i={a['i']}, hidden {h}, "
             f"{nl} of {a['n_heads']} heads of {d}, {S} tokens, causal", "",
             "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             f"Per-dispatch durations from the kernel trace: the four kernels of each of the "
             f"{len(calls)} `tp_attn_shard` calls at this configuration (the run also times the "
             "FFN step and the layer row, whose kernels are left out).", "",
             "| kernel | role | workgroups | calls | avg us | min us | max us |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for n, v in per.items():
        r = next((t for key, t in role.items() if key in n), "")
        lines.append(f"| `{n}` | {r} | {grids[n]} | {len(v)} | {statistics.mean(v):.1f} | "
                     f"{min(v):.1f} | {max(v):.1f} |")
    lines += ["", f"One attention shard call, first kernel start to last kernel end: {med:.1f} us "
              f"median ({statistics.mean(calls):.1f} us mean); {flop/1e9:.1f} GFLOP algorithmic "
              f"work, {flop/med/1e6:.0f} TFLOP/s at the median, {flop/med/1e6/2516.6:.1%} of the "
              "bf16 MFMA peak."]
    with open(os.path.join(ROOT, "profiles", "kernel_stats_attn_shard_h8192_t8.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote attention profile ({len(calls)} calls, median {med:.1f} us)")


def summarize_layer_profile(trace_csv, cmd):
    """Write profiles/kernel_stats_layer_t4_h12288.md from a rocprofv3 kernel
    trace of `bench.py --layer-only`: every kernel of the layer row (four
    attention shards, their sum, the bf16 copy of X1, four FFN shards, their
    sum), grouped by kernel and grid, per layer call (the trace's calls
    counted by the FFN shards' GeLU products, four per layer)."""
    import csv
    import statistics
    rows = list(csv.DictReader(open(trace_csv)))
    wg = lambda r: int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    per = {}
    for r in rows:
        if "at::" in r["Kernel_Name"]:
            continue      # the row's input generation (torch kernels)
        per.setdefault((_short(r["Kernel_Name"]), wg(r)), []).append(dur(r))
    n_layers = sum(len(v) for (n, g), v in per.items() if "EpiGelu" in n) // 4
    total = sum(sum(v) for v in per.values()) / n_layers
    roles = [("EpiQkv", "attention: QKV projection [8192 x 12288] x [12288 x 9216]"),
             ("attn_fwd", "attention: causal attention, 24 local heads, 256-query blocks"),
             ("attn_combine", "attention: merge of split query blocks"),
             ("EpiStore, true, 2", "attention: output projection (O fp16 + bf8) [8192 x 3072] x [3072 x 12288]"),
             ("EpiGelu", "FFN: GEMM1 + GeLU [8192 x 12288] x [12288 x 12288]"),
             ("EpiStore", "FFN: GEMM2 [8192 x 12288] x [12288 x 12288]"),
             ("reduce_kernel<0, 1, 0", "sum: 4 fp32 attention partials + X (bf16) -> X1 (fp32)"),
             ("reduce_kernel<1, 0, 0", "sum: 4 bf16 FFN partials + X1 -> X2 (fp32)"),
             ("reduce_kernel<0, 2, 1", "copy: X1 -> bf16, the FFN input"),
             ("vt_pad", "attention: zero the V^T padding")]
    lines = ["# Kernel durations: one transformer layer on one GPU, t=4 "
             "(hidden 12288, 96 heads of 128, ffn 49152, 4 x 2048 causal tokens)", "",
             "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             f"Per-dispatch durations from the kernel trace, grouped by kernel and grid; "
             f"{n_layers} layer calls (warm-up and timed) in the trace. Per layer: the "
             "kernel's dispatches per layer call and their summed time.", "",
             "| kernel | role | workgroups | per layer | avg us | us per layer | share |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for (n, g), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        r = next((t for key, t in roles if key in n), "")
        lines.append(f"| `{n}` | {r} | {g} | {len(v) / n_layers:.0f} | "
                     f"{statistics.mean(v):.1f} | {sum(v) / n_layers:.0f} | "
                     f"{sum(v) / n_layers / total:.1%} |")
    fl = 4 * attn_flops(4, 2048, 12288, 96, 128, 4) + 4 * ffn_flops(8192, 12288, 49152, 4)
    lines += ["", f"Kernel time per layer: {total / 1e3:.2f} ms for {fl / 1e12:.2f} TFLOP "
              f"algorithmic, {fl / (total * 1e-6) / 1e12:.0f} TFLOP/s "
              f"({fl / (total * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1%} of the bf16 MFMA peak)."]
    with open(os.path.join(ROOT, "profiles", "kernel_stats_layer_t4_h12288.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote layer profile ({n_layers} layers, {total / 1e3:.2f} ms of kernels per layer)")


# First products of FFN shards (t = 1) whose tile plans are single kinds of
# one tile per CU: [tokens, ffn] -> 128x192, 256x192, 256x256 and 256x128
# tiles (X read as given: the K = 32 kinds through A pairs); K (the hidden
# size) from 2048 to 16384.
TILE_SWEEP = ((2048, 3072), (2048, 6144), (2048, 8192), (4096, 2048))
TILE_SWEEP_K = (2048, 4096, 8192, 16384)
TILE_SWEEP_CALLS = 12


def tile_sweep(k_values):
    """The workload of --summarize-tile-sweep: TILE_SWEEP_CALLS calls of the
    FFN shard (t = 1, bf16 out) per [tokens, ffn] of TILE_SWEEP and hidden in
    k_values, in that order, on device-seeded inputs."""
    import torch
    from attention_shards_amd import binding as B
    g = torch.Generator(device="cuda").manual_seed(5)
    for tok, fs in TILE_SWEEP:
        for h in k_values:
            X = torch.randn(tok, h, device="cuda", generator=g).to(torch.bfloat16)
            W1 = (torch.randn(h, fs, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
            W2 = (torch.randn(fs, h, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
            Y = torch.empty(tok, h, device="cuda", dtype=torch.bfloat16)
            ws = torch.empty(max(16, B.tp_ffn_shard_workspace_bytes(tok, h, fs, 1, B.TP_BF16)),
                             dtype=torch.uint8, device="cuda")
            for _ in range(TILE_SWEEP_CALLS):
                B.tp_ffn_shard(X, W1, W2, Y, 0, 1, workspace=ws)
            torch.cuda.synchronize()
            print(f"tile sweep: tokens {tok}, ffn {fs}, hidden {h}", file=sys.stderr, flush=True)
            del X, W1, W2, Y, ws


def _gelu_groups(rows, n_groups):
    """The first-product (GeLU epilogue) dispatches of a tile-sweep run, in
    order, cut into n_groups groups of TILE_SWEEP_CALLS (one per shape)."""
    g1 = [r for r in rows if "EpiGelu" in r["Kernel_Name"]]
    if len(g1) != n_groups * TILE_SWEEP_CALLS:
        raise SystemExit(f"expected {n_groups * TILE_SWEEP_CALLS} first-product dispatches, "
                         f"found {len(g1)}")
    return [g1[k * TILE_SWEEP_CALLS:(k + 1) * TILE_SWEEP_CALLS] for k in range(n_groups)]


def summarize_tile_sweep(trace_csv, counter_csv, cmd_trace, cmd_pmc):
    """profiles/gemm_tile_kinds_one_tile_per_cu.md from a kernel trace of
    --tile-sweep (all K) and a --pmc run of --tile-sweep --tile-sweep-k 16384:
    per tile kind, the first product's median time at each K, a straight-line
    fit time = fixed + K x per-K (the per-tile costs that do not grow with K,
    and the steady rate of the main loop), and, at K = 16384, the per-CU
    vector-memory counters (TA/TD busy, TA stalled by the L1, mean L2 read
    latency) with the matrix pipes' busy fraction at the measured clock."""
    import csv
    import numpy as np
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    groups = _gelu_groups(rows, len(TILE_SWEEP) * len(TILE_SWEEP_K))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
    ncu = 256
    lines = ["# First product of one-tile-per-CU FFN shards: fixed and steady cost per tile "
             "kind, per-CU memory-path counters", "",
             "Commands (from the repository root, on one MI355X): the kernel trace", "", "```",
             cmd_trace, "```", "", "and the counters (K = 16384 only):", "", "```", cmd_pmc,
             "```", "",
             "Each shape is the FFN shard at t = 1 ([tokens, hidden] x [hidden, ffn], GeLU "
             "epilogue, bf16 out); its tile plan is one kind with one tile per CU (256 tiles). "
             "Times: median of the last 10 of 12 dispatches of the first product. The fit "
             "time = fixed + per-K x K over K = 2048..16384 separates what each tile pays "
             "once (launch, first loads, the epilogue) from the main loop's steady rate.", "",
             "| tile (A operand) | tokens x ffn | " +
             " | ".join(f"K={k} us" for k in TILE_SWEEP_K) + " | fixed us | steady TFLOP/s |",
             "|---|---|" + "---:|" * (len(TILE_SWEEP_K) + 2)]
    kinds = {}
    for s_i, (tok, fs) in enumerate(TILE_SWEEP):
        ts = []
        for k_i, K in enumerate(TILE_SWEEP_K):
            grp = groups[s_i * len(TILE_SWEEP_K) + k_i]
            ts.append(statistics.median(dur(r) for r in grp[2:]))
        kind = _short(groups[s_i * len(TILE_SWEEP_K)][0]["Kernel_Name"])
        # <BM, BN, WM, WN, KS, NSL, Epi, AKB, NA, AP>
        prm = [x.strip() for x in kind.split("<")[1].rstrip(">").split(",")]
        tile = f"{prm[0]}x{prm[1]}"
        a_op = ("K-blocked" if prm[7] == "true" else
                "row-major, A pairs" if len(prm) > 9 and prm[9] == "true" else "row-major")
        kinds[(tok, fs)] = (tile, a_op)
        slope, fixed = np.polyfit(np.array(TILE_SWEEP_K, float), np.array(ts), 1)
        steady = 2 * tok * fs / (slope * 1e-6) / 1e12
        lines.append(f"| {tile} ({a_op}) | {tok} x {fs} | " + " | ".join(f"{t:.1f}" for t in ts) +
                     f" | {fixed:.1f} | {steady:.0f} |")
    if counter_csv:
        per, names, grids = _read_counters(counter_csv)
        ids = sorted(per, key=int)
        cgroups = _gelu_groups([{"Kernel_Name": names[d], "id": d} for d in ids], len(TILE_SWEEP))
        lines += ["", "Counters at K = 16384 (mean of the last 10 of 12 dispatches; per CU = the "
                  "summed counter / 256 CUs; cycles = `GRBM_GUI_ACTIVE` / 8 XCDs). TA: the "
                  "texture addresser, which takes every vector-memory instruction's addresses "
                  "(a 1 KiB buffer load to LDS needs at least 16 of its cycles at 64 B/clk); "
                  "TD: the data return path that writes the loads into LDS; the L1's misses go "
                  "to L2 with the latency shown. Bytes per CU-cycle: the tile's operands "
                  "(K x (rows + columns) x 2 B) over the cycles.", "",
                  "| tile (A operand) | tokens x ffn | clock GHz | operand B/CU-cycle | TA busy | "
                  "TA stalled by L1 | TD busy | mean L2 read latency (cycles) | MFMA busy at clock |",
                  "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
        trace_k = {(tok, fs): statistics.median(
            dur(r) for r in groups[s_i * len(TILE_SWEEP_K) + len(TILE_SWEEP_K) - 1][2:])
            for s_i, (tok, fs) in enumerate(TILE_SWEEP)}
        for s_i, (tok, fs) in enumerate(TILE_SWEEP):
            ds = [per[r["id"]] for r in cgroups[s_i][2:]]
            m = lambda c: sum(d.get(c, 0.0) for d in ds) / len(ds)
            cyc = m("GRBM_GUI_ACTIVE") / 8
            tile, a_op = kinds[(tok, fs)]
            bm, bn = (int(x) for x in tile.split("x"))
            clk = cyc / (trace_k[(tok, fs)] * 1e-6) / 1e9
            opb = TILE_SWEEP_K[-1] * (bm + bn) * 2 / cyc
            lat = m("TCP_TCC_READ_REQ_LATENCY_sum") / max(1.0, m("TCP_TCC_READ_REQ_sum"))
            lines.append(f"| {tile} ({a_op}) | {tok} x {fs} | {clk:.2f} | {opb:.1f} | "
                         f"{m('TA_TA_BUSY_sum') / ncu / cyc:.0%} | "
                         f"{m('TA_ADDR_STALLED_BY_TC_CYCLES_sum') / ncu / cyc:.0%} | "
                         f"{m('TD_TD_BUSY_sum') / ncu / cyc:.0%} | {lat:.0f} | "
                         f"{m('SQ_VALU_MFMA_BUSY_CYCLES') / (4 * ncu) / cyc:.0%} |")
    lines += ["", f"GEMM source hash: `{src_hash('gemm.hip')}`"]
    with open(os.path.join(ROOT, "profiles", "gemm_tile_kinds_one_tile_per_cu.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/gemm_tile_kinds_one_tile_per_cu.md")


def summarize_clock_counters(csvs, cmd):
    """profiles/counters_mfma_clock.md from one rocprofv3 run with --pmc
    SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_INSTS_LDS
    SQ_LDS_BANK_CONFLICT and --kernel-trace over the headline, the t=8 step
    and the attention shard: per kernel and grid, the duration, the MFMA busy
    fraction at the measured clock and at the nominal 2.4 GHz, and the
    shader clock implied by GRBM_GUI_ACTIVE."""
    import csv
    import statistics
    per, names, grids, dur = {}, {}, {}, {}
    for k in range(0, len(csvs) - 1, 2):   # dispatch ids are per run: prefix the run
        p_, n_, g_ = _read_counters(csvs[k])
        per.update({f"{k}:{d}": v for d, v in p_.items()})
        names.update({f"{k}:{d}": v for d, v in n_.items()})
        grids.update({f"{k}:{d}": v for d, v in g_.items()})
        for r in csv.DictReader(open(csvs[k + 1])):
            dur[f"{k}:{r['Dispatch_Id']}"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    groups = {}
    for d, c in per.items():
        n = _short(names[d])
        if n.startswith("at::") or "copyBuffer" in n or "fillBuffer" in n or d not in dur:
            continue
        groups.setdefault((n, grids[d]), []).append((dur[d], c))
    simds = 256 * 4
    lines = ["# MFMA utilisation and shader clock per kernel", "",
             "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             "Per dispatch: duration from the kernel trace of the same run; `GRBM_GUI_ACTIVE` "
             "counts GPU clock cycles while the GPU is busy, summed over the 8 XCDs, so "
             "`GRBM_GUI_ACTIVE / 8 / duration` is the shader clock the kernel ran at (memory-bound "
             "kernels read 2.1-2.3 GHz this way, against the nominal 2.4 GHz); the counting "
             "window is a few microseconds longer than the kernel, so the clock (and the busy "
             "fraction at it) is given only for kernels of a millisecond or more. "
             "`SQ_VALU_MFMA_BUSY_CYCLES` is the matrix pipes' busy cycles summed over the "
             "1024 SIMDs (a 32x32x16 bf16 MFMA keeps a SIMD's pipe busy 32 cycles), so "
             "busy / (1024 x cycles at the measured clock) is the fraction of time the matrix "
             "pipes worked, and busy / (1024 x duration x 2.4 GHz) the fraction of the nominal "
             "peak. LDS bank conflicts per LDS instruction from `SQ_LDS_BANK_CONFLICT / "
             "SQ_INSTS_LDS`. Medians over the run's dispatches of each kernel and grid.", "",
             "| kernel | workgroups | dispatches | median us | clock GHz | MFMA busy at clock | "
             "MFMA busy at 2.4 GHz | LDS conflict cycles / instr |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (n, wg), v in sorted(groups.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
        d = statistics.median(x[0] for x in v)
        clk = statistics.median(x[1].get("GRBM_GUI_ACTIVE", 0) / 8 / x[0] for x in v)
        busy = statistics.median(x[1].get("SQ_VALU_MFMA_BUSY_CYCLES", 0) for x in v)
        at_clk = busy / (simds * d * clk) if clk else 0.0
        nominal = busy / (simds * d * 2.4e9)
        ins = sum(x[1].get("SQ_INSTS_LDS", 0) for x in v)
        conf = sum(x[1].get("SQ_LDS_BANK_CONFLICT", 0) for x in v)
        # the counting window exceeds the kernel by a few us: the clock is
        # read only for kernels of a millisecond or more
        long_ = d >= 1e-3
        lines.append(f"| `{n}` | {wg} | {len(v)} | {d*1e6:.1f} | "
                     f"{(f'{clk/1e9:.2f}' if long_ else '-')} | "
                     f"{(f'{at_clk:.1%}' if long_ else '-')} | "
                     f"{nominal:.1%} | {(conf / ins if ins else 0.0):.3f} |")
    lines += ["", f"GEMM source hash: `{src_hash('gemm.hip')}`, attention: "
              f"`{src_hash('attention.hip')}`"]
    with open(os.path.join(ROOT, "profiles", "counters_mfma_clock.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/counters_mfma_clock.md")


def summarize_sweep(path, cmd):
    """Write profiles/sweep_ffn_shard_tokens2048.md from a --sweep JSONL file."""
    recs = [json.loads(line) for line in open(path) if line.strip()]
    by = {}
    for r in recs:
        by.setdefault(r["hidden"], {})[r["t"]] = r
    ts = sorted({r["t"] for r in recs})
    lines = ["# FFN shard TFLOP/s vs hidden size (2048 tokens, ffn = 4h, bf16, shard 0 of t)",
             "", "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             "Each cell: this library's `tp_ffn_shard` (GEMM1 + fused GeLU, GEMM2) / the same",
             "shard through torch (hipBLASLt GEMMs and a separate exact-erf GeLU kernel), in",
             "TFLOP/s of the algorithmic 4·M·h·f/t FLOPs; device-seeded inputs, HIP-event",
             "timing of each call. Fraction of the 2516.6 TFLOP/s bf16 peak in brackets.", "",
             "| hidden | " + " | ".join(f"t={t}" for t in ts) + " |",
             "|---:|" + "---:|" * len(ts)]
    for h in sorted(by):
        cells = []
        for t in ts:
            r = by[h].get(t)
            cells.append("" if r is None else
                         f"{r['tflops']:.0f} / {r['torch_tflops']:.0f} ({r['frac_peak']:.2f})")
        lines.append(f"| {h} | " + " | ".join(cells) + " |")
    wins = sum(1 for r in recs if r["tflops"] > r["torch_tflops"])
    best = max(recs, key=lambda r: r["tflops"])
    lines += ["", f"This library is faster at {wins} of {len(recs)} points; its best point is "
              f"{best['tflops']:.0f} TFLOP/s ({best['frac_peak']:.1%} of peak) at hidden "
              f"{best['hidden']}, t={best['t']}."]
    with open(os.path.join(ROOT, "profiles", "sweep_ffn_shard_tokens2048.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote profiles/sweep_ffn_shard_tokens2048.md ({len(recs)} points)")




def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline FFN shard only (profiling runs)")
    ap.add_argument("--reduce-only", action="store_true",
                    help="time the two rotated reduce rows only (profiling runs)")
    ap.add_argument("--attn-only", action="store_true",
                    help="time the attention shard row only (profiling runs)")
    ap.add_argument("--step-only", action="store_true",
                    help="time the t=8 hidden-4096 FFN step row only (profiling runs)")
    ap.add_argument("--layer-only", action="store_true",
                    help="time the whole-layer row only (profiling runs)")
    ap.add_argument("--summarize-layer-profile", metavar="KERNEL_TRACE_CSV", default=None)
    ap.add_argument("--summarize-clock-counters", nargs="+", metavar="CSV",
                    help="COUNTER_CSV TRACE_CSV pairs (one per run): write the per-kernel "
                         "MFMA-utilisation / clock table")
    ap.add_argument("--no-sweep-torch", action="store_true",
                    help="skip the torch (hipBLASLt) comparison at each sweep point")
    ap.add_argument("--sweep-out", metavar="JSONL", default=None,
                    help="also write the sweep records to this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (counter calibration)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="run the one-tile-per-CU first-product workload only (profiling runs)")
    ap.add_argument("--tile-sweep-k", type=int, nargs="+", default=list(TILE_SWEEP_K))
    ap.add_argument("--summarize-tile-sweep", nargs=2, metavar=("TRACE_CSV", "COUNTER_CSV"))
    ap.add_argument("--summarize-attn-profile", metavar="KERNEL_TRACE_CSV", default=None)
    ap.add_argument("--summarize-sweep", metavar="SWEEP_JSONL", default=None)
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_CSV", "FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-reduce-traffic", nargs=3,
                    metavar=("TRACE_CSV", "FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--profile-commands", nargs=2, default=["", ""],
                    metavar=("STATS_CMD", "PMC_CMD"))
    args = ap.parse_args()
    if args.summarize_tile_sweep:
        summarize_tile_sweep(*args.summarize_tile_sweep, *args.profile_commands)
        return
    if args.summarize_attn_profile:
        summarize_attn_profile(args.summarize_attn_profile, args.profile_commands[0])
        return
    if args.summarize_layer_profile:
        summarize_layer_profile(args.summarize_layer_profile, args.profile_commands[0])
        return
    if args.summarize_sweep:
        summarize_sweep(args.summarize_sweep, args.profile_commands[0])
        return
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, *args.profile_commands)
        return
    if args.summarize_clock_counters:
        summarize_clock_counters(args.summarize_clock_counters, args.profile_commands[0])
        return
    if args.summarize_reduce_traffic:
        summarize_reduce_traffic(*args.summarize_reduce_traffic, *args.profile_commands)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's shard only: this library runs on a single "
              "GPU and has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from attention_shards_amd import binding as B
    B.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    K, W = args.steps, args.warmup
    if args.copy_calibration:
        copy_calibration()
    if args.reduce_only:
        for t, rows, cols in REDUCE_SHAPES:
            log(json.dumps(reduce_rotated(t, rows, cols, K, W)))
        log(json.dumps(sp_layernorm_rotated(4, 8192, 12288, K, W)))
        return
    if args.attn_only:
        log(json.dumps(attn_row(K, W)))
        return
    if args.step_only:
        log(json.dumps(ffn_step_row(K, W, fused=False)[0]))
        return
    if args.layer_only:
        log(json.dumps(layer_row(K, W)))
        return
    if args.tile_sweep:
        tile_sweep(args.tile_sweep_k)
        return

    # ---------------- headline: the sweep's hidden-22528, t=1 FFN shard ----------------
    p = HEADLINE
    M, h, f, t, i = p["tokens"], p["hidden"], p["ffn"], p["t"], p["i"]
    log(f"headline inputs: hidden {h}, ffn {f}, {M} tokens (seed {p['seed']})")
    d = headline_inputs()
    from attention_shards_amd import synthetic as syn
    X = dev_tensor(d["X"], syn.BF16)
    W1 = dev_tensor(d["W1"], syn.BF16)
    W2 = dev_tensor(d["W2"], syn.BF16)
    Y = torch.empty(M, h, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.tp_ffn_shard_workspace_bytes(M, h, f, t, B.TP_BF16),
                     dtype=torch.uint8, device="cuda")

    def ffn():
        B.tp_ffn_shard(X, W1, W2, Y, i, t, workspace=ws)

    settle(ffn)
    for _ in range(W):
        ffn()
    torch.cuda.synchronize()
    # the K timed steps: launches only, nothing else on the stream
    t0 = time.perf_counter()
    for _ in range(K):
        ffn()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / K * 1e3
    # per-call durations: the same K steps again with events around each call
    ms = time_calls(ffn, K, 2)
    fl = ffn_flops(M, h, f, t)
    med, mean = statistics.median(ms), statistics.mean(ms)
    value = fl / (med * 1e-3) / 1e12
    log(f"headline: median {med:.4f} ms, min {min(ms):.4f} ms, {value:.1f} TFLOP/s")
    del X, W1, W2, Y, ws
    torch.cuda.empty_cache()

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64 normals: activations N(0,1), weights N(0,0.02^2))",
        "config": {"workload": f"ffn_shard_t{t}_i{i}_h{h}_f{f}_tokens{M}",
                   "tokens": M, "hidden": h, "ffn": f, "t": t, "i": i, "seed": p["seed"],
                   "in_dtype": "bf16", "out_dtype": "f32",
                   "timing": "value = FLOPs / median per-call time (HIP events)",
                   **stats(ms)},
        "roofline": {"bound": "mfma", "kernel": "tp_ffn_shard (GEMM1+GeLU, GEMM2)",
                     "achieved": round(fl / (mean * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fl / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(), "per_launch_flop": fl,
                     "avg_launch_ms": round(mean, 5)},
        "rows": {},
    }
    if not args.headline_only:
        rows = res["rows"]
        log("sweep (44 points)")
        sw = sweep_rows(max(5, K // 5), 3, with_torch=not args.no_sweep_torch, log=log)
        rows["sweep"] = sw
        if args.sweep_out:
            with open(args.sweep_out, "w") as fo:
                for r in sw:
                    fo.write(json.dumps(r) + "\n")
        rows["sweep_summary"] = {
            "points": len(sw), "min_tflops": min(r["tflops"] for r in sw),
            "max_tflops": max(r["tflops"] for r in sw),
            "points_at_or_above_60pct": sum(1 for r in sw if r["frac_peak"] >= 0.6),
            "points_faster_than_torch": sum(1 for r in sw if r["tflops"] >= r.get("torch_tflops", 0))}
        log("FFN step (t=8, hidden 4096) and reduce")
        step, sl, fused = ffn_step_row(K, W)
        rows["ffn_step_h4096_t8"] = step
        rows["partial_reduce_slice"] = sl
        for t_, r_, c_ in REDUCE_SHAPES:
            log(f"reduce rotated t={t_} [{r_},{c_}]")
            rows[f"partial_reduce_t{t_}_h{c_}"] = reduce_rotated(t_, r_, c_, K, W)
        log("sequence-parallel sum + LayerNorm t=4 [8192,12288]")
        rows["sp_reduce_layernorm_t4_h12288"] = sp_layernorm_rotated(4, 8192, 12288, K, W)
        if fused is not None:
            fused["large"] = fused_vs_unfused_large(max(5, K // 5), 3)
        rows["ffn_shard_reduce_fused"] = fused
        log("attention shard")
        rows["attn_shard"] = attn_row(K, W)
        log("layer")
        rows["layer"] = layer_row(max(3, K // 10), 2)
        rows["device"] = device_info()
    if not args.no_cpu_baseline and not args.headline_only:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
