#!/usr/bin/env python3
"""Throughput of one GPU's share of a tensor-parallel FFN sub-layer on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--sweep OUT.jsonl]
    python bench.py --summarize-{profiles,attn-profile,counters,sweep} ...
                    (write profiles/*.md from rocprofv3 output or a sweep)

Workload (one "step"): FFN shard i=3 of t=8 at hidden 4096, ffn 16384,
4096 tokens (2 sequences of 2048), bf16 inputs with fp32 accumulation:
  1. tp_ffn_shard: Z_3 = X W1_3 (W1_3 a zero-copy column view of the full W1),
     GeLU in the epilogue, Y_3 = GeLU(Z_3) W2_3 -> bf16 partial;
  2. tp_partial_reduce: out = sum of the 8 partials + residual (fp32 out).
     The other seven partials are the other shards' results, computed once
     before timing: they stand for what the peers would contribute.
value = algorithmic FFN FLOPs of the shard (4*M*h*f/t) / wall time per step.
Every timed row starts after about 0.1 s of the same work, untimed, so that
the GPU has left its idle clock state, then W warmup steps.

The same run also times, under "rows": the reduce-scatter block shard i
would own (tp_partial_reduce_slice; rows.partial_reduce_slice), the step
with the sum fused into the second GEMM's epilogue (tp_ffn_shard_reduce;
rows.ffn_shard_reduce_fused), the attention shard (t=8, 8 of 64 heads of
128, hidden 8192, 2048 tokens, causal; rows.attn_shard) and a whole layer
of four shards on this GPU (hidden 12288, 96 heads, 8192 tokens;
rows.layer).  On rank 0 at N=1 it also times the fp64 CPU oracle on a
bounded sample of the FFN workload ("cpu_baseline").  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "TP-shard FFN TFLOP/s vs hidden size (bf16, 1 GPU); % of MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ffn_shard_h4096_t8.json")

FFN = dict(tokens=4096, hidden=4096, ffn=16384, t=8, i=3, seed=2)
ATTN = dict(batch=1, seq=2048, hidden=8192, n_heads=64, head_dim=128, t=8, i=0, seed=4)


def ffn_flops(M, h, f, t):
    return 4.0 * M * h * f / t


def attn_flops(batch, seq, hidden, n_heads, head_dim, t):
    nl = n_heads // t
    S = seq
    qkv = 2.0 * batch * S * hidden * 3 * nl * head_dim
    core = 4.0 * head_dim * (S * (S + 1) / 2) * nl * batch      # causal pairs only
    out = 2.0 * batch * S * nl * head_dim * hidden
    return qkv + core + out


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
    """HBM bytes per FFN-shard call from the committed rocprofv3 counter runs,
    or None when the kernels changed since those counters were taken."""
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
    timed row starts from a settled clock; W warmup steps follow."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def time_events(fn, steps, warmup):
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
    return sum(a.elapsed_time(b) for a, b in ev) / steps


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


def cpu_baseline(d, budget_s=12.0):
    """fp64 oracle on a bounded row sample of the FFN shard workload."""
    import numpy as np
    import oracle
    from attention_shards_amd import synthetic as syn
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = 1
    p = FFN
    cols = syn.column_slice(p["ffn"], p["i"], p["t"])
    W1_i = syn.to_f64(d["W1"][:, cols], syn.BF16)
    W2_i = syn.to_f64(d["W2"][cols, :], syn.BF16)
    rows_done, block = 0, 256
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        r0 = rows_done % p["tokens"]
        Xb = syn.to_f64(d["X"][r0:r0 + block], syn.BF16)
        oracle.ffn_shard(Xb, W1_i, W2_i)
        rows_done += Xb.shape[0]
    dt = time.perf_counter() - t0
    fl = ffn_flops(rows_done, p["hidden"], p["ffn"], p["t"])
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{rows_done} token rows ({rows_done / p['tokens']:.2f} passes over the "
                      f"{p['tokens']} rows) of the FFN shard, fp64 numpy, {dt:.1f} s"}


def sweep(path, steps, warmup):
    """Hidden-size sweep h = 2048..22528 step 2048, t in {1,2,4,8}, 2048 tokens.
    Timing only (device-seeded inputs); parity of sweep points is in tests."""
    import torch
    from attention_shards_amd import binding as B
    g = torch.Generator(device="cuda")
    with open(path, "w") as out:
        for h in range(2048, 22528 + 1, 2048):
            g.manual_seed(300 + h // 2048)
            f = 4 * h
            X = torch.randn(2048, h, device="cuda", generator=g).to(torch.bfloat16)
            for t in (1, 2, 4, 8):
                fs = f // t
                W1 = (torch.randn(h, fs, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
                W2 = (torch.randn(fs, h, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
                Y = torch.empty(2048, h, device="cuda")
                ws = torch.empty(B.tp_ffn_shard_workspace_bytes(2048, h, f, t, B.TP_BF16),
                                 dtype=torch.uint8, device="cuda")
                ms = time_events(lambda: B.tp_ffn_shard(X, W1, W2, Y, 0, t, workspace=ws),
                                 steps, warmup)
                tf = ffn_flops(2048, h, f, t) / (ms * 1e-3) / 1e12
                # context: the same shard through torch (hipBLASLt GEMMs, a
                # separate exact-erf GeLU kernel, bf16 between them)
                tms = time_events(lambda: torch.nn.functional.gelu(X @ W1) @ W2, steps, warmup)
                rec = {"hidden": h, "t": t, "ms": round(ms, 5), "tflops": round(tf, 2),
                       "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                       "torch_ms": round(tms, 5),
                       "torch_tflops": round(ffn_flops(2048, h, f, t) / (tms * 1e-3) / 1e12, 2)}
                out.write(json.dumps(rec) + "\n")
                print(json.dumps(rec), file=sys.stderr, flush=True)
                del W1, W2, Y, ws
            del X
            torch.cuda.empty_cache()


COPY_BYTES = 1 << 30


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
    un_ms = time_events(unfused, steps, warmup)
    fu_ms = time_events(lambda: B.tp_ffn_shard_reduce(X, W1, W2, peers, R, out, i, workspace=ws),
                        steps, warmup)
    fl = ffn_flops(M, h, f, t)
    del X, W1, W2, R, parts, peers, out, ws
    torch.cuda.empty_cache()
    return {"workload": "t4_i0_h12288_f49152_tokens8192", "unfused_ms": round(un_ms, 4),
            "fused_ms": round(fu_ms, 4), "unfused_tflops": round(fl / (un_ms * 1e-3) / 1e12, 1),
            "fused_tflops": round(fl / (fu_ms * 1e-3) / 1e12, 1)}


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

    ms = time_events(step, steps, warmup)
    fl = t * attn_flops(batch, seq, h, nh, d, t) + t * ffn_flops(M, h, f, t)
    del X, Wqkv, Wo, W1, W1v, W2v
    torch.cuda.empty_cache()
    return {"workload": "layer_t4_h12288_96x128heads_f49152_b4x2048_causal",
            "ms": round(ms, 3), "flop": fl, "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "frac_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


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
    """{kernel: {counter: [per-dispatch values]}} from a rocprofv3 counter CSV."""
    import collections
    import csv
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[key[0]][key[1]] += float(r["Counter_Value"])
            names[key[0]] = r["Kernel_Name"]
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for disp, counters in per.items():
        for c, v in counters.items():
            out[names[disp]][c].append(v)
    return out


def _short(name):
    n = name.replace("tp::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0] if "<" not in n.split("(")[0] else n[:n.index(">(") + 1]


def summarize_profiles(stats_csv, fetch_csv, write_csv, cmd_stats, cmd_pmc):
    """Write profiles/*.md and the traffic record bench.py reads."""
    import csv
    gemm_src = src_hash("gemm.hip")
    # Per-dispatch durations from the kernel trace next to the stats file,
    # grouped by kernel and grid size (the bench launches the reduce kernel
    # both over whole tensors and over row blocks).
    trace_csv = stats_csv.replace("kernel_stats", "kernel_trace")
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total_us = sum(sum(v) for v in groups.values())
    lines = ["# Kernel durations: FFN shard t=8 i=3, hidden 4096, ffn 16384, 4096 tokens",
             "", "Command (from the repository root, on one MI355X):", "",
             "```", cmd_stats, "```", "",
             "Per-dispatch durations from the kernel trace of the same run, grouped by kernel",
             "and number of workgroups (the partial reduce runs over the whole 4096 x 4096",
             "output and, in the block row, over one eighth of its rows).", "",
             "| kernel | workgroups | calls | avg us | min us | max us | share |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for (name, wgs), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {wgs} | {len(v)} | {sum(v)/len(v):.1f} | {min(v):.1f} | "
                     f"{max(v):.1f} | {100*sum(v)/total_us:.1f}% |")
    with open(os.path.join(ROOT, "profiles", "kernel_stats_ffn_shard_h4096_t8.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fe, wr = _read_counters(fetch_csv), _read_counters(write_csv)

    def mean(d, kname, c):
        vals = [v for k, cs in d.items() if kname in k for v in cs.get(c, [])]
        return sum(vals) / len(vals) if vals else None
    copy_fetch = mean(fe, "copyBuffer", "FETCH_SIZE")
    copy_write = mean(wr, "copyBuffer", "WRITE_SIZE")
    f_fac = (COPY_BYTES / 1024) / copy_fetch
    w_fac = (COPY_BYTES / 1024) / copy_write
    p = FFN
    M, h, fs = p["tokens"], p["hidden"], p["ffn"] // p["t"]
    kernels = {"GEMM1 + GeLU": "EpiGelu", "GEMM2": "EpiStore"}
    table = ["# HBM traffic per launch: FFN shard t=8 i=3, hidden 4096, ffn 16384, 4096 tokens",
             "", "Commands (from the repository root, one MI355X, one counter per run):", "",
             "```", cmd_pmc.replace("COUNTER", "FETCH_SIZE"), cmd_pmc.replace("COUNTER", "WRITE_SIZE"),
             "```", "",
             f"Calibration: a {COPY_BYTES >> 20} MiB device copy read FETCH_SIZE {copy_fetch:.0f} KiB "
             f"and WRITE_SIZE {copy_write:.0f} KiB, so the counters are scaled by "
             f"{f_fac:.3f} (fetch) and {w_fac:.3f} (write).", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB read | scaled MB written |",
             "|---|---:|---:|---:|---:|"]
    total = 0.0
    for label, tag in kernels.items():
        fk = mean(fe, tag, "FETCH_SIZE")
        wk = mean(wr, tag, "WRITE_SIZE")
        rb_, wb_ = fk * 1024 * f_fac, wk * 1024 * w_fac
        total += rb_ + wb_
        table.append(f"| {label} | {fk:.0f} | {wk:.0f} | {rb_/1e6:.1f} | {wb_/1e6:.1f} |")
    alg = 2 * (M * h + h * fs + M * fs) + 2 * (M * fs + fs * h) + 2 * M * h
    table += ["", f"Sum for one tp_ffn_shard call: {total/1e6:.1f} MB of HBM traffic; the "
              f"algorithmic minimum (X, W1_i, GeLU(Z) written and re-read, W2_i, bf16 Y) is "
              f"{alg/1e6:.1f} MB.", "", f"GEMM source hash: `{gemm_src}`"]
    with open(os.path.join(ROOT, "profiles", "traffic_ffn_shard_h4096_t8.md"), "w") as f:
        f.write("\n".join(table) + "\n")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"kernel_source_sha": gemm_src, "traffic_bytes": round(total),
                   "fetch_factor": f_fac, "write_factor": w_fac,
                   "algorithmic_bytes": alg}, f, indent=1)
    print(f"wrote profiles (traffic {total/1e6:.1f} MB per call, algorithmic {alg/1e6:.1f} MB)")


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
    role = {"EpiQkv": f"QKV projection [{S} x {h}] x [{h} x {3 * nl * d}], Q/K hi/lo rows, "
                      "V^T hi/lo as 16-byte runs along the sequence",
            "attn_fwd": "causal attention (query blocks of 128 or 256 x up to a chunk of 64-key tiles each)",
            "attn_combine": "merge of the split query blocks",
            "EpiStore": f"output projection [{S} x {2 * nl * d} (O hi, O lo)] x [{nl * d} x {h}], "
                        "fp32 partial"}
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


def summarize_counters(counter_csv, cmd):
    """Write profiles/counters_mfma_lds_ffn_attn.md from a rocprofv3 --pmc run
    of MfmaUtil, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_LDS_BANK_CONFLICT
    and SQ_INSTS_LDS over a bench run: per kernel (and grid size), the mean of
    rocprofv3's MfmaUtil and the LDS bank-conflict cycles per LDS instruction."""
    import csv
    per = {}
    for r in csv.DictReader(open(counter_csv)):
        d = per.setdefault(r["Dispatch_Id"], {"name": _short(r["Kernel_Name"]),
                                              "wg": int(r["Grid_Size"]) // int(r["Workgroup_Size"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    groups = {}
    for d in per.values():
        if d["name"].startswith("at::") or "copyBuffer" in d["name"]:
            continue
        groups.setdefault((d["name"], d["wg"]), []).append(d)
    lines = ["# MFMA utilisation and LDS bank conflicts per kernel (FFN step and attention shard)",
             "", "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             "`MfmaUtil` is rocprofv3's derived metric: the summed per-SIMD "
             "`SQ_VALU_MFMA_BUSY_CYCLES` over `GRBM_GUI_ACTIVE` times the SIMD count, in "
             "percent (the GPU-busy cycles count at the reference clock, so it is close to the "
             "fraction of the nominal MFMA peak). Conflicts: `SQ_LDS_BANK_CONFLICT` cycles per "
             "`SQ_INSTS_LDS` instruction. Means over the run's dispatches of each kernel and "
             "grid size.", "",
             "| kernel | workgroups | dispatches | MfmaUtil % | LDS conflict cycles / LDS instr |",
             "|---|---:|---:|---:|---:|"]
    for (name, wg), ds in sorted(groups.items(), key=lambda kv: -sum(x.get("GRBM_GUI_ACTIVE", 0)
                                                                      for x in kv[1])):
        mu = sum(x.get("MfmaUtil", 0.0) for x in ds) / len(ds)
        conf = sum(x.get("SQ_LDS_BANK_CONFLICT", 0.0) for x in ds)
        insts = sum(x.get("SQ_INSTS_LDS", 0.0) for x in ds)
        lines.append(f"| `{name}` | {wg} | {len(ds)} | {mu:.1f} | "
                     f"{(conf / insts if insts else 0.0):.3f} |")
    with open(os.path.join(ROOT, "profiles", "counters_mfma_lds_ffn_attn.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote profiles/counters_mfma_lds_ffn_attn.md ({len(per)} dispatches)")


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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the attention row (profiling runs of the FFN step)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused-step rows (profiling runs of the FFN step)")
    ap.add_argument("--sweep", metavar="OUT_JSONL", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (counter calibration)")
    ap.add_argument("--summarize-counters", metavar="COUNTER_CSV", default=None,
                    help="write the MFMA-utilisation / LDS-conflict table from a --pmc run")
    ap.add_argument("--summarize-attn-profile", metavar="KERNEL_TRACE_CSV", default=None,
                    help="write the attention-shard kernel table from a rocprofv3 trace")
    ap.add_argument("--summarize-sweep", metavar="SWEEP_JSONL", default=None,
                    help="write profiles/sweep_*.md from a --sweep output and exit")
    ap.add_argument("--summarize-profiles", nargs=3,
                    metavar=("STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/ summaries from rocprofv3 CSVs and exit")
    ap.add_argument("--profile-commands", nargs=2, default=["", ""],
                    metavar=("STATS_CMD", "PMC_CMD"))
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.profile_commands[0])
        return
    if args.summarize_attn_profile:
        summarize_attn_profile(args.summarize_attn_profile, args.profile_commands[0])
        return
    if args.summarize_sweep:
        summarize_sweep(args.summarize_sweep, args.profile_commands[0])
        return
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, *args.profile_commands)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's shard only: this library runs on a single "
              "GPU and has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from attention_shards_amd import binding as B
    from attention_shards_amd import synthetic as syn
    B.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration()
    if args.sweep:
        sweep(args.sweep, max(5, args.steps // 5), 3)

    # ---------------- FFN sub-layer step ----------------
    p = FFN
    M, h, f, t, i = p["tokens"], p["hidden"], p["ffn"], p["t"], p["i"]
    fs = f // t
    d = syn.make_ffn_inputs(p["seed"], M, h, f, syn.BF16, residual=True)
    X = dev_tensor(d["X"], syn.BF16)
    W1 = dev_tensor(d["W1"], syn.BF16)
    W2 = dev_tensor(d["W2"], syn.BF16)
    R = dev_tensor(d["R"], syn.BF16)
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

    settle(lambda: (ffn(), red()))
    for _ in range(args.warmup):
        ffn()
        red()
    torch.cuda.synchronize()
    # The K timed steps: launches only, nothing else on the stream.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ffn()
        red()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    # Per-call durations: the same K steps again with events around each call.
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
          for _ in range(args.steps)]
    for e0, e1, e2 in ev:
        e0.record()
        ffn()
        e1.record()
        red()
        e2.record()
    torch.cuda.synchronize()
    ffn_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    red_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
    fl = ffn_flops(M, h, f, t)
    value = fl / (ms_step * 1e-3) / 1e12
    ffn_tf = fl / (ffn_ms * 1e-3) / 1e12
    red_bytes = (t * 2 + 2 + 4) * M * h
    red_gbs = red_bytes / (red_ms * 1e-3) / 1e9

    # The reduce-scatter half of the all-reduce on this GPU: one row block
    # (rows [j*M/t, (j+1)*M/t) of every partial) per call, j rotating over the
    # t blocks so that successive calls do not find their inputs in the
    # Infinity Cache (one block is 46 MB; all t together 369 MB).
    nxt = [0]

    def one_slice():
        B.tp_partial_reduce_slice(parts, R, out, nxt[0] % t, t)
        nxt[0] += 1

    slice_ms = time_batched(one_slice, args.steps, args.warmup)
    slice_bytes = (t * 2 + 2 + 4) * (M // t) * h
    slice_row = {"slices": "rotating 0..t-1", "nslices": t, "ms": round(slice_ms, 5),
                 "bytes": slice_bytes,
                 "gbs": round(slice_bytes / (slice_ms * 1e-3) / 1e9, 1),
                 "frac_hbm_peak": round(slice_bytes / (slice_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    # The same step with the sum fused into GEMM2's epilogue: this shard's
    # partial is added from the accumulators and never stored or re-read.
    fused_row = None
    if not args.no_fused:
        peers = [None if j == i else parts[j] for j in range(t)]
        wsf = torch.empty(B.tp_ffn_shard_reduce_workspace_bytes(M, h, f, t, B.TP_BF16),
                          dtype=torch.uint8, device="cuda")
        fused_ms = time_events(lambda: B.tp_ffn_shard_reduce(X, W1v[i], W2v[i], peers, R, out,
                                                             i, workspace=wsf),
                               args.steps, args.warmup)
        fused_row = {"ms": round(fused_ms, 5),
                     "tflops": round(fl / (fused_ms * 1e-3) / 1e12, 2),
                     "unfused_ms": round(ffn_ms + red_ms, 5),
                     "hbm_bytes_saved": 2 * 2 * M * h}
        del peers, wsf
    del parts, W1v, W2v, W1, W2, ws, out
    torch.cuda.empty_cache()
    if fused_row is not None:
        fused_row["large"] = fused_vs_unfused_large(max(5, args.steps // 5), 3)

    # ---------------- attention shard ----------------
    attn_row = None
    if not args.no_attention:
        a = ATTN
        ad = syn.make_attn_inputs(a["seed"], a["batch"], a["seq"], a["hidden"], a["n_heads"],
                                  a["head_dim"])
        nl = a["n_heads"] // a["t"]
        Xa = dev_tensor(ad["X"], syn.BF16)
        Wqkv = dev_tensor(syn.qkv_held_shard(ad["WQ"], ad["WK"], ad["WV"], a["n_heads"],
                                             a["head_dim"], a["i"], a["t"]), syn.BF16)
        Wo = dev_tensor(np.ascontiguousarray(
            ad["WO"][syn.head_slice(a["n_heads"], a["head_dim"], a["i"], a["t"]), :]), syn.BF16)
        Ya = torch.empty(a["batch"] * a["seq"], a["hidden"], dtype=torch.float32, device="cuda")
        wsa = torch.empty(B.tp_attn_shard_workspace_bytes(a["batch"], a["seq"], a["n_heads"],
                                                          a["head_dim"], a["t"]),
                          dtype=torch.uint8, device="cuda")
        attn_ms = time_events(lambda: B.tp_attn_shard(Xa, Wqkv, Wo, Ya, a["batch"], a["seq"],
                                                      a["n_heads"], a["head_dim"], a["i"], a["t"],
                                                      True, workspace=wsa),
                              args.steps, args.warmup)
        afl = attn_flops(a["batch"], a["seq"], a["hidden"], a["n_heads"], a["head_dim"], a["t"])
        attn_tf = afl / (attn_ms * 1e-3) / 1e12
        del ad
        attn_row = {"workload": "t8_i0_h8192_64x128heads_seq2048_causal",
                    "ms": round(attn_ms, 5), "flop": afl, "tflops": round(attn_tf, 2),
                    "frac_peak": round(attn_tf / PEAK_BF16_TFLOPS, 4)}

    layer = None if args.no_attention else layer_row(max(3, args.steps // 40), 2)

    traffic = load_traffic()
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64 normals: activations N(0,1), weights N(0,0.02^2))",
        "config": {"workload": "ffn_shard_t8_i3_h4096_f16384_tokens4096_plus_reduce8",
                   "tokens": M, "hidden": h, "ffn": f, "t": t, "i": i,
                   "partial_dtype": "bf16", "reduce_out_dtype": "f32"},
        "roofline": {"bound": "mfma", "kernel": "tp_ffn_shard (GEMM1+GeLU, GEMM2)",
                     "achieved": round(ffn_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ffn_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "per_launch_flop": fl,
                     "avg_launch_ms": round(ffn_ms, 5)},
        "rows": {
            "ffn_shard": {"ms": round(ffn_ms, 5), "tflops": round(ffn_tf, 2),
                          "frac_peak": round(ffn_tf / PEAK_BF16_TFLOPS, 4)},
            "partial_reduce": {"ms": round(red_ms, 5), "bytes": red_bytes,
                               "gbs": round(red_gbs, 1),
                               "frac_hbm_peak": round(red_gbs / PEAK_HBM_GBS, 4),
                               "bound": "hbm"},
            "partial_reduce_slice": slice_row,
            "ffn_shard_reduce_fused": fused_row,
            "attn_shard": attn_row,
            "layer": layer,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
