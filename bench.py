#!/usr/bin/env python3
"""Throughput of Kimi Delta Attention forward + backward on one MI355X.

One step = kda_fwd followed by kda_bwd (every kernel of the path) over one
batch of seeded synthetic inputs already resident in HBM: the varlen workload
of 8 packed sequences with lengths drawn from U[1K, 32K] (~128K tokens),
H=16, dk=dv=128, bf16 inputs, fp32 states and accumulation, outputs and
gradients stored in their primal's dtype (bf16; --out-dtype f32 stores them
in fp32).

Prints one JSON line: tokens/s for the whole step, the roofline of the
dominant kernel (HIP-event durations recorded live around every launch of the
timed steps), the whole-step HBM and bf16-MFMA rooflines with achieved TFLOP/s,
the float64 CPU oracle timed on a bounded sample of the same workload on this
host's cores, and (configs_fwd) the forward pass of the three single-sequence
workloads (T = 4K, 32K with the sharp gate, 128K; H=16, d=128, bf16) timed in
the same run.  Algorithmic bytes count outputs and gradients at the inputs'
storage size (the primal dtype): 1,282 B forward and 2,308 B backward per
token-head at d = 128, plus the states.

    python bench.py [--steps K] [--warmup W] [--config 4] [--fwd-only] [--no-extra-configs]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
METRIC = "KDA fwd(+bwd) tokens/s and % MFMA/HBM roofline, H=16 d=128 bf16, T=4K\u2013128K"

CSRC = os.path.join(ROOT, "gated_delta_rule_79_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(workload):
    """Counter summary (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled) of one workload."""
    return os.path.join(PROFILES, f"hbm_traffic_{workload}.json")


CONV_SOURCES = ("kda_conv.hip", "kda_conv.hpp")


def sources_digest(workload=""):
    """sha256 over the sources a workload's kernels are built from: counters taken from other sources
    are stale.  The convolution workload hashes its own kernel files; the KDA workloads every other file."""
    import hashlib
    h = hashlib.sha256()
    conv = workload.startswith("conv_")
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".hpp", ".cpp", ".h")):
            continue
        if (name in CONV_SOURCES) != conv and not (conv and name in ("kda_common.hpp", "kda_internal.hpp",
                                                                      "kda_api.cpp")):
            continue
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _counter_rows(path):
    import csv
    out = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def _bools(name):
    """Bool template arguments of a kernel name, in order: mangled 'Lb1E' and demangled 'true'
    (rocprofv3 can print a name half-demangled, with both forms in it)."""
    import re
    return [(m[0] == "1") if m[0] else (m[1] == "true") for m in re.findall(r"Lb([01])(?:E|(?=\)))|\b(true|false)\b", name)]


def _ints(name):
    """Integer template arguments of a kernel name, in order: mangled 'Li64E' and demangled ', 64'."""
    import re
    return [int(m[0] or m[1]) for m in re.findall(r"Li(\d+)E|(?:<|,)\s*(\d+)\s*(?=[,>])", name)]


def _short_name(name, train=True):
    """rocprofv3 kernel name -> the timing name the library uses (train: the forward saves for
    the backward, so the prep that keeps T etc. is the forward's)."""
    if "kda_state_rev" in name:
        b = _bools(name)   # kda_state_rev<E, DK, DV, DVS, LOCAL>
        return "kda_seg_rev_local" if b and b[-1] else "kda_state_bwd_revpass"
    if "kda_segment_rscan" in name:
        return "kda_seg_rscan"
    if "kda_segment_scan" in name:
        return "kda_seg_scan"
    if "kda_bwd_chunk" in name:
        # kda_bwd_chunk<E, O, DK, DV, QKN, PATH>: bf16 inputs run the flagged (steep) chunk-heads in
        # a PATH 1 launch of their own; fp32 inputs run every chunk-head through PATH 1
        ints = _ints(name)
        steep = bool(ints) and ints[-1] == 1 and ("DF16b" in name or "bf16" in name or "__bf16" in name)
        return "kda_bwd_chunk_steep" if steep else "kda_bwd_chunk"
    if "kda_grad_absmax" in name:
        return "kda_grad_absmax"
    if "kda_grad_scale" in name:
        return "kda_grad_scale"
    if "kda_chunk_map" in name:
        return "kda_chunk_map"
    if "kda_decode_step" in name:
        return "kda_decode_step"
    for k in ("fwd", "bwd", "final", "dinit", "reduce", "decode"):
        if f"kda_conv_{k}_k" in name:
            return f"kda_conv_{k}"
    if "kda_prep" in name:
        bwd = (_bools(name) or [False])[0]   # <..., BWD, QKN[, GATE][, PATH]>
        if "kda_prep8" in name:
            ints = _ints(name)
            if ints and ints[-1] == 1:   # the 8-token-group walk over the flagged chunk-heads
                return "kda_prep_steep"
        return ("kda_prep_save" if train else "kda_prep_bwd") if bwd else "kda_prep"
    if "kda_state" in name:
        # kda_state<E, O, DK, DV, DVS, OUT, SAVE, PF, MODE, UF>: the bools are OUT, SAVE, UF and the
        # last integer argument is MODE (2: a stretch's run from zero with its transfer)
        b = _bools(name)
        out, save = (b[0], b[1]) if len(b) >= 2 else (True, False)
        ints = _ints(name)
        if ints and ints[-1] == 2:
            return "kda_seg_local_transfer"
        if out:
            return "kda_state_fwd_save" if save else "kda_state_fwd"
        return "kda_state_bwd_fwdpass"
    return None


def ingest_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, workload):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (one bench step, and a plain copy of
    copy_bytes bytes) into per-kernel HBM bytes per launch, scaled by the copy's calibration."""
    cf = _counter_rows(copy_fetch_csv)
    cw = _counter_rows(copy_write_csv)
    copy_name = next(n for n in cf if "copyBuffer" in n)
    f_kib = sum(cf[copy_name]) / len(cf[copy_name])
    w_kib = sum(cw[copy_name]) / len(cw[copy_name])
    scale_f = copy_bytes / (f_kib * 1024.0)   # bytes per counted KiB-unit, reads
    scale_w = copy_bytes / (w_kib * 1024.0)
    kf, kw = _counter_rows(fetch_csv), _counter_rows(write_csv)
    kernels = {}
    for name in kf:
        short = _short_name(name)
        if not short or name not in kw:
            continue
        fk = sum(kf[name]) / len(kf[name])
        wk = sum(kw[name]) / len(kw[name])
        kernels[short] = {"fetch_kib": fk, "write_kib": wk,
                          "read_bytes": fk * 1024.0 * scale_f, "write_bytes": wk * 1024.0 * scale_w,
                          "bytes": fk * 1024.0 * scale_f + wk * 1024.0 * scale_w}
    doc = {"workload": workload, "sources_sha256": sources_digest(workload),
           "calibration": {"copy_bytes": copy_bytes, "copy_fetch_kib": f_kib, "copy_write_kib": w_kib,
                           "fetch_scale": scale_f, "write_scale": scale_w},
           "kernels": kernels}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(workload), "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
        f.write("\n")
    return doc


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counters, or None when absent or stale."""
    try:
        doc = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None
    if doc.get("workload") != workload or doc.get("sources_sha256") != sources_digest(workload):
        return None
    k = doc.get("kernels", {}).get(kernel)
    return int(k["bytes"]) if k else None


def algorithmic_bytes(w, tokens, n_seqs, fwd_only):
    """Compulsory HBM bytes of the path: inputs read once, outputs written once.  Outputs and
    gradients are counted at the inputs' storage size (the primal dtype, 1,282 B forward and
    2,308 B backward per token-head at d = 128 in bf16) whatever dtype a run stores them in, so
    fp32 outputs cost time without earning bytes."""
    H, dk, dv = w.H, w.dk, w.dv
    e = 2 if w.dtype == "bf16" else 4
    th = tokens * H
    state = n_seqs * H * dk * dv * 4
    fwd = th * (e * (2 * dk + dk + dv) + e) + th * e * dv + 2 * state      # q,k,la,v,beta -> o; S0 in, S_T out
    if fwd_only:
        return fwd, {"fwd": fwd}
    bwd = (th * (e * (2 * dk + dk + dv) + e + e * dv)                       # q,k,la,v,beta,dO
           + th * e * (2 * dk + dk + dv + 1)                                # dq,dk,dla,dv,dbeta
           + 3 * state)                                                     # S0, dS_T in; dS0 out
    return fwd + bwd, {"fwd": fwd, "bwd": bwd}


def flops_per_token_head(d, C=64):
    """Algorithmic flops per token-head of the chunked form (triangular products counted once):
    forward = Gram blocks A_kk, A_qk + W, U~ (4 x C/2 x d x 2) + W S, Qt S, Kh^T U (3 x 2 d^2)
    + Aqk U (C/2 x d x 2) + the triangular inverse (C^2 / 3); 141 kFLOP at d = 128.  The
    backward is 2.75 times the forward (387 kFLOP at d = 128): dU, dS over the chain, the
    value-side contractions, the T products and the gated products."""
    fwd = 4 * (C // 2) * d * 2 + 3 * 2 * d * d + (C // 2) * d * 2 + C * C / 3
    return fwd, 2.75 * fwd


def algorithmic_flops(w, tokens, fwd_only):
    f, b = flops_per_token_head(w.dk)
    return (f if fwd_only else f + b) * tokens * w.H


def kernel_alg_bytes(name, w, tokens, n_seqs):
    """Compulsory bytes one launch of a kernel must move: its share of the path's own inputs
    and outputs (intermediates in the workspace are not counted; outputs at the primal size)."""
    H, dk, dv = w.H, w.dk, w.dv
    e = 2 if w.dtype == "bf16" else 4
    th = tokens * H
    state = n_seqs * H * dk * dv * 4
    table = {
        "kda_prep": th * (e * (3 * dk + dv) + e),                         # reads q, k, log_alpha, v, beta
        "kda_prep_bwd": th * (e * (3 * dk + dv) + e),                     # same reads, backward recompute
        "kda_prep_save": th * (e * (3 * dk + dv) + e),                    # forward prep keeping the backward's data
        "kda_state_fwd_save": th * e * dv + 2 * state,                    # as kda_state_fwd
        "kda_state_fwd": th * e * dv + 2 * state,                         # writes o; reads S0, writes S_T
        "kda_state_bwd_fwdpass": state,                                   # reads S0
        "kda_state_bwd_revpass": th * e * dv + 2 * state,                 # reads dO, dS_T; writes dS0
        # reads q, k, log_alpha, v, dO, beta; writes dq, dk, dlog_alpha, dv, dbeta
        "kda_bwd_chunk": th * (e * (3 * dk + 2 * dv) + e + e * (3 * dk + dv + 1)),
        "kda_chunk_map": 0,
    }
    return table.get(name, 0)


def kernel_alg_flops(name, w, tokens):
    """Algorithmic flops of one launch (chunk C=64, triangular products counted once)."""
    dk, dv, C = w.dk, w.dv, 64
    per = {
        "kda_prep": 2 * C * dk + C * dk + C * dv,                          # Gram Akk, Aqk; W, U~
        "kda_prep_bwd": 2 * C * dk + C * dk + C * dv,
        "kda_prep_save": 2 * C * dk + C * dk + C * dv,
        "kda_state_fwd_save": 3 * 2 * dk * dv + C * dv,
        "kda_state_fwd": 3 * 2 * dk * dv + C * dv,                         # W S, Qt S, Kh^T U; Aqk U
        "kda_state_bwd_fwdpass": 2 * 2 * dk * dv,                          # W S, Kh^T U
        "kda_state_bwd_revpass": 3 * 2 * dk * dv + C * dv,                 # Kh dS', Qt^T dO, W^T dU; Aqk^T dO
        # dO S^T, U dS'^T, dU S^T; dO U^T, dU V^T, T^T dU; T^T dW, dW K+^T, T-products, gated products
        "kda_bwd_chunk": 3 * 2 * dk * dv + 4 * C * dv + 3 * C * dk + 2 * C * C + 4 * C * dk,
    }.get(name, 0)
    return per * tokens * w.H


def cpu_baseline(inp, w, with_bwd, prepped=False):
    """The float64 oracle (untuned) on a bounded sample: heads 0-3 of every sequence, fwd (+bwd)
    (about 10-15 s on 16 host threads for the varlen training step).
    prepped: the inputs are raw and the oracle applies the same input preparation."""
    import oracle
    n_seq = len(inp["lengths"])
    heads = [0, 1, 2, 3]
    units = [(s, h) for h in heads for s in range(n_seq)]
    threads = oracle.default_threads()
    fwd = oracle.kda_fwd_prepped if prepped else oracle.kda_fwd
    bwd = oracle.kda_bwd_prepped if prepped else oracle.kda_bwd
    t0 = time.perf_counter()
    fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"],
        init_state=inp["init_state"], units=units, nthreads=threads)
    if with_bwd:
        bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["cu_seqlens"], inp["d_out"],
            init_state=inp["init_state"], d_final_state=inp["d_final_state"], units=units, nthreads=threads)
    dt = time.perf_counter() - t0
    token_heads = sum(inp["lengths"]) * len(heads)
    return {
        "value": token_heads / w.H / dt,
        "unit": "tokens/s",
        "cores": min(threads, len(units)),
        "kind": "oracle",
        "sample": f"heads {heads[0]}-{heads[-1]} of all {n_seq} sequences ({token_heads} token-heads, "
                  f"{'fwd+bwd' if with_bwd else 'fwd'}), {dt:.1f} s; value = sample token-heads / H / s",
    }


DECODE_METRIC = "KDA decode/replay step tokens/s and % HBM roofline, H=16 d=128 bf16, fp32 state pool"


def decode_bench(args, dev) -> int:
    """One step = one kda_decode call: B sequences advance T tokens from pool slots and commit them."""
    import numpy as np
    import torch

    import gated_delta_rule_79_amd as kda
    import kda_inputs as ki
    B, T = (int(x) for x in args.decode.split(","))
    H, dk, dv = 16, 128, 128
    P = B
    odt = torch.bfloat16 if (args.out_dtype == "bf16") else torch.float32
    print(f"[bench] decode inputs B={B} T={T}", file=sys.stderr, flush=True)
    inp = ki.decode_inputs(B, T, H, dk, dv, P, dtype="bf16", seed=99)
    idx_np = np.random.default_rng(99).permutation(P)[:B].astype(np.int32)
    t = {n: torch.from_numpy(inp[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v", "log_alpha", "beta")}
    pool = torch.from_numpy(inp["state_pool"]).to(dev)
    idx = torch.from_numpy(idx_np).to(dev)
    out = torch.empty((B, T, H, dv), dtype=odt, device=dev)

    def step():
        kda.decode(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], pool, state_indices=idx, out=out,
                   out_dtype=odt)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} decode steps", file=sys.stderr, flush=True)
    kda.timing_enable(True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    kt = kda.timing_read()
    kda.timing_enable(False)
    tot_ms, n_launch = kt["kda_decode_step"]
    avg_ms = tot_ms / max(n_launch, 1)
    # algorithmic bytes: each (sequence, head) state read and written once (fp32), the tokens' q, k,
    # log_alpha, v, beta read (bf16) and outputs written, plus the index list
    # (outputs counted at the inputs' bf16 size, whatever out_dtype stores them in)
    ab = B * H * (2 * dk * dv * 4 + T * (2 * (3 * dk + dv) + 2 + 2 * dv)) + 4 * B
    ach = ab / (avg_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic("kda_decode_step", f"decode_B{B}_T{T}"),
            "kernel": "kda_decode_step", "avg_launch_ms": round(avg_ms, 5), "launches": n_launch,
            "alg_bytes_per_launch": int(ab)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nb = min(B, 64)
        t0 = time.perf_counter()
        oracle.kda_decode(inp["q"][:nb], inp["k"][:nb], inp["v"][:nb], inp["log_alpha"][:nb], inp["beta"][:nb],
                          inp["state_pool"], state_indices=idx_np[:nb])
        dt_cpu = time.perf_counter() - t0
        cpu = {"value": round(nb * T / dt_cpu, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"first {nb} of the {B} sequences, all {H} heads, {T} tokens each (float64, one thread), "
                         f"{dt_cpu:.1f} s"}
    line = {
        "metric": DECODE_METRIC, "value": round(B * T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode_B{B}_T{T}", "sequences": B, "tokens_per_sequence": T, "H": H, "dk": dk,
                   "dv": dv, "out_dtype": "bf16" if (args.out_dtype == "bf16") else "f32", "commit": "all tokens"},
        "roofline": roof, "kernels_ms_per_step": {k: round(v[0] / args.steps, 5) for k, v in kt.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


CONV_METRIC = "short causal convolution fwd+bwd tokens/s and % HBM roofline, D=6144 W=4 SiLU bf16"


def conv_bench(args, dev) -> int:
    """One step = kda_conv_fwd then kda_conv_bwd over the training step's eight packed sequences
    (lengths of the varlen workload), D = 3 x 16 heads x 128 channels (the q, k, v channels a
    short convolution precedes KDA with), W = 4, SiLU, bf16 inputs, fp32 states and weights."""
    import numpy as np
    import torch

    import gated_delta_rule_79_amd as kda
    import kda_inputs as ki
    D, W = 6144, 4
    lengths = list(ki.config(4).lengths)
    tokens, N = int(sum(lengths)), len(lengths)
    odt = torch.bfloat16 if (args.out_dtype == "bf16") else torch.float32
    print(f"[bench] conv inputs: {N} sequences, {tokens} tokens, D={D}, W={W}", file=sys.stderr, flush=True)
    c = ki.conv_inputs(lengths, D, W, dtype="bf16", seed=4)
    g = {n: torch.from_numpy(c[n]).to(dev, torch.bfloat16).unsqueeze(0) for n in ("x", "dy")}
    p = {n: torch.from_numpy(c[n]).to(dev) for n in ("weight", "bias", "init_state", "d_final_state")}
    cu = torch.from_numpy(c["cu_seqlens"]).to(dev)
    y = torch.empty((1, tokens, D), dtype=odt, device=dev)
    fin = torch.empty((N, W - 1, D), dtype=torch.float32, device=dev)
    dx = torch.empty((1, tokens, D), dtype=odt, device=dev)
    dw = torch.empty((D, W), dtype=torch.float32, device=dev)
    db = torch.empty((D,), dtype=torch.float32, device=dev)
    dinit = torch.empty_like(fin)
    ws = torch.empty(max(kda.conv_workspace_bytes(1, tokens, D, W, torch.bfloat16), 1), dtype=torch.uint8,
                     device=dev)

    def step():
        kda.conv_fwd(g["x"], p["weight"], p["bias"], p["init_state"], cu_seqlens=cu, silu=True, out=y,
                     final_state=fin, out_dtype=odt)
        kda.conv_bwd(g["x"], p["weight"], g["dy"], p["bias"], p["init_state"], p["d_final_state"], cu_seqlens=cu,
                     silu=True, out_dtype=odt, workspace=ws, dx=dx, dweight=dw, dbias=db, d_init=dinit)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} conv steps", file=sys.stderr, flush=True)
    kda.timing_enable(True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    kt = kda.timing_read()
    kda.timing_enable(False)
    # algorithmic bytes per launch: the forward reads x and writes y; the backward reads x and dy and
    # writes dx, outputs counted at the inputs' bf16 size (states, weights and the per-channel sums are
    # under 0.1% and left out)
    alg = {"kda_conv_fwd": tokens * D * (2 + 2), "kda_conv_bwd": tokens * D * (2 + 2 + 2)}
    step_bytes = sum(alg.values())
    dom = max(alg, key=lambda k: kt[k][0])
    tot_ms, n_launch = kt[dom]
    avg_ms = tot_ms / max(n_launch, 1)
    ach = alg[dom] / (avg_ms * 1e-3) / 1e9
    wl = f"conv_varlen8_D{D}_W{W}"
    roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom, wl), "kernel": dom,
            "avg_launch_ms": round(avg_ms, 5), "launches": n_launch, "alg_bytes_per_launch": int(alg[dom])}
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import short_conv as sc
        nch = 1536
        ch = np.arange(0, D, D // nch)[:nch]
        sub = lambda a: np.ascontiguousarray(a[..., ch])  # noqa: E731
        t0 = time.perf_counter()
        sc.short_conv_fwd(sub(c["x"]), c["weight"][ch], c["cu_seqlens"], bias=c["bias"][ch],
                          init_state=sub(c["init_state"]), silu=True)
        sc.short_conv_bwd(sub(c["x"]), c["weight"][ch], c["cu_seqlens"], sub(c["dy"]), bias=c["bias"][ch],
                          init_state=sub(c["init_state"]), d_final_state=sub(c["d_final_state"]), silu=True)
        dt_cpu = time.perf_counter() - t0
        cpu = {"value": round(tokens * nch / D / dt_cpu, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{nch} of the {D} channels (every {D // nch}th), all {tokens} tokens, fwd+bwd "
                         f"(float64 numpy, one thread), {dt_cpu:.1f} s; value = tokens x {nch}/{D} / s"}
    line = {
        "metric": CONV_METRIC, "value": round(tokens / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl, "tokens": tokens, "sequences": N, "D": D, "W": W, "activation": "silu",
                   "out_dtype": "bf16" if (args.out_dtype == "bf16") else "f32", "pass": "fwd+bwd"},
        "roofline": roof,
        "step_roofline": {"alg_bytes": int(step_bytes), "roofline_ms": round(step_bytes / HBM_PEAK_GBS / 1e6, 4),
                          "frac": round(step_bytes / HBM_PEAK_GBS / 1e6 / ms_step, 4), "bound": "hbm"},
        "kernels_ms_per_step": {k: round(v[0] / args.steps, 5) for k, v in kt.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload index (4 = varlen fwd+bwd)")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward pass only")
    ap.add_argument("--train", action="store_true",
                    help="time the training step (forward + backward) on a forward-only workload too "
                         "(dO and dS_final drawn as for the varlen workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the forward timings of the T = 4K, 32K and 128K single-sequence workloads that "
                         "the default training-step run adds under configs_fwd")
    ap.add_argument("--out-dtype", choices=("bf16", "f32"), default="bf16",
                    help="storage of outputs and gradients: the primal dtype (bf16, default) or fp32; states and "
                         "accumulation are fp32 either way")
    ap.add_argument("--recompute", action="store_true",
                    help="self-contained backward (recomputes the forward) instead of the training step in which "
                         "the forward keeps the backward's intermediates")
    ap.add_argument("--fused-prep", action="store_true",
                    help="raw q, k and gate inputs: L2 norm and logsigmoid inside the kernels (forward and backward)")
    ap.add_argument("--decode", default=None, metavar="B,T",
                    help="time the decode / replay step instead: B sequences x T tokens (e.g. 512,4), H=16, "
                         "d=128, bf16, states gathered from a pool through a permuted index list, all T committed")
    ap.add_argument("--conv", action="store_true",
                    help="time the short causal convolution (forward + backward) on the varlen workload's lengths, "
                         "D=6144, W=4, SiLU, instead")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (HBM counter calibration)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from rocprofv3 --pmc counter_collection CSVs "
                         "(one bench step; a --copy-probe 1024 run); needs no GPU")
    args = ap.parse_args()
    if args.ingest_counters:
        import kda_inputs as ki
        wl = ("decode_B{}_T{}".format(*args.decode.split(",")) if args.decode else
              "conv_varlen8_D6144_W4" if args.conv else ki.config(args.config).name)
        doc = ingest_counters(*args.ingest_counters, copy_bytes=1024 << 20, workload=wl)
        print(json.dumps(doc["calibration"]))
        for k, v in sorted(doc["kernels"].items()):
            print(f"{k:24s} read {v['read_bytes'] / 1e9:8.3f} GB  write {v['write_bytes'] / 1e9:8.3f} GB")
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}); the multi-GPU path is not "
              f"part of this build", file=sys.stderr)
        return 2

    import torch

    import gated_delta_rule_79_amd as kda
    import kda_inputs as ki

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return 0
    kda.load_library()
    if args.decode:
        return decode_bench(args, dev)
    if args.conv:
        return conv_bench(args, dev)

    w = ki.config(args.config)
    res = run_workload(args, dev, w, with_cpu=not args.no_cpu_baseline, steps=args.steps, warmup=args.warmup)
    line = res["line"]
    if args.config == 4 and not args.fwd_only and not args.no_extra_configs:
        # the forward of the three single-sequence workloads (T = 4K, 32K with the sharp gate, 128K),
        # timed in the same run; not the headline value, which is the training step above
        extra = {}
        for c in (1, 2, 3):
            r = run_workload(args, dev, ki.config(c), with_cpu=False, steps=max(1, min(args.steps, 10)),
                             warmup=max(1, min(args.warmup, 2)), force_fwd=True)
            extra[str(c)] = r["summary"]
            del r
            torch.cuda.empty_cache()
        line["configs_fwd"] = extra
    print(json.dumps(line), flush=True)
    return 0


def run_workload(args, dev, w, with_cpu, steps, warmup, force_fwd=False):
    """Time `steps` steps of workload w (forward, or forward + backward) with inputs resident in HBM."""
    import torch

    import gated_delta_rule_79_amd as kda
    import kda_inputs as ki

    fwd_only = force_fwd or args.fwd_only or not (w.backward or args.train)
    print(f"[bench] generating inputs for {w.name}", file=sys.stderr, flush=True)
    inp = ki.make_inputs(w, with_grads=not fwd_only, raw=args.fused_prep)
    prep = dict(qk_l2norm=True, gate_logsigmoid=True) if args.fused_prep else {}
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    odt = torch.bfloat16 if (args.out_dtype == "bf16") else torch.float32
    t = {k: torch.from_numpy(inp[k]).to(dev, dt).unsqueeze(0) for k in ("q", "k", "v", "log_alpha", "beta")}
    init = torch.from_numpy(inp["init_state"]).to(dev) if inp["init_state"] is not None else None
    varlen = w.lengths is not None
    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev) if varlen else None
    if not varlen:
        t = {k: v.reshape(w.B, w.T, *v.shape[2:]) for k, v in t.items()}
    tokens = int(sum(inp["lengths"]))
    n_seqs = len(inp["lengths"])
    d_out = d_fin = None
    if not fwd_only:
        d_out = torch.from_numpy(inp["d_out"]).to(dev, dt).unsqueeze(0)
        if not varlen:
            d_out = d_out.reshape(w.B, w.T, *d_out.shape[2:])
        d_fin = torch.from_numpy(inp["d_final_state"]).to(dev)
    B, T = t["q"].shape[0], t["q"].shape[1]
    ws = torch.empty(kda.workspace_bytes(B, T, w.H, w.dk, w.dv, dt, num_seqs=n_seqs if varlen else 0,
                                         backward=not fwd_only, **prep), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, w.H, w.dv), dtype=odt, device=dev)
    fin = torch.empty((n_seqs, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    grads = dinit = None
    if not fwd_only:
        grads = tuple(torch.empty(x.shape, dtype=odt, device=dev) for x in (t["q"], t["k"], t["v"], t["log_alpha"],
                                                                            t["beta"]))
        dinit = torch.empty_like(fin)

    train = not fwd_only and not args.recompute

    def step():
        kda.fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], init_state=init, cu_seqlens=cu, out=out,
                final_state=fin, workspace=ws, out_dtype=odt, save_for_backward=train, **prep)
        if not fwd_only:
            kda.bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], d_out, init_state=init, d_final_state=d_fin,
                    cu_seqlens=cu, workspace=ws, out_dtype=odt, grads=grads, d_init=dinit, use_saved=train, **prep)

    print(f"[bench] {w.name}: warmup {warmup} steps", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    print(f"[bench] {w.name}: timing {steps} steps", file=sys.stderr, flush=True)
    kda.timing_enable(True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    kt = kda.timing_read()
    kda.timing_enable(False)
    ms_step = ms_total / steps
    value = tokens / (ms_step * 1e-3)

    # dominant kernel roofline: algorithmic bytes (and flops) of one launch over its average duration,
    # the duration from HIP events recorded around every launch on the launch stream
    dom = max(kt.items(), key=lambda kv: kv[1][0]) if kt else None
    roof = None
    if dom:
        name, (tot_ms, n_launch) = dom
        avg_ms = tot_ms / max(n_launch, 1)
        ab = kernel_alg_bytes(name, w, tokens, n_seqs)
        af = kernel_alg_flops(name, w, tokens)
        gbs = ab / (avg_ms * 1e-3) / 1e9
        tfs = af / (avg_ms * 1e-3) / 1e12
        if ab / (HBM_PEAK_GBS * 1e9) >= af / (BF16_PEAK_TFLOPS * 1e12):
            roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4)}
        else:
            roof = {"bound": "mfma", "achieved": round(tfs, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tfs / BF16_PEAK_TFLOPS, 4)}
        roof.update({"traffic": measured_traffic(name, w.name), "kernel": name, "avg_launch_ms": round(avg_ms, 4),
                     "launches": n_launch, "alg_bytes_per_launch": int(ab), "alg_flops_per_launch": int(af),
                     "mfma": {"achieved_tflops": round(tfs, 3), "peak_tflops": BF16_PEAK_TFLOPS,
                              "frac": round(tfs / BF16_PEAK_TFLOPS, 5)}})
    total_bytes, parts = algorithmic_bytes(w, tokens, n_seqs, fwd_only)
    flops = algorithmic_flops(w, tokens, fwd_only)
    t_hbm = total_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (BF16_PEAK_TFLOPS * 1e12)
    tflops = flops / (ms_step * 1e-3) / 1e12
    step_roof = {"alg_bytes": int(total_bytes), "alg_flops": int(flops),
                 "roofline_ms": round(max(t_hbm, t_mfma) * 1e3, 4),
                 "frac": round(max(t_hbm, t_mfma) / (ms_step * 1e-3), 4), "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                 "hbm": {"achieved_gbs": round(total_bytes / (ms_step * 1e-3) / 1e9, 1), "peak_gbs": HBM_PEAK_GBS,
                         "frac": round(t_hbm / (ms_step * 1e-3), 4)},
                 "mfma": {"achieved_tflops": round(tflops, 2), "peak_tflops": BF16_PEAK_TFLOPS,
                          "frac": round(tflops / BF16_PEAK_TFLOPS, 5)}}

    cpu = None
    if with_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, w, not fwd_only, prepped=args.fused_prep)

    kernels = {k: round(v[0] / steps, 4) for k, v in kt.items()}
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": tokens, "sequences": n_seqs, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "out_dtype": "bf16" if (args.out_dtype == "bf16") else "f32", "pass": "fwd" if fwd_only else "fwd+bwd",
                   "backward": None if fwd_only else ("recomputes the forward" if args.recompute
                                                      else "uses the forward's saved intermediates"),
                   "input_prep": "fused (raw q, k, gate)" if args.fused_prep else "inputs already prepared"},
        "roofline": roof,
        "step_roofline": step_roof,
        "tflops": round(tflops, 2),
        "kernels_ms_per_step": kernels,
        "cpu_baseline": cpu,
        "wall_s_timed": round(t_wall, 3),
    }
    summary = {"workload": w.name, "tokens": tokens, "steps": steps, "ms_per_step": round(ms_step, 4),
               "tokens_per_s": round(value, 1), "tflops": round(tflops, 2),
               "hbm_frac": step_roof["hbm"]["frac"], "mfma_frac": step_roof["mfma"]["frac"],
               "roofline_ms": step_roof["roofline_ms"], "kernels_ms_per_step": kernels,
               "dominant": roof}
    return {"line": line, "summary": summary}


if __name__ == "__main__":
    sys.exit(main())
