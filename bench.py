"""Benchmark of the chunkwise KDA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu-baseline]

A step is one full forward pass (stage 1+2 then stage 3+4, through the C
ABI) over the headline workload: B=1, H=32, T=32768, K=V=128, bf16 inputs,
fp32 state, random initial state. Inputs are synthetic (seeded) and already
resident in HBM when timing starts. W untimed warmup steps, then exactly K
timed steps bracketed by device synchronisation; HIP events on the stream the
kernels run on give the step time and, in separate loops, each kernel's
average duration for the roofline entry.

Prints ONE JSON line. Throughput `value` is tokens/s (B*T per step).
Rooflines use MI355X's published peaks (HBM3E 8 TB/s, dense bf16 MFMA
2.5 PFLOP/s) and the algorithmic traffic of each kernel:
  stage 1+2: reads q,k,v,g (4 x 256 B) + beta (2 B), writes its workspace
             record (1128 B)                     -> 2154 B per token-head
  stage 3+4: reads the record (1128 B), writes o (256 B) -> 1384 B per token-head
  algorithmic FLOPs: 6CKV + C(C+1)(3K+2V) + C^3/3 per chunk-head (C = 64).
The CPU baseline times the float64 oracle on a bounded sample of the same
workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # bytes/s
PEAK_BF16 = 2.5e15         # dense bf16 MFMA FLOP/s
PEAK_FP32 = 157.3e12       # dense fp32 MFMA FLOP/s
METRIC = "KDA chunk-fwd tokens/s at H=32,K=V=128,T=32k bf16; % MFMA peak"


def alg_flops_per_chunk_head(C, K, V):
    return 6 * C * K * V + C * (C + 1) * (3 * K + 2 * V) + C ** 3 / 3


def alg_bytes_per_token_head(K, V, elem, gelem, belem):
    s12 = (2 * K) * elem + V * elem + K * gelem + belem          # q, k, v, g, beta
    rec = (3 * K + 48 + V) * elem + 4 * K / 64                  # W, qg, kg, Aqk (6 of 8 blocks), U, gamma
    s34 = rec + V * elem                                          # record in, o out
    return s12 + rec, s34


KERNEL_SOURCES = {
    "stage12": ["kda_stage12.hip", "kda_device.h", "kda_layout.h", "kda_kernels.h"],
    "stage34": ["kda_stage34.hip", "kda_device.h", "kda_layout.h", "kda_kernels.h"],
    "bwd": ["kda_bwd.hip", "kda_device.h", "kda_layout.h", "kda_kernels.h"],
}


def kernel_source_hash(kernel):
    import hashlib
    m = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        m.update(open(os.path.join(ROOT, "kimi_delta_attention_03_amd", "csrc", f), "rb").read())
    return m.hexdigest()[:16]


def measured_traffic(workload_name, kernel):
    """Calibrated HBM bytes per launch from the committed rocprofv3 counter runs,
    or None when they were taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", f"traffic_kda_fwd_{workload_name}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get("kernels", {}).get(kernel)
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return rec["traffic_bytes"]


def time_loop(fn, reps, torch):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def host_info():
    """CPU model, usable cores and the BLAS numpy calls (for the CPU baseline record)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name')} {b.get('version')}".strip()
    except Exception:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    return {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0)), "blas": blas, "blas_threads": threads}


def build_info():
    """Provenance of the loaded library (written next to it at build time)."""
    p = os.path.join(ROOT, "kimi_delta_attention_03_amd", "_build_info.json")
    try:
        return json.load(open(p))
    except (OSError, ValueError):
        return None


def copy_rate(torch, nbytes=1 << 30, reps=5):
    """Measured device-to-device copy rate (read + write bytes per second)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ms = time_loop(lambda: dst.copy_(src), reps, torch)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms / 1e3)


def cpu_baseline(x, target_s=15.0):
    """Time the float64 chunkwise oracle on a bounded sample of the workload."""
    import oracle.kda_oracle as orc
    H = x.q.shape[2]
    heads = [0, 1]
    T = x.q.shape[1]
    tok = 1024
    # grow the sample until it takes a measurable time, then run the bounded one
    while True:
        t0 = time.perf_counter()
        c0 = time.process_time()
        orc.kda_chunkwise(x.q[:, :tok], x.k[:, :tok], x.v[:, :tok], x.g[:, :tok], x.beta[:, :tok],
                          x.scale, 64, None if x.initial_state is None else x.initial_state,
                          heads=heads)
        wall = time.perf_counter() - t0
        cpu = time.process_time() - c0
        if wall * 2 >= target_s or tok * 2 > T:
            break
        tok = min(T, tok * max(2, int(target_s / max(wall, 1e-3) / 2)))
        tok = max(64, tok // 64 * 64)
    token_heads = tok * len(heads)
    tps = token_heads / wall / H       # tokens/s of the full-H workload
    hi = host_info()
    return {
        "value": tps, "unit": "tokens/s", "cores": hi["blas_threads"] or hi["usable_cores"], "kind": "oracle",
        "sample": f"float64 chunkwise oracle on heads {heads} of {H}, first {tok} of {T} tokens "
                  f"({token_heads} token-heads, {wall:.1f} s wall, {cpu:.1f} s CPU, "
                  f"{cpu / wall:.1f} cores busy on average); tokens/s scaled to all {H} heads",
        **hi,
    }


def bench_decode(args, torch, kda):
    """One decode step for B sequences: the state (fp32 [B, H, K, V]) is read
    and written once; q, k, g (K each), v, o (V each) and beta per (sequence,
    head) are read or written once -> 8 K V + 2 (3 K + 2 V) + 2 bytes per head."""
    B, H, K = 256, 32, 128
    from kimi_delta_attention_03_amd.synthetic import core_inputs
    x = core_inputs(B, 1, H, K, K, dtype="bf16", seed=1101, init_std=0.1)
    dev = "cuda:0"
    sl = lambda a: torch.from_numpy(a[:, 0].copy()).to(torch.bfloat16).to(dev)
    q, k, v, g, beta = (sl(a) for a in (x.q, x.k, x.v, x.g, x.beta))
    st = torch.from_numpy(x.initial_state).to(dev)
    o = torch.empty((B, H, K), dtype=torch.bfloat16, device=dev)
    step = lambda: kda.decode_step(q, k, v, g, beta, st, scale=x.scale, out=o)
    for _ in range(args.warmup):
        step()
    ms = time_loop(step, args.steps, torch)
    nbytes = B * H * (8 * K * K + 2 * (3 * K + 2 * K) + 2)
    gbps = nbytes / (ms / 1e3) / 1e9
    print(json.dumps({
        "metric": "KDA decode step tokens/s (one token per sequence)", "value": B / (ms / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "dtype": "bf16 (fp32 state)", "data": "synthetic (seeded numpy generators)",
        "config": {"workload": f"decode_bf16_B{B}_H{H}_K{K}", "B": B, "H": H, "K": K, "V": K},
        "roofline": {"kernel": "decode", "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": gbps * 1e9 / PEAK_HBM, "traffic": None, "alg_bytes_per_launch": nbytes},
    }), flush=True)


def bench_affine(args, torch, kda, WORKLOADS, workload):
    """Affine summaries of a core workload: stage 1+2 (reads the inputs, writes
    the records), then two stage-3+4 passes without output (zero start -> N,
    identity start -> M) that each read the records' W, kg, U and gamma
    (2K + V elements + 4K/64 bytes per token-head) and write their K x V states."""
    x = workload(args.workload)
    dev = "cuda:0"
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    to = lambda a: torch.from_numpy(a).to(dt).to(dev)
    q, k, v, g, beta = (to(a) for a in (x.q, x.k, x.v, x.g, x.beta))
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(dev)
    run = lambda: kda.affine_summary(q, k, v, g, beta, scale=x.scale, cu_seqlens=cu)
    for _ in range(args.warmup):
        run()
    ms = time_loop(run, args.steps, torch)
    B, T, H, K = x.q.shape
    elem = 2 if x.dtype == "bf16" else 4
    b12, _ = alg_bytes_per_token_head(K, K, elem, elem, elem)
    summ = (2 * K + K) * elem + 4 * K / 64       # W, kg, U, gamma
    nseq = B if cu is None else len(x.cu_seqlens) - 1
    nbytes = B * T * H * (b12 + 2 * summ) + 2 * nseq * H * K * K * 4
    gbps = nbytes / (ms / 1e3) / 1e9
    print(json.dumps({
        "metric": "KDA affine chunk summaries tokens/s", "value": B * T / (ms / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "dtype": x.dtype, "data": "synthetic (seeded numpy generators)",
        "config": {"workload": WORKLOADS[args.workload]["name"], "B": B, "T": T, "H": H, "K": K, "V": K},
        "roofline": {"kernel": "stage12 + 2 x stage34 (summary)", "bound": "hbm", "achieved": gbps,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": gbps * 1e9 / PEAK_HBM, "traffic": None,
                     "alg_bytes_per_launch": nbytes},
    }), flush=True)


def bench_gated(args, torch, kda, WORKLOADS, workload):
    """The forward with the gate activation inside stage 1+2 (lower-bound
    sigmoid, bound -5, or softplus with --gate softplus) on a core workload's
    shape: g holds raw gate values (N(0,1) clipped to [-3, 2]) and A_log, dt_bias
    are per head / per (head, channel). Same bytes as the plain forward (the raw
    gate replaces the log decay) plus A_log and dt_bias; the roofline entry is
    the whole step's algorithmic bytes over the step time."""
    from kimi_delta_attention_03_amd.synthetic import gate_inputs
    x = workload(args.workload)
    dev = "cuda:0"
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    to = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(d).to(dev)
    B, T, H, K = x.q.shape
    raw, A_log, dt_bias = gate_inputs(B, T, H, K, seed=WORKLOADS[args.workload]["seed"] + 70, dtype=x.dtype)
    q, k, v, graw, beta = (to(a, dt) for a in (x.q, x.k, x.v, raw, x.beta))
    init = None if x.initial_state is None else to(x.initial_state, torch.float32)
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(dev)
    mode = "softplus" if args.gate == "softplus" else "lower_bound_sigmoid"
    fwd = kda.KdaForward(q, k, v, graw, beta, scale=x.scale, initial_state=init, cu_seqlens=cu, gate_mode=mode,
                         A_log=to(A_log, torch.float32), dt_bias=to(dt_bias, torch.float32), gate_lower_bound=-5.0)
    for _ in range(args.warmup):
        fwd()
    ms = time_loop(fwd, args.steps, torch)
    elem = 2 if x.dtype == "bf16" else 4
    b12, b34 = alg_bytes_per_token_head(K, K, elem, elem, elem)
    nbytes = B * T * H * (b12 + b34) + 4 * H * (K + 1)
    gbps = nbytes / (ms / 1e3) / 1e9
    print(json.dumps({
        "metric": f"KDA chunk-fwd with in-kernel gate activation ({mode}) tokens/s", "value": B * T / (ms / 1e3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "dtype": x.dtype, "data": "synthetic (seeded numpy generators)",
        "config": {"workload": WORKLOADS[args.workload]["name"] + "_gated", "B": B, "T": T, "H": H, "K": K,
                   "V": K, "gate": mode},
        "roofline": {"kernel": "stage12 (gate inside) + stage34, whole step", "bound": "hbm", "achieved": gbps,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": gbps * 1e9 / PEAK_HBM, "traffic": None,
                     "alg_bytes_per_launch": nbytes},
    }), flush=True)


def bwd_flops_per_chunk_head(C, K, V):
    """Algorithmic FLOPs of each backward launch per (chunk, head), causal
    triangles counted as triangles (tri = C(C+1)/2 pairs):
      prep         Aqk, M (2 tri K each), the unit-triangular inverse (C^3/3),
                   W = A Kb and U = A Vb (2 tri K, 2 tri V)
      states_fwd   Vn = U - W S and S' = gamma S + KG^T Vn (2 C K V each)
      states_bwd   dVn = Aqk^T dO + KG dS' (2 tri V + 2 C K V),
                   dS = Qg^T dO - W^T dVn (2 x 2 C K V)
      chunk        Vn, dVn (as above), dQg, dW, dKG (3 x 2 C K V), dAqk (2 tri V),
                   dgamma (2 K V), dA (2 tri (K + V)), dKb, dVb (2 tri K, 2 tri V),
                   A^T dA A^T (2 C^3 / 3), four gated sums (4 x 2 tri K), ~20 C K
                   elementwise"""
    tri = C * (C + 1) / 2
    ckv = 2.0 * C * K * V
    return {
        "prep": 4 * tri * K + C ** 3 / 3 + 2 * tri * (K + V),
        "states_fwd": 2 * ckv,
        "states_bwd": 2 * tri * V + 3 * ckv,
        "chunk": (ckv + 2 * tri * V + ckv + 3 * ckv + 2 * tri * V + 2 * K * V + 2 * tri * (K + V)
                  + 2 * tri * (K + V) + 2 * C ** 3 / 3 + 8 * tri * K + 20 * C * K),
    }


def bwd_chunk_alg_bytes_per_token_head(K, V, e):
    """Bytes the chunk-gradient stage cannot avoid per token-head, with
    inputs of e bytes per element: the chunk's inputs q, k, g (K each), v and
    dO (V each) and beta, the chunk-start state S and the end-state gradient
    dS' (K x V fp32 each, once per 64-token chunk), and the fp32 gradients dq,
    dk, dg, dv and dbeta it writes. At K = V = 128 with bf16 inputs: 3330 B
    read + 2052 B written."""
    reads = (3 * K + 2 * V + 1) * e + 2 * K * V * 4 / 64
    writes = (3 * K + V + 1) * 4
    return reads + writes


def bench_backward(args, torch, kda, WORKLOADS, workload):
    """The backward (kda_chunk_bwd) on a core workload's shape: one step = all
    four launches for d_o ~ N(0,1) and d_final ~ N(0,1); each launch is also
    timed alone (in order, over one workspace) for the roofline entry."""
    from kimi_delta_attention_03_amd.synthetic import grad_inputs
    x = workload(args.workload)
    dev = "cuda:0"
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    to = lambda a, d: torch.from_numpy(a).to(d).to(dev)
    q, k, v, g, beta = (to(a, dt) for a in (x.q, x.k, x.v, x.g, x.beta))
    init = None if x.initial_state is None else to(x.initial_state, torch.float32)
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(dev)
    B, T, H, K = x.q.shape
    V = x.v.shape[3]
    N = B if cu is None else len(x.cu_seqlens) - 1
    d_o, d_f = grad_inputs(B, T, H, V, N, K=K, seed=WORKLOADS[args.workload]["seed"] + 50, dtype=x.dtype)
    call = kda.KdaBackward(q, k, v, g, beta, to(d_o, dt), scale=x.scale, initial_state=init, cu_seqlens=cu,
                           d_final_state=to(d_f, torch.float32))
    for _ in range(args.warmup):
        call()
    ms = time_loop(call, args.steps, torch)
    names = {1: "prep", 2: "states_fwd", 4: "states_bwd", 8: "chunk"}
    reps = max(1, min(args.kernel_reps, 5))
    stage_ms = {}
    for bit, nm in names.items():
        # every stage reads what the earlier ones wrote: run the earlier ones first, then time this one
        if bit > 1:
            call(bit - 1)
        stage_ms[nm] = time_loop(lambda: call(bit), reps, torch)
    if cu is not None:
        nchunk_heads = int(sum(-(-int(L) // 64) for L in np.diff(x.cu_seqlens))) * H
    else:
        nchunk_heads = B * (T // 64) * H
    fl = bwd_flops_per_chunk_head(64, K, V)
    dom = max(stage_ms, key=stage_ms.get)
    cpu = None if args.no_cpu_baseline else cpu_baseline_bwd(x, d_o, d_f)
    # measured HBM bytes of the dominant launch(es) from the committed counter runs, if taken on this source
    traffic = None
    tp = os.path.join(ROOT, "profiles", f"traffic_kda_bwd_{WORKLOADS[args.workload]['name']}.json")
    if os.path.exists(tp):
        rec = json.load(open(tp))
        chunk = (["bwd_chunk_fused_kernel"] if x.dtype == "bf16" else ["bwd_chunk_mm_kernel", "bwd_chunk_elem_kernel"])
        names = {"prep": ["bwd_prep_kernel"], "states_fwd": ["bwd_states_fwd_kernel"],
                 "states_bwd": ["bwd_states_bwd_kernel"], "chunk": chunk}
        if rec.get("source_sha256_16") == kernel_source_hash("bwd") and all(n in rec["kernels"] for n in names[dom]):
            traffic = sum(rec["kernels"][n]["traffic_bytes"] for n in names[dom])
    ach = fl[dom] * nchunk_heads / (stage_ms[dom] / 1e3) / 1e12
    if dom == "chunk":
        # the chunk-gradient launch(es) stream their operands through the fp32
        # slab (for bf16 inputs one fused kernel with its products on MFMA): bound
        # by memory traffic, so the roofline is HBM on the bytes they cannot avoid
        # (see bwd_chunk_alg_bytes_per_token_head), with the measured bytes beside them
        ntok_heads = (int(x.cu_seqlens[-1]) if cu is not None else B * T) * H
        alg_b = bwd_chunk_alg_bytes_per_token_head(K, V, 2 if x.dtype == "bf16" else 4) * ntok_heads
        gbps = alg_b / (stage_ms[dom] / 1e3) / 1e9
        kname = "bwd_chunk_fused" if x.dtype == "bf16" else "bwd_chunk (chunk_mm + chunk_elem)"
        roof = {"kernel": kname, "bound": "hbm", "achieved": gbps,
                "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": gbps * 1e9 / PEAK_HBM, "traffic": traffic,
                "alg_bytes_per_launch": alg_b, "traffic_over_alg": None if traffic is None else traffic / alg_b,
                "flop_rate_TFLOPs": ach}
    else:
        roof = {"kernel": f"bwd_{dom}", "bound": "alu", "achieved": ach, "peak": PEAK_FP32 / 1e12,
                "unit": "TFLOP/s", "frac": ach * 1e12 / PEAK_FP32, "traffic": traffic,
                "alg_flops_per_launch": fl[dom] * nchunk_heads}
    print(json.dumps({
        "metric": "KDA chunk-bwd tokens/s (dq, dk, dv, dg, dbeta, dh0)", "value": B * T / (ms / 1e3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16 inputs; chunk and state-gradient products on bf16 MFMA operands with f32 accumulation; "
                  "f32 states and gradients"
                  if x.dtype == "bf16" else "f32 inputs, f32 arithmetic and gradients"),
        "data": "synthetic (seeded numpy generators)",
        "config": {"workload": WORKLOADS[args.workload]["name"] + "_backward", "B": B, "T": T, "H": H, "K": K,
                   "V": V},
        "stage_ms": stage_ms,
        "roofline": roof,
        "cpu_baseline": cpu,
    }), flush=True)


def cpu_baseline_bwd(x, d_o, d_f, target_s=10.0):
    """Time the float64 backward oracle (reverse-mode differentiation of the token
    recurrence) on one head of the workload, over a prefix grown to about
    target_s of work; tokens/s scaled to all heads."""
    import oracle.kda_oracle as orc
    B, T, H, K = x.q.shape
    tok = 128
    while True:
        t0 = time.perf_counter()
        c0 = time.process_time()
        sl = lambda a: a[:1, :tok, :1]
        orc.kda_recurrent_vjp(sl(x.q), sl(x.k), sl(x.v), sl(x.g), x.beta[:1, :tok, :1], x.scale, sl(d_o),
                              d_f[:1, :1], None if x.initial_state is None else x.initial_state[:1, :1])
        wall = time.perf_counter() - t0
        cpu = time.process_time() - c0
        if wall * 2 >= target_s or tok * 2 > T:
            break
        tok = min(T, tok * max(2, int(target_s / max(wall, 1e-3) / 2)))
    hi = host_info()
    import torch
    return {
        "value": tok / wall / H, "unit": "tokens/s", "cores": torch.get_num_threads(), "kind": "oracle",
        "sample": f"float64 backward oracle (torch autograd over the token recurrence) on head 0 of {H}, "
                  f"first {tok} of {T} tokens ({wall:.1f} s wall, {cpu:.1f} s CPU, {cpu / wall:.1f} cores busy "
                  f"on average); tokens/s scaled to all {H} heads",
        **hi,
    }


def bench_layer(args, torch, kda):
    """The KDA layer around the core (workload 4): one step = the whole layer
    forward over a [B, T, M] bf16 input, inputs and weights resident in HBM."""
    from kimi_delta_attention_03_amd.synthetic import WORKLOADS, layer_inputs
    cfg = WORKLOADS[4]
    B, T, M, H, D = cfg["B"], cfg["T"], cfg["M"], cfg["H"], cfg["D"]
    x, w = layer_inputs(B=B, T=T, M=M, H=H, D=D, seed=cfg["seed"])
    bf = ("Wqkv", "Wb", "Wad", "Wau", "Wgd", "Wgu", "Wo")
    wd = {n: torch.from_numpy(a).to(torch.bfloat16 if n in bf else torch.float32).to("cuda:0") for n, a in w.items()}
    xd = torch.from_numpy(x).to(torch.bfloat16).to("cuda:0")
    # the input-projection weights packed back to back once, as at model load:
    # the layer then reads them in place
    layer = kda.KdaLayer(kda.pack_layer_weights(wd), B, T, H, D)
    for _ in range(args.warmup):
        layer(xd)
    ms = time_loop(lambda: layer(xd), args.steps, torch)
    r, rg, HD = w["Wad"].shape[0], w["Wgd"].shape[0], H * D
    NP = 3 * HD + H + r + rg
    BT = B * T
    gemm = 2.0 * BT * (M * NP + r * HD + rg * HD + HD * M)
    core = alg_flops_per_chunk_head(64, D, D) * B * (T // 64) * H
    print(json.dumps({
        "metric": "KDA layer forward tokens/s (workload 4)", "value": BT / (ms / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "dtype": "bf16 (fp32 core)", "data": "synthetic (seeded numpy generators; random-init weights)",
        "config": {"workload": cfg["name"], "B": B, "T": T, "M": M, "H": H, "D": D, "gate_rank": int(r),
                   "out_gate_rank": int(rg)},
        "gemm_tflops": gemm / (ms / 1e3) / 1e12, "core_gflop": core / 1e9,
        "roofline": {"kernel": "whole layer (projection FLOPs over the step)", "bound": "mfma",
                     "achieved": gemm / (ms / 1e3) / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                     "frac": gemm / (ms / 1e3) / PEAK_BF16, "traffic": None},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--mode", choices=["forward", "decode", "affine", "backward", "gated"], default="forward",
                    help="decode: one kda_decode_step over B=256 sequences x H=32 (K=V=128, bf16); "
                         "affine: stage 1+2 plus the affine summaries on the workload's shape; "
                         "backward: kda_chunk_bwd on the workload's shape; "
                         "gated: the forward with the gate activation inside stage 1+2")
    ap.add_argument("--gate", choices=["lower_bound_sigmoid", "softplus"], default="lower_bound_sigmoid")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the KDA forward here is a single-GPU kernel path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        ms = time_loop(lambda: dst.copy_(src), 5, torch)
        print(json.dumps({"copy_bytes": n, "ms": ms, "GBps_read_plus_write": 2 * n / ms / 1e6}), flush=True)
        return
    import kimi_delta_attention_03_amd as kda
    from kimi_delta_attention_03_amd.synthetic import WORKLOADS, workload
    if args.workload == 4:
        return bench_layer(args, torch, kda)
    if args.mode == "decode":
        return bench_decode(args, torch, kda)
    if args.mode == "affine":
        return bench_affine(args, torch, kda, WORKLOADS, workload)
    if args.mode == "backward":
        return bench_backward(args, torch, kda, WORKLOADS, workload)
    if args.mode == "gated":
        return bench_gated(args, torch, kda, WORKLOADS, workload)

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    x = workload(args.workload)
    t_gen = time.perf_counter() - t_gen
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    to = lambda a, d: torch.from_numpy(a).to(d).to(dev)
    q, k, v, g, beta = (to(a, dt) for a in (x.q, x.k, x.v, x.g, x.beta))
    init = None if x.initial_state is None else to(x.initial_state, torch.float32)
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(dev)
    B, T, H, K = x.q.shape
    V = x.v.shape[3]
    fwd = kda.KdaForward(q, k, v, g, beta, scale=x.scale, initial_state=init, cu_seqlens=cu)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    ms_step = time_loop(fwd, args.steps, torch)

    # per-kernel durations on the launch stream. kda_chunk_fwd runs long
    # fixed-length inputs in segments along T (stage 1+2 then stage 3+4 of each
    # segment, the state handed over in fp32); the same launches are replayed
    # here segment by segment (B = 1: each segment is a contiguous view) with
    # HIP events around each, giving the average duration of one launch.
    info = kda.workspace_layout(fwd.params)
    nseg = int(info.segments)
    if nseg > 1 and B == 1:
        ts = int(info.segment_chunks) * 64
        seg_calls, states = [], [init] + [torch.empty((1, H, K, V), dtype=torch.float32, device=dev)
                                          for _ in range(nseg)]
        seg_ws = None
        for i in range(nseg):
            sl = slice(i * ts, min(T, (i + 1) * ts))
            c = kda.KdaForward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], scale=x.scale,
                               initial_state=states[i], out=fwd.o[:, sl], workspace=seg_ws)
            c.final_state = states[i + 1]
            seg_ws = c.workspace
            seg_calls.append(c)
        t12 = t34 = 0.0
        reps = max(1, args.kernel_reps)
        for _ in range(reps):
            for c in seg_calls:
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(); c.stage12(); e1.record(); c.stage34(); e2.record()
                torch.cuda.synchronize()
                t12 += e0.elapsed_time(e1)
                t34 += e1.elapsed_time(e2)
        ms12, ms34 = t12 / (reps * nseg), t34 / (reps * nseg)     # per launch
        launches = nseg
        seg_token_heads = [min(T, (i + 1) * ts) - i * ts for i in range(nseg)]
        del seg_calls, states
    else:
        ms12 = time_loop(fwd.stage12, args.kernel_reps, torch)
        ms34 = time_loop(fwd.stage34, args.kernel_reps, torch)
        launches = 1
        seg_token_heads = [T]

    tokens = B * T
    token_heads = tokens * H
    elem = 2 if x.dtype == "bf16" else 4
    b12, b34 = alg_bytes_per_token_head(K, V, elem, elem, elem)
    if cu is not None:
        nchunk_heads = int(sum(-(-int(L) // 64) for L in np.diff(x.cu_seqlens))) * H
    else:
        nchunk_heads = B * (T // 64) * H
    flops = alg_flops_per_chunk_head(64, K, V) * nchunk_heads
    bytes_total = (b12 + b34) * token_heads
    peak_mma = PEAK_BF16 if x.dtype == "bf16" else PEAK_FP32
    s_step = ms_step / 1e3
    dom = "stage12" if ms12 >= ms34 else "stage34"
    # algorithmic bytes of one launch (the average segment)
    dom_bytes = (b12 if dom == "stage12" else b34) * token_heads / launches
    dom_ms = ms12 if dom == "stage12" else ms34
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9

    cfg = WORKLOADS[args.workload]
    copy_Bps = copy_rate(torch)
    if cu is not None:
        lens = np.diff(x.cu_seqlens).astype(np.int64)
        seg = {"num_seqs": int(len(lens)), "min": int(lens.min()), "median": float(np.median(lens)),
               "max": int(lens.max()), "mean": float(lens.mean())}
        aligned = int(sum(-(-int(L) // 64) * 64 for L in lens))
    else:
        seg = None
        aligned = tokens
    result = {
        "metric": METRIC,
        "value": tokens / s_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic (seeded numpy generators; no dataset)",
        "config": {"workload": cfg["name"], "B": B, "T": T, "H": H, "K": K, "V": V, "chunk": 64,
                   "state": "fp32", "initial_state": init is not None, "varlen": cu is not None},
        "tflops": flops / s_step / 1e12,
        "mfma_frac": flops / s_step / peak_mma,
        "hbm_alg_GBps": bytes_total / s_step / 1e9,
        "hbm_alg_frac": bytes_total / s_step / PEAK_HBM,
        "kernels_ms": {"stage12": ms12, "stage34": ms34, "launches_per_step": launches,
                       "per": "one launch (one segment along T)" if launches > 1 else "one launch"},
        "hbm_alg_frac_of_copy": bytes_total / s_step / copy_Bps,
        "copy_GBps_measured": copy_Bps / 1e9,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": achieved * 1e9 / PEAK_HBM,
                     "traffic": measured_traffic(cfg["name"], dom),
                     "alg_bytes_per_launch": dom_bytes, "launch_ms": dom_ms},
        "record": {"library": build_info(),
                   "tokens_logical": tokens, "tokens_chunk_aligned": aligned, "sequence_lengths": seg,
                   "t_segments": {"count": nseg, "chunks_per_segment": int(info.segment_chunks) if nseg > 1 else None},
                   "flags": {"use_qk_l2norm": False, "gate": "log_decay (g given)",
                             "initial_state": init is not None, "final_state": True, "chunk_size": 64},
                   "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                   "device": torch.cuda.get_device_name(0),
                   "cus": torch.cuda.get_device_properties(0).multi_processor_count,
                   "sync": "torch.cuda.synchronize + HIP events on the launch stream",
                   "timed": "end to end per step: one kda_chunk_fwd call (chunk map if varlen, stage 1+2, "
                            "stage 3+4) per step, inputs resident, workspace preallocated; kernels_ms times "
                            "each stage alone",
                   "input_gen_s": round(t_gen, 1)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
