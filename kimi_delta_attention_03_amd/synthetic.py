"""Seeded synthetic inputs for the KDA forward (shared by tests and benchmark).

This module only draws random numbers and shapes them; it performs none of
the attention arithmetic. Both the HIP path and the float64 oracle consume
the arrays it returns. All arrays are numpy float32; when a workload is
"bf16" every float array except the initial state already holds values that
are exactly representable in bfloat16 (round-to-nearest-even), so handing it
to either side is exact.

Recipe (per workload; numpy PCG64, fixed draw order
lengths -> q -> k -> v -> g -> beta -> initial_state -> layer weights):
  q, k  ~ N(0, 1), L2-normalised over the head dim in fp32 (then rounded)
  v     ~ N(0, 1)
  g     = -5 * sigmoid(N(0, 1))  per channel, natural-log decay in (-5, 0)
  beta  = sigmoid(N(0, 1))
  initial_state ~ N(0, 0.1^2) fp32 when requested, else none (zeros)
  varlen lengths ~ Uniform{1..8192}, multiples of 64 redrawn
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["round_bf16", "CoreInputs", "core_inputs", "workload", "WORKLOADS",
           "layer_inputs", "varlen_lengths", "gate_inputs"]


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _sigmoid32(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float32)))).astype(np.float32)


@dataclass
class CoreInputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    scale: float
    dtype: str                     # "bf16" or "fp32": element type of q, k, v, g, beta
    initial_state: np.ndarray | None = None
    cu_seqlens: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.q.shape


def varlen_lengths(rng, n, max_len, chunk=64):
    """n lengths uniform in [1, max_len], none a multiple of `chunk`."""
    out = []
    while len(out) < n:
        L = int(rng.integers(1, max_len + 1))
        if L % chunk != 0:
            out.append(L)
    return np.asarray(out, dtype=np.int64)


def core_inputs(B, T, H, K, V, dtype="bf16", seed=0, init_std=None, lengths=None,
                normalize=True, scale=None, g_low=-5.0):
    """Draw one KDA-core workload.

    lengths: if given, B must be 1 and T is ignored; the sequences are packed
    along T with cu_seqlens = [0, cumsum(lengths)] and one initial state per
    sequence. g_low sets the most negative decay (g = g_low * sigmoid(N)).
    """
    rng = np.random.default_rng(seed)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        if B != 1:
            raise ValueError("packed variable-length input needs B == 1")
        T = int(lengths.sum())
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        N = len(lengths)
    else:
        cu = None
        N = B

    def normal(shape):
        return rng.standard_normal(shape, dtype=np.float32)

    q = normal((B, T, H, K))
    k = normal((B, T, H, K))
    if normalize:
        q /= np.maximum(np.sqrt(np.sum(q * q, axis=-1, keepdims=True)), 1e-6)
        k /= np.maximum(np.sqrt(np.sum(k * k, axis=-1, keepdims=True)), 1e-6)
    v = normal((B, T, H, V))
    g = (g_low * _sigmoid32(normal((B, T, H, K)))).astype(np.float32)
    beta = _sigmoid32(normal((B, T, H)))
    init = None
    if init_std is not None:
        init = (init_std * normal((N, H, K, V))).astype(np.float32)
    if dtype == "bf16":
        q, k, v, g, beta = (round_bf16(x) for x in (q, k, v, g, beta))
    elif dtype != "fp32":
        raise ValueError(dtype)
    if scale is None:
        scale = float(K) ** -0.5
    return CoreInputs(q=q, k=k, v=v, g=g, beta=beta, scale=scale, dtype=dtype,
                      initial_state=init, cu_seqlens=cu,
                      meta={"seed": seed, "B": B, "T": T, "H": H, "K": K, "V": V})


def grad_inputs(B, T, H, V, N, K=None, seed=0, dtype="bf16", final=True):
    """Incoming gradients for the backward: d_o [B, T, H, V] ~ N(0,1) (rounded to
    bf16 for dtype "bf16") and d_final [N, H, K, V] ~ N(0,1) fp32 (or None)."""
    rng = np.random.default_rng(seed)
    d_o = rng.standard_normal((B, T, H, V), dtype=np.float32)
    if dtype == "bf16":
        d_o = round_bf16(d_o)
    d_final = rng.standard_normal((N, H, K if K is not None else V, V), dtype=np.float32) if final else None
    return d_o, d_final


# The five workloads of this project, smallest first. Index 2 is the headline.
WORKLOADS = {
    0: dict(name="tiny_fp32", B=1, H=2, T=256, K=64, V=64, dtype="fp32", init_std=None, seed=1000),
    1: dict(name="core_bf16_B2_H16_T4096", B=2, H=16, T=4096, K=128, V=128, dtype="bf16",
            init_std=None, seed=1001),
    2: dict(name="core_bf16_B1_H32_T32768", B=1, H=32, T=32768, K=128, V=128, dtype="bf16",
            init_std=0.1, seed=1002),
    3: dict(name="varlen_bf16_16seq_H32", B=1, H=32, T=None, K=128, V=128, dtype="bf16",
            init_std=0.1, seed=1003, nseq=16, max_len=8192),
    4: dict(name="layer_B4_T8192_M2048_H16_D128", B=4, T=8192, M=2048, H=16, D=128, seed=1004),
}


def workload(i, seed=None, **over):
    """Inputs of core workload i (0-3), optionally overriding fields."""
    cfg = dict(WORKLOADS[i])
    cfg.update(over)
    seed = cfg["seed"] if seed is None else seed
    if i == 3:
        rng = np.random.default_rng(seed)
        lengths = varlen_lengths(rng, cfg["nseq"], cfg["max_len"])
        # the rest of the draws continue from a derived seed so that the
        # length draw comes first and everything stays reproducible
        return core_inputs(1, None, cfg["H"], cfg["K"], cfg["V"], cfg["dtype"],
                           seed=seed + 7919, init_std=cfg["init_std"], lengths=lengths)
    if i == 4:
        raise ValueError("workload 4 is the layer; use layer_inputs()")
    return core_inputs(cfg["B"], cfg["T"], cfg["H"], cfg["K"], cfg["V"], cfg["dtype"],
                       seed=seed, init_std=cfg["init_std"])


def gate_inputs(B, T, H, K, seed=0, a_log_range=(0.5, 1.5), bias_std=0.5, dtype="bf16", clip=(-3.0, 2.0)):
    """Raw gate values [B, T, H, K] ~ N(0,1) clipped to `clip` (rounded to bf16
    for dtype "bf16"), A_log = log U[a_log_range] per head and dt_bias ~
    N(0, bias_std^2) per (head, channel) as fp32."""
    rng = np.random.default_rng(seed)
    raw = np.clip(rng.standard_normal((B, T, H, K), dtype=np.float32), *clip).astype(np.float32)
    if dtype == "bf16":
        raw = round_bf16(raw)
    A_log = np.log(rng.uniform(*a_log_range, size=H)).astype(np.float32)
    dt_bias = (bias_std * rng.standard_normal((H, K))).astype(np.float32)
    return raw, A_log, dt_bias


def layer_inputs(B=4, T=8192, M=2048, H=16, D=128, rank=128, seed=1004):
    """x ~ N(0,1) and random-init layer weights, all bf16-representable float32.

    Linear weights are [out, in] with N(0, 1/fan_in) entries; depthwise conv
    weights N(0, 0.5^2); A_log = log U[1, 16]; dt_bias = inverse softplus of
    dt = exp(U[ln 1e-3, ln 1e-1]); RMSNorm weight ones. A_log and dt_bias
    stay fp32.
    """
    rng = np.random.default_rng(seed)
    HD = H * D

    def lin(o, i):
        return round_bf16(rng.standard_normal((o, i), dtype=np.float32) * np.float32(i ** -0.5))

    x = round_bf16(rng.standard_normal((B, T, M), dtype=np.float32))
    w = {
        "Wqkv": lin(3 * HD, M),
        "conv_q": round_bf16(0.5 * rng.standard_normal((HD, 4), dtype=np.float32)),
        "conv_k": round_bf16(0.5 * rng.standard_normal((HD, 4), dtype=np.float32)),
        "conv_v": round_bf16(0.5 * rng.standard_normal((HD, 4), dtype=np.float32)),
        "Wb": lin(H, M),
        "Wad": lin(rank, M),
        "Wau": lin(HD, rank),
        "A_log": np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32),
    }
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=HD))
    w["dt_bias"] = (dt + np.log(-np.expm1(-dt))).astype(np.float32)   # softplus^-1(dt)
    w["Wgd"] = lin(D, M)
    w["Wgu"] = lin(HD, D)
    w["norm_w"] = np.ones(D, dtype=np.float32)
    w["Wo"] = lin(M, HD)
    return x, w
