"""Shared helpers for the GPU tests: tensor transfer, error metric, workspace decoding."""
from __future__ import annotations

import numpy as np

# tolerances on max|gpu - oracle| / max|oracle|, per tensor
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def to_dev(x, dtype):
    """numpy float32 array -> torch tensor on cuda:0 (exact for bf16-representable values)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype).to("cuda:0")


def dev_inputs(x):
    """CoreInputs -> dict of device tensors for chunk_fwd."""
    import torch
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    d = dict(q=to_dev(x.q, dt), k=to_dev(x.k, dt), v=to_dev(x.v, dt), g=to_dev(x.g, dt),
             beta=to_dev(x.beta, dt))
    d["initial_state"] = None if x.initial_state is None else to_dev(x.initial_state, torch.float32)
    d["cu_seqlens"] = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to("cuda:0")
    return d


def host(t):
    return t.float().cpu().numpy()


def phys(g, t):
    return 4 * g + t if t < 4 else 16 + 4 * g + t - 4


def _frag_index_tables():
    lanes = np.arange(64)
    g, i = lanes >> 4, lanes & 15
    rows = np.repeat(i[:, None], 8, 1)                                  # [lane, t]
    cols = np.array([[phys(gg, t) for t in range(8)] for gg in g])      # [lane, t]
    return rows, cols


_FR, _FC = _frag_index_tables()


def decode_frag8(arr, n_rt, n_kb):
    """[n_rt][n_kb][64][8] fragment array -> dense [16 n_rt, 32 n_kb] matrix."""
    a = np.asarray(arr, np.float64).reshape(n_rt, n_kb, 64, 8)
    out = np.zeros((16 * n_rt, 32 * n_kb))
    for rt in range(n_rt):
        for kb in range(n_kb):
            out[16 * rt + _FR, 32 * kb + _FC] = a[rt, kb]
    return out


def decode_acc(arr, n_vb, n_rt=4):
    """U fragments [n_vb][n_rt][64][4] -> dense [16 n_rt, 16 n_vb]."""
    a = np.asarray(arr, np.float64).reshape(n_vb, n_rt, 64, 4)
    lanes = np.arange(64)
    g, i = lanes >> 4, lanes & 15
    out = np.zeros((16 * n_rt, 16 * n_vb))
    for vb in range(n_vb):
        for rt in range(n_rt):
            for r in range(4):
                out[16 * rt + 4 * g + r, 16 * vb + i] = a[vb, rt, :, r]
    return out


def decode_aq(arr):
    """The 6 stored Aqk fragments -> dense [64, 64]; fragment (rt, kb) sits at
    index rt for rt < 2 (kb = 0 only) and 2 rt - 2 + kb otherwise."""
    a = np.asarray(arr, np.float64).reshape(6, 64, 8)
    out = np.zeros((64, 64))
    for rt in range(4):
        for kb in range(2 if rt >= 2 else 1):
            idx = rt if rt < 2 else 2 * rt - 2 + kb
            out[16 * rt + _FR, 32 * kb + _FC] = a[idx]
    return out


def decode_record(ws_bytes, info, h, p, K, V, bf16, H):
    """Decode the stage-1+2 record of (head h, chunk slot p) into dense matrices
    (records are chunk-major: index p * H + h)."""
    import torch
    base = info.records_offset + (p * H + h) * info.record_bytes
    rec = ws_bytes[base:base + info.record_bytes]

    def elems(off, n):
        raw = rec[off:off + n * info.elem_bytes]
        if bf16:
            t = torch.from_numpy(raw.copy()).view(torch.bfloat16).float()
            return t.numpy()
        return raw.copy().view(np.float32)

    C = 64
    out = {
        "W": decode_frag8(elems(info.off_w, C * K), 4, K // 32),
        "qg": decode_frag8(elems(info.off_qg, C * K), 4, K // 32),
        "kgT": decode_frag8(elems(info.off_kg, C * K), K // 16, 2),
        "Aqk": decode_aq(elems(info.off_aq, 6 * 512)),
        "U": decode_acc(elems(info.off_u, C * V), V // 16),
        "gamma": rec[info.off_gamma:info.off_gamma + 4 * K].copy().view(np.float32).astype(np.float64),
    }
    return out
