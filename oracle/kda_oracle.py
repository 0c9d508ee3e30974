"""Float64 CPU oracle for the chunkwise Kimi Delta Attention (KDA) forward.

TEST INFRASTRUCTURE ONLY. This module is the independent reference that the
HIP path is checked against. Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code, constants or helpers with the HIP library.

Everything is computed in numpy float64. Inputs given in bf16 or fp32 are
widened exactly, so the oracle sees the very values the GPU sees.

Sources (the three pages this work is based on):
  [Blog]     "KDA Doesn't Care About the Future" (drisspg.github.io), sections
             "Chunkwise KDA in Broad Strokes", "Chunkwise Aqk",
             "Trace Aqk back to the base recurrence".
  [K3]       "KDAChunkwise" (Kimi K3 docs), sections "FP32 core and log-space
             decay", "Constructing the triangular interaction system",
             "Carrying one state between chunks", "Returning to the model
             dimension".
  [Tokamax]  Tokamax "chunk_kda_fwd design doc" (openxla.org), sections
             3.5, 4.3.2, 9.1.2 (Paper Eq. 1), 9.1.3, 9.1.5 (Paper Eq. 6-7),
             9.1.6 (Paper Eq. 8-9), 9.1.7, 9.1.8.

Tensor conventions (token-major, the layout the HIP library uses too):
  q, k, g : [B, T, H, K]   g is the natural-log decay, g <= 0
  v       : [B, T, H, V]
  beta    : [B, T, H]
  initial_state / final_state : [N, H, K, V] with N = B (fixed length) or the
  number of sequences (variable length, B == 1 and cu_seqlens = [N + 1]).

The steps are small module-level functions on purpose: the test suite swaps
single steps for plausible mistakes and checks that the pins catch them.

Parity status:
  kda_recurrent, kda_chunkwise, varlen handling, l2norm,
  chunk_affine_summary     -> pinned (closed forms, invariants, exact recall,
                              brute force and cross-checks in tests/).
  kda_recurrent_vjp        -> pinned (central finite differences of
                              kda_recurrent, the beta = 0 closed form and
                              the varlen / l2norm cases in tests/).
  kda_layer_ref            -> pinned: its steps (conv against numpy.convolve,
                              RMSNorm by closed forms with eps != 0, the gate
                              by closed forms) and their composition (a
                              single-token closed form worked by hand, a
                              reduced-weight case composed from the pinned
                              token recurrence, per-head RMS, causality), with
                              planted mistakes in each step caught in tests/.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular
from scipy.special import expit

__all__ = [
    "l2norm",
    "kda_recurrent",
    "kda_chunkwise",
    "chunk_terms",
    "chunk_affine_summary",
    "compose_affine",
    "segments",
    "kda_layer_ref",
    "depthwise_causal_conv",
    "silu",
    "sigmoid",
    "rms_norm",
    "short_conv_silu",
    "qk_features",
    "head_rms_norm",
    "output_gate",
    "decay_gate",
    "gate_activation",
    "kda_recurrent_vjp",
]


# --------------------------------------------------------------------------
# small elementwise pieces
# --------------------------------------------------------------------------
def l2norm(x, eps=1e-6):
    """x / max(||x||_2, eps) over the last axis.

    [K3] "FP32 core and log-space decay": q and k are unit-normalised along the
    head dimension with F.normalize and eps=1e-6; [Tokamax] 3.1 lists the same
    optional q/k L2 normalisation in preprocessing.
    """
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def sigmoid(x):
    return expit(np.asarray(x, dtype=np.float64))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def gate_activation(g_raw, A_log, dt_bias, mode, lower_bound=None):
    """Log decay from a raw gate ([Tokamax] 9.1.3, gate inside the kernel).

    g_raw: [B, T, H, K]; A_log: [H]; dt_bias: [H, K] (or [H*K], or None).
    x = g_raw + dt_bias and lambda_h = exp(A_log_h); then
      mode "softplus":            g = -lambda_h * softplus(x)
      mode "lower_bound_sigmoid": g = lower_bound * sigmoid(lambda_h * x)
    softplus(x) = log(1 + e^x), evaluated as logaddexp(0, x).
    """
    x = _f64(g_raw)
    H, K = x.shape[-2], x.shape[-1]
    if dt_bias is not None:
        x = x + _f64(dt_bias).reshape(H, K)
    lam = np.exp(_f64(A_log)).reshape(H, 1)
    if mode == "softplus":
        return -lam * np.logaddexp(0.0, x)
    if mode == "lower_bound_sigmoid":
        return float(lower_bound) * expit(lam * x)
    raise ValueError(mode)


def segments(B, T, cu_seqlens):
    """List of (batch_row, start, end) segments.

    Fixed length: one segment [0, T) per batch row. Variable length
    ([Tokamax] 9.1.7): B must be 1 and segment n is [cu[n], cu[n+1]).
    """
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    if B != 1:
        raise ValueError("variable-length input requires B == 1")
    if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu[:-1], cu[1:])):
        raise ValueError("cu_seqlens must be non-decreasing from 0 to T")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


# --------------------------------------------------------------------------
# Oracle R: token recurrence ([Tokamax] 9.1.2, Paper Eq. 1, delta-correction
# form; [Blog] "Chunkwise KDA in Broad Strokes", steps 0-5)
# --------------------------------------------------------------------------
def decay_state(S, g_t):
    """S_bar = Diag(alpha_t) S with alpha_t = exp(g_t), per key channel."""
    return np.exp(g_t)[..., :, None] * S


def prediction_error(S_bar, k_t, v_t):
    """e_t = v_t - S_bar^T k_t  (read the value stored at key k_t)."""
    return v_t - np.einsum("hkv,hk->hv", S_bar, k_t)


def delta_write(S_bar, k_t, e_t, beta_t):
    """S_t = S_bar + beta_t k_t e_t^T  (rank-1 correction at key k_t)."""
    return S_bar + beta_t[:, None, None] * k_t[:, :, None] * e_t[:, None, :]


def read_output(S_t, q_t, scale):
    """o_t = scale * S_t^T q_t  (read after this token's write)."""
    return scale * np.einsum("hkv,hk->hv", S_t, q_t)


def kda_recurrent(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
                  use_qk_l2norm=False, eps=1e-6):
    """Token-by-token KDA recurrence, float64. Returns (o, final_state).

    For each segment and head, S starts at initial_state (zeros if None) and
    every token applies decay -> prediction error -> delta write -> read, the
    order fixed by [Tokamax] 9.1.2 ("decay, then correct") and [Blog] steps
    (0)-(5) (the read uses the state after the current token's write).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    if use_qk_l2norm:
        q, k = l2norm(q, eps), l2norm(k, eps)
    segs = segments(B, T, cu_seqlens)
    o = np.zeros((B, T, H, V))
    final = np.zeros((len(segs), H, K, V))
    init = _f64(initial_state)
    for n, (b, s0, s1) in enumerate(segs):
        S = np.zeros((H, K, V)) if init is None else init[n].copy()
        for t in range(s0, s1):
            S_bar = decay_state(S, g[b, t])
            e = prediction_error(S_bar, k[b, t], v[b, t])
            S = delta_write(S_bar, k[b, t], e, beta[b, t])
            o[b, t] = read_output(S, q[b, t], scale)
        final[n] = S
    return o, final


# --------------------------------------------------------------------------
# Oracle C: chunkwise form ([Tokamax] 9.1.3-9.1.6, Paper Eq. 6-9;
# [K3] "Constructing the triangular interaction system",
# "Carrying one state between chunks")
# --------------------------------------------------------------------------
def chunk_cumsum(g_chunk):
    """Chunk-local inclusive cumulative log decay, natural log.

    [Tokamax] 9.1.3: G^r sums the gates of positions 1..r of this chunk (the
    current token included), restarted in every chunk. Kept in natural log
    here; the pages' log2 form only rescales it.
    """
    return np.cumsum(g_chunk, axis=0)


def decay_ratio(G):
    """rho[i, j] = exp(G_i - G_j) for j <= i, 0 above the diagonal.

    [Tokamax] 9.1.3 defines the ratio as the decay a write at j sees by
    position i; [Blog] "Chunkwise Aqk" explains the j+1..i span. Masked
    exponents are replaced before exp, so nothing non-finite is formed.
    Shape: (c, c, H, K).
    """
    c = G.shape[0]
    diff = G[:, None] - G[None, :]
    causal = np.tril(np.ones((c, c), dtype=bool))
    diff = np.where(causal[:, :, None, None], diff, -np.inf)
    return np.exp(diff)


def relation_qk(qc, kc, rho, scale):
    """Aqk[h, i, j] = scale * sum_d q_{i,d} k_{j,d} rho[i,j,d], j <= i.

    [Blog] "Chunkwise Aqk" (diagonal included); [Tokamax] 9.1.5 includes the
    attention scale in Aqk.
    """
    return scale * np.einsum("ihd,jhd,ijhd->hij", qc, kc, rho)


def relation_kk(kc, bc, rho):
    """L[h, i, j] = beta_i * sum_d k_{i,d} k_{j,d} rho[i,j,d], j < i.

    [Tokamax] 9.1.5: L = StrictTril(D_beta K+ (K-)^T); the beta of the later
    position i multiplies row i ([K3], section "Constructing the triangular
    interaction system", states the same row scaling).
    """
    c = kc.shape[0]
    strict = np.tril(np.ones((c, c)), -1)
    return bc.T[:, :, None] * np.einsum("ihd,jhd,ijhd->hij", kc, kc, rho) * strict


def solve_unit_lower(Lmat):
    """A = (I + L)^{-1} for each head, L strictly lower triangular.

    [Tokamax] 9.1.5 ("A_c = (I + L_c)^{-1}"), computed as an exact triangular
    solve against the identity ([K3]: a batched triangular solve, not a
    generic inverse).
    """
    H, c, _ = Lmat.shape
    I = np.eye(c)
    return np.stack([solve_triangular(I + Lmat[h], I, lower=True, unit_diagonal=True)
                     for h in range(H)])


def wy_factors(A, kc, vc, bc, G):
    """W = A (D_beta K+), U = A (D_beta V) with K+ = k * exp(G).

    [Tokamax] 9.1.5, Paper Eq. 6-7: M = (I + L)^{-1} D_beta, W = M K+,
    U = M V; beta multiplies on the right of the inverse ([K3]: T_b is
    T_UT Diag(beta), not Diag(beta) T_UT).
    """
    Kplus = kc * np.exp(G)
    bK = (bc[..., None] * Kplus).transpose(1, 0, 2)  # (H, c, K)
    bV = (bc[..., None] * vc).transpose(1, 0, 2)     # (H, c, V)
    return A @ bK, A @ bV


def gated_keys(kc, G):
    """kg_r = k_r * exp(G_C - G_r): each write carried to the chunk end.

    [Tokamax] 9.1.5 (bar K); [K3], section "Carrying one state between
    chunks": the decayed keys move every key of the chunk forward to the
    chunk's last position. Shape (H, c, K).
    """
    return (kc * np.exp(G[-1][None] - G)).transpose(1, 0, 2)


def gated_queries(qc, G, scale):
    """scale * q * exp(G): the read of the chunk-start state ([Tokamax] 9.1.6)."""
    return (scale * qc * np.exp(G)).transpose(1, 0, 2)


def chunk_terms(qc, kc, vc, gc, bc, scale):
    """Everything one chunk contributes, independent of the incoming state.

    Inputs are one chunk of one segment: qc, kc, gc (c, H, K), vc (c, H, V),
    bc (c, H), with c <= chunk size. Returns a dict with G (natural log),
    Aqk, L, A, W, U, kg, qg (head-first) and gamma = exp(G_C).
    """
    G = chunk_cumsum(gc)
    rho = decay_ratio(G)
    Aqk = relation_qk(qc, kc, rho, scale)
    Lmat = relation_kk(kc, bc, rho)
    A = solve_unit_lower(Lmat)
    W, U = wy_factors(A, kc, vc, bc, G)
    return {
        "G": G.transpose(1, 0, 2), "Aqk": Aqk, "L": Lmat, "A": A, "W": W, "U": U,
        "kg": gated_keys(kc, G), "qg": gated_queries(qc, G, scale),
        "gamma": np.exp(G[-1]),
    }


def chunk_step(S, terms):
    """One chunk of the ordered state recurrence, [Tokamax] 4.3.2 / 9.1.6.

    V_new = U - W S (uses the chunk-start state); O = qg S + Aqk V_new;
    S_next = Diag(gamma) S + kg^T V_new. Returns (O (H, c, V), S_next).
    """
    Vn = terms["U"] - terms["W"] @ S
    O = terms["qg"] @ S + terms["Aqk"] @ Vn
    S_next = terms["gamma"][:, :, None] * S + terms["kg"].transpose(0, 2, 1) @ Vn
    return O, S_next


def kda_chunkwise(q, k, v, g, beta, scale, chunk_size=64, initial_state=None,
                  cu_seqlens=None, use_qk_l2norm=False, eps=1e-6, heads=None,
                  return_terms=False):
    """Chunkwise KDA forward, float64. Returns (o, final_state[, terms]).

    Each segment is cut into chunks of `chunk_size` tokens starting at the
    segment start; a short last chunk is processed with its real length, so
    no chunk spans two segments ([Tokamax] 3.5, 9.1.7). `heads` restricts
    the computation to a subset of heads (o and final_state then carry only
    those heads, in the given order). With return_terms, the per-chunk
    `chunk_terms` dicts are also returned as a list of (segment, start,
    terms).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    if heads is not None:
        heads = list(heads)
        q, k, v, g, beta = (x[:, :, heads] for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    if use_qk_l2norm:
        q, k = l2norm(q, eps), l2norm(k, eps)
    segs = segments(B, T, cu_seqlens)
    init = _f64(initial_state)
    if init is not None and heads is not None:
        init = init[:, heads]
    o = np.zeros((B, T, H, V))
    final = np.zeros((len(segs), H, K, V))
    all_terms = []
    for n, (b, s0, s1) in enumerate(segs):
        S = np.zeros((H, K, V)) if init is None else init[n].copy()
        for c0 in range(s0, s1, chunk_size):
            c1 = min(c0 + chunk_size, s1)
            terms = chunk_terms(q[b, c0:c1], k[b, c0:c1], v[b, c0:c1], g[b, c0:c1],
                                beta[b, c0:c1], scale)
            O, S = chunk_step(S, terms)
            o[b, c0:c1] = O.transpose(1, 0, 2)
            if return_terms:
                all_terms.append((n, c0, terms))
        final[n] = S
    if return_terms:
        return o, final, all_terms
    return o, final


# --------------------------------------------------------------------------
# Affine state summaries ([Tokamax] 9.1.8)
# --------------------------------------------------------------------------
def chunk_affine_summary(terms):
    """S_next = Phi S + Psi with Phi = Diag(gamma) - kg^T W, Psi = kg^T U."""
    kgT = terms["kg"].transpose(0, 2, 1)
    Kdim = kgT.shape[1]
    Phi = terms["gamma"][:, :, None] * np.eye(Kdim)[None] - kgT @ terms["W"]
    Psi = kgT @ terms["U"]
    return Phi, Psi


def compose_affine(first, second):
    """Summary of `first` followed by `second`: (Phi_b Phi_a, Phi_b Psi_a + Psi_b)."""
    Pa, Sa = first
    Pb, Sb = second
    return Pb @ Pa, Pb @ Sa + Sb


# --------------------------------------------------------------------------
# Backward: the vector-Jacobian product of the token recurrence ([Tokamax]
# 4.3.4 and 6.1: the backward returns dq, dk, dv, dg, dbeta and the optional
# dh0 of the same forward map (O, S_final) = F(Q, K, V, G, D_beta, S_0))
# --------------------------------------------------------------------------
def kda_recurrent_vjp(q, k, v, g, beta, scale, d_o, d_final=None, initial_state=None,
                      cu_seqlens=None, use_qk_l2norm=False, eps=1e-6):
    """Gradients of <d_o, o> + <d_final, final_state> for kda_recurrent.

    The forward is the same token recurrence (decay, prediction error, delta
    write, read after the write), restated with torch float64 CPU tensors so
    that reverse-mode differentiation (torch.autograd, a library routine)
    gives the exact vector-Jacobian product. With use_qk_l2norm the gradients
    are those of the un-normalised q and k. Returns a dict with dq, dk, dv,
    dg, dbeta (shapes of the inputs) and dh0 ([N, H, K, V]), float64 numpy.
    """
    import torch

    def leaf(a):
        return torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)

    qt, kt, vt, gt, bt = (leaf(a) for a in (q, k, v, g, beta))
    B, T, H, K = qt.shape
    V = vt.shape[-1]
    segs = segments(B, T, cu_seqlens)
    h0 = leaf(np.zeros((len(segs), H, K, V)) if initial_state is None else initial_state)
    qn, kn = qt, kt
    if use_qk_l2norm:
        qn = qt / torch.clamp(torch.sqrt((qt * qt).sum(-1, keepdim=True)), min=eps)
        kn = kt / torch.clamp(torch.sqrt((kt * kt).sum(-1, keepdim=True)), min=eps)
    outs = [[None] * T for _ in range(B)]
    finals = []
    for n, (b, s0, s1) in enumerate(segs):
        S = h0[n]
        for t in range(s0, s1):
            S_bar = torch.exp(gt[b, t])[:, :, None] * S
            e = vt[b, t] - torch.einsum("hkv,hk->hv", S_bar, kn[b, t])
            S = S_bar + bt[b, t][:, None, None] * kn[b, t][:, :, None] * e[:, None, :]
            outs[b][t] = scale * torch.einsum("hkv,hk->hv", S, qn[b, t])
        finals.append(S)
    zero_row = torch.zeros((H, V), dtype=torch.float64)
    o = torch.stack([torch.stack([r if r is not None else zero_row for r in row]) for row in outs]) \
        if T > 0 else torch.zeros((B, 0, H, V), dtype=torch.float64)
    loss = (o * torch.as_tensor(np.asarray(d_o, dtype=np.float64))).sum()
    if d_final is not None and finals:
        fin = torch.stack(finals)
        loss = loss + (fin * torch.as_tensor(np.asarray(d_final, dtype=np.float64))).sum()
    leaves = (qt, kt, vt, gt, bt, h0)
    if loss.requires_grad:
        grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    else:
        grads = (None,) * len(leaves)
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    return {nm: (np.zeros(lf.shape) if gr is None else gr.detach().numpy())
            for nm, lf, gr in zip(names, leaves, grads)}


# --------------------------------------------------------------------------
# KDA layer around the core ([K3] "From the hidden states to causal Q, K, and
# V", "FP32 core and log-space decay", "Returning to the model dimension";
# [Tokamax] 9.1.3 lower-bound sigmoid gate)
# --------------------------------------------------------------------------
def depthwise_causal_conv(x, w):
    """Depthwise causal 1-D convolution along T with left zero padding.

    x: [B, T, C]; w: [C, k]. out[t, c] = sum_m w[c, m] x[t + m - (k-1), c]:
    a Conv1d with groups = channels applied after padding k-1 zeros on the
    left, so position t only sees positions <= t ([K3] "From the hidden
    states to causal Q, K, and V").
    """
    x = _f64(x)
    w = _f64(w)
    B, T, C = x.shape
    kw = w.shape[1]
    xp = np.concatenate([np.zeros((B, kw - 1, C)), x], axis=1)
    out = np.zeros_like(x)
    for m in range(kw):
        out += w[:, m][None, None, :] * xp[:, m:m + T, :]
    return out


def rms_norm(x, weight, eps):
    """x / sqrt(mean(x^2) + eps) * weight over the last axis (eps inside the root)."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(weight)


def short_conv_silu(p, conv_w):
    """One feature stream of the layer: causal depthwise conv, then SiLU
    ([K3] "From the hidden states to causal Q, K, and V": the projection is
    convolved along time first and the activation follows)."""
    return silu(depthwise_causal_conv(p, conv_w))


def qk_features(p, conv_w, num_heads, head_dim, eps):
    """q or k of the layer: conv -> SiLU, then split into heads and
    L2-normalised over the head dimension ([K3] "FP32 core and log-space
    decay": the normalisation acts on the activated features)."""
    B, T, _ = p.shape
    return l2norm(short_conv_silu(p, conv_w).reshape(B, T, num_heads, head_dim), eps)


def head_rms_norm(o, weight, eps):
    """RMSNorm of the core output per (token, head) over the head dimension
    ([K3] "Returning to the model dimension": the norm is per head, with a
    weight of length D shared by the heads). o: [B, T, H, D]."""
    return rms_norm(o, weight, eps)


def output_gate(x, Wgd, Wgu, num_heads, head_dim):
    """Low-rank output gate sigmoid(x Wgd^T Wgu^T), split into heads
    ([K3] "Returning to the model dimension")."""
    B, T, _ = x.shape
    return sigmoid((_f64(x) @ _f64(Wgd).T) @ _f64(Wgu).T).reshape(B, T, num_heads, head_dim)


def decay_gate(x, w, num_heads, head_dim, lower_bound):
    """Log decay of the layer, the lower-bound sigmoid form of [Tokamax]
    9.1.3: g = a * sigmoid(exp(A_log_h) * (x Wad^T Wau^T + dt_bias))."""
    B, T, _ = x.shape
    raw = (_f64(x) @ _f64(w["Wad"]).T) @ _f64(w["Wau"]).T
    return gate_activation(raw.reshape(B, T, num_heads, head_dim), w["A_log"],
                           _f64(w["dt_bias"]).reshape(num_heads, head_dim), "lower_bound_sigmoid",
                           lower_bound)


def kda_layer_ref(x, w, num_heads, head_dim, chunk_size=64, gate_lower_bound=-5.0,
                  norm_eps=1e-6, l2_eps=1e-6, heads=None):
    """KDA layer forward with the low-rank output gate, float64.

    x: [B, T, M]. `w` maps names to arrays (Linear weights are [out, in]):
      Wqkv [3*H*D, M]; conv_q, conv_k, conv_v [H*D, 4]; Wb [H, M];
      Wad [r, M]; Wau [H*D, r]; A_log [H]; dt_bias [H*D];
      Wgd [D, M]; Wgu [H*D, D]; norm_w [D]; Wo [M, H*D].
    Steps ([K3]), each a function of this module:
      QKV projection -> short_conv_silu per stream (q and k through
      qk_features, L2-normalised over D) -> beta = sigmoid(x Wb^T) ->
      decay_gate -> chunkwise core with scale D^-1/2 and zero state ->
      head_rms_norm -> * output_gate -> Wo.
    `heads` restricts the core to a subset of heads (then x_new is not
    formed and is returned as None; the intermediates carry those heads).
    Returns (x_new [B, T, M], dict of intermediates q, k, v, g, beta, o).
    """
    x = _f64(x)
    B, T, M = x.shape
    H, D = num_heads, head_dim
    HD = H * D
    qkv = x @ _f64(w["Wqkv"]).T
    qp, kp, vp = qkv[..., :HD], qkv[..., HD:2 * HD], qkv[..., 2 * HD:]
    q = qk_features(qp, w["conv_q"], H, D, l2_eps)
    k = qk_features(kp, w["conv_k"], H, D, l2_eps)
    v = short_conv_silu(vp, w["conv_v"]).reshape(B, T, H, D)
    beta = sigmoid(x @ _f64(w["Wb"]).T)
    g = decay_gate(x, w, H, D, gate_lower_bound)
    if heads is not None:
        hs = list(heads)
        q, k, v, g, beta = q[:, :, hs], k[:, :, hs], v[:, :, hs], g[:, :, hs], beta[:, :, hs]
    o, _ = kda_chunkwise(q, k, v, g, beta, D ** -0.5, chunk_size)
    inter = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "o": o}
    if heads is not None:
        return None, inter
    y = head_rms_norm(o, w["norm_w"], norm_eps) * output_gate(x, w["Wgd"], w["Wgu"], H, D)
    x_new = y.reshape(B, T, HD) @ _f64(w["Wo"]).T
    return x_new, inter
