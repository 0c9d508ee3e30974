"""MI355X (gfx950) chunkwise Kimi Delta Attention forward.

Python binding of the C ABI in include/kda.h. This module only checks and
marshals arguments; every step of the forward runs in the HIP kernels of
libkda_mi355x.so. torch provides device memory and the current HIP stream.

    o, final_state = chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None,
                               cu_seqlens=None, output_final_state=True,
                               use_qk_l2norm=False)

Layouts: q, k, g [B, T, H, K]; v [B, T, H, V]; beta [B, T, H]; states
[N, H, K, V] fp32 (N = B, or the number of sequences with cu_seqlens, B = 1).
g is the natural-log decay (<= 0, >= -5).
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import KdaError, KdaValueError, KdaFwdParams, KdaWorkspaceInfo

__all__ = ["chunk_fwd", "KdaForward", "KdaError", "KdaValueError", "make_params", "workspace_layout",
           "KdaLayer", "layer_fwd", "decode_step", "affine_summary", "affine_apply",
           "chunk_bwd", "KdaBackward", "validate_inputs", "chunk_fwd_noalloc"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return _lib.KDA_DTYPE_F32
    raise KdaValueError(1, f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def make_params(B, T, H, K, V, qkv_dtype, g_dtype, beta_dtype, scale, chunk_size=64,
                use_qk_l2norm=False, l2norm_eps=1e-6, num_seqs=0) -> KdaFwdParams:
    p = KdaFwdParams()
    p.B, p.T, p.H, p.K, p.V = int(B), int(T), int(H), int(K), int(V)
    p.qkv_dtype, p.g_dtype, p.beta_dtype = int(qkv_dtype), int(g_dtype), int(beta_dtype)
    p.scale = float(scale)
    p.chunk_size = int(chunk_size)
    p.use_qk_l2norm = 1 if use_qk_l2norm else 0
    p.l2norm_eps = float(l2norm_eps)
    p.num_seqs = int(num_seqs)
    return p


def workspace_layout(p: KdaFwdParams) -> KdaWorkspaceInfo:
    info = KdaWorkspaceInfo()
    _lib.check(_lib.load().kda_workspace_layout(ctypes.byref(p), ctypes.byref(info)))
    return info


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _core_params(q, k, v, g, beta, scale, chunk_size, initial_state, cu_seqlens, use_qk_l2norm, l2norm_eps):
    """Shape, dtype and placement checks shared by the forward and backward
    bindings; returns the kda_fwd_params and the number of sequences N."""
    torch = _torch()
    if q.dim() != 4 or k.shape != q.shape or g.shape != q.shape:
        raise KdaValueError(1, "q, k, g must be [B, T, H, K] with equal shapes")
    B, T, H, K = q.shape
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, T, H):
        raise KdaValueError(1, "v must be [B, T, H, V]")
    V = v.shape[3]
    if tuple(beta.shape) != (B, T, H):
        raise KdaValueError(1, "beta must be [B, T, H]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise KdaValueError(1, "q, k, v must share a dtype")
    tensors = [q, k, v, g, beta]
    for t in tensors:
        if not t.is_cuda:
            raise KdaValueError(1, "inputs must be on the GPU")
        if not t.is_contiguous():
            raise KdaValueError(1, "inputs must be contiguous")
    num_seqs = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
            raise KdaValueError(1, "cu_seqlens must be a 1-D int32 GPU tensor")
        num_seqs = cu_seqlens.numel() - 1
        if num_seqs < 1:
            raise KdaValueError(1, "cu_seqlens needs at least 2 entries")
    N = num_seqs if num_seqs else B
    if initial_state is not None:
        if (tuple(initial_state.shape) != (N, H, K, V) or initial_state.dtype != torch.float32
                or not initial_state.is_cuda or not initial_state.is_contiguous()):
            raise KdaValueError(1, f"initial_state must be contiguous fp32 [{N}, {H}, {K}, {V}] on the GPU")
    if scale is None:
        scale = K ** -0.5
    params = make_params(B, T, H, K, V, _dtype_code(q), _dtype_code(g), _dtype_code(beta), scale,
                         chunk_size, use_qk_l2norm, l2norm_eps, num_seqs)
    return params, N


def chunk_fwd_noalloc(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None, out=None,
                      final_state=None, use_qk_l2norm=False, l2norm_eps=1e-6):
    """kda_chunk_fwd_noalloc: the forward with the library's static device
    workspace (no workspace allocation; the problem must fit
    KDA_NOALLOC_SCRATCH_BYTES). `out` and `final_state` may be preallocated
    (final_state None: not written). Returns (o, final_state)."""
    torch = _torch()
    lib = _lib.load()
    params, N = _core_params(q, k, v, g, beta, scale, 64, initial_state, cu_seqlens, use_qk_l2norm, l2norm_eps)
    B, T, H, K = q.shape
    o = out if out is not None else torch.empty((B, T, H, v.shape[3]), dtype=q.dtype, device=q.device)
    _lib.check(lib.kda_chunk_fwd_noalloc(
        ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
        _ptr(cu_seqlens), _ptr(o), _ptr(final_state), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    return o, final_state


def validate_inputs(g, beta, cu_seqlens=None, scratch=None):
    """Check the fast path's value preconditions on the GPU (kda_validate_inputs):
    g in [-5, 0], beta in [0, 1] (all finite), cu_seqlens[0] == 0, non-decreasing,
    cu_seqlens[-1] == T. g: [B, T, H, K], beta: [B, T, H]. Synchronises the
    current stream. Returns (ok, message, report dict); report["failed"] names
    the first failed precondition (0: none, 1: non-finite g, 2: g range,
    3: non-finite beta, 4: beta range, 5: cu_seqlens)."""
    torch = _torch()
    lib = _lib.load()
    if g.dim() != 4 or beta.dim() != 3 or tuple(beta.shape) != tuple(g.shape[:3]):
        raise KdaValueError(1, "g must be [B, T, H, K] and beta [B, T, H]")
    for t in (g, beta) + (() if cu_seqlens is None else (cu_seqlens,)):
        if not t.is_cuda or not t.is_contiguous():
            raise KdaValueError(1, "g, beta and cu_seqlens must be contiguous GPU tensors")
    num_seqs = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise KdaValueError(1, "cu_seqlens must be a 1-D int32 tensor with at least 2 entries")
        num_seqs = cu_seqlens.numel() - 1
    B, T, H, K = g.shape
    p = make_params(B, T, H, K, K, _lib.KDA_DTYPE_F32, _dtype_code(g), _dtype_code(beta), 1.0, num_seqs=num_seqs)
    if scratch is None:
        scratch = torch.empty(_lib.KDA_VALIDATE_SCRATCH_BYTES, dtype=torch.uint8, device=g.device)
    rep = _lib.KdaInputReport()
    st = lib.kda_validate_inputs(ctypes.byref(p), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(scratch),
                                 scratch.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                 ctypes.byref(rep))
    if rep.failed < 0:          # an argument error: the check did not run
        _lib.check(st)
    msg = lib.kda_last_error().decode(errors="replace")
    report = {n: getattr(rep, n) for n, _ in _lib.KdaInputReport._fields_}
    return st == 0, msg, report


class KdaForward:
    """A bound forward call: checked inputs, preallocated outputs and workspace.

    Calling the object runs both stages on the current stream; stage12() and
    stage34() run them one at a time (same workspace), e.g. to time each.
    """

    def __init__(self, q, k, v, g, beta, scale=None, chunk_size=64, initial_state=None,
                 cu_seqlens=None, output_final_state=True, use_qk_l2norm=False, l2norm_eps=1e-6,
                 out=None, workspace=None, gate_mode=None, A_log=None, dt_bias=None, gate_lower_bound=-5.0):
        torch = _torch()
        lib = _lib.load()
        self.params, N = _core_params(q, k, v, g, beta, scale, chunk_size, initial_state, cu_seqlens,
                                      use_qk_l2norm, l2norm_eps)
        B, T, H, K = q.shape
        V = v.shape[3]
        nbytes = ctypes.c_size_t(0)
        _lib.check(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(self.params), ctypes.byref(nbytes)))
        dev = q.device
        if workspace is None or workspace.numel() < nbytes.value:
            workspace = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self.o = out if out is not None else torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
        self.final_state = (torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
                            if output_final_state else None)
        self.inputs = (q, k, v, g, beta)
        # optional gate activation inside stage 1+2 (g then holds the raw gate)
        if gate_mode not in _lib.GATE_MODES:
            raise KdaValueError(1, f"unknown gate_mode {gate_mode!r}")
        self.gate = None
        if _lib.GATE_MODES[gate_mode]:
            for name, t, shp in (("A_log", A_log, (H,)), ("dt_bias", dt_bias, (H, K))):
                if t is None and name == "dt_bias":
                    continue
                if (t is None or not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous()
                        or t.numel() != (H if name == "A_log" else H * K)):
                    raise KdaValueError(1, f"{name} must be a contiguous fp32 GPU tensor of shape {shp}")
            self.gate = _lib.KdaGateParams(_lib.GATE_MODES[gate_mode], float(gate_lower_bound),
                                           A_log.data_ptr(), None if dt_bias is None else dt_bias.data_ptr())
            self._gate_tensors = (A_log, dt_bias)
        self.initial_state = initial_state
        self.cu_seqlens = cu_seqlens
        self._lib = lib

    def _stream(self):
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)

    def stage12(self):
        q, k, v, g, beta = self.inputs
        _lib.check(self._lib.kda_chunk_fwd_stage12(
            ctypes.byref(self.params), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(self.cu_seqlens),
            _ptr(self.workspace), self.workspace.numel(), self._stream()))

    def stage34(self):
        _lib.check(self._lib.kda_chunk_fwd_stage34(
            ctypes.byref(self.params), _ptr(self.initial_state), _ptr(self.cu_seqlens), _ptr(self.o),
            _ptr(self.final_state), _ptr(self.workspace), self.workspace.numel(), self._stream()))

    def __call__(self):
        q, k, v, g, beta = self.inputs
        if self.gate is not None:
            _lib.check(self._lib.kda_chunk_fwd_gated(
                ctypes.byref(self.params), ctypes.byref(self.gate), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                _ptr(self.initial_state), _ptr(self.cu_seqlens), _ptr(self.o), _ptr(self.final_state),
                _ptr(self.workspace), self.workspace.numel(), self._stream()))
            return self.o, self.final_state
        _lib.check(self._lib.kda_chunk_fwd(
            ctypes.byref(self.params), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(self.initial_state),
            _ptr(self.cu_seqlens), _ptr(self.o), _ptr(self.final_state), _ptr(self.workspace),
            self.workspace.numel(), self._stream()))
        return self.o, self.final_state


def chunk_fwd(q, k, v, g, beta, scale=None, chunk_size=64, initial_state=None, cu_seqlens=None,
              output_final_state=True, use_qk_l2norm=False, l2norm_eps=1e-6, gate_mode=None, A_log=None,
              dt_bias=None, gate_lower_bound=-5.0):
    """Chunkwise KDA forward on the GPU. Returns (o, final_state or None).

    gate_mode None: g is the natural-log decay. "softplus" or
    "lower_bound_sigmoid": g is the raw gate, activated inside stage 1+2 with
    A_log [H] and dt_bias [H, K] (fp32, dt_bias optional)."""
    return KdaForward(q, k, v, g, beta, scale, chunk_size, initial_state, cu_seqlens,
                      output_final_state, use_qk_l2norm, l2norm_eps, gate_mode=gate_mode, A_log=A_log,
                      dt_bias=dt_bias, gate_lower_bound=gate_lower_bound)()


class KdaBackward:
    """A bound backward call (kda_chunk_bwd): the gradients of
    <d_o, o> + <d_final_state, final_state> for the forward with the same
    arguments. Outputs dq, dk, dv, dg, dbeta (fp32, the inputs' shapes) and
    dh0 ([N, H, K, V] fp32, when requested) are preallocated; calling the
    object runs the backward on the current stream and returns them as a dict.
    """

    def __init__(self, q, k, v, g, beta, d_o, scale=None, initial_state=None, cu_seqlens=None,
                 d_final_state=None, use_qk_l2norm=False, l2norm_eps=1e-6, output_dh0=True, workspace=None):
        torch = _torch()
        self._lib = _lib.load()
        self.params, N = _core_params(q, k, v, g, beta, scale, 64, initial_state, cu_seqlens, use_qk_l2norm,
                                      l2norm_eps)
        B, T, H, K = q.shape
        V = v.shape[3]
        if (tuple(d_o.shape) != (B, T, H, V) or d_o.dtype != q.dtype or not d_o.is_cuda
                or not d_o.is_contiguous()):
            raise KdaValueError(1, "d_o must be contiguous [B, T, H, V] in q's dtype on the GPU")
        if d_final_state is not None and (tuple(d_final_state.shape) != (N, H, K, V)
                                          or d_final_state.dtype != torch.float32 or not d_final_state.is_cuda
                                          or not d_final_state.is_contiguous()):
            raise KdaValueError(1, f"d_final_state must be contiguous fp32 [{N}, {H}, {K}, {V}] on the GPU")
        nbytes = ctypes.c_size_t(0)
        _lib.check(self._lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(self.params), ctypes.byref(nbytes)))
        dev = q.device
        if workspace is None or workspace.numel() < nbytes.value:
            workspace = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=dev)
        self.workspace = workspace
        f32 = torch.float32
        self.grads = {
            "dq": torch.empty((B, T, H, K), dtype=f32, device=dev),
            "dk": torch.empty((B, T, H, K), dtype=f32, device=dev),
            "dv": torch.empty((B, T, H, V), dtype=f32, device=dev),
            "dg": torch.empty((B, T, H, K), dtype=f32, device=dev),
            "dbeta": torch.empty((B, T, H), dtype=f32, device=dev),
            "dh0": torch.empty((N, H, K, V), dtype=f32, device=dev) if output_dh0 else None,
        }
        self.inputs = (q, k, v, g, beta, d_o)
        self.initial_state = initial_state
        self.d_final_state = d_final_state
        self.cu_seqlens = cu_seqlens

    def __call__(self, stages=15):
        """Run the backward (or, for timing, the launches in the `stages` bit
        mask: 1 chunk terms, 2 chunk-start states, 4 state gradients, 8 chunk
        gradients) and return the gradients."""
        q, k, v, g, beta, d_o = self.inputs
        gr = self.grads
        _lib.check(self._lib.kda_chunk_bwd_stages(
            ctypes.byref(self.params), stages, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(self.initial_state),
            _ptr(self.cu_seqlens), _ptr(d_o), _ptr(self.d_final_state), _ptr(gr["dq"]), _ptr(gr["dk"]),
            _ptr(gr["dv"]), _ptr(gr["dg"]), _ptr(gr["dbeta"]), _ptr(gr["dh0"]), _ptr(self.workspace),
            self.workspace.numel(), ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)))
        return gr


def chunk_bwd(q, k, v, g, beta, d_o, scale=None, initial_state=None, cu_seqlens=None, d_final_state=None,
              use_qk_l2norm=False, l2norm_eps=1e-6):
    """Backward of chunk_fwd (g is the log decay). Returns a dict of fp32
    gradients dq, dk, dv, dg, dbeta and dh0."""
    return KdaBackward(q, k, v, g, beta, d_o, scale, initial_state, cu_seqlens, d_final_state,
                       use_qk_l2norm, l2norm_eps)()


def affine_summary(q, k, v, g, beta, scale=None, cu_seqlens=None, use_qk_l2norm=False, l2norm_eps=1e-6,
                   **gate):
    """Affine summary (M, N) of each sequence (include/kda.h, kda_chunk_affine_summary):
    for any initial state S0 the final state is M @ S0 + N. Runs stage 1+2 on
    the inputs, then the summary; returns fp32 M [N, H, K, K] and N [N, H, K, V]."""
    torch = _torch()
    f = KdaForward(q, k, v, g, beta, scale, cu_seqlens=cu_seqlens, output_final_state=False,
                   use_qk_l2norm=use_qk_l2norm, l2norm_eps=l2norm_eps, **gate)
    if f.gate is not None:
        raise KdaValueError(1, "affine_summary takes the activated log decay g (no gate_mode)")
    f.stage12()
    p = f.params
    N = p.num_seqs if p.num_seqs else p.B
    M = torch.empty((N, p.H, p.K, p.K), dtype=torch.float32, device=q.device)
    Nst = torch.empty((N, p.H, p.K, p.V), dtype=torch.float32, device=q.device)
    _lib.check(f._lib.kda_chunk_affine_summary(ctypes.byref(p), _ptr(cu_seqlens), _ptr(M), _ptr(Nst),
                                               _ptr(f.workspace), f.workspace.numel(), f._stream()))
    return M, Nst


def affine_apply(M, N, S0, out=None):
    """S = M @ S0 + N per (sequence, head) on the GPU (include/kda.h, kda_affine_apply)."""
    torch = _torch()
    lib = _lib.load()
    n, H, K, V = N.shape
    for t, shp in ((M, (n, H, K, K)), (S0, (n, H, K, V))):
        if tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise KdaValueError(1, f"expected contiguous fp32 GPU tensor of shape {shp}")
    out = out if out is not None else torch.empty_like(S0)
    p = make_params(n, 1, H, K, V, _lib.KDA_DTYPE_F32, _lib.KDA_DTYPE_F32, _lib.KDA_DTYPE_F32, 1.0)
    _lib.check(lib.kda_affine_apply(ctypes.byref(p), _ptr(M), _ptr(N), _ptr(S0), _ptr(out),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    return out


def decode_step(q, k, v, g, beta, state, scale=None, use_qk_l2norm=False, l2norm_eps=1e-6, out=None):
    """One token per sequence through the KDA recurrence (include/kda.h,
    kda_decode_step). q, k, g: [B, H, K]; v: [B, H, V]; beta: [B, H];
    state: fp32 [B, H, K, V], updated in place. Returns o [B, H, V] in q's dtype."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 3 or k.shape != q.shape or g.shape != q.shape:
        raise KdaValueError(1, "q, k, g must be [B, H, K] with equal shapes")
    B, H, K = q.shape
    if v.dim() != 3 or tuple(v.shape[:2]) != (B, H):
        raise KdaValueError(1, "v must be [B, H, V]")
    V = v.shape[2]
    if tuple(beta.shape) != (B, H):
        raise KdaValueError(1, "beta must be [B, H]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise KdaValueError(1, "q, k, v must share a dtype")
    for t in (q, k, v, g, beta, state):
        if not t.is_cuda or not t.is_contiguous():
            raise KdaValueError(1, "inputs and state must be contiguous GPU tensors")
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, K, V):
        raise KdaValueError(1, f"state must be fp32 [{B}, {H}, {K}, {V}]")
    if scale is None:
        scale = K ** -0.5
    p = make_params(B, 1, H, K, V, _dtype_code(q), _dtype_code(g), _dtype_code(beta), scale, 64,
                    use_qk_l2norm, l2norm_eps, 0)
    o = out if out is not None else torch.empty((B, H, V), dtype=q.dtype, device=q.device)
    _lib.check(lib.kda_decode_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                   _ptr(o), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    return o


# bf16 projection weights and fp32 small parameters of the layer (include/kda_layer.h)
_LAYER_BF16 = ("Wqkv", "Wb", "Wad", "Wau", "Wgd", "Wgu", "Wo")
_LAYER_F32 = ("conv_q", "conv_k", "conv_v", "A_log", "dt_bias", "norm_w")


class KdaLayer:
    """A bound KDA layer forward (include/kda_layer.h): checked weights,
    preallocated output and workspace. Calling it with x (bf16 [B, T, M] on the
    GPU) runs the whole layer on the current stream and returns x_new (bf16)."""

    def __init__(self, weights, B, T, H, D, gate_lower_bound=-5.0, norm_eps=1e-6, l2_eps=1e-6,
                 keep_core_output=False):
        torch = _torch()
        lib = _lib.load()
        for n in _lib.LAYER_WEIGHT_NAMES:
            if n not in weights:
                raise KdaValueError(1, f"missing layer weight {n}")
            t = weights[n]
            want = torch.bfloat16 if n in _LAYER_BF16 else torch.float32
            if not t.is_cuda or t.dtype != want or not t.is_contiguous():
                raise KdaValueError(1, f"layer weight {n} must be a contiguous {want} GPU tensor")
        M = weights["Wqkv"].shape[1]
        p = _lib.KdaLayerParams()
        p.B, p.T, p.M, p.H, p.D = int(B), int(T), int(M), int(H), int(D)
        p.gate_rank = int(weights["Wad"].shape[0])
        p.out_gate_rank = int(weights["Wgd"].shape[0])
        p.conv_size = int(weights["conv_q"].shape[1])
        p.gate_lower_bound, p.norm_eps, p.l2_eps = float(gate_lower_bound), float(norm_eps), float(l2_eps)
        HD = H * D
        shapes = {"Wqkv": (3 * HD, M), "conv_q": (HD, p.conv_size), "conv_k": (HD, p.conv_size),
                  "conv_v": (HD, p.conv_size), "Wb": (H, M), "Wad": (p.gate_rank, M), "Wau": (HD, p.gate_rank),
                  "A_log": (H,), "dt_bias": (HD,), "Wgd": (p.out_gate_rank, M), "Wgu": (HD, p.out_gate_rank),
                  "norm_w": (D,), "Wo": (M, HD)}
        for n, shp in shapes.items():
            if tuple(weights[n].shape) != shp:
                raise KdaValueError(1, f"layer weight {n} must have shape {shp}, got {tuple(weights[n].shape)}")
        self.params = p
        nbytes = ctypes.c_size_t(0)
        _lib.check(lib.kda_layer_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(nbytes)))
        dev = weights["Wqkv"].device
        self.workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
        self.x_new = torch.empty((B, T, M), dtype=torch.bfloat16, device=dev)
        self.core_out = (torch.empty((B, T, H, D), dtype=torch.float32, device=dev) if keep_core_output else None)
        self.weights = dict(weights)
        self.cw = _lib.KdaLayerWeights(*[t.data_ptr() for t in (weights[n] for n in _lib.LAYER_WEIGHT_NAMES)])
        self._lib = lib

    def core_inputs(self):
        """Views into the workspace of the last call's fp32 core inputs and
        output (kda_layer_workspace_layout): q, k, v [B, T, H, D], the raw
        decay gate g_raw [B, T, H, D] (before dt_bias and the activation),
        beta [B, T, H] and the core output o [B, T, H, D] (when no core_out)."""
        torch = _torch()
        p = self.params
        info = _lib.KdaLayerWorkspaceInfo()
        _lib.check(self._lib.kda_layer_workspace_layout(ctypes.byref(p), ctypes.byref(info)))
        B, T, H, D = p.B, p.T, p.H, p.D

        def view(off, shape):
            n = 1
            for d in shape:
                n *= d
            return self.workspace[off:off + 4 * n].view(torch.float32).view(shape)

        full = (B, T, H, D)
        return {"q": view(info.off_q, full), "k": view(info.off_k, full), "v": view(info.off_v, full),
                "g_raw": view(info.off_g_raw, full), "beta": view(info.off_beta, (B, T, H)),
                "o": self.core_out if self.core_out is not None else view(info.off_o, full)}

    def __call__(self, x):
        torch = _torch()
        p = self.params
        if (not x.is_cuda or x.dtype != torch.bfloat16 or not x.is_contiguous()
                or tuple(x.shape) != (p.B, p.T, p.M)):
            raise KdaValueError(1, f"x must be a contiguous bf16 GPU tensor of shape {(p.B, p.T, p.M)}")
        _lib.check(self._lib.kda_layer_fwd(
            ctypes.byref(p), ctypes.byref(self.cw), _ptr(x), _ptr(self.x_new), _ptr(self.core_out),
            _ptr(self.workspace), self.workspace.numel(),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        return self.x_new


def pack_layer_weights(weights):
    """A copy of the weight dict whose input-projection matrices Wqkv, Wad, Wgd
    and Wb are views of one bf16 allocation, back to back in that order
    (include/kda_layer.h): kda_layer_fwd then reads them in place instead of
    copying them at every call. One device copy, at load time."""
    torch = _torch()
    names = ("Wqkv", "Wad", "Wgd", "Wb")
    for n in names:
        t = weights[n]
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 2:
            raise KdaValueError(1, f"layer weight {n} must be a 2-D bf16 GPU tensor")
    M = weights["Wqkv"].shape[1]
    if any(weights[n].shape[1] != M for n in names):
        raise KdaValueError(1, "Wqkv, Wad, Wgd and Wb must have the same number of columns")
    buf = torch.cat([weights[n].contiguous() for n in names], dim=0)
    out = dict(weights)
    at = 0
    for n in names:
        rows = weights[n].shape[0]
        out[n] = buf[at:at + rows]
        at += rows
    return out


def layer_fwd(x, weights, H, D, **kw):
    """KDA layer forward on the GPU: x bf16 [B, T, M] -> x_new bf16 [B, T, M]."""
    B, T, _ = x.shape
    return KdaLayer(weights, B, T, H, D, **kw)(x)
