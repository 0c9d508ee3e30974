"""Host-side checks of the C ABI (no GPU needed; no kernel is launched).

The library must load, export every function include/*.h declares, size
the workspace as documented and reject bad arguments before any launch.
"""
import ctypes
import os
import re

import pytest

from kimi_delta_attention_03_amd import _lib, make_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_abi_version(lib):
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    v = int(re.search(r"#define KDA_ABI_VERSION (\d+)", text).group(1))
    assert lib.kda_abi_version() == v


def P(**kw):
    d = dict(B=1, T=128, H=2, K=128, V=128, qkv_dtype=1, g_dtype=1, beta_dtype=1, scale=0.088,
             chunk_size=64, use_qk_l2norm=False, l2norm_eps=1e-6, num_seqs=0)
    d.update(kw)
    return make_params(**d)


def ws_bytes(lib, p):
    n = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def test_workspace_size_formula(lib):
    # record = (3 C K + 6 * 512 + C V) elements + 4 K bytes, rounded to 256; C = 64
    # (6 stored Aqk fragments of 16 x 32)
    for (K, dt, elem) in ((128, 1, 2), (128, 0, 4), (64, 1, 2), (64, 0, 4)):
        p = P(K=K, V=K, qkv_dtype=dt, g_dtype=dt, beta_dtype=dt, B=3, T=256, H=5)
        st, n = ws_bytes(lib, p)
        assert st == 0
        rec = (3 * 64 * K + 6 * 512 + 64 * K) * elem + 4 * K
        rec = (rec + 255) // 256 * 256
        info = _lib.KdaWorkspaceInfo()
        assert lib.kda_workspace_layout(ctypes.byref(p), ctypes.byref(info)) == 0
        # metadata: header, chunk table, sequence table, order, then a 256-byte sink
        meta = ((64 + 8 * 12 + 8 * 3 + 4 * 3 + 255) // 256) * 256 + 256
        assert info.records_offset == meta and info.record_bytes == rec
        assert n == meta + rec * (3 * 256 // 64) * 5
    # varlen: ceil(T/64) + N chunk slots per head
    p = P(T=1000, num_seqs=7)
    st, n = ws_bytes(lib, p)
    info = _lib.KdaWorkspaceInfo()
    assert lib.kda_workspace_layout(ctypes.byref(p), ctypes.byref(info)) == 0
    assert info.chunk_slots == 16 + 7 and info.record_bytes == 72192
    assert n == info.total_bytes == info.records_offset + 72192 * 23 * 2


@pytest.mark.parametrize("kw,status", [
    (dict(T=100), 1),                 # fixed length needs T % 64 == 0
    (dict(K=96, V=96), 2),            # unsupported head dim
    (dict(K=128, V=64), 2),           # K != V
    (dict(K=512, V=512), 1),          # K > 256
    (dict(chunk_size=32), 2),         # chunk size fixed at 64
    (dict(qkv_dtype=7), 1),           # unknown dtype
    (dict(H=0), 1),
    (dict(num_seqs=3, B=2), 1),       # varlen needs B == 1
    (dict(use_qk_l2norm=True, l2norm_eps=0.0), 1),
])
def test_invalid_params_rejected(lib, kw, status):
    st, _ = ws_bytes(lib, P(**kw))
    assert st == status
    assert lib.kda_last_error().decode()


def test_forward_rejects_before_launch(lib):
    """Bad pointers, sizes and workspace are reported without touching a GPU."""
    p = P()
    null = None
    # workspace missing
    st = lib.kda_chunk_fwd(ctypes.byref(p), null, null, null, null, null, null, null, null, null,
                           null, 0, null)
    assert st == 3
    # workspace too small (a fake, aligned address is never dereferenced)
    fake = ctypes.c_void_p(1 << 20)
    st = lib.kda_chunk_fwd(ctypes.byref(p), null, null, null, null, null, null, null, null, null,
                           fake, 1024, null)
    assert st == 3 and b"too small" in lib.kda_last_error()
    # inputs missing
    st, n = ws_bytes(lib, p)
    st = lib.kda_chunk_fwd(ctypes.byref(p), null, null, null, null, null, null, null, null, null,
                           fake, n, null)
    assert st == 1
    # misaligned input
    mis = ctypes.c_void_p((1 << 20) + 2)
    st = lib.kda_chunk_fwd(ctypes.byref(p), mis, mis, mis, mis, mis, null, null, fake, null,
                           fake, n, null)
    assert st == 1 and b"aligned" in lib.kda_last_error()
    # cu_seqlens without num_seqs and the reverse
    st = lib.kda_chunk_fwd_stage12(ctypes.byref(p), null, null, null, null, null, fake, fake, n, null)
    assert st == 1
    pv = P(num_seqs=2, T=100)
    st, nv = ws_bytes(lib, pv)
    st = lib.kda_chunk_fwd_stage12(ctypes.byref(pv), null, null, null, null, null, null, fake, nv, null)
    assert st == 1


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.kda_status_string(code).decode() == name


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "missing.so"))


# ---------------------------------------------------------------- layer ABI

def LP(**kw):
    p = _lib.KdaLayerParams()
    d = dict(B=2, T=128, M=256, H=2, D=128, gate_rank=32, out_gate_rank=128, conv_size=4,
             gate_lower_bound=-5.0, norm_eps=1e-6, l2_eps=1e-6)
    d.update(kw)
    for k, v in d.items():
        setattr(p, k, v)
    return p


def test_layer_workspace_formula(lib):
    p = LP()
    n = ctypes.c_size_t(0)
    assert lib.kda_layer_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
    BT, HD = 256, 256
    NP = (3 * 256 + 2 + 32 + 128 + 7) // 8 * 8
    up = lambda x: (x + 255) // 256 * 256
    core = make_params(2, 128, 2, 128, 128, 0, 0, 0, 128 ** -0.5)
    cb = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(core), ctypes.byref(cb)) == 0
    want = (up(NP * 256 * 2) + up(BT * NP * 2) + 5 * up(BT * HD * 4) + up(BT * 2 * 4) + up(BT * HD * 2) +
            up(cb.value))
    assert n.value == want
    info = _lib.KdaLayerWorkspaceInfo()
    assert lib.kda_layer_workspace_layout(ctypes.byref(p), ctypes.byref(info)) == 0
    assert info.total_bytes == want
    offs = [info.off_q, info.off_k, info.off_v, info.off_g_raw, info.off_beta, info.off_o]
    sizes = [BT * HD * 4] * 4 + [BT * 2 * 4, BT * HD * 4]
    spans = sorted(zip(offs, sizes))
    assert all(o % 256 == 0 for o in offs)
    assert all(a + sa <= b for (a, sa), (b, _) in zip(spans, spans[1:])) and spans[-1][0] + spans[-1][1] <= want


@pytest.mark.parametrize("kw,status", [
    (dict(T=100), 1),                 # T % 64
    (dict(D=96), 2),                  # head dim
    (dict(conv_size=3), 2),           # conv width
    (dict(M=100), 1),                 # M % 8
    (dict(gate_rank=0), 1),
    (dict(gate_lower_bound=-6.0), 1), # outside the core's decay range
    (dict(gate_lower_bound=0.0), 1),
    (dict(norm_eps=0.0), 1),
    (dict(B=0), 1),
])
def test_layer_rejects_bad_params(lib, kw, status):
    p = LP(**kw)
    n = ctypes.c_size_t(0)
    assert lib.kda_layer_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == status
    assert lib.kda_last_error()


def test_layer_rejects_null_pointers_before_launch(lib):
    p = LP()
    w = _lib.KdaLayerWeights()
    st = lib.kda_layer_fwd(ctypes.byref(p), ctypes.byref(w), ctypes.c_void_p(256), ctypes.c_void_p(512), None,
                           ctypes.c_void_p(1 << 20), 1 << 40, None)
    assert st == 1 and b"weight" in lib.kda_last_error()


def test_decode_rejects_bad_params_before_launch(lib):
    vp = ctypes.c_void_p(4096)
    p = make_params(2, 64, 4, 128, 128, 1, 1, 1, 0.1)          # T must be 1
    assert lib.kda_decode_step(ctypes.byref(p), vp, vp, vp, vp, vp, vp, vp, None) == 1
    assert b"T == 1" in lib.kda_last_error()
    p = make_params(2, 1, 4, 96, 96, 1, 1, 1, 0.1)             # unsupported head dim
    assert lib.kda_decode_step(ctypes.byref(p), vp, vp, vp, vp, vp, vp, vp, None) == 2
    p = make_params(2, 1, 4, 128, 128, 1, 1, 1, 0.1)
    assert lib.kda_decode_step(ctypes.byref(p), vp, vp, vp, vp, vp, None, vp, None) == 1
    p = make_params(0, 1, 4, 128, 128, 1, 1, 1, 0.1)           # empty batch: nothing to do
    assert lib.kda_decode_step(ctypes.byref(p), None, None, None, None, None, None, None, None) == 0


def test_backward_workspace_formula(lib):
    """Backward workspace = forward metadata + one fp32 slab per (chunk slot, head):
    8 [64 x K] + 6 [64 x V] + 7 [64 x 64] matrices, 3 row vectors, 2 [K] vectors and
    2 [K x V] states, rounded up to 64 floats."""
    for K in (64, 128):
        p = P(K=K, V=K, B=2, T=256, H=3)
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
        info = _lib.KdaWorkspaceInfo()
        assert lib.kda_workspace_layout(ctypes.byref(p), ctypes.byref(info)) == 0
        slab = 8 * 64 * K + 6 * 64 * K + 7 * 64 * 64 + 3 * 64 + 2 * K + 2 * K * K
        slab = (slab + 63) // 64 * 64
        assert n.value == info.records_offset + info.chunk_slots * 3 * slab * 4


def test_segment_plan_bf16_only(lib):
    """Long fixed-length bf16 inputs are planned in segments along T; fp32 and
    variable-length inputs in one pass."""
    from kimi_delta_attention_03_amd import make_params, workspace_layout
    bf = workspace_layout(make_params(1, 32768, 32, 128, 128, 1, 1, 1, 128 ** -0.5))
    assert bf.segments == 8 and bf.segment_chunks == 64
    f32 = workspace_layout(make_params(4, 8192, 16, 128, 128, 0, 0, 0, 128 ** -0.5))
    assert f32.segments == 1
    var = workspace_layout(make_params(1, 32768, 32, 128, 128, 1, 1, 1, 128 ** -0.5, num_seqs=4))
    assert var.segments == 1


def test_backward_rejects_before_launch(lib):
    """Bad stage masks, workspace, pointers and alignment are reported without a launch."""
    p = P()
    null = None
    fake = ctypes.c_void_p(1 << 20)
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
    args = [null] * 15                            # q, k, v, g, beta, h0, cu, d_o, d_final, 6 gradients
    assert lib.kda_chunk_bwd(ctypes.byref(p), *args, null, 0, null) == 3          # no workspace
    assert lib.kda_chunk_bwd(ctypes.byref(p), *args, fake, 1024, null) == 3       # too small
    assert b"too small" in lib.kda_last_error()
    assert lib.kda_chunk_bwd(ctypes.byref(p), *args, fake, n.value, null) == 1    # inputs missing
    vp = ctypes.c_void_p(4096)
    ins = [vp] * 5 + [null, null, vp, null]      # q, k, v, g, beta, h0, cu, d_o, d_final
    assert lib.kda_chunk_bwd(ctypes.byref(p), *ins, null, null, null, null, null, null, fake, n.value, null) == 1
    assert b"dq" in lib.kda_last_error()          # gradient outputs missing
    mis = ctypes.c_void_p(4096 + 1)               # odd: misaligned for bf16 and fp32 alike
    outs = [vp] * 5 + [null]
    assert lib.kda_chunk_bwd(ctypes.byref(p), mis, *ins[1:], *outs, fake, n.value, null) == 1
    assert b"aligned" in lib.kda_last_error()
    for bad in (0, 16, -1):
        assert lib.kda_chunk_bwd_stages(ctypes.byref(p), bad, *ins, *outs, fake, n.value, null) == 1
    pv = P(num_seqs=2, T=100)                      # varlen without cu_seqlens
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(pv), ctypes.byref(n)) == 0
    assert lib.kda_chunk_bwd(ctypes.byref(pv), *ins, *outs, fake, n.value, null) == 1


# ------------------------------------------- output / state checks before any launch
# These pass fake device addresses: they run only where no GPU is visible, so that
# an address can never reach a device even if a check were missing (on a machine
# without a GPU a launch fails with KDA_ERR_HIP, so status 1 also shows that the
# check ran before the first launch).

def _gpu_visible():
    import torch
    return torch.cuda.is_available()


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses must never reach a real device")


@no_gpu
@pytest.mark.parametrize("which", ["o", "initial_state", "final_state"])
@pytest.mark.parametrize("entry", ["fwd", "gated", "stage34", "stage34_varlen"])
def test_misaligned_output_or_state_rejected_before_launch(lib, which, entry):
    """kda_chunk_fwd, kda_chunk_fwd_gated and kda_chunk_fwd_stage34 with aligned
    inputs and one misaligned o, initial_state or final_state: KDA_ERR_INVALID_ARG,
    nothing launched (the varlen stage 3+4 used to launch its chunk map first)."""
    p = P(num_seqs=2, T=100) if entry == "stage34_varlen" else P()
    _, n = ws_bytes(lib, p)
    ok = ctypes.c_void_p(1 << 24)
    mis = ctypes.c_void_p((1 << 24) + 8)          # 8-byte aligned, not 16
    ws = ctypes.c_void_p(1 << 30)
    o, h0, hf = ok, ok, ok
    if which == "o":
        o = mis
    elif which == "initial_state":
        h0 = mis
    else:
        hf = mis
    cu = ok if entry == "stage34_varlen" else None
    if entry == "fwd":
        st = lib.kda_chunk_fwd(ctypes.byref(p), ok, ok, ok, ok, ok, h0, None, o, hf, ws, n, None)
    elif entry == "gated":
        st = lib.kda_chunk_fwd_gated(ctypes.byref(p), None, ok, ok, ok, ok, ok, h0, None, o, hf, ws, n, None)
    else:
        st = lib.kda_chunk_fwd_stage34(ctypes.byref(p), h0, cu, o, hf, ws, n, None)
    assert st == 1, lib.kda_last_error()
    assert b"aligned" in lib.kda_last_error()


@no_gpu
def test_forward_needs_o_before_launch(lib):
    p = P()
    _, n = ws_bytes(lib, p)
    ok = ctypes.c_void_p(1 << 24)
    st = lib.kda_chunk_fwd(ctypes.byref(p), ok, ok, ok, ok, ok, None, None, None, None, ctypes.c_void_p(1 << 30), n,
                           None)
    assert st == 1 and b"o must be non-NULL" in lib.kda_last_error()


@no_gpu
def test_affine_summary_rejects_aliased_outputs(lib):
    p = P()
    _, n = ws_bytes(lib, p)
    m = ctypes.c_void_p(1 << 24)
    assert lib.kda_chunk_affine_summary(ctypes.byref(p), None, m, m, ctypes.c_void_p(1 << 30), n, None) == 1
    assert b"alias" in lib.kda_last_error()


def test_backward_stage_mask_message(lib):
    """A bad stage mask is reported with its own message, not a stale one."""
    lib.kda_chunk_fwd_workspace_bytes(None, None)            # leaves "params is NULL"
    p = P()
    args = [None] * 15
    assert lib.kda_chunk_bwd_stages(ctypes.byref(p), 0, *args, None, 0, None) == 1
    assert b"stages" in lib.kda_last_error()


# ------------------------------------------------------------- kda_validate_inputs

def _report():
    return _lib.KdaInputReport()


def test_validate_rejects_bad_arguments_before_launch(lib):
    """Argument errors are reported without a launch; report.failed stays -1."""
    vp = ctypes.c_void_p(1 << 24)
    p = P()
    r = _report()
    assert lib.kda_validate_inputs(ctypes.byref(p), vp, vp, None, vp, 16384, None, None) == 1
    assert lib.kda_validate_inputs(ctypes.byref(p), vp, vp, None, None, 16384, None, ctypes.byref(r)) == 3
    assert r.failed == -1
    assert lib.kda_validate_inputs(ctypes.byref(p), vp, vp, None, vp, 1024, None, ctypes.byref(r)) == 3
    assert b"scratch" in lib.kda_last_error()
    odd = ctypes.c_void_p((1 << 24) + 1)
    assert lib.kda_validate_inputs(ctypes.byref(p), odd, vp, None, vp, 16384, None, ctypes.byref(r)) == 1
    assert b"aligned" in lib.kda_last_error() and r.failed == -1
    assert lib.kda_validate_inputs(ctypes.byref(p), vp, vp, vp, vp, 16384, None, ctypes.byref(r)) == 1
    assert b"num_seqs == 0" in lib.kda_last_error()
    pv = P(num_seqs=3, T=100)
    assert lib.kda_validate_inputs(ctypes.byref(pv), vp, vp, None, vp, 16384, None, ctypes.byref(r)) == 1
    assert b"needs cu_seqlens" in lib.kda_last_error()
    assert lib.kda_validate_inputs(ctypes.byref(P()), None, None, None, vp, 16384, None, ctypes.byref(r)) == 1


def test_validate_report_layout_matches_header():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    body = text[:text.index("} kda_input_report;")]
    body = body[body.rindex("typedef struct {") + len("typedef struct {"):]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"(\w+)\s*[,;]", body)
    assert names == [n for n, _ in _lib.KdaInputReport._fields_]
    assert ctypes.sizeof(_lib.KdaInputReport) == 48
    assert int(re.search(r"#define KDA_VALIDATE_SCRATCH_BYTES (\d+)", text).group(1)) == \
        _lib.KDA_VALIDATE_SCRATCH_BYTES


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=12), 1, b"multiples of 8"),
    (dict(lda=4), 1, b"multiples of 8"),
    (dict(ldc=3), 1, b"ldc >= N"),
    (dict(lda=(1 << 21) + 8), 2, b"2^21"),
    (dict(ldb=(1 << 22)), 2, b"2^21"),
    (dict(c_dtype=7), 1, b"c_dtype"),
    (dict(A=None), 1, b"non-NULL"),
    (dict(A=(1 << 24) + 8), 1, b"16-byte"),
])
def test_gemm_rejects_bad_arguments_before_launch(lib, kw, status, msg):
    """kda_gemm_bf16_nt checks shapes, strides (the kernel's 32-bit buffer
    offsets bound lda and ldb by 2^21), dtype, NULL and alignment on the host
    and launches nothing when a check fails (every case here fails one, so the
    fake addresses never reach a device)."""
    a = dict(M=300, N=200, K=64, A=1 << 24, lda=64, B=1 << 25, ldb=64, C=1 << 26, ldc=200, c_dtype=1)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    st = lib.kda_gemm_bf16_nt(a["M"], a["N"], a["K"], vp(a["A"]), a["lda"], vp(a["B"]), a["ldb"], vp(a["C"]),
                              a["ldc"], a["c_dtype"], None)
    assert st == status, lib.kda_last_error()
    assert msg in lib.kda_last_error()
