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
    want = (up(NP * 256 * 2) + up(BT * NP * 2) + 5 * up(BT * HD * 4) + up(BT * 2 * 4) + up(cb.value))
    assert n.value == want


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
    14 [64 x K] + 6 [64 x V] + 7 [64 x 64] matrices, 3 row vectors, 2 [K] vectors and
    2 [K x V] states, rounded up to 64 floats."""
    for K in (64, 128):
        p = P(K=K, V=K, B=2, T=256, H=3)
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
        info = _lib.KdaWorkspaceInfo()
        assert lib.kda_workspace_layout(ctypes.byref(p), ctypes.byref(info)) == 0
        slab = 14 * 64 * K + 6 * 64 * K + 7 * 64 * 64 + 3 * 64 + 2 * K + 2 * K * K
        slab = (slab + 63) // 64 * 64
        assert n.value == info.records_offset + info.chunk_slots * 3 * slab * 4


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
