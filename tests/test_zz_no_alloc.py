"""kda_chunk_fwd_noalloc (the forward on the library's static device workspace)
against kda_chunk_fwd (caller workspace) through the C ABI: two calls in a row,
the second on a smaller problem, each bitwise equal to the caller-workspace
forward on the same inputs (both run the same kernels), and a problem larger
than the static workspace rejected before any launch."""
import ctypes
import sys

import numpy as np
import pytest

from helpers import dev_inputs, host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(x):
    import torch
    import kimi_delta_attention_03_amd as kda
    d = dev_inputs(x)
    N = d["initial_state"].shape[0] if d["initial_state"] is not None else (
        x.q.shape[0] if d["cu_seqlens"] is None else len(x.cu_seqlens) - 1)
    B, T, H, K = x.q.shape
    o_ref, f_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=x.scale,
                                 initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    fs = torch.full((N, H, K, x.v.shape[3]), float("nan"), dtype=torch.float32, device="cuda:0")
    o, fs = kda.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=x.scale,
                                  initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], final_state=fs)
    torch.cuda.synchronize()
    return o_ref, f_ref, o, fs


def test_noalloc_matches_caller_workspace_twice():
    from kimi_delta_attention_03_amd.synthetic import core_inputs
    import torch
    # first call: fixed length, bf16, K = V = 128, random initial state (18.5 MB of workspace)
    _say("noalloc call 1: B=2 T=1024 H=8 K=128 bf16")
    x1 = core_inputs(2, 1024, 8, 128, 128, dtype="bf16", seed=901, init_std=0.1)
    o_ref, f_ref, o, fs = _both(x1)
    assert torch.equal(o, o_ref) and torch.equal(fs, f_ref)
    # second call, smaller: packed ragged sequences, fp32, K = V = 64; the static
    # array still holds the first call's records
    _say("noalloc call 2: varlen 3 sequences T=200 H=3 K=64 fp32")
    x2 = core_inputs(1, 0, 3, 64, 64, dtype="fp32", seed=902, init_std=0.1, lengths=[1, 129, 70])
    o_ref2, f_ref2, o2, fs2 = _both(x2)
    assert torch.equal(o2, o_ref2) and torch.equal(fs2, f_ref2)
    assert np.isfinite(host(o2)).all()


def test_noalloc_rejects_a_problem_larger_than_the_scratch():
    """Workspace need above KDA_NOALLOC_SCRATCH_BYTES: KDA_ERR_WORKSPACE, nothing launched
    (the pointers are never looked at)."""
    from kimi_delta_attention_03_amd import _lib, make_params
    lib = _lib.load()
    p = make_params(1, 32768, 32, 128, 128, 1, 1, 1, 128 ** -0.5)
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value > _lib.KDA_NOALLOC_SCRATCH_BYTES
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None)
    assert st == 3 and b"static scratch" in lib.kda_last_error()
