"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Metric: max|gpu - oracle| / max|oracle| per tensor, <= 1e-4 for fp32 inputs
and <= 2e-2 for bf16 inputs, on both o and final_state.
"""
import sys

import numpy as np
import pytest

import oracle.kda_oracle as orc
from helpers import TOL, decode_record, dev_inputs, host, rel_err
from kimi_delta_attention_03_amd.synthetic import core_inputs, workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(x, **kw):
    import kimi_delta_attention_03_amd as kda
    import torch
    d = dev_inputs(x)
    o, fs = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=x.scale,
                          initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return host(o), (None if fs is None else host(fs))


def check(x, tol=None, heads=None, **kw):
    tol = tol or TOL[x.dtype]
    o, fs = run_gpu(x, **kw)
    o_ref, f_ref = orc.kda_chunkwise(x.q, x.k, x.v, x.g, x.beta, x.scale, 64, x.initial_state,
                                     cu_seqlens=x.cu_seqlens, heads=heads,
                                     use_qk_l2norm=kw.get("use_qk_l2norm", False))
    if heads is not None:
        o, fs = o[:, :, heads], fs[:, heads]
    eo, ef = rel_err(o, o_ref), rel_err(fs, f_ref)
    _say(f"  rel err o={eo:.3e} final={ef:.3e} (tol {tol})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(fs))
    assert eo <= tol and ef <= tol
    return o, fs


@pytest.mark.parametrize("dtype,K", [("fp32", 64), ("fp32", 128), ("bf16", 64), ("bf16", 128)])
def test_small_multi_chunk(dtype, K):
    """B=2, 5 chunks per row, several heads, zero and non-zero initial state."""
    _say(f"small multi-chunk {dtype} K={K}")
    x = core_inputs(2, 320, 3, K, K, dtype=dtype, seed=100 + K, init_std=0.1)
    check(x)


@pytest.mark.parametrize("varlen", [False, True], ids=["fixed", "varlen"])
def test_fp32_more_workgroups_than_cus(varlen):
    """fp32 at K = 128 with more (sequence, head) pairs than one stage 3+4
    workgroup per CU covers (8 column blocks each, 256 CUs), so the workgroups
    run in rounds; the variable-length case adds ragged last chunks and empty
    and one-token sequences."""
    if varlen:
        lengths = np.random.default_rng(31).integers(0, 260, size=40)
        lengths[[2, 17]] = [0, 1]
        x = core_inputs(1, None, 2, 128, 128, dtype="fp32", seed=32, init_std=0.1, lengths=lengths)
    else:
        x = core_inputs(3, 320, 12, 128, 128, dtype="fp32", seed=33, init_std=0.1)
    _say(f"fp32 K=128 many units varlen={varlen} q={x.q.shape}")
    check(x)


def test_workload0_tiny_fp32():
    _say("workload 0: B=1 H=2 T=256 K=V=64 fp32")
    check(workload(0))


def test_workload1_bf16():
    _say("workload 1: B=2 H=16 T=4096 K=V=128 bf16")
    check(workload(1))


def test_workload2_headline_sampled_heads():
    """Full headline shape on the GPU, oracle on 3 of the 32 heads (whole sequence)."""
    _say("workload 2: B=1 H=32 T=32768 K=V=128 bf16 (heads 0, 13, 31 vs oracle)")
    check(workload(2), heads=[0, 13, 31])


def test_workload3_varlen_sampled_heads():
    _say("workload 3: 16 packed sequences, H=32, bf16 (heads 5, 30 vs oracle)")
    check(workload(3), heads=[5, 30])


def test_varlen_ragged_small():
    """Lengths around chunk boundaries, an empty sequence and a single token."""
    for dtype in ("fp32", "bf16"):
        _say(f"varlen ragged {dtype}")
        x = core_inputs(1, None, 2, 64, 64, dtype=dtype, seed=7, init_std=0.2,
                        lengths=[1, 63, 64, 65, 0, 130, 200, 2])
        check(x)


def test_l2norm_flag():
    for dtype in ("fp32", "bf16"):
        _say(f"in-kernel q/k L2 norm {dtype}")
        x = core_inputs(1, 192, 2, 128, 128, dtype=dtype, seed=8, init_std=0.1, normalize=False)
        check(x, use_qk_l2norm=True)


def test_no_final_state_and_zero_length():
    import kimi_delta_attention_03_amd as kda
    import torch
    _say("final_state omitted; T=0 returns the initial state")
    x = core_inputs(1, 128, 2, 64, 64, dtype="bf16", seed=9)
    d = dev_inputs(x)
    o, fs = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], output_final_state=False)
    assert fs is None and o.shape == (1, 128, 2, 64)
    z = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    zb = torch.zeros((1, 0, 2), dtype=torch.bfloat16, device="cuda:0")
    s0 = torch.randn((1, 2, 64, 64), device="cuda:0")
    o, fs = kda.chunk_fwd(z, z, z, z, zb, initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 2, 64) and torch.equal(fs, s0)


def gamma_err(gpu, ref):
    """Per-channel relative error of the chunk-end decay where fp32 can hold it;
    below ~1e-30 the true value underflows and only |gpu| <= 1e-29 is asked."""
    small = ref < 1e-30
    assert np.all(np.abs(gpu[small]) <= 1e-29)
    big = ~small
    return float(np.max(np.abs(gpu[big] - ref[big]) / ref[big])) if big.any() else 0.0


def test_stage12_intermediates_match_oracle():
    """Decode the workspace records and compare W, U, qg, kg, Aqk, gamma per chunk."""
    import kimi_delta_attention_03_amd as kda
    import torch
    for dtype in ("fp32", "bf16"):
        _say(f"stage 1+2 intermediates {dtype}")
        K = 128
        x = core_inputs(1, 128, 2, K, K, dtype=dtype, seed=11)
        d = dev_inputs(x)
        f = kda.KdaForward(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=x.scale)
        f.workspace.zero_()
        f.stage12()
        torch.cuda.synchronize()
        ws = f.workspace.cpu().numpy()
        info = kda.workspace_layout(f.params)
        _, _, terms = orc.kda_chunkwise(x.q, x.k, x.v, x.g, x.beta, x.scale, 64, return_terms=True)
        tol = 1e-5 if dtype == "fp32" else 1e-2
        for (_, c0, t) in terms:
            p = c0 // 64
            for h in range(2):
                r = decode_record(ws, info, h, p, K, K, dtype == "bf16", 2)
                errs = {
                    "W": rel_err(r["W"], t["W"][h]), "U": rel_err(r["U"], t["U"][h]),
                    "qg": rel_err(r["qg"], t["qg"][h]), "kg": rel_err(r["kgT"].T, t["kg"][h]),
                    "Aqk": rel_err(r["Aqk"], t["Aqk"][h]), "gamma": gamma_err(r["gamma"], t["gamma"][h]),
                }
                _say(f"  chunk {p} head {h}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
                assert max(errs.values()) <= tol, errs


def test_prefix_invariance_bitwise():
    """Perturbing tokens after n leaves o[0..n] bit-identical (same chunk and later chunks)."""
    import torch
    for dtype in ("fp32", "bf16"):
        _say(f"prefix invariance {dtype}")
        x = core_inputs(1, 256, 4, 128, 128, dtype=dtype, seed=12, init_std=0.1)
        y = core_inputs(1, 256, 4, 128, 128, dtype=dtype, seed=13, init_std=0.1)
        o1, _ = run_gpu(x)
        for n in (5, 70, 191):
            z = core_inputs(1, 256, 4, 128, 128, dtype=dtype, seed=12, init_std=0.1)
            for name in ("q", "k", "v", "g", "beta"):
                getattr(z, name)[:, n + 1:] = getattr(y, name)[:, n + 1:]
            o2, _ = run_gpu(z)
            assert np.array_equal(o1[:, :n + 1], o2[:, :n + 1]), f"prefix {n} changed"
            assert not np.array_equal(o1[:, n + 1:], o2[:, n + 1:])


def test_deterministic_bitwise():
    x = core_inputs(1, 512, 8, 128, 128, dtype="bf16", seed=14, init_std=0.1)
    _say("determinism")
    o1, f1 = run_gpu(x)
    o2, f2 = run_gpu(x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_continuation_through_state():
    """run(0..T) == run(t..T) started from run(0..t).final_state (t on a chunk boundary)."""
    import kimi_delta_attention_03_amd as kda
    import torch
    _say("state continuation")
    x = core_inputs(1, 384, 2, 128, 128, dtype="fp32", seed=15, init_std=0.1)
    d = dev_inputs(x)
    o, f = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"])
    t = 128
    sl = lambda a, s: a[:, s].contiguous()
    oa, fa = kda.chunk_fwd(*(sl(d[n], slice(0, t)) for n in ("q", "k", "v", "g", "beta")),
                           initial_state=d["initial_state"])
    ob, fb = kda.chunk_fwd(*(sl(d[n], slice(t, None)) for n in ("q", "k", "v", "g", "beta")), initial_state=fa)
    torch.cuda.synchronize()
    assert rel_err(host(torch.cat([oa, ob], 1)), host(o)) < 1e-5
    assert rel_err(host(fb), host(f)) < 1e-5


def test_invalid_arguments_raise():
    import kimi_delta_attention_03_amd as kda
    import torch
    q = torch.zeros((1, 100, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    b = torch.zeros((1, 100, 2), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        kda.chunk_fwd(q, q, q, q, b)          # T % 64 != 0 without cu_seqlens
    q2 = torch.zeros((1, 64, 2, 96), dtype=torch.bfloat16, device="cuda:0")
    b2 = torch.zeros((1, 64, 2), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        kda.chunk_fwd(q2, q2, q2, q2, b2)     # unsupported head dim


def test_varlen_many_sequences_unsorted_path():
    """5000 packed sequences: more than the varlen map ranks longest first
    (4096), so the map keeps the given order. Sequences are independent, so
    the GPU results of the first and last 200 must equal oracle runs on just
    those sequences."""
    import kimi_delta_attention_03_amd as kda
    import torch
    rng = np.random.default_rng(123)
    lengths = rng.integers(0, 80, size=5000)
    lengths[[3, 4000]] = 0
    x = core_inputs(1, None, 2, 64, 64, dtype="bf16", seed=124, init_std=0.1, lengths=lengths)
    _say(f"varlen {len(lengths)} sequences, T={x.q.shape[1]}")
    o, fs = run_gpu(x)
    cu = x.cu_seqlens
    for lo, hi in ((0, 200), (4800, 5000)):
        t0, t1 = int(cu[lo]), int(cu[hi])
        sub = lambda a: a[:, t0:t1]
        o_ref, f_ref = orc.kda_chunkwise(sub(x.q), sub(x.k), sub(x.v), sub(x.g), sub(x.beta), x.scale, 64,
                                         x.initial_state[lo:hi], cu_seqlens=cu[lo:hi + 1] - cu[lo])
        eo, ef = rel_err(o[:, t0:t1], o_ref), rel_err(fs[lo:hi], f_ref)
        _say(f"  sequences {lo}..{hi}: rel err o={eo:.2e} final={ef:.2e}")
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    # zero-length sequences return their initial state exactly
    assert np.array_equal(fs[[3, 4000]], x.initial_state[[3, 4000]])


@pytest.mark.parametrize("dtype,B,T,H,nseg", [("bf16", 3, 67 * 64, 16, 2), ("bf16", 1, 280 * 64, 16, 3)])
def test_segmented_forward_bitwise_equals_one_pass(dtype, B, T, H, nseg):
    """Long fixed-length bf16 inputs run in segments along T with the fp32 state
    handed over in the workspace (kda_chunk_fwd); stage 1+2 and stage 3+4 called
    once each over the whole problem (kda_chunk_fwd_stage12 / _stage34) compute the
    same chunks. The two must agree bitwise, with and without final_state; the
    shapes give 2 uneven segments (34 + 33 chunks) and 3 (94 + 94 + 92)."""
    import kimi_delta_attention_03_amd as kda
    import torch
    _say(f"segmented vs one pass {dtype} B={B} T={T} H={H}")
    x = core_inputs(B, T, H, 128, 128, dtype=dtype, seed=16, init_std=0.1)
    d = dev_inputs(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    fwd = kda.KdaForward(*args, scale=x.scale, initial_state=d["initial_state"])
    assert kda.workspace_layout(fwd.params).segments == nseg
    o1, f1 = fwd()
    o1, f1 = o1.clone(), f1.clone()
    fwd.o.zero_()
    fwd.final_state.zero_()
    fwd.stage12()
    fwd.stage34()
    torch.cuda.synchronize()
    assert torch.equal(o1, fwd.o) and torch.equal(f1, fwd.final_state)
    o3, f3 = kda.chunk_fwd(*args, scale=x.scale, initial_state=d["initial_state"], output_final_state=False)
    torch.cuda.synchronize()
    assert f3 is None and torch.equal(o3, o1)
    # and the oracle on one head over the whole length
    h = H - 1
    o_ref, f_ref = orc.kda_chunkwise(x.q, x.k, x.v, x.g, x.beta, x.scale, 64, x.initial_state, heads=[h])
    eo, ef = rel_err(host(o1)[:, :, [h]], o_ref), rel_err(host(f1)[:, [h]], f_ref)
    _say(f"  head {h}: rel err o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
