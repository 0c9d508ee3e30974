"""GPU parity of the affine chunk summaries (kda_chunk_affine_summary) and the
merge step (kda_affine_apply) against the float64 oracle's per-chunk
summaries composed in order ([Tokamax] 4.2, 9.1.8), through the C ABI; and
the one-GPU part of context parallelism: a sequence split in two halves,
each summarised on its own, merged, and continued.

Metric: max|gpu - oracle| / max|oracle| per tensor, <= 1e-4 (fp32 inputs),
<= 2e-2 (bf16 inputs).
"""
import sys

import numpy as np
import pytest

import oracle.kda_oracle as orc
from helpers import TOL, host, rel_err, to_dev
from kimi_delta_attention_03_amd.synthetic import core_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dt(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def oracle_summary(x):
    """Per sequence and head: (M, N) composed from the oracle's chunk summaries."""
    _, _, terms = orc.kda_chunkwise(x.q, x.k, x.v, x.g, x.beta, x.scale, 64, None, cu_seqlens=x.cu_seqlens,
                                    return_terms=True)
    H, K, V = x.q.shape[2], x.q.shape[3], x.v.shape[3]
    nseq = len(x.cu_seqlens) - 1 if x.cu_seqlens is not None else x.q.shape[0]
    # terms are in segment order, chunk order within a segment
    M = np.broadcast_to(np.eye(K), (nseq, H, K, K)).copy()
    N = np.zeros((nseq, H, K, V))
    bounds = (list(zip(x.cu_seqlens[:-1], x.cu_seqlens[1:])) if x.cu_seqlens is not None
              else [(0, x.q.shape[1])] * nseq)
    it = iter(terms)
    for n, (s0, s1) in enumerate(bounds):
        for _ in range(-(-(int(s1) - int(s0)) // 64)):
            _, _, t = next(it)
            Phi, Psi = orc.chunk_affine_summary(t)
            M[n], N[n] = orc.compose_affine((M[n], N[n]), (Phi, Psi))
    return M, N


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("varlen", [False, True])
def test_affine_summary_matches_oracle(dtype, K, varlen):
    import kimi_delta_attention_03_amd as kda
    import torch
    lengths = [130, 64, 1, 0, 200] if varlen else None
    # mild decay (g in [-0.05, 0]): with the usual g in [-5, 0] the product of the
    # chunk decays, and so M, is far below the fp32 range
    x = core_inputs(1 if varlen else 2, None if varlen else 192, 3, K, K, dtype=dtype, seed=71 + K, lengths=lengths,
                    g_low=-0.05)
    _say(f"affine summary {dtype} K={K} varlen={varlen}")
    dt = _dt(dtype)
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to("cuda:0")
    M, N = kda.affine_summary(to_dev(x.q, dt), to_dev(x.k, dt), to_dev(x.v, dt), to_dev(x.g, dt),
                              to_dev(x.beta, dt), scale=x.scale, cu_seqlens=cu)
    torch.cuda.synchronize()
    M_ref, N_ref = oracle_summary(x)
    em, en = rel_err(host(M), M_ref), rel_err(host(N), N_ref)
    _say(f"  rel err M={em:.2e} N={en:.2e}")
    assert em <= TOL[dtype] and en <= TOL[dtype]


def test_affine_summary_fp32_many_sequences():
    """40 sequences x 2 heads in fp32 at K = 128: more stage 3+4 workgroups than
    CUs, so the summary passes run in rounds."""
    import kimi_delta_attention_03_amd as kda
    import torch
    lengths = np.random.default_rng(72).integers(0, 200, size=40)
    x = core_inputs(1, None, 2, 128, 128, dtype="fp32", seed=73, lengths=lengths, g_low=-0.05)
    _say("affine summary fp32 K=128, 40 sequences")
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32)).to("cuda:0")
    M, N = kda.affine_summary(to_dev(x.q, torch.float32), to_dev(x.k, torch.float32), to_dev(x.v, torch.float32),
                              to_dev(x.g, torch.float32), to_dev(x.beta, torch.float32), scale=x.scale, cu_seqlens=cu)
    torch.cuda.synchronize()
    M_ref, N_ref = oracle_summary(x)
    em, en = rel_err(host(M), M_ref), rel_err(host(N), N_ref)
    _say(f"  rel err M={em:.2e} N={en:.2e}")
    assert em <= TOL["fp32"] and en <= TOL["fp32"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_context_parallel_merge_on_one_gpu(dtype):
    """Two halves of each sequence summarised independently (as two ranks would),
    merged with kda_affine_apply, then the second half continued from the
    merged state: the outputs and the final state match one full pass."""
    import kimi_delta_attention_03_amd as kda
    import torch
    T, half = 512, 256
    x = core_inputs(2, T, 4, 128, 128, dtype=dtype, seed=81, init_std=0.1, g_low=-0.01)
    dt = _dt(dtype)
    dev = lambda a, sl: to_dev(np.ascontiguousarray(a[:, sl]), dt)
    first, second = slice(0, half), slice(half, T)
    M1, N1 = kda.affine_summary(*(dev(a, first) for a in (x.q, x.k, x.v, x.g, x.beta)), scale=x.scale)
    M2, N2 = kda.affine_summary(*(dev(a, second) for a in (x.q, x.k, x.v, x.g, x.beta)), scale=x.scale)
    S0 = to_dev(x.initial_state, torch.float32)
    S_mid = kda.affine_apply(M1, N1, S0)
    S_end = kda.affine_apply(M2, N2, S_mid)
    o2, f2 = kda.chunk_fwd(*(dev(a, second) for a in (x.q, x.k, x.v, x.g, x.beta)), scale=x.scale,
                           initial_state=S_mid)
    torch.cuda.synchronize()
    o_ref, f_ref = orc.kda_chunkwise(x.q, x.k, x.v, x.g, x.beta, x.scale, 64, x.initial_state)
    eo, ef, em = rel_err(host(o2), o_ref[:, half:]), rel_err(host(S_end), f_ref), rel_err(host(f2), f_ref)
    _say(f"CP merge {dtype}: rel err o(second half)={eo:.2e} merged final={ef:.2e} continued final={em:.2e}")
    assert max(eo, ef, em) <= TOL[dtype]
