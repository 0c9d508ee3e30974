"""Host-side checks of bench.py's accounting (no GPU): the algorithmic bytes and
FLOPs behind every roofline figure, tied to the library's actual record layout
and to their derivations, and the one-GPU guard of --gpus."""
import importlib.util
import os
import subprocess
import sys

import pytest

from kimi_delta_attention_03_amd import make_params, workspace_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("elem", [2, 4])
def test_record_bytes_match_the_library_layout(bench, K, elem):
    """The stage boundary bench.py prices (W, qg, kg, U, the 6 stored Aqk blocks,
    gamma) is exactly the record the library writes per 64-token chunk."""
    dt = 1 if elem == 2 else 0
    info = workspace_layout(make_params(1, 4096, 2, K, K, dt, dt, dt, K ** -0.5))
    s12, s34 = bench.alg_bytes_per_token_head(K, K, elem, elem, elem)
    rec = info.record_bytes / 64
    inputs = 3 * K * elem + K * elem + elem          # q, k, g (K each), v (V), beta
    assert s12 == pytest.approx(inputs + rec)
    assert s34 == pytest.approx(rec + K * elem)       # the record in, o out


def test_headline_bytes_and_flops(bench):
    """K = V = 128 with bf16 inputs: 1026 B read by stage 1+2, a 1128 B record,
    256 B of o, and the causal-triangle FLOP count of one chunk-head."""
    s12, s34 = bench.alg_bytes_per_token_head(128, 128, 2, 2, 2)
    assert (s12, s34) == (1026 + 1128, 1128 + 256)
    C, K, V = 64, 128, 128
    want = 6 * C * K * V + C * (C + 1) * (3 * K + 2 * V) + C ** 3 / 3
    assert bench.alg_flops_per_chunk_head(C, K, V) == pytest.approx(want)
    assert want == pytest.approx(9.04e6, rel=1e-3)


def test_backward_chunk_bytes(bench):
    """The backward's chunk pair: inputs q, k, g, v, dO, beta, the fp32 state
    and end-state gradient once per chunk, fp32 gradients out."""
    assert bench.bwd_chunk_alg_bytes_per_token_head(128, 128, 2) == 1282 + 2048 + 2052
    assert bench.bwd_chunk_alg_bytes_per_token_head(64, 64, 4) == (
        (3 * 64 + 2 * 64 + 1) * 4 + 2 * 64 * 64 * 4 / 64 + (3 * 64 + 64 + 1) * 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout.strip()
