"""The layer's projection GEMM (kda_gemm_bf16_nt: bf16 operands, fp32
accumulation, hand-written MFMA kernel) against a plain PyTorch fp32 matmul of
the same bf16 values, through the C ABI. Shapes cover partial tiles along M, N
and K, strided operands (the layer reads slices of its projection buffer in
place) and the layer's own projection shapes.

Metric: max|C - C_ref| / max|C_ref|: <= 1e-5 for fp32 C (only the summation
order differs) and <= 4e-3 for bf16 C (one rounding to bf16, 2^-9 relative,
plus the order)."""
import ctypes
import sys

import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gemm(A, B, out_f32, lda=None, ldb=None, C=None, ldc=None):
    import torch
    from kimi_delta_attention_03_amd import _lib
    M, K = A.shape
    N = B.shape[0]
    lda = lda or A.stride(0)
    ldb = ldb or B.stride(0)
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=A.device)
    ldc = ldc or C.stride(0)
    st = _lib.load().kda_gemm_bf16_nt(M, N, K, ctypes.c_void_p(A.data_ptr()), lda, ctypes.c_void_p(B.data_ptr()),
                                      ldb, ctypes.c_void_p(C.data_ptr()), ldc, 0 if out_f32 else 1,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st)
    return C


def ref(A, B):
    return A.float() @ B.float().t().contiguous()


def rel(x, y):
    return float((x.float() - y).abs().max() / y.abs().max())


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (300, 200, 136), (256, 256, 64), (511, 513, 520), (1024, 96, 2048)])
@pytest.mark.parametrize("out_f32", [True, False])
def test_gemm_shapes(M, N, K, out_f32):
    import torch
    _say(f"gemm M={M} N={N} K={K} out_f32={out_f32}")
    g = torch.Generator(device="cuda:0").manual_seed(M * 7 + N * 3 + K)
    A = torch.randn(M, K, device="cuda:0", generator=g).to(torch.bfloat16)
    B = torch.randn(N, K, device="cuda:0", generator=g).to(torch.bfloat16)
    C = gemm(A, B, out_f32)
    torch.cuda.synchronize()
    e = rel(C, ref(A, B))
    _say(f"  rel err {e:.2e}")
    assert e <= (1e-5 if out_f32 else 4e-3)


def test_gemm_strided_slices():
    """A is a column slice of a wider buffer (row stride > K) and C lands in a
    wider buffer, as the layer's low-rank projections do; columns outside C's
    window stay untouched."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(5)
    P = torch.randn(700, 400, device="cuda:0", generator=g).to(torch.bfloat16)
    A = P[:, 136:136 + 128]
    B = torch.randn(300, 128, device="cuda:0", generator=g).to(torch.bfloat16)
    Cbuf = torch.full((700, 320), 7.0, device="cuda:0")
    C = Cbuf[:, 8:308]
    gemm(A, B, True, lda=400, C=C, ldc=320)
    torch.cuda.synchronize()
    assert rel(C, ref(A.contiguous(), B)) <= 1e-5
    assert torch.all(Cbuf[:, :8] == 7.0) and torch.all(Cbuf[:, 308:] == 7.0)


@pytest.mark.parametrize("ldc,c0", [(320, 8), (322, 8), (320, 4)],
                         ids=["aligned_rows", "odd_row_stride", "misaligned_start"])
def test_gemm_strided_bf16_output(ldc, c0):
    """bf16 C inside a wider buffer: 16-byte aligned rows take the staged
    row-piece stores (with pieces crossing N written element by element),
    other strides or starts the element stores; columns outside C's window and
    rows past M stay untouched."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(11)
    M, N, K = 700, 300, 200
    A = torch.randn(M, K, device="cuda:0", generator=g).to(torch.bfloat16)
    B = torch.randn(N, K, device="cuda:0", generator=g).to(torch.bfloat16)
    Cbuf = torch.full((M + 1, ldc), 7.0, device="cuda:0").to(torch.bfloat16)
    C = Cbuf[:M, c0:c0 + N]
    gemm(A, B, False, C=C, ldc=ldc)
    torch.cuda.synchronize()
    assert rel(C, ref(A, B)) <= 4e-3
    assert torch.all(Cbuf[:, :c0] == 7.0) and torch.all(Cbuf[:, c0 + N:] == 7.0) and torch.all(Cbuf[M] == 7.0)


@pytest.mark.parametrize("M,N,K,out_f32", [(32768, 6416, 2048, False), (32768, 2048, 128, True),
                                           (32768, 2048, 2048, False)],
                         ids=["input_projection", "low_rank_up", "output_projection"])
def test_gemm_layer_shapes(M, N, K, out_f32):
    """The layer's projections at workload 4 (B T = 32768 tokens, M = 2048)."""
    import torch
    _say(f"gemm layer shape M={M} N={N} K={K}")
    g = torch.Generator(device="cuda:0").manual_seed(9)
    A = (torch.randn(M, K, device="cuda:0", generator=g) * 0.5).to(torch.bfloat16)
    B = (torch.randn(N, K, device="cuda:0", generator=g) * K ** -0.5).to(torch.bfloat16)
    C = gemm(A, B, out_f32)
    torch.cuda.synchronize()
    e = rel(C, ref(A, B))
    _say(f"  rel err {e:.2e}")
    assert e <= (1e-5 if out_f32 else 4e-3)
