// Launch interface of the layer's projection GEMM (kda_gemm.hip). Internal
// to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct GemmArgs {
  const void* A;       // bf16 [M, K], row stride lda (elements)
  const void* B;       // bf16 [N, K], row stride ldb
  void* C;             // [M, N], row stride ldc, bf16 or fp32
  int64_t M, N, K, lda, ldb, ldc;
  int ntm, ntn;        // tiles along M and N (set by the launcher)
  int vec_out;         // C rows 16-byte aligned: bf16 C staged for row stores (set by the launcher)
  int vec4;            // runs of 4 elements of C aligned to their size: vector stores (set by the launcher)
  // optional output-gate epilogue (bf16 C only): with norm_o set, the product G
  // is not stored; instead C[m, n] = o[m, n] * rsqrt(mean over n's head of o^2
  // + norm_eps) * norm_w[n % norm_d] * sigmoid(G[m, n]), heads of norm_d columns
  const float* norm_o; // fp32 [M, N], row stride ldo
  const float* norm_w; // fp32 [norm_d]
  int64_t ldo;
  int norm_d;          // 64 or 128
  float norm_eps;
};

// C = A B^T on MFMA (bf16 operands, fp32 accumulation); out_f32 selects fp32 C.
// K <= 128 takes a kernel of its own (whole K per pass, several workgroups per
// CU), larger K the 256 x 256 tiled pipeline.
// With a.norm_o set (bf16 C, 16-byte aligned rows of C and o, ldc and ldo
// multiples of 8, N a multiple of norm_d) the output-gate epilogue runs instead
// of the plain store; hipErrorInvalidValue if those conditions do not hold.
hipError_t launch_gemm_bf16(const GemmArgs& a, int out_f32, hipStream_t s);

}  // namespace kda
