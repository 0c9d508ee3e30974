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
  int vec_out;         // C rows 4-element aligned: full tiles use vector stores (set by the launcher)
};

// C = A B^T on MFMA (bf16 operands, fp32 accumulation); out_f32 selects fp32 C
hipError_t launch_gemm_bf16(const GemmArgs& a, int out_f32, hipStream_t s);

}  // namespace kda
