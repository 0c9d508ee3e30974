/*
 * kda_layer.h - C ABI of the KDA layer forward around the chunkwise core, for
 * one MI355X (gfx950). Part of libkda_mi355x.so; include kda.h first.
 *
 * What it computes ("KDAChunkwise" docs, sections "From the hidden states to
 * causal Q, K, and V", "FP32 core and log-space decay", "Returning to the
 * model dimension"; the gate is the lower-bound sigmoid variant of the
 * Tokamax "chunk_kda_fwd design doc", section 9.1.3). For x [B, T, M]:
 *   P      = x Wqkv^T                               [B, T, 3 H D]
 *   q,k,v  = SiLU(causal depthwise conv_4(P_{q,k,v})) per channel, left zero
 *            padding inside each batch row; q, k <- x / max(||x||_2, l2_eps)
 *            over D for every (token, head)
 *   beta   = sigmoid(x Wb^T)                        [B, T, H]
 *   g      = lb * sigmoid(exp(A_log_h) * (x Wad^T Wau^T + dt_bias))  [B, T, H, D]
 *   o      = chunkwise KDA core in fp32 (scale D^-1/2, zero initial state)
 *   y      = RMSNorm_D(o) * norm_w * sigmoid(x Wgd^T Wgu^T)
 *   x_new  = y Wo^T                                 [B, T, M]
 *
 * Implementation: every step runs in this library's HIP kernels: the
 * projections on its bf16 MFMA GEMM (fp32 accumulation, kda_gemm_bf16_nt),
 * conv + SiLU + L2 norm and beta in an elementwise kernel, the decay-gate
 * activation inside the core's first stage, the RMSNorm and output gate in the
 * epilogue of the output-gate up-projection GEMM (the gate factor rounded to
 * fp16 before it scales the normalised o), and the core on the same two-kernel
 * path as kda_chunk_fwd with fp32 q, k, v, g and beta.
 *
 * Conventions:
 *  - Every tensor pointer is a DEVICE pointer; row-major and contiguous.
 *    Linear weights are [out, in]. The caller owns every buffer.
 *  - Work is enqueued on `stream`; the call does not synchronise and
 *    allocates nothing (the caller's workspace holds every intermediate), so
 *    it can be captured in a HIP graph. It keeps no state between calls and
 *    may be called from several threads at once on different workspaces.
 *  - Shapes and sizes are checked on the host before any launch; a failed
 *    check returns a non-zero kda_status and launches nothing.
 *  - Value preconditions are not checked (finite inputs are assumed).
 */
#ifndef KDA_MI355X_LAYER_H
#define KDA_MI355X_LAYER_H

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t B, T;            /* batch rows and tokens per row; T % 64 == 0 */
  int32_t M;               /* model width (multiple of 8) */
  int32_t H, D;            /* heads and head dim; D in {64, 128} */
  int32_t gate_rank;       /* rank r of the decay gate (Wad [r, M], Wau [H D, r]); multiple of 8 */
  int32_t out_gate_rank;   /* rank of the output gate (Wgd [rg, M], Wgu [H D, rg]); multiple of 8 */
  int32_t conv_size;       /* depthwise causal conv width; must be 4 */
  float gate_lower_bound;  /* lb of the decay gate, e.g. -5 (g in [lb, 0]) */
  float norm_eps;          /* RMSNorm eps, e.g. 1e-6 */
  float l2_eps;            /* q / k L2-normalisation eps, e.g. 1e-6 */
} kda_layer_params;

typedef struct {
  const void* Wqkv;        /* bf16 [3 H D, M]: rows 0..HD-1 -> q, HD..2HD-1 -> k, then v */
  const float* conv_q;     /* fp32 [H D, conv_size]; tap conv_size-1 multiplies the current token */
  const float* conv_k;     /* fp32 [H D, conv_size] */
  const float* conv_v;     /* fp32 [H D, conv_size] */
  const void* Wb;          /* bf16 [H, M] */
  const void* Wad;         /* bf16 [gate_rank, M] */
  const void* Wau;         /* bf16 [H D, gate_rank] */
  const float* A_log;      /* fp32 [H] */
  const float* dt_bias;    /* fp32 [H D] */
  const void* Wgd;         /* bf16 [out_gate_rank, M] */
  const void* Wgu;         /* bf16 [H D, out_gate_rank] */
  const float* norm_w;     /* fp32 [D] */
  const void* Wo;          /* bf16 [M, H D] */
} kda_layer_weights;
/* The input projection multiplies x by the row concatenation [Wqkv; Wad; Wgd;
 * Wb] ([3 H D + gate_rank + out_gate_rank + H, M]). If the four matrices
 * already sit back to back in that order in one allocation (Wad starting where
 * Wqkv ends, and so on) with Wqkv 16-byte aligned, the GEMM reads them in
 * place; otherwise each call first copies them into the workspace (four
 * device-to-device copies on `stream`). */

/* The layer's projection GEMM on its own (bf16 operands, fp32 accumulation,
 * hand-written MFMA kernel): C[m, n] = sum_k A[m, k] B[n, k] for A [M, K] and
 * B [N, K], both row-major with K contiguous (activations [tokens, features]
 * and Linear weights [out, in], as in the "KDAChunkwise" docs' projections),
 * row strides lda, ldb, ldc in elements. c_dtype is KDA_DTYPE_BF16 (rounded to
 * nearest even) or KDA_DTYPE_F32. Device pointers; A and B 16-byte aligned with
 * K, lda and ldb multiples of 8 and lda, ldb <= 2^21 (KDA_ERR_UNSUPPORTED
 * beyond); C must not overlap A or B. Asynchronous on `stream`, no allocation;
 * errors as for the other entry points. */
kda_status kda_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, void* C, int64_t ldc, int32_t c_dtype, hipStream_t stream);

/* Device workspace bytes kda_layer_fwd needs (pure host computation). */
kda_status kda_layer_fwd_workspace_bytes(const kda_layer_params* p, size_t* bytes);

/* Where kda_layer_fwd leaves the core's fp32 inputs in its workspace (byte
 * offsets): q, k, v [B, T, H, D] (after conv, SiLU and, for q and k, the L2
 * norm), the raw decay gate x Wad^T Wau^T [B, T, H, D] (before dt_bias and the
 * activation, which run inside the core), beta [B, T, H], and the core output
 * o [B, T, H, D] (used when core_out is NULL). They hold the last call's
 * values until the workspace is reused. Pure host computation. */
typedef struct {
  size_t total_bytes;
  size_t off_q, off_k, off_v, off_g_raw, off_beta, off_o;
} kda_layer_workspace_info;

kda_status kda_layer_workspace_layout(const kda_layer_params* p, kda_layer_workspace_info* info);

/* x: bf16 [B, T, M]; x_new: bf16 [B, T, M] (must not alias x).
 * If core_out is not NULL it receives the fp32 core output o [B, T, H, D]
 * (before the norm), for inspection. */
kda_status kda_layer_fwd(const kda_layer_params* p, const kda_layer_weights* w, const void* x,
                         void* x_new, float* core_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_MI355X_LAYER_H */
