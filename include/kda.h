/*
 * kda.h - C ABI of the MI355X (gfx950) chunkwise Kimi Delta Attention forward.
 *
 * The operation (all three sources agree on it):
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 * per (sequence, head), with a K x V fp32 state S and a per-channel natural-log
 * decay g <= 0. Defined as Paper Eq. 1 in the Tokamax "chunk_kda_fwd design
 * doc" (openxla.org), section 9.1.2, and as steps (0)-(5) in "KDA Doesn't Care
 * About the Future" (drisspg.github.io), section "Chunkwise KDA in Broad
 * Strokes". The library evaluates it chunkwise (chunk size 64): Tokamax design
 * doc sections 4.1 (stage 1+2: gate cumsum, relation matrices, unit
 * lower-triangular solve, W/U factors) and 4.3 (stage 3+4: ordered state
 * recurrence and output), Paper Eq. 6-9 (section 9.1.5-9.1.6).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers on the current HIP device; the caller
 *    owns every buffer, the library keeps no pointer after the call returns
 *    and allocates nothing.
 *  - Work is enqueued on `stream` and the call returns without synchronising,
 *    so calls can be captured in a HIP graph.
 *  - Shapes, dtypes, sizes and alignment are checked on the host before any
 *    launch; a failed check returns a non-zero kda_status and launches
 *    nothing. kda_last_error() then gives a message (thread-local).
 *  - Value preconditions are NOT checked on the fast path: g in [-5, 0]
 *    (the lower bound of the pages; it keeps the rebased operands inside the
 *    fp32 range), beta in [0, 1], cu_seqlens non-decreasing from 0 to T.
 *    Values outside give undefined numbers but never an out-of-bounds access.
 *    kda_validate_inputs checks them on request (it synchronises).
 *
 * Layouts (row-major, contiguous, token-major like the layer projections):
 *   q, k, g : [B, T, H, K]     v, o : [B, T, H, V]     beta : [B, T, H]
 *   initial_state, final_state : [N, H, K, V] fp32, N = B (fixed length) or
 *   num_seqs (variable length).
 * Variable length (Tokamax design doc section 3.5 and 9.1.7): B must be 1,
 * the sequences are packed along T and cu_seqlens[0..num_seqs] (int32,
 * device) gives their boundaries. Every sequence is cut into chunks from its
 * own start, so no chunk spans two sequences; a short last chunk is padded
 * virtually with q = k = v = beta = 0, g = 0 (zero writes, identity decay).
 */
#ifndef KDA_MI355X_H
#define KDA_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 2

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1,   /* bad shape, dtype, pointer, alignment or size */
  KDA_ERR_UNSUPPORTED = 2,   /* valid request the GPU path does not implement */
  KDA_ERR_WORKSPACE = 3,     /* workspace missing or too small */
  KDA_ERR_HIP = 4            /* a HIP runtime call failed (launch error) */
} kda_status;

typedef struct {
  int64_t B, T, H;       /* batch, tokens per row (total packed tokens if varlen), heads */
  int32_t K, V;          /* head dims; the GPU path supports K == V in {64, 128} */
  int32_t qkv_dtype;     /* kda_dtype of q, k, v and of the output o */
  int32_t g_dtype;       /* kda_dtype of g */
  int32_t beta_dtype;    /* kda_dtype of beta */
  float scale;           /* output scale, usually K^-1/2 */
  int32_t chunk_size;    /* must be 64 */
  int32_t use_qk_l2norm; /* 1: q, k <- x / max(||x||_2, l2norm_eps) per token and head
                            ("KDAChunkwise" docs, section "FP32 core and log-space decay") */
  float l2norm_eps;      /* eps of the L2 normalisation (1e-6 by convention) */
  int32_t num_seqs;      /* 0: fixed length (T % 64 == 0, cu_seqlens NULL);
                            > 0: variable length with that many sequences (B == 1) */
} kda_fwd_params;

/* Bytes of device workspace kda_chunk_fwd needs for these parameters.
 * Returns KDA_ERR_* if the parameters are invalid. Pure host computation. */
kda_status kda_chunk_fwd_workspace_bytes(const kda_fwd_params* p, size_t* bytes);

/* Full forward: stage 1+2 then stage 3+4 on `stream`.
 *   q, k, v, g, beta : inputs as laid out above (16-byte aligned, beta 4-byte)
 *   initial_state    : [N, H, K, V] fp32 or NULL (zeros)
 *   cu_seqlens       : [num_seqs + 1] int32 or NULL (fixed length)
 *   o                : output, dtype qkv_dtype, same layout as v
 *   final_state      : [N, H, K, V] fp32 or NULL (not written)
 *   workspace        : device buffer of at least kda_chunk_fwd_workspace_bytes
 * A zero-length sequence writes final_state = initial_state (or zeros). */
kda_status kda_chunk_fwd(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, const float* initial_state,
                         const int32_t* cu_seqlens, void* o, float* final_state,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gate activation applied inside stage 1+2 (Tokamax "chunk_kda_fwd design
 * doc", section 9.1.3). With x = g_raw + dt_bias (per channel) and
 * lambda = exp(A_log_h):
 *   KDA_GATE_SOFTPLUS:             g = -lambda * softplus(x)
 *   KDA_GATE_LOWER_BOUND_SIGMOID:  g = lower_bound * sigmoid(lambda * x)
 * The lower-bound form keeps g in (lower_bound, 0) by construction; for the
 * softplus form the g >= -5 precondition of the fast path becomes
 * lambda * softplus(x) <= 5 (documented, not checked). */
typedef enum {
  KDA_GATE_LOG_DECAY = 0,            /* g is already the natural-log decay */
  KDA_GATE_SOFTPLUS = 1,
  KDA_GATE_LOWER_BOUND_SIGMOID = 2
} kda_gate_mode;

typedef struct {
  int32_t mode;           /* kda_gate_mode */
  float lower_bound;      /* KDA_GATE_LOWER_BOUND_SIGMOID: in [-5, 0) */
  const float* A_log;     /* [H] fp32, device; required for modes 1 and 2 */
  const float* dt_bias;   /* [H, K] fp32, device, or NULL (no bias) */
} kda_gate_params;

/* kda_chunk_fwd with the gate activation fused into stage 1+2: `g` holds the
 * raw gate (dtype p->g_dtype, layout [B, T, H, K]). gate may be NULL (same as
 * mode KDA_GATE_LOG_DECAY). Same workspace, stream and error rules. */
kda_status kda_chunk_fwd_gated(const kda_fwd_params* p, const kda_gate_params* gate, const void* q,
                               const void* k, const void* v, const void* g, const void* beta,
                               const float* initial_state, const int32_t* cu_seqlens, void* o,
                               float* final_state, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Stage 1+2 alone (Tokamax design doc section 4.1): chunk-local gate cumsum,
 * rebased Aqk / L relation tiles, (I + L)^{-1}, W, U, gated keys and queries,
 * written into the workspace (layout: kda_workspace_info). With cu_seqlens
 * it first builds the chunk map from cu_seqlens. Same argument rules as
 * kda_chunk_fwd. */
kda_status kda_chunk_fwd_stage12(const kda_fwd_params* p, const void* q, const void* k,
                                 const void* v, const void* g, const void* beta,
                                 const int32_t* cu_seqlens, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Stage 3+4 alone (Tokamax design doc section 4.3): reads a workspace filled
 * by kda_chunk_fwd_stage12 with the same parameters and writes o and
 * final_state. With cu_seqlens it rebuilds the chunk map first, so a workspace
 * that stage 1+2 has not filled yields meaningless values but no access outside
 * the buffers. */
kda_status kda_chunk_fwd_stage34(const kda_fwd_params* p, const float* initial_state,
                                 const int32_t* cu_seqlens, void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Where stage 1+2 puts its outputs inside the workspace (for inspection).
 * All offsets are in bytes. For head h and physical chunk p the record starts
 * at records_offset + (p * H + h) * record_bytes (chunk-major) and holds, in
 * the stored element type (bf16 for bf16 q/k/v, else fp32):
 *   W, QG (qg), KG (kg^T), AQ (Aqk, the 6 causally non-zero fragments) as
 *   16-row x 32-wide MFMA fragments and U in accumulator-tile order, then
 *   gamma (fp32, K values). The fragment orders are documented in
 *   kimi_delta_attention_03_amd/csrc/kda_layout.h. */
typedef struct {
  size_t total_bytes, records_offset, record_bytes, chunk_slots;
  size_t off_w, off_qg, off_kg, off_aq, off_u, off_gamma;
  int32_t elem_bytes;
  size_t off_chunk_table;  /* varlen: int32 pairs (first token, valid length) per chunk slot */
  size_t off_seq_table;    /* varlen: int32 pairs (first chunk slot, chunk count) per sequence */
  size_t off_order;        /* varlen: sequences ordered longest first */
  int32_t segments;        /* kda_chunk_fwd runs fixed-length bf16 inputs in this many segments along T
                              (1 for fp32 and variable-length inputs) */
  int32_t segment_chunks;  /* chunks per row in each segment (the last may be shorter); the records
                              of one segment fill the chunk slots from 0 */
} kda_workspace_info;

kda_status kda_workspace_layout(const kda_fwd_params* p, kda_workspace_info* info);

/* Affine summary of each sequence's chunks (Tokamax "chunk_kda_fwd design
 * doc", sections 4.2 and 9.1.8): the recurrence is affine in the state, so for
 * every initial state S0 the final state is M S0 + N, with
 * M = prod over chunks of (Diag(gamma) - kg^T W) and N the final state reached
 * from S0 = 0. Reads a workspace filled by kda_chunk_fwd_stage12 with the same
 * parameters; writes M [N_seq, H, K, K] and N [N_seq, H, K, V] fp32 (N_seq = B
 * or num_seqs). This is the per-rank building block of context parallelism
 * along T. Requires K == V. */
kda_status kda_chunk_affine_summary(const kda_fwd_params* p, const int32_t* cu_seqlens, float* M, float* N,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Merge step: S_out = M S0 + N for every (sequence, head), fp32, shapes as
 * above (S0 and S_out [N_seq, H, K, V]); S_out must not alias S0 or M. Uses
 * B (or num_seqs), H, K, V of p only. */
kda_status kda_affine_apply(const kda_fwd_params* p, const float* M, const float* N, const float* S0, float* S_out,
                            hipStream_t stream);

/* One decode step of the token recurrence for B independent sequences
 * ("KDA Doesn't Care About the Future", section "Chunkwise KDA in Broad
 * Strokes", steps (0)-(5); Tokamax "chunk_kda_fwd design doc" section 9.1.2,
 * Paper Eq. 1), with the same state layout as the chunked path:
 *   S <- (I - beta k k^T) Diag(exp g) S + beta k v^T,   o = scale * S^T q
 * p->T must be 1 (one token per batch row), p->num_seqs 0; chunk_size is
 * ignored. q, k, g: [B, 1, H, K]; v, o: [B, 1, H, V]; beta: [B, 1, H];
 * state: [B, H, K, V] fp32, read and overwritten in place (the state after
 * the token). use_qk_l2norm normalises q and k as in kda_chunk_fwd. Needs
 * no workspace; same stream and error conventions as the other calls. */
kda_status kda_decode_step(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, float* state, void* o, hipStream_t stream);

/* Backward of kda_chunk_fwd: the gradients of <d_o, o> + <d_final_state, final_state>
 * with respect to q, k, v, g, beta and initial_state (Tokamax "chunk_kda_fwd design doc",
 * sections 4.3.4 and 6.1: the backward returns dq, dk, dv, dg, dbeta and the optional dh0
 * of the same forward map, rebuilding the chunk intermediates from the inputs rather than
 * keeping them from the forward).
 *   p, q, k, v, g, beta, initial_state, cu_seqlens: exactly as passed to kda_chunk_fwd
 *     (g is the log decay: the gate activation of kda_chunk_fwd_gated has no backward here).
 *   d_o:           [B, T, H, V] in qkv_dtype, the gradient of o (rows of every token used),
 *                  16-byte aligned; q, k, v, g, beta aligned to their element size.
 *   d_final_state: [N, H, K, V] fp32 or NULL (zero).
 *   dq, dk, dg:    [B, T, H, K] fp32;  dv: [B, T, H, V] fp32;  dbeta: [B, T, H] fp32.
 *     With use_qk_l2norm, dq and dk are the gradients of the un-normalised q and k.
 *   d_initial_state: [N, H, K, V] fp32 or NULL (not written).
 * All arithmetic is fp32. Every pointer is a device pointer owned by the caller; inputs
 * are not modified. The workspace (kda_chunk_bwd_workspace_bytes, 256-byte aligned) holds
 * the chunk map and one fp32 slab per (chunk, head) of intermediates. Asynchronous on
 * `stream`; no allocation, no host synchronisation. Errors: as kda_chunk_fwd; nothing is
 * launched when a check fails. */
kda_status kda_chunk_bwd_workspace_bytes(const kda_fwd_params* p, size_t* bytes);
kda_status kda_chunk_bwd(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, const float* initial_state,
                         const int32_t* cu_seqlens, const void* d_o, const float* d_final_state,
                         float* dq, float* dk, float* dv, float* dg, float* dbeta,
                         float* d_initial_state, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* kda_chunk_bwd split into its four launches, for timing each: `stages` is a bit mask
 * (1: rebuild the chunk terms into the workspace, 2: chunk-start states, 4: state
 * gradients and d_initial_state, 8: every other gradient). Each stage reads what the
 * earlier ones left in the same workspace, so stages run in increasing order over one
 * workspace reproduce kda_chunk_bwd exactly; 15 is kda_chunk_bwd. With cu_seqlens every
 * call rebuilds the chunk map, so a stage run on a workspace the earlier stages have not
 * filled yields meaningless values but no access outside the buffers. Arguments, errors and
 * ownership as kda_chunk_bwd; KDA_ERR_INVALID_ARG for a mask outside [1, 15]. */
kda_status kda_chunk_bwd_stages(const kda_fwd_params* p, int32_t stages, const void* q, const void* k,
                                const void* v, const void* g, const void* beta,
                                const float* initial_state, const int32_t* cu_seqlens,
                                const void* d_o, const float* d_final_state, float* dq, float* dk,
                                float* dv, float* dg, float* dbeta, float* d_initial_state,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Value preconditions of the fast path, checked on the GPU (Tokamax
 * "chunk_kda_fwd design doc", section 5.3 "Required Runtime Invariants": the
 * log decay inside the lower bound [-5, 0] and beta in [0, 1]; section 3.5:
 * cu_seqlens[0] == 0, non-decreasing, cu_seqlens[num_seqs] == T). The lower
 * bound matters: below g = -5 the rebased in-chunk key factors leave the fp32
 * range ("KDA Doesn't Care About the Future", section "What's the catch?").
 *   p          : as for kda_chunk_fwd (B, T, H, K, g_dtype, beta_dtype and
 *                num_seqs are used)
 *   g          : [B, T, H, K] log decay (dtype g_dtype), device
 *   beta       : [B, T, H] (dtype beta_dtype), device
 *   cu_seqlens : [num_seqs + 1] int32, device, or NULL when num_seqs == 0
 *   scratch    : device buffer of >= KDA_VALIDATE_SCRATCH_BYTES, 16-byte
 *                aligned, owned by the caller (contents overwritten)
 *   report     : host struct; report->failed is -1 until the check has run
 * SYNCHRONISES `stream` (it copies the reduction back to the host). Returns
 * KDA_OK when every precondition holds, KDA_ERR_INVALID_ARG naming the first
 * failed one (non-finite g, g range, non-finite beta, beta range, cu_seqlens)
 * in kda_last_error(), or the usual argument / HIP errors. Reads only the
 * elements of the three inputs; any values, however malformed, are safe. */
#define KDA_VALIDATE_SCRATCH_BYTES 16384
typedef struct {
  float g_min, g_max;          /* over the finite entries of g (+inf / -inf if there are none) */
  float beta_min, beta_max;    /* over the finite entries of beta */
  int64_t g_nonfinite;         /* NaN or infinite entries of g */
  int64_t beta_nonfinite;      /* NaN or infinite entries of beta */
  int64_t cu_first_bad;        /* -1, or the first index of cu_seqlens that breaks the conditions */
  int32_t failed;              /* -1: not run (argument error); 0: every precondition holds;
                                  1: non-finite g, 2: g outside [-5, 0], 3: non-finite beta,
                                  4: beta outside [0, 1], 5: cu_seqlens (the first that fails) */
} kda_input_report;

kda_status kda_validate_inputs(const kda_fwd_params* p, const void* g, const void* beta,
                               const int32_t* cu_seqlens, void* scratch, size_t scratch_bytes,
                               hipStream_t stream, kda_input_report* report);

/* kda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same forward, with the workspace taken from a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends. Arguments, results, stream and error rules as
 * kda_chunk_fwd, without the workspace arguments. Problems whose
 * kda_chunk_fwd_workspace_bytes exceeds KDA_NOALLOC_SCRATCH_BYTES return
 * KDA_ERR_WORKSPACE (128 MiB holds e.g. 1850 bf16 chunk-heads at K = V = 128,
 * 118k token-heads). Nothing is allocated or freed. Every call on one GPU uses
 * that GPU's single array: calls that overlap on one GPU (several streams or
 * threads) race and must be serialised by the caller. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
kda_status kda_chunk_fwd_noalloc(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, void* o, float* final_state,
                                 hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* kda_status_string(kda_status s);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the built library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_MI355X_H */
