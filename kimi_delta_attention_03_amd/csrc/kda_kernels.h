// Launch interface between the host dispatcher (kda_api.cpp) and the gfx950
// kernels. Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"
#include "kda_layout.h"

namespace kda {

struct Stage12Args {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  int g_f32;        // 1: g is fp32, 0: bf16
  int beta_f32;     // 1: beta is fp32, 0: bf16
  int H;
  float scale;
  int l2norm;
  float l2eps;
  int varlen;       // 1: chunk table in the workspace metadata
  int gate_mode;    // 0: g is the log decay; 1: softplus; 2: lower-bound sigmoid (raw gate in g)
  float gate_lb;    // lower bound of mode 2
  const float* A_log;    // [H] (modes 1, 2)
  const float* dt_bias;  // [H, K] or null (modes 1, 2)
  char* ws;         // workspace base
  size_t meta_bytes, rec_bytes, ncp;
  size_t off_chunk_tab;
  size_t off_w, off_qg, off_kg, off_aq, off_u, off_gam;
  // fixed length: chunk slot p holds chunk p % nt_seg of batch row p / nt_seg of
  // the segment starting at token seg_t0 of every row (rows are row_T tokens long)
  int64_t row_T, seg_t0;
  int nt_seg;
};

struct Stage34Args {
  const float* init;   // [N, H, K, V] or null
  float* final_state;  // [N, H, K, V] or null
  void* o;             // or null: no output (affine summaries)
  int init_identity;   // 1: the state starts at the identity (K == V)
  int zero_u;          // 1: U is taken as zero (the linear part of the affine map)
  int H;
  int nunits;          // N * H
  int nt;              // fixed length: chunks per batch row in this segment
  int64_t row_T;       // fixed length: tokens per batch row of the tensors
  int64_t seg_t0;      // fixed length: first token of the segment in every row
  int varlen;
  const char* ws;
  size_t meta_bytes, rec_bytes, ncp;
  size_t off_chunk_tab, off_seq_tab, off_order, off_sink;
  size_t off_w, off_qg, off_kg, off_aq, off_u, off_gam;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  float* state;        // [N, H, K, V], in place
  void* o;
  float scale;
  int l2norm;
  float l2eps;
  int nunits;          // N * H
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const void* d_o;          // [B, T, H, V], q's dtype
  const float* init;        // [N, H, K, V] or null
  const float* d_final;     // [N, H, K, V] or null
  float* dq;                // [B, T, H, K]
  float* dk;
  float* dv;                // [B, T, H, V]
  float* dg;                // [B, T, H, K]
  float* dbeta;             // [B, T, H]
  float* dh0;               // [N, H, K, V] or null
  int bf16_qkv, g_f32, beta_f32;
  int H;
  float scale;
  int l2norm;
  float l2eps;
  int varlen;
  int nunits;               // N * H
  int nt;                   // fixed length: chunks per batch row
  char* ws;
  size_t meta_bytes, ncp;
  size_t off_chunk_tab, off_seq_tab;
  BwdSlab sl;
};

// bf16 == 1 selects the bf16 instantiation (bf16 q/k/v, bf16 intermediates).
hipError_t launch_stage12(const Stage12Args& a, int K, int bf16, int nblocks, hipStream_t s);
hipError_t launch_stage34(const Stage34Args& a, int K, int bf16, hipStream_t s);
hipError_t launch_varlen_map(const int32_t* cu, int nseq, int64_t T, char* ws, size_t ncp,
                             size_t off_chunk_tab, size_t off_seq_tab, size_t off_order,
                             hipStream_t s);

// S_out = M S0 + N for each of nunits (sequence, head) pairs, K == V
hipError_t launch_affine_apply(const float* M, const float* N, const float* S0, float* S_out, int nunits, int K,
                               hipStream_t s);
// backward: chunk-term recompute, chunk-start states, state gradients, chunk gradients
// stages: bit mask of the four launches (1 prep, 2 states, 4 state gradients, 8 chunk gradients)
hipError_t launch_bwd(const BwdArgs& a, int K, int nitems, int stages, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int K, int bf16_qkv, int g_f32, int b_f32, hipStream_t s);

// sets the thread-local message returned by kda_last_error and returns s
kda_status fail_msg(kda_status s, const char* fmt, ...);
void clear_msg();

}  // namespace kda
