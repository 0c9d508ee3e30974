// Host side of the C ABI declared in include/kda.h: argument validation,
// workspace sizing and kernel dispatch. Nothing here allocates or
// synchronises; every launch goes to the caller's stream.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda_kernels.h"
#include "kda_layout.h"

namespace {

thread_local char g_msg[512] = "";

kda_status fail(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kda_status check_params(const kda_fwd_params* p) {
  g_msg[0] = 0;
  if (!p) return fail(KDA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 0 || p->T < 0 || p->H <= 0) return fail(KDA_ERR_INVALID_ARG, "need B >= 0, T >= 0, H > 0");
  if (p->K <= 0 || p->V <= 0) return fail(KDA_ERR_INVALID_ARG, "need K > 0 and V > 0");
  if (p->K > 256) return fail(KDA_ERR_INVALID_ARG, "K must be <= 256 (got %d)", p->K);
  if (!(p->K == p->V && (p->K == 64 || p->K == 128)))
    return fail(KDA_ERR_UNSUPPORTED, "GPU path supports K == V in {64, 128} (got K=%d V=%d)", p->K, p->V);
  for (int32_t d : {p->qkv_dtype, p->g_dtype, p->beta_dtype})
    if (d != KDA_DTYPE_F32 && d != KDA_DTYPE_BF16) return fail(KDA_ERR_INVALID_ARG, "unknown dtype %d", d);
  if (p->chunk_size != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk_size must be 64 (got %d)", p->chunk_size);
  if (p->use_qk_l2norm && !(p->l2norm_eps > 0.f)) return fail(KDA_ERR_INVALID_ARG, "l2norm_eps must be > 0");
  if (p->num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (p->num_seqs > 0) {
    if (p->B != 1) return fail(KDA_ERR_INVALID_ARG, "variable-length input needs B == 1 (got %lld)", (long long)p->B);
  } else if (p->T % 64 != 0) {
    return fail(KDA_ERR_INVALID_ARG, "fixed-length T must be a multiple of 64 (got %lld); pass cu_seqlens for ragged input",
                (long long)p->T);
  }
  // 32-bit indexing limits of the kernels' tables
  const int64_t tokens = p->B * p->T;
  if (tokens > (int64_t)INT32_MAX / 2 || p->H > 16384 || tokens * p->H * p->K > ((int64_t)1 << 40))
    return fail(KDA_ERR_UNSUPPORTED, "problem too large");
  if (p->num_seqs > (1 << 24)) return fail(KDA_ERR_UNSUPPORTED, "too many sequences");
  return KDA_OK;
}

kda::Layout layout_of(const kda_fwd_params* p) {
  const int elem = p->qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
  return kda::make_layout(p->K, p->V, elem, p->B, p->T, p->H, p->num_seqs);
}

kda_status check_common(const kda_fwd_params* p, const int32_t* cu, void* ws, size_t ws_bytes, kda::Layout* L) {
  kda_status s = check_params(p);
  if (s != KDA_OK) return s;
  if (p->num_seqs > 0 && !cu) return fail(KDA_ERR_INVALID_ARG, "num_seqs > 0 needs cu_seqlens");
  if (p->num_seqs == 0 && cu) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens given but num_seqs == 0");
  if (cu && !aligned(cu, 4)) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
  *L = layout_of(p);
  if (!ws) return fail(KDA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L->total_bytes)
    return fail(KDA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L->total_bytes);
  return KDA_OK;
}

bool empty_problem(const kda_fwd_params* p) { return p->B == 0 || (p->num_seqs == 0 && p->T == 0); }

kda_status check_gate(const kda_gate_params* gp) {
  if (!gp || gp->mode == KDA_GATE_LOG_DECAY) return KDA_OK;
  if (gp->mode != KDA_GATE_SOFTPLUS && gp->mode != KDA_GATE_LOWER_BOUND_SIGMOID)
    return fail(KDA_ERR_INVALID_ARG, "unknown gate mode %d", gp->mode);
  if (!gp->A_log) return fail(KDA_ERR_INVALID_ARG, "gate activation needs A_log");
  if (!aligned(gp->A_log, 4) || (gp->dt_bias && !aligned(gp->dt_bias, 4)))
    return fail(KDA_ERR_INVALID_ARG, "A_log and dt_bias must be 4-byte aligned");
  if (gp->mode == KDA_GATE_LOWER_BOUND_SIGMOID && !(gp->lower_bound >= -5.f && gp->lower_bound < 0.f))
    return fail(KDA_ERR_INVALID_ARG, "lower_bound must be in [-5, 0) (got %g)", (double)gp->lower_bound);
  return KDA_OK;
}

// Host-only checks of the stage 1+2 inputs. Every entry point runs them (and
// check_stage34 for its outputs) before its first launch, so that a failed
// check launches nothing.
kda_status check_stage12(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const kda::Layout& L) {
  if (p->T > 0 && p->B > 0) {
    if (!q || !k || !v || !g || !beta) return fail(KDA_ERR_INVALID_ARG, "q, k, v, g and beta must be non-NULL");
    for (const void* t : {q, k, v, g})
      if (!aligned(t, 16)) return fail(KDA_ERR_INVALID_ARG, "q, k, v and g must be 16-byte aligned");
    if (!aligned(beta, 4)) return fail(KDA_ERR_INVALID_ARG, "beta must be 4-byte aligned");
  }
  if (L.ncp * (size_t)p->H > (size_t)INT32_MAX) return fail(KDA_ERR_UNSUPPORTED, "grid too large");
  return KDA_OK;
}

// Host-only checks of the stage 3+4 outputs and states; need_o: the call
// writes o (every forward entry point; not the affine summaries).
kda_status check_stage34(const kda_fwd_params* p, const void* o, bool need_o, const float* init, const float* fin) {
  const int64_t nseq = p->num_seqs > 0 ? p->num_seqs : p->B;
  if (need_o && p->T > 0 && p->B > 0 && !o) return fail(KDA_ERR_INVALID_ARG, "o must be non-NULL");
  if (o && !aligned(o, 16)) return fail(KDA_ERR_INVALID_ARG, "o must be 16-byte aligned");
  if ((init && !aligned(init, 16)) || (fin && !aligned(fin, 16)))
    return fail(KDA_ERR_INVALID_ARG, "initial_state and final_state must be 16-byte aligned");
  if (nseq * p->H > INT32_MAX / 16) return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
  return KDA_OK;
}

// A fixed-length segment: chunks [c0, c0 + nc) of every batch row. Its records
// occupy chunk slots 0 .. B nc - 1 of the workspace (slot b nc + c).
struct Segment {
  int64_t c0;
  int nc;
};

Segment whole(const kda_fwd_params* p) { return {0, p->num_seqs > 0 ? 1 : (int)(p->T / 64)}; }

// Launches only: the arguments have passed check_common and check_stage12.
kda_status do_stage12(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                      const void* beta, const int32_t* cu, void* ws, const kda::Layout& L, hipStream_t stream,
                      const kda_gate_params* gp = nullptr, Segment sg = {-1, 0}) {
  if (sg.c0 < 0) sg = whole(p);
  char* w = static_cast<char*>(ws);
  const int varlen = p->num_seqs > 0;
  if (varlen) {
    hipError_t e = kda::launch_varlen_map(cu, p->num_seqs, p->T, w, L.ncp, L.off_chunk_tab, L.off_seq_tab,
                                          L.off_order, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "varlen map launch: %s", hipGetErrorString(e));
  }
  if (empty_problem(p) || p->T == 0) return KDA_OK;
  kda::Stage12Args a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.g_f32 = p->g_dtype == KDA_DTYPE_F32;
  a.beta_f32 = p->beta_dtype == KDA_DTYPE_F32;
  a.H = (int)p->H;
  a.scale = p->scale;
  a.l2norm = p->use_qk_l2norm != 0;
  a.l2eps = p->l2norm_eps;
  a.varlen = varlen;
  if (gp && gp->mode != KDA_GATE_LOG_DECAY) {
    a.gate_mode = gp->mode;
    a.gate_lb = gp->lower_bound;
    a.A_log = gp->A_log;
    a.dt_bias = gp->dt_bias;
  }
  a.ws = w;
  a.meta_bytes = L.meta_bytes; a.rec_bytes = L.rec_bytes; a.ncp = L.ncp;
  a.off_chunk_tab = L.off_chunk_tab;
  a.off_w = L.off_w; a.off_qg = L.off_qg; a.off_kg = L.off_kg; a.off_aq = L.off_aq; a.off_u = L.off_u;
  a.off_gam = L.off_gam;
  a.row_T = p->T;
  a.seg_t0 = sg.c0 * 64;
  a.nt_seg = sg.nc;
  if (!varlen) a.ncp = (size_t)p->B * sg.nc;
  const size_t nblocks = a.ncp * (size_t)p->H;
  hipError_t e = kda::launch_stage12(a, p->K, p->qkv_dtype == KDA_DTYPE_BF16, (int)nblocks, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "stage 1+2 launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

// Launches only: the arguments have passed check_common and check_stage34.
// build_map: (re)build the variable-length chunk map first. The entry points that
// run stage 3+4 on its own do, so that a workspace not prepared by stage 1+2 still
// holds valid tables and every access stays in bounds.
kda_status do_stage34(const kda_fwd_params* p, const float* init, void* o, float* fin, void* ws,
                      const kda::Layout& L, hipStream_t stream, int affine_linear = 0, bool build_map = false,
                      const int32_t* cu = nullptr, Segment sg = {-1, 0}) {
  if (sg.c0 < 0) sg = whole(p);
  const int64_t nseq = p->num_seqs > 0 ? p->num_seqs : p->B;
  if (nseq == 0) return KDA_OK;
  if (build_map && p->num_seqs > 0) {
    hipError_t e = kda::launch_varlen_map(cu, p->num_seqs, p->T, static_cast<char*>(ws), L.ncp, L.off_chunk_tab,
                                          L.off_seq_tab, L.off_order, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "varlen map launch: %s", hipGetErrorString(e));
  }
  kda::Stage34Args a{};
  a.init = init;
  a.final_state = fin;
  a.o = o;
  a.init_identity = affine_linear;
  a.zero_u = affine_linear;
  a.H = (int)p->H;
  a.nunits = (int)(nseq * p->H);
  a.nt = p->num_seqs > 0 ? 0 : sg.nc;
  a.row_T = p->T;
  a.seg_t0 = p->num_seqs > 0 ? 0 : sg.c0 * 64;
  a.varlen = p->num_seqs > 0;
  a.ws = static_cast<const char*>(ws);
  a.meta_bytes = L.meta_bytes; a.rec_bytes = L.rec_bytes; a.ncp = L.ncp;
  a.off_chunk_tab = L.off_chunk_tab; a.off_seq_tab = L.off_seq_tab; a.off_order = L.off_order;
  a.off_sink = L.off_sink;
  a.off_w = L.off_w; a.off_qg = L.off_qg; a.off_kg = L.off_kg; a.off_aq = L.off_aq; a.off_u = L.off_u;
  a.off_gam = L.off_gam;
  hipError_t e = kda::launch_stage34(a, p->K, p->qkv_dtype == KDA_DTYPE_BF16, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "stage 3+4 launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

// Fixed-length bf16 inputs are processed in segments of whole chunks along T:
// stage 1+2 of a segment, then stage 3+4 of it, the fp32 state handed from one
// segment to the next through two buffers in the workspace (an exact hand-off:
// stage 3+4 keeps the state in fp32 throughout). A segment's records (about
// kSegmentRecordBytes) are read back by stage 3+4 while they still sit in the
// 256 MB memory-side cache, instead of from HBM after the whole problem's
// records have streamed through it: with bf16 operands stage 3+4 is bound by
// the delivery of its records. With fp32 operands it is bound by its fp32
// products instead, and the segments' extra launch ramps cost more than the
// cache saves, so fp32 inputs run in one pass. The result is bitwise the same
// for any segmentation, since every chunk's arithmetic is unchanged.
constexpr size_t kSegmentRecordBytes = (size_t)144 << 20;

struct SegmentPlan {
  int nseg;          // 1: one pass over the whole problem
  int nc;            // chunks per segment (the last may be shorter)
  size_t off_state;  // two state buffers at off_state and off_state + state_bytes
  size_t state_bytes;
};

SegmentPlan plan_segments(const kda_fwd_params* p, const kda::Layout& L) {
  SegmentPlan sp{1, 0, 0, 0};
  if (p->num_seqs > 0 || p->B == 0 || p->T == 0 || p->qkv_dtype != KDA_DTYPE_BF16) return sp;
  const int64_t nt = p->T / 64;
  sp.nc = (int)nt;
  const size_t per_chunk = (size_t)p->B * (size_t)p->H * L.rec_bytes;  // records of one chunk index
  const int64_t nc_max = std::max<int64_t>(1, (int64_t)(kSegmentRecordBytes / per_chunk));
  const int64_t nseg = (nt + nc_max - 1) / nc_max;
  if (nseg <= 1) return sp;
  const int64_t nc = (nt + nseg - 1) / nseg;
  const size_t state_bytes = kda::round_up((size_t)p->B * p->H * p->K * p->V * sizeof(float), 256);
  const size_t off_state = L.meta_bytes + kda::round_up(per_chunk * nc, 256);
  if (off_state + 2 * state_bytes > L.total_bytes) return sp;
  sp.nseg = (int)((nt + nc - 1) / nc);
  sp.nc = (int)nc;
  sp.off_state = off_state;
  sp.state_bytes = state_bytes;
  return sp;
}

// Both stages over the whole problem (segmented for long fixed-length inputs).
// The arguments have passed every check.
kda_status run_forward(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const float* init, const int32_t* cu, void* o, float* fin, void* ws,
                       const kda::Layout& L, hipStream_t stream, const kda_gate_params* gp) {
  const SegmentPlan sp = plan_segments(p, L);
  if (sp.nseg <= 1) {
    kda_status s = do_stage12(p, q, k, v, g, beta, cu, ws, L, stream, gp);
    if (s != KDA_OK) return s;
    return do_stage34(p, init, o, fin, ws, L, stream);
  }
  char* w = static_cast<char*>(ws);
  float* st[2] = {reinterpret_cast<float*>(w + sp.off_state),
                  reinterpret_cast<float*>(w + sp.off_state + sp.state_bytes)};
  const int64_t nt = p->T / 64;
  for (int i = 0; i < sp.nseg; ++i) {
    const Segment sg{(int64_t)i * sp.nc, (int)std::min<int64_t>(sp.nc, nt - (int64_t)i * sp.nc)};
    const float* si = i == 0 ? init : st[(i - 1) & 1];
    float* so = i == sp.nseg - 1 ? fin : st[i & 1];
    kda_status s = do_stage12(p, q, k, v, g, beta, cu, ws, L, stream, gp, sg);
    if (s != KDA_OK) return s;
    s = do_stage34(p, si, o, so, ws, L, stream, 0, false, nullptr, sg);
    if (s != KDA_OK) return s;
  }
  return KDA_OK;
}

}  // namespace

namespace kda {
kda_status fail_msg(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}
void clear_msg() { g_msg[0] = 0; }
}  // namespace kda

extern "C" {

kda_status kda_chunk_fwd_workspace_bytes(const kda_fwd_params* p, size_t* bytes) {
  kda_status s = check_params(p);
  if (s != KDA_OK) return s;
  if (!bytes) return fail(KDA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout_of(p).total_bytes;
  return KDA_OK;
}

kda_status kda_workspace_layout(const kda_fwd_params* p, kda_workspace_info* info) {
  kda_status s = check_params(p);
  if (s != KDA_OK) return s;
  if (!info) return fail(KDA_ERR_INVALID_ARG, "info is NULL");
  const kda::Layout L = layout_of(p);
  info->total_bytes = L.total_bytes;
  info->records_offset = L.meta_bytes;
  info->record_bytes = L.rec_bytes;
  info->chunk_slots = L.ncp;
  info->off_w = L.off_w;
  info->off_qg = L.off_qg;
  info->off_kg = L.off_kg;
  info->off_aq = L.off_aq;
  info->off_u = L.off_u;
  info->off_gamma = L.off_gam;
  info->elem_bytes = L.elem;
  info->off_chunk_table = L.off_chunk_tab;
  info->off_seq_table = L.off_seq_tab;
  info->off_order = L.off_order;
  const SegmentPlan sp = plan_segments(p, L);
  info->segments = sp.nseg;
  info->segment_chunks = sp.nc;
  return KDA_OK;
}

kda_status kda_chunk_fwd_stage12(const kda_fwd_params* p, const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const int32_t* cu_seqlens, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  kda::Layout L;
  kda_status s = check_common(p, cu_seqlens, workspace, workspace_bytes, &L);
  if (s != KDA_OK) return s;
  s = check_stage12(p, q, k, v, g, beta, L);
  if (s != KDA_OK) return s;
  return do_stage12(p, q, k, v, g, beta, cu_seqlens, workspace, L, stream);
}

kda_status kda_chunk_fwd_stage34(const kda_fwd_params* p, const float* initial_state, const int32_t* cu_seqlens,
                                 void* o, float* final_state, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  kda::Layout L;
  kda_status s = check_common(p, cu_seqlens, workspace, workspace_bytes, &L);
  if (s != KDA_OK) return s;
  s = check_stage34(p, o, true, initial_state, final_state);
  if (s != KDA_OK) return s;
  return do_stage34(p, initial_state, o, final_state, workspace, L, stream, 0, true, cu_seqlens);
}

kda_status kda_chunk_fwd(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, const int32_t* cu_seqlens, void* o,
                         float* final_state, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  kda::Layout L;
  kda_status s = check_common(p, cu_seqlens, workspace, workspace_bytes, &L);
  if (s != KDA_OK) return s;
  s = check_stage12(p, q, k, v, g, beta, L);
  if (s != KDA_OK) return s;
  s = check_stage34(p, o, true, initial_state, final_state);
  if (s != KDA_OK) return s;
  return run_forward(p, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state, workspace, L, stream, nullptr);
}

kda_status kda_decode_step(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                           const void* beta, float* state, void* o, hipStream_t stream) {
  g_msg[0] = 0;
  if (!p) return fail(KDA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 0 || p->H <= 0) return fail(KDA_ERR_INVALID_ARG, "need B >= 0 and H > 0");
  if (p->T != 1) return fail(KDA_ERR_INVALID_ARG, "a decode step takes T == 1 (got %lld)", (long long)p->T);
  if (p->num_seqs != 0) return fail(KDA_ERR_INVALID_ARG, "a decode step takes num_seqs == 0 (one token per row)");
  if (p->K <= 0 || p->V <= 0 || p->K > 256) return fail(KDA_ERR_INVALID_ARG, "need 0 < K <= 256 and V > 0");
  if (!(p->K == p->V && (p->K == 64 || p->K == 128)))
    return fail(KDA_ERR_UNSUPPORTED, "GPU path supports K == V in {64, 128} (got K=%d V=%d)", p->K, p->V);
  for (int32_t d : {p->qkv_dtype, p->g_dtype, p->beta_dtype})
    if (d != KDA_DTYPE_F32 && d != KDA_DTYPE_BF16) return fail(KDA_ERR_INVALID_ARG, "unknown dtype %d", d);
  if (p->use_qk_l2norm && !(p->l2norm_eps > 0.f)) return fail(KDA_ERR_INVALID_ARG, "l2norm_eps must be > 0");
  const int64_t units = p->B * p->H;
  if (units > (int64_t)INT32_MAX / 4) return fail(KDA_ERR_UNSUPPORTED, "problem too large");
  if (units == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state || !o)
    return fail(KDA_ERR_INVALID_ARG, "q, k, v, g, beta, state and o must be non-NULL");
  if (!aligned(state, 16)) return fail(KDA_ERR_INVALID_ARG, "state must be 16-byte aligned");
  kda::DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
  a.scale = p->scale;
  a.l2norm = p->use_qk_l2norm != 0;
  a.l2eps = p->l2norm_eps;
  a.nunits = (int)units;
  hipError_t e = kda::launch_decode(a, p->K, p->qkv_dtype == KDA_DTYPE_BF16, p->g_dtype == KDA_DTYPE_F32,
                                    p->beta_dtype == KDA_DTYPE_F32, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_chunk_bwd_workspace_bytes(const kda_fwd_params* p, size_t* bytes) {
  kda_status s = check_params(p);
  if (s != KDA_OK) return s;
  if (!bytes) return fail(KDA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = kda::bwd_workspace_bytes(layout_of(p), p->H);
  return KDA_OK;
}

kda_status kda_chunk_bwd_stages(const kda_fwd_params* p, int32_t stages, const void* q, const void* k,
                                const void* v, const void* g, const void* beta, const float* initial_state,
                                const int32_t* cu_seqlens, const void* d_o, const float* d_final_state, float* dq,
                                float* dk, float* dv, float* dg, float* dbeta, float* d_initial_state,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_msg[0] = 0;
  if (stages < 1 || stages > 15) return fail(KDA_ERR_INVALID_ARG, "stages must be a mask in [1, 15] (got %d)", stages);
  kda_status s = check_params(p);
  if (s != KDA_OK) return s;
  if (p->num_seqs > 0 && !cu_seqlens) return fail(KDA_ERR_INVALID_ARG, "num_seqs > 0 needs cu_seqlens");
  if (p->num_seqs == 0 && cu_seqlens) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens given but num_seqs == 0");
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
  const kda::Layout L = layout_of(p);
  const size_t need = kda::bwd_workspace_bytes(L, p->H);
  if (!workspace) return fail(KDA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < need) return fail(KDA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  const bool any_tokens = p->B > 0 && p->T > 0;
  if (any_tokens) {
    if (!q || !k || !v || !g || !beta || !d_o)
      return fail(KDA_ERR_INVALID_ARG, "q, k, v, g, beta and d_o must be non-NULL");
    if (!dq || !dk || !dv || !dg || !dbeta)
      return fail(KDA_ERR_INVALID_ARG, "dq, dk, dv, dg and dbeta must be non-NULL");
    const size_t ea = p->qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    for (const void* t : {q, k, v})
      if (!aligned(t, ea)) return fail(KDA_ERR_INVALID_ARG, "q, k, v and d_o must be aligned to their element size");
    if (!aligned(d_o, 16)) return fail(KDA_ERR_INVALID_ARG, "d_o must be 16-byte aligned");
    if (!aligned(g, p->g_dtype == KDA_DTYPE_BF16 ? 2 : 4) || !aligned(beta, p->beta_dtype == KDA_DTYPE_BF16 ? 2 : 4))
      return fail(KDA_ERR_INVALID_ARG, "g and beta must be aligned to their element size");
    for (const float* t : {dq, dk, dv, dg, dbeta})
      if (!aligned(t, 4)) return fail(KDA_ERR_INVALID_ARG, "gradient outputs must be 4-byte aligned");
  }
  for (const float* t : {initial_state, d_final_state, (const float*)d_initial_state})
    if (t && !aligned(t, 4)) return fail(KDA_ERR_INVALID_ARG, "states must be 4-byte aligned");
  const int64_t nseq = p->num_seqs > 0 ? p->num_seqs : p->B;
  const int64_t nunits = nseq * p->H;
  if ((nunits + 8) * (p->V / 16) > INT32_MAX) return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
  char* w = static_cast<char*>(workspace);
  const int varlen = p->num_seqs > 0;
  if (varlen) {  // every call: later stages alone still see valid chunk tables
    hipError_t e = kda::launch_varlen_map(cu_seqlens, p->num_seqs, p->T, w, L.ncp, L.off_chunk_tab, L.off_seq_tab,
                                          L.off_order, stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "varlen map launch: %s", hipGetErrorString(e));
  }
  kda::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.d_o = d_o;
  a.init = initial_state;
  a.d_final = d_final_state;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = d_initial_state;
  a.bf16_qkv = p->qkv_dtype == KDA_DTYPE_BF16;
  a.g_f32 = p->g_dtype == KDA_DTYPE_F32;
  a.beta_f32 = p->beta_dtype == KDA_DTYPE_F32;
  a.H = (int)p->H;
  a.scale = p->scale;
  a.l2norm = p->use_qk_l2norm != 0;
  a.l2eps = p->l2norm_eps;
  a.varlen = varlen;
  a.nunits = (int)nunits;
  a.nt = varlen ? 0 : (int)(p->T / 64);
  a.ws = w;
  a.meta_bytes = L.meta_bytes;
  a.ncp = L.ncp;
  a.off_chunk_tab = L.off_chunk_tab;
  a.off_seq_tab = L.off_seq_tab;
  a.sl = kda::make_bwd_slab(p->K, p->V);
  const size_t nitems = any_tokens ? L.ncp * (size_t)p->H : 0;
  if (nitems > (size_t)INT32_MAX) return fail(KDA_ERR_UNSUPPORTED, "grid too large");
  hipError_t e = kda::launch_bwd(a, p->K, (int)nitems, stages, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_chunk_bwd(const kda_fwd_params* p, const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state, const int32_t* cu_seqlens, const void* d_o,
                         const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                         float* d_initial_state, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return kda_chunk_bwd_stages(p, 15, q, k, v, g, beta, initial_state, cu_seqlens, d_o, d_final_state, dq, dk, dv, dg,
                              dbeta, d_initial_state, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_gated(const kda_fwd_params* p, const kda_gate_params* gate, const void* q, const void* k,
                               const void* v, const void* g, const void* beta, const float* initial_state,
                               const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  kda::Layout L;
  kda_status s = check_common(p, cu_seqlens, workspace, workspace_bytes, &L);
  if (s != KDA_OK) return s;
  s = check_gate(gate);
  if (s != KDA_OK) return s;
  s = check_stage12(p, q, k, v, g, beta, L);
  if (s != KDA_OK) return s;
  s = check_stage34(p, o, true, initial_state, final_state);
  if (s != KDA_OK) return s;
  return run_forward(p, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state, workspace, L, stream, gate);
}

kda_status kda_chunk_affine_summary(const kda_fwd_params* p, const int32_t* cu_seqlens, float* M, float* N,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  kda::Layout L;
  kda_status s = check_common(p, cu_seqlens, workspace, workspace_bytes, &L);
  if (s != KDA_OK) return s;
  if (!M || !N) return fail(KDA_ERR_INVALID_ARG, "M and N must be non-NULL");
  if (!aligned(M, 16) || !aligned(N, 16)) return fail(KDA_ERR_INVALID_ARG, "M and N must be 16-byte aligned");
  if (M == N) return fail(KDA_ERR_INVALID_ARG, "M and N must not alias");
  s = check_stage34(p, nullptr, false, nullptr, N);
  if (s != KDA_OK) return s;
  // N: the state reached from a zero start; M: the recurrence run on an identity
  // start with U taken as zero (the linear part). No output is written.
  s = do_stage34(p, nullptr, nullptr, N, workspace, L, stream, 0, true, cu_seqlens);
  if (s != KDA_OK) return s;
  return do_stage34(p, nullptr, nullptr, M, workspace, L, stream, 1);
}

kda_status kda_affine_apply(const kda_fwd_params* p, const float* M, const float* N, const float* S0, float* S_out,
                            hipStream_t stream) {
  g_msg[0] = 0;
  if (!p) return fail(KDA_ERR_INVALID_ARG, "params is NULL");
  if (p->H <= 0 || p->B < 0 || p->num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "bad B, H or num_seqs");
  if (!(p->K == p->V && (p->K == 64 || p->K == 128)))
    return fail(KDA_ERR_UNSUPPORTED, "GPU path supports K == V in {64, 128} (got K=%d V=%d)", p->K, p->V);
  const int64_t nunits = (p->num_seqs > 0 ? p->num_seqs : p->B) * p->H;
  if (nunits == 0) return KDA_OK;
  if (nunits > INT32_MAX / 4) return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
  if (!M || !N || !S0 || !S_out) return fail(KDA_ERR_INVALID_ARG, "M, N, S0 and S_out must be non-NULL");
  if (S_out == S0 || S_out == M) return fail(KDA_ERR_INVALID_ARG, "S_out must not alias S0 or M");
  hipError_t e = kda::launch_affine_apply(M, N, S0, S_out, (int)nunits, p->K, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "affine apply launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_msg; }

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
