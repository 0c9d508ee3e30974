// KDA layer forward around the chunkwise core on gfx950 ("KDAChunkwise" docs,
// sections "From the hidden states to causal Q, K, and V", "FP32 core and
// log-space decay", "Returning to the model dimension"; lower-bound sigmoid
// gate of the Tokamax "chunk_kda_fwd design doc", section 9.1.3).
//
// Order of work on the caller's stream (BT = B * T tokens, HD = H * D):
//   1. Wcat = [Wqkv; Wad; Wgd; Wb] (device copies, rows of width M): the
//      low-rank slices of P start at 16-byte aligned columns
//   2. P    = x Wcat^T                     GEMM, bf16 x bf16 (fp32 accumulation) -> bf16 [BT, NP]
//   3. prologue kernel: q, k, v = SiLU(conv4(P_qkv)) (+ L2 norm for q, k) in
//      fp32, beta = sigmoid(P_b)
//   4. g    = P_a Wau^T                    GEMM -> fp32 [BT, HD] (raw gate; P_a read in place)
//   5. core: the two-kernel chunkwise forward on fp32 q, k, v, beta with the
//      decay g = lb * sigmoid(exp(A_log_h) (g_raw + dt_bias)) applied inside
//      stage 1+2 (no separate pass over g)
//   6+7. y = RMSNorm_D(o) * norm_w * sigmoid(P_g Wgu^T) -> bf16 [BT, HD]: one
//      GEMM whose epilogue applies the norm and the gate
//   8. x_new = y Wo^T                      GEMM, bf16 x bf16 -> bf16 [BT, M]
// The projections run on this library's MFMA GEMM (kda_gemm.hip); every other
// step is a kernel of this file or of the core. The elementwise kernels are HBM-bound: each reads
// its inputs once with coalesced vector loads and writes its outputs once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "kda.h"
#include "kda_layer.h"
#include "kda_kernels.h"
#include "kda_gemm.h"

namespace kda {
namespace {

constexpr int kWave = 64;
constexpr int kLayerThreads = 256;
constexpr int kTile = 64;  // tokens per prologue wave

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

struct PrologueArgs {
  const uint16_t* P;   // [BT, ldp] bf16 bits
  int64_t ldp;
  const float* conv[3];
  float* out[3];       // q, k, v [BT, HD]
  float* beta;         // [BT, H]
  int64_t T;           // tokens per batch row
  int H, nt;           // heads, 64-token tiles per row
  int off_b;
  float l2eps;
  int64_t nwaves;      // B * nt * H * 3
};

// One wave per (batch row, 64-token tile, head, stream q/k/v): a sliding
// window of the last 3 pre-activations per channel in registers, so P is read
// once. Lane l holds channels CPL l .. CPL l + CPL - 1 of the head.
template <int D>
__global__ __launch_bounds__(kLayerThreads) void layer_prologue_kernel(PrologueArgs a) {
  constexpr int CPL = D / kWave;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * (kLayerThreads / kWave) + (threadIdx.x >> 6);
  if (wid >= a.nwaves) return;
  const int s = (int)(wid % 3);
  int64_t r = wid / 3;
  const int h = (int)(r % a.H);
  r /= a.H;
  const int tile = (int)(r % a.nt);
  const int64_t b = r / a.nt;
  const int HD = a.H * D;
  const int c0 = h * D + CPL * lane;
  const int64_t row0 = b * a.T + (int64_t)tile * kTile;  // first token row of the tile
  const uint16_t* src = a.P + s * HD + c0;
  float wgt[CPL][4];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const float4 w4 = *reinterpret_cast<const float4*>(a.conv[s] + (size_t)(c0 + j) * 4);
    wgt[j][0] = w4.x; wgt[j][1] = w4.y; wgt[j][2] = w4.z; wgt[j][3] = w4.w;
  }
  // window: x[m] = P at token t - 3 + m (zero before the row start)
  float win[CPL][3];
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int64_t t = (int64_t)tile * kTile - 3 + m;
#pragma unroll
    for (int j = 0; j < CPL; ++j) win[j][m] = t >= 0 ? bf16f(src[(row0 - 3 + m) * a.ldp + j]) : 0.f;
  }
  float* dst = a.out[s] + c0;
  for (int tb = 0; tb < kTile; tb += 8) {
    float xin[8][CPL];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (CPL == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(src + (row0 + tb + i) * a.ldp);
        xin[i][0] = __uint_as_float(v << 16);
        xin[i][1] = __uint_as_float(v & 0xffff0000u);
      } else {
        xin[i][0] = bf16f(src[(row0 + tb + i) * a.ldp]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y[CPL];
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const float c = wgt[j][0] * win[j][0] + wgt[j][1] * win[j][1] + wgt[j][2] * win[j][2] + wgt[j][3] * xin[i][j];
        win[j][0] = win[j][1];
        win[j][1] = win[j][2];
        win[j][2] = xin[i][j];
        y[j] = c * sigmoidf_(c);  // SiLU
        ss += y[j] * y[j];
      }
      if (s < 2) {  // wave-uniform: q and k are L2-normalised over the head dim
        const float inv = 1.f / fmaxf(sqrtf(wave_sum(ss)), a.l2eps);
#pragma unroll
        for (int j = 0; j < CPL; ++j) y[j] *= inv;
      }
      float* o = dst + (row0 + tb + i) * HD;
      if constexpr (CPL == 2) *reinterpret_cast<float2*>(o) = make_float2(y[0], y[1]);
      else o[0] = y[0];
    }
  }
  if (s == 0) {
    // beta of the tile's 64 tokens for this head, one token per lane
    const int64_t row = row0 + lane;
    a.beta[row * a.H + h] = sigmoidf_(bf16f(a.P[row * a.ldp + a.off_b + h]));
  }
}

// ------------------------------------------------------------------ host side

struct LayerLayout {
  int64_t BT;
  int HD, NP;
  size_t off_wcat, off_P, off_q, off_k, off_v, off_g, off_beta, off_o, off_y, off_core, total;
  size_t core_bytes;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

kda_fwd_params core_params(const kda_layer_params* p) {
  kda_fwd_params c{};
  c.B = p->B; c.T = p->T; c.H = p->H; c.K = p->D; c.V = p->D;
  c.qkv_dtype = KDA_DTYPE_F32; c.g_dtype = KDA_DTYPE_F32; c.beta_dtype = KDA_DTYPE_F32;
  c.scale = 1.f / sqrtf((float)p->D);
  c.chunk_size = 64;
  c.use_qk_l2norm = 0;
  c.l2norm_eps = 1e-6f;
  c.num_seqs = 0;
  return c;
}

kda_status check_layer(const kda_layer_params* p, LayerLayout* L) {
  clear_msg();
  if (!p) return fail_msg(KDA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 1 || p->T < 1 || p->M < 1 || p->H < 1) return fail_msg(KDA_ERR_INVALID_ARG, "need B, T, M, H >= 1");
  if (p->T % 64) return fail_msg(KDA_ERR_INVALID_ARG, "T must be a multiple of 64 (got %lld)", (long long)p->T);
  if (!(p->D == 64 || p->D == 128)) return fail_msg(KDA_ERR_UNSUPPORTED, "D must be 64 or 128 (got %d)", p->D);
  if (p->conv_size != 4) return fail_msg(KDA_ERR_UNSUPPORTED, "conv_size must be 4 (got %d)", p->conv_size);
  if (p->M % 8 || p->gate_rank < 8 || p->gate_rank % 8 || p->out_gate_rank < 8 || p->out_gate_rank % 8)
    return fail_msg(KDA_ERR_INVALID_ARG, "M and both gate ranks must be positive multiples of 8");
  if (!(p->norm_eps > 0.f) || !(p->l2_eps > 0.f)) return fail_msg(KDA_ERR_INVALID_ARG, "eps values must be > 0");
  if (!(p->gate_lower_bound < 0.f) || p->gate_lower_bound < -5.f)
    return fail_msg(KDA_ERR_INVALID_ARG, "gate_lower_bound must be in [-5, 0) (the core's decay range)");
  L->BT = p->B * p->T;
  L->HD = p->H * p->D;
  // P's row stride, padded to 8 columns so that every row starts 16-byte aligned
  L->NP = (int)((3 * (int64_t)L->HD + p->H + p->gate_rank + p->out_gate_rank + 7) / 8 * 8);
  if (L->BT > INT32_MAX / 2 || (int64_t)L->NP * p->M > INT32_MAX || (int64_t)L->HD > 65536 || p->M > (1 << 21) ||
      p->gate_rank > (1 << 21) || p->out_gate_rank > (1 << 21))
    return fail_msg(KDA_ERR_UNSUPPORTED, "layer too large for 32-bit GEMM sizes");
  kda_fwd_params c = core_params(p);
  size_t cb = 0;
  kda_status s = kda_chunk_fwd_workspace_bytes(&c, &cb);
  if (s != KDA_OK) return s;
  L->core_bytes = cb;
  const size_t BT = (size_t)L->BT, HD = (size_t)L->HD;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = up256(off + bytes); return o; };
  L->off_wcat = take((size_t)L->NP * p->M * 2);
  L->off_P = take(BT * L->NP * 2);        // bf16
  // q, k, v, the raw gate and beta are the core's inputs; nothing later overwrites
  // them, so they can be inspected after the call (kda_layer_workspace_layout)
  L->off_q = take(BT * HD * 4);
  L->off_k = take(BT * HD * 4);
  L->off_v = take(BT * HD * 4);
  L->off_g = take(BT * HD * 4);
  L->off_beta = take(BT * p->H * 4);
  L->off_o = take(BT * HD * 4);
  L->off_y = take(BT * HD * 2);           // y [BT, HD] bf16, the output projection's input
  L->off_core = take(cb);
  L->total = off;
  return KDA_OK;
}

// Y[n_rows, N] = X[n_rows, Kd] W[N, Kd]^T, row-major, on this library's MFMA GEMM
kda_status gemm_nt(const void* W, int64_t ldw, const void* X, int64_t ldx, void* Y, int64_t ldy, bool y_f32,
                   int64_t N, int64_t n_rows, int64_t Kd, hipStream_t stream, const char* what) {
  GemmArgs g{};
  g.A = X; g.lda = ldx;
  g.B = W; g.ldb = ldw;
  g.C = Y; g.ldc = ldy;
  g.M = n_rows; g.N = N; g.K = Kd;
  const hipError_t e = launch_gemm_bf16(g, y_f32 ? 1 : 0, stream);
  if (e != hipSuccess) return fail_msg(KDA_ERR_HIP, "GEMM (%s) launch: %s", what, hipGetErrorString(e));
  return KDA_OK;
}

}  // namespace
}  // namespace kda

extern "C" {

kda_status kda_layer_fwd_workspace_bytes(const kda_layer_params* p, size_t* bytes) {
  kda::LayerLayout L;
  kda_status s = kda::check_layer(p, &L);
  if (s != KDA_OK) return s;
  if (!bytes) return kda::fail_msg(KDA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = L.total;
  return KDA_OK;
}

kda_status kda_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, void* C, int64_t ldc, int32_t c_dtype, hipStream_t stream) {
  using namespace kda;
  clear_msg();
  if (M < 0 || N < 0 || K < 0) return fail_msg(KDA_ERR_INVALID_ARG, "need M, N, K >= 0");
  if (c_dtype != KDA_DTYPE_BF16 && c_dtype != KDA_DTYPE_F32) return fail_msg(KDA_ERR_INVALID_ARG, "unknown c_dtype");
  if (M == 0 || N == 0) return KDA_OK;
  if (K % 8 || lda % 8 || ldb % 8 || lda < K || ldb < K || ldc < N)
    return fail_msg(KDA_ERR_INVALID_ARG, "K, lda, ldb must be multiples of 8 with lda, ldb >= K and ldc >= N");
  // the kernel addresses a 256-row operand tile through a buffer resource with
  // 32-bit byte offsets (up to 512 lda bytes)
  if (lda > ((int64_t)1 << 21) || ldb > ((int64_t)1 << 21))
    return fail_msg(KDA_ERR_UNSUPPORTED, "lda and ldb must be at most 2^21 elements");
  if (!A || !B || !C) return fail_msg(KDA_ERR_INVALID_ARG, "A, B and C must be non-NULL");
  if (reinterpret_cast<uintptr_t>(A) % 16 || reinterpret_cast<uintptr_t>(B) % 16 ||
      reinterpret_cast<uintptr_t>(C) % (c_dtype == KDA_DTYPE_F32 ? 4 : 2))
    return fail_msg(KDA_ERR_INVALID_ARG, "A and B must be 16-byte aligned, C aligned to its element size");
  if ((M + 255) / 256 * ((N + 255) / 256) > (int64_t)1 << 26) return fail_msg(KDA_ERR_UNSUPPORTED, "GEMM too large");
  GemmArgs g{};
  g.A = A; g.B = B; g.C = C;
  g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc;
  const hipError_t e = launch_gemm_bf16(g, c_dtype == KDA_DTYPE_F32, stream);
  if (e != hipSuccess) return fail_msg(KDA_ERR_HIP, "GEMM launch: %s", hipGetErrorString(e));
  return KDA_OK;
}

kda_status kda_layer_workspace_layout(const kda_layer_params* p, kda_layer_workspace_info* info) {
  kda::LayerLayout L;
  kda_status s = kda::check_layer(p, &L);
  if (s != KDA_OK) return s;
  if (!info) return kda::fail_msg(KDA_ERR_INVALID_ARG, "info is NULL");
  info->total_bytes = L.total;
  info->off_q = L.off_q;
  info->off_k = L.off_k;
  info->off_v = L.off_v;
  info->off_g_raw = L.off_g;
  info->off_beta = L.off_beta;
  info->off_o = L.off_o;
  return KDA_OK;
}

kda_status kda_layer_fwd(const kda_layer_params* p, const kda_layer_weights* w, const void* x, void* x_new,
                         float* core_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace kda;
  LayerLayout L;
  kda_status s = check_layer(p, &L);
  if (s != KDA_OK) return s;
  if (!w || !x || !x_new) return fail_msg(KDA_ERR_INVALID_ARG, "weights, x and x_new must be non-NULL");
  const void* ptrs[] = {w->Wqkv, w->conv_q, w->conv_k, w->conv_v, w->Wb, w->Wad, w->Wau,
                        w->A_log, w->dt_bias, w->Wgd, w->Wgu, w->norm_w, w->Wo};
  for (const void* q : ptrs)
    if (!q) return fail_msg(KDA_ERR_INVALID_ARG, "every weight pointer must be non-NULL");
  for (const void* q : {(const void*)w->conv_q, (const void*)w->conv_k, (const void*)w->conv_v,
                        (const void*)w->dt_bias})
    if (reinterpret_cast<uintptr_t>(q) % 16) return fail_msg(KDA_ERR_INVALID_ARG, "conv weights and dt_bias must be 16-byte aligned");
  if (x == x_new) return fail_msg(KDA_ERR_INVALID_ARG, "x_new must not alias x");
  if (core_out && reinterpret_cast<uintptr_t>(core_out) % 16)
    return fail_msg(KDA_ERR_INVALID_ARG, "core_out must be 16-byte aligned");
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail_msg(KDA_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail_msg(KDA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  const int M = p->M, H = p->H, D = p->D, HD = L.HD, NP = L.NP;
  const int BT = (int)L.BT;
  const int r = p->gate_rank, rg = p->out_gate_rank;
  uint16_t* wcat = reinterpret_cast<uint16_t*>(ws + L.off_wcat);
  uint16_t* P = reinterpret_cast<uint16_t*>(ws + L.off_P);
  const int off_r = 3 * HD;      // column of the first low-rank activation in P
  float* q = reinterpret_cast<float*>(ws + L.off_q);
  float* k = reinterpret_cast<float*>(ws + L.off_k);
  float* v = reinterpret_cast<float*>(ws + L.off_v);
  float* g = reinterpret_cast<float*>(ws + L.off_g);
  float* beta = reinterpret_cast<float*>(ws + L.off_beta);
  float* o = core_out ? core_out : reinterpret_cast<float*>(ws + L.off_o);

  // 1. concatenated input projections (rows of width M): read in place when the
  // caller keeps [Wqkv; Wad; Wgd; Wb] back to back, else copied
  const size_t rowb = (size_t)M * 2;
  const struct { const void* src; size_t rows; } parts[] = {
      {w->Wqkv, (size_t)3 * HD}, {w->Wad, (size_t)r}, {w->Wgd, (size_t)rg}, {w->Wb, (size_t)H}};
  bool adjacent = reinterpret_cast<uintptr_t>(w->Wqkv) % 16 == 0;
  for (int i = 1; i < 4; ++i)
    adjacent = adjacent && static_cast<const char*>(parts[i].src) ==
                               static_cast<const char*>(parts[i - 1].src) + parts[i - 1].rows * rowb;
  const void* wproj = adjacent ? w->Wqkv : static_cast<const void*>(wcat);
  if (!adjacent) {
    size_t at = 0;
    for (const auto& pt : parts) {
      if (hipMemcpyAsync(reinterpret_cast<char*>(wcat) + at, pt.src, pt.rows * rowb, hipMemcpyDeviceToDevice,
                         stream) != hipSuccess)
        return fail_msg(KDA_ERR_HIP, "weight copy failed");
      at += pt.rows * rowb;
    }
  }
  // 2. P = x Wcat^T
  const int NW = 3 * HD + r + rg + H;  // rows of Wcat (columns of P in use)
  s = gemm_nt(wproj, M, x, M, P, NP, false, NW, BT, M, stream, "input projections");
  if (s != KDA_OK) return s;
  // 3. prologue
  {
    PrologueArgs a{};
    a.P = P; a.ldp = NP;
    a.conv[0] = w->conv_q; a.conv[1] = w->conv_k; a.conv[2] = w->conv_v;
    a.out[0] = q; a.out[1] = k; a.out[2] = v;
    a.beta = beta;
    a.T = p->T; a.H = H; a.nt = (int)(p->T / kTile);
    a.off_b = 3 * HD + r + rg;
    a.l2eps = p->l2_eps;
    a.nwaves = p->B * a.nt * (int64_t)H * 3;
    const int wpb = kLayerThreads / kWave;
    const dim3 grid((unsigned)((a.nwaves + wpb - 1) / wpb));
    if (D == 128) hipLaunchKernelGGL(layer_prologue_kernel<128>, grid, dim3(kLayerThreads), 0, stream, a);
    else hipLaunchKernelGGL(layer_prologue_kernel<64>, grid, dim3(kLayerThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return fail_msg(KDA_ERR_HIP, "prologue launch failed");
  }
  // 4. decay-gate up projection (raw gate)
  s = gemm_nt(w->Wau, r, P + off_r, NP, g, HD, true, HD, BT, r, stream, "decay gate");
  if (s != KDA_OK) return s;
  // 5. the chunkwise core in fp32, gate activation inside stage 1+2
  {
    kda_fwd_params c = core_params(p);
    kda_gate_params gp{};
    gp.mode = KDA_GATE_LOWER_BOUND_SIGMOID;
    gp.lower_bound = p->gate_lower_bound;
    gp.A_log = w->A_log;
    gp.dt_bias = w->dt_bias;
    s = kda_chunk_fwd_gated(&c, &gp, q, k, v, g, beta, nullptr, nullptr, o, nullptr, ws + L.off_core, L.core_bytes,
                            stream);
    if (s != KDA_OK) return s;
  }
  // 6-7. output-gate up projection fused with RMSNorm * gate -> y (bf16): the
  // GEMM's epilogue reads o and writes y = RMSNorm_D(o) * norm_w *
  // sigmoid(P_g Wgu^T) into a buffer of its own, so y never overlaps P, which
  // the same GEMM is still reading (o's rows are 16-byte aligned: the core has
  // checked them)
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.off_y);
  {
    GemmArgs g{};
    g.A = P + off_r + r; g.lda = NP;
    g.B = w->Wgu; g.ldb = rg;
    g.C = y; g.ldc = HD;
    g.M = BT; g.N = HD; g.K = rg;
    g.norm_o = o; g.ldo = HD; g.norm_w = w->norm_w; g.norm_d = D; g.norm_eps = p->norm_eps;
    const hipError_t e = launch_gemm_bf16(g, 0, stream);
    if (e != hipSuccess) return fail_msg(KDA_ERR_HIP, "GEMM (output gate + norm) launch: %s", hipGetErrorString(e));
  }
  // 8. x_new = y Wo^T
  return gemm_nt(w->Wo, HD, y, HD, x_new, M, false, M, BT, HD, stream, "output projection");
}

}  // extern "C"
