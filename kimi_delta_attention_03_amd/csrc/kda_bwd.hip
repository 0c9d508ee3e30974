// Backward of the chunkwise KDA forward on gfx950: dq, dk, dv, dg, dbeta and
// dh0 for a given dO and d(final state) (Tokamax "chunk_kda_fwd design doc",
// sections 4.3.4 and 6.1: the backward returns these six gradients of the same
// forward map and reconstructs the chunk intermediates instead of keeping them).
//
// All arithmetic is fp32 with natural-log gates. Per chunk (C = 64 rows, the
// rows past the end of a short chunk are zero tokens with g = 0), with
// G = chunk-local inclusive cumsum of g, E_ij = exp(G_i - G_j) per channel and
// Gl = G of the last row:
//   Aqk = s Tril(sum_d q_i k_j E_ij),  M = StrictTril(sum_d k_i k_j E_ij),
//   A = (I + Diag(beta) M)^-1,  Kb = beta k e^G,  Vb = beta v,
//   W = A Kb,  U = A Vb,  Qg = s q e^G,  KG = k e^(Gl - G),  gamma = e^Gl
//   forward step: Vn = U - W S,  O = Qg S + Aqk Vn,  S' = Diag(gamma) S + KG^T Vn
// (Paper Eq. 6-9 of the design doc, written in the natural-log base). Its
// reverse, for the chunk-start state S and the gradient dS' of the chunk-end
// state:
//   dVn = Aqk^T dO + KG dS'                 dS = Qg^T dO + Diag(gamma) dS' - W^T dVn
//   dQg = dO S^T   dW = -dVn S^T   dKG = Vn dS'^T   dAqk = Tril(dO Vn^T)
//   dgamma = rowsum(S * dS')   dA = dW Kb^T + dVn Vb^T
//   dKb = A^T dW   dVb = A^T dVn   dL = -StrictTril(A^T dA A^T)
// and the elementwise and gated-sum rules of the definitions above take these
// to dq, dk, dv, dg (reverse cumsum of dG), dbeta; with the optional L2 norm,
// dq = (dq^ - q^ (q^ . dq^)) / |q| (or dq^ / eps where the norm is clamped).
//
// Four launches:
//   prep        per (chunk, head): the chunk terms above, from the inputs
//   states_fwd  per (sequence, head, 16 columns): chunk-start states, in order
//   states_bwd  per (sequence, head, 16 columns): dS' per chunk, in reverse; dh0
//   chunk       per (chunk, head): every other gradient
// Every intermediate lives in a per-(chunk, head) fp32 slab of the workspace.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int kBT = 256;  // threads per workgroup
constexpr int C = kChunk;

__device__ __forceinline__ float ldx(const void* p, size_t i, int f32) {
  return f32 ? reinterpret_cast<const float*>(p)[i] : to_f32(reinterpret_cast<const bf16*>(p)[i]);
}

struct ItemB {
  int p, h, len;
  int64_t tok0;
};

__device__ __forceinline__ int items_in_use(const BwdArgs& a) {
  return (a.varlen ? *reinterpret_cast<const int*>(a.ws) : (int)a.ncp) * a.H;
}

__device__ __forceinline__ ItemB chunk_of(const BwdArgs& a, int p, int h) {
  ItemB r;
  r.p = p;
  r.h = h;
  if (a.varlen) {
    const int2 ct = reinterpret_cast<const int2*>(a.ws + a.off_chunk_tab)[p];
    r.tok0 = ct.x;
    r.len = ct.y;
  } else {
    r.tok0 = (int64_t)p * C;
    r.len = C;
  }
  return r;
}

__device__ __forceinline__ float* slab_of(const BwdArgs& a, int p, int h) {
  return reinterpret_cast<float*>(a.ws + a.meta_bytes) + ((size_t)p * a.H + h) * a.sl.floats;
}

// first chunk slot and chunk count of sequence seq
__device__ __forceinline__ void seq_chunks(const BwdArgs& a, int seq, int& p0, int& nch) {
  if (a.varlen) {
    const int2 st = reinterpret_cast<const int2*>(a.ws + a.off_seq_tab)[seq];
    p0 = st.x;
    nch = st.y;
  } else {
    p0 = seq * a.nt;
    nch = a.nt;
  }
}

// out(i, j) = sum_kk fa(i, kk) fb(kk, j) for an M x N result, 4 x 4 outputs per
// thread and pass
template <int M, int N, typename FA, typename FB, typename FO>
__device__ __forceinline__ void wg_mm(int KD, FA fa, FB fb, FO fo) {
  constexpr int TN = N / 4;
  constexpr int NT = (M / 4) * TN;
  for (int t = threadIdx.x; t < NT; t += kBT) {
    const int i0 = (t / TN) * 4, j0 = (t % TN) * 4;
    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
    for (int kk = 0; kk < KD; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = fa(i0 + r, kk);
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = fb(kk, j0 + c);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] += av[r] * bv[c];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) fo(i0 + r, j0 + c, acc[r][c]);
  }
}

// ---------------------------------------------------------------- prep
template <int K>
__global__ __launch_bounds__(kBT) void bwd_prep_kernel(BwdArgs a) {
  constexpr int V = K;
  constexpr int KP = K + 1;
  constexpr int CP = C + 1;
  __shared__ float sQ[C * KP], sK[C * KP], sG[C * KP];
  __shared__ float sL[C * CP], sA[C * CP];
  __shared__ float sB[C];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= items_in_use(a)) return;
  const ItemB it = chunk_of(a, (int)blockIdx.x / a.H, (int)blockIdx.x % a.H);
  const BwdSlab& o = a.sl;
  float* sl = slab_of(a, it.p, it.h);
  const int H = a.H;
  const int qf32 = !a.bf16_qkv;

  // rows of q, k, g (rows past the chunk end are zero tokens)
  for (int e = tid; e < C * K; e += kBT) {
    const int r = e / K, d = e % K;
    float qv = 0.f, kv = 0.f, gv = 0.f;
    if (r < it.len) {
      const size_t idx = ((size_t)(it.tok0 + r) * H + it.h) * K + d;
      qv = ldx(a.q, idx, qf32);
      kv = ldx(a.k, idx, qf32);
      gv = ldx(a.g, idx, a.g_f32);
    }
    sQ[r * KP + d] = qv;
    sK[r * KP + d] = kv;
    sG[r * KP + d] = gv;
  }
  if (tid < C) sB[tid] = tid < it.len ? ldx(a.beta, (size_t)(it.tok0 + tid) * H + it.h, a.beta_f32) : 0.f;
  __syncthreads();

  // row norms (kept for the backward of the optional L2 norm); gate cumsum
  if (tid < 2 * C) {
    float* X = tid < C ? sQ : sK;
    const int r = tid % C;
    float ss = 0.f;
    for (int d = 0; d < K; ++d) ss += X[r * KP + d] * X[r * KP + d];
    const float nrm = sqrtf(ss);
    sl[(tid < C ? o.nq : o.nk) + r] = nrm;
    if (a.l2norm) {
      const float inv = 1.f / fmaxf(nrm, a.l2eps);
      for (int d = 0; d < K; ++d) X[r * KP + d] *= inv;
    }
  } else if (tid - 2 * C < K) {
    const int d = tid - 2 * C;
    float run = 0.f;
    for (int r = 0; r < C; ++r) {
      run += sG[r * KP + d];
      sG[r * KP + d] = run;
    }
  }
  __syncthreads();

  // elementwise terms
  for (int e = tid; e < C * K; e += kBT) {
    const int r = e / K, d = e % K;
    const float G = sG[r * KP + d], Gl = sG[(C - 1) * KP + d];
    const float qn = sQ[r * KP + d], kn = sK[r * KP + d];
    const float eg = __expf(G);
    sl[o.qn + e] = qn;
    sl[o.kn + e] = kn;
    sl[o.G + e] = G;
    sl[o.qg + e] = a.scale * qn * eg;
    sl[o.kg + e] = kn * __expf(Gl - G);
    sl[o.kb + e] = sB[r] * kn * eg;
  }
  for (int e = tid; e < C * V; e += kBT) {
    const int r = e / V, d = e % V;
    const float vv = r < it.len ? ldx(a.v, ((size_t)(it.tok0 + r) * H + it.h) * V + d, qf32) : 0.f;
    sl[o.vb + e] = sB[r] * vv;
  }
  if (tid < K) sl[o.gam + tid] = __expf(sG[(C - 1) * KP + tid]);
  if (tid < C) sl[o.beta + tid] = sB[tid];

  // relation tiles: thread -> row i, columns j = tid % 4 + 4 m
  {
    const int i = tid >> 2;
    for (int m = 0; m < C / 4; ++m) {
      const int j = (tid & 3) + 4 * m;
      float aq = 0.f, mm = 0.f;
      if (j <= i) {
        for (int d = 0; d < K; ++d) {
          const float kj = sK[j * KP + d] * __expf(sG[i * KP + d] - sG[j * KP + d]);
          aq += sQ[i * KP + d] * kj;
          mm += sK[i * KP + d] * kj;
        }
      }
      const float mv = j < i ? mm : 0.f;
      sl[o.aqk + i * C + j] = a.scale * aq;
      sl[o.m + i * C + j] = mv;
      sL[i * CP + j] = sB[i] * mv;
    }
  }
  __syncthreads();

  // A = (I + L)^-1 by forward substitution, thread j -> column j
  if (tid < C) {
    const int j = tid;
    for (int i = 0; i < C; ++i) {
      float x = (i == j) ? 1.f : 0.f;
      for (int m = j; m < i; ++m) x -= sL[i * CP + m] * sA[m * CP + j];
      sA[i * CP + j] = i >= j ? x : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < C * C; e += kBT) sl[o.a + e] = sA[(e / C) * CP + e % C];

  // W = A Kb, U = A Vb: thread -> channel d, rows i = tid / K + (256 / K) m
  {
    const int d = tid % K;
    constexpr int RS = kBT / K;
    float kb[C], vb[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      kb[j] = sB[j] * sK[j * KP + d] * __expf(sG[j * KP + d]);
      vb[j] = sl[o.vb + j * V + d];
    }
    for (int i = tid / K; i < C; i += RS) {
      float w = 0.f, u = 0.f;
#pragma unroll
      for (int j = 0; j < C; ++j) {  // A is zero above the diagonal
        const float aij = sA[i * CP + j];
        w += aij * kb[j];
        u += aij * vb[j];
      }
      sl[o.w + i * K + d] = w;
      sl[o.u + i * V + d] = u;
    }
  }
}

// ---------------------------------------------------------- chunk-start states
template <int K>
__global__ __launch_bounds__(kBT) void bwd_states_fwd_kernel(BwdArgs a) {
  constexpr int V = K, KP = K + 1, NVB = V / 16;
  __shared__ float sW[C * KP], sKG[C * KP];
  __shared__ float sU[C * 17], sVn[C * 17], sS[K * 17], sGam[K];
  const int tid = threadIdx.x;
  const int u = (int)blockIdx.x / NVB, vb = (int)blockIdx.x % NVB;
  if (u >= a.nunits) return;
  const int seq = u / a.H, h = u % a.H;
  const BwdSlab& o = a.sl;
  int p0, nch;
  seq_chunks(a, seq, p0, nch);
  const int c = tid & 15;
  const int col = 16 * vb + c;
  for (int d = tid >> 4; d < K; d += 16) sS[d * 17 + c] = a.init ? a.init[((size_t)u * K + d) * V + col] : 0.f;
  __syncthreads();
  for (int cc = 0; cc < nch; ++cc) {
    float* sl = slab_of(a, p0 + cc, h);
    for (int d = tid >> 4; d < K; d += 16) sl[o.S + d * V + col] = sS[d * 17 + c];
    for (int e = tid; e < C * K; e += kBT) {
      const int r = e / K, d = e % K;
      sW[r * KP + d] = sl[o.w + e];
      sKG[r * KP + d] = sl[o.kg + e];
    }
    for (int e = tid; e < C * 16; e += kBT) sU[(e >> 4) * 17 + (e & 15)] = sl[o.u + (e >> 4) * V + 16 * vb + (e & 15)];
    if (tid < K) sGam[tid] = sl[o.gam + tid];
    __syncthreads();
    for (int i = tid >> 4; i < C; i += 16) {
      float acc = 0.f;
      for (int d = 0; d < K; ++d) acc += sW[i * KP + d] * sS[d * 17 + c];
      sVn[i * 17 + c] = sU[i * 17 + c] - acc;
    }
    __syncthreads();
    for (int d = tid >> 4; d < K; d += 16) {
      float acc = sGam[d] * sS[d * 17 + c];
      for (int i = 0; i < C; ++i) acc += sKG[i * KP + d] * sVn[i * 17 + c];
      sS[d * 17 + c] = acc;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ state gradients
template <int K>
__global__ __launch_bounds__(kBT) void bwd_states_bwd_kernel(BwdArgs a) {
  constexpr int V = K, KP = K + 1, CP = C + 1, NVB = V / 16;
  __shared__ float sAq[C * CP], sKG[C * KP], sQG[C * KP], sW[C * KP];
  __shared__ float sdO[C * 17], sdVn[C * 17], sdS[K * 17], sGam[K];
  const int tid = threadIdx.x;
  const int u = (int)blockIdx.x / NVB, vb = (int)blockIdx.x % NVB;
  if (u >= a.nunits) return;
  const int seq = u / a.H, h = u % a.H;
  const BwdSlab& o = a.sl;
  int p0, nch;
  seq_chunks(a, seq, p0, nch);
  const int c = tid & 15;
  const int col = 16 * vb + c;
  const int qf32 = !a.bf16_qkv;
  for (int d = tid >> 4; d < K; d += 16)
    sdS[d * 17 + c] = a.d_final ? a.d_final[((size_t)u * K + d) * V + col] : 0.f;
  __syncthreads();
  for (int cc = nch - 1; cc >= 0; --cc) {
    const ItemB it = chunk_of(a, p0 + cc, h);
    float* sl = slab_of(a, p0 + cc, h);
    for (int d = tid >> 4; d < K; d += 16) sl[o.dS + d * V + col] = sdS[d * 17 + c];
    for (int e = tid; e < C * K; e += kBT) {
      const int r = e / K, d = e % K;
      sKG[r * KP + d] = sl[o.kg + e];
      sQG[r * KP + d] = sl[o.qg + e];
      sW[r * KP + d] = sl[o.w + e];
    }
    for (int e = tid; e < C * C; e += kBT) sAq[(e / C) * CP + e % C] = sl[o.aqk + e];
    for (int e = tid; e < C * 16; e += kBT) {
      const int r = e >> 4, cl = e & 15;
      sdO[r * 17 + cl] = r < it.len ? ldx(a.d_o, ((size_t)(it.tok0 + r) * a.H + h) * V + 16 * vb + cl, qf32) : 0.f;
    }
    if (tid < K) sGam[tid] = sl[o.gam + tid];
    __syncthreads();
    for (int i = tid >> 4; i < C; i += 16) {
      float acc = 0.f;
      for (int r = i; r < C; ++r) acc += sAq[r * CP + i] * sdO[r * 17 + c];
      for (int d = 0; d < K; ++d) acc += sKG[i * KP + d] * sdS[d * 17 + c];
      sdVn[i * 17 + c] = acc;
    }
    __syncthreads();
    for (int d = tid >> 4; d < K; d += 16) {
      float acc = sGam[d] * sdS[d * 17 + c];
      for (int r = 0; r < C; ++r) acc += sQG[r * KP + d] * sdO[r * 17 + c] - sW[r * KP + d] * sdVn[r * 17 + c];
      sdS[d * 17 + c] = acc;
    }
    __syncthreads();
  }
  if (a.dh0)
    for (int d = tid >> 4; d < K; d += 16) a.dh0[((size_t)u * K + d) * V + col] = sdS[d * 17 + c];
}

// ------------------------------------------------------------ chunk gradients
template <int K>
__global__ __launch_bounds__(kBT) void bwd_chunk_kernel(BwdArgs a) {
  constexpr int V = K;
  __shared__ float sDot[2 * C];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= items_in_use(a)) return;
  const ItemB it = chunk_of(a, (int)blockIdx.x / a.H, (int)blockIdx.x % a.H);
  const BwdSlab& o = a.sl;
  float* sl = slab_of(a, it.p, it.h);
  const int H = a.H;
  const int qf32 = !a.bf16_qkv;
  const float s = a.scale;
  float* const QN = sl + o.qn;
  float* const KN = sl + o.kn;
  float* const G = sl + o.G;
  float* const QG = sl + o.qg;
  float* const KG = sl + o.kg;
  float* const W = sl + o.w;
  float* const KB = sl + o.kb;
  float* const U = sl + o.u;
  float* const VB = sl + o.vb;
  float* const AQK = sl + o.aqk;
  float* const A = sl + o.a;
  float* const Mm = sl + o.m;
  float* const BETA = sl + o.beta;
  float* const GAM = sl + o.gam;
  float* const S = sl + o.S;
  float* const DS = sl + o.dS;
  float* const DO = sl + o.dO;
  float* const VN = sl + o.vn;
  float* const DVN = sl + o.dvn;
  float* const DVB = sl + o.dvb;
  float* const DQG = sl + o.dqg;
  float* const DW = sl + o.dw;
  float* const DKG = sl + o.dkg;
  float* const DKB = sl + o.dkb;
  float* const DQN = sl + o.dqn;
  float* const DKN = sl + o.dkn;
  float* const DG = sl + o.dG;
  float* const DAQK = sl + o.daqk;
  float* const DA = sl + o.da;
  float* const T1 = sl + o.t1;
  float* const DL = sl + o.dl;
  float* const DGAM = sl + o.dgam;

  for (int e = tid; e < C * V; e += kBT) {
    const int r = e / V, d = e % V;
    DO[e] = r < it.len ? ldx(a.d_o, ((size_t)(it.tok0 + r) * H + it.h) * V + d, qf32) : 0.f;
  }
  __syncthreads();
  // Vn = U - W S;  dVn = Aqk^T dO + KG dS'
  wg_mm<C, V>(K, [&](int i, int kk) { return W[i * K + kk]; }, [&](int kk, int j) { return S[kk * V + j]; },
              [&](int i, int j, float x) { VN[i * V + j] = U[i * V + j] - x; });
  wg_mm<C, V>(C + K,
              [&](int i, int kk) { return kk < C ? AQK[kk * C + i] : KG[i * K + kk - C]; },
              [&](int kk, int j) { return kk < C ? DO[kk * V + j] : DS[(kk - C) * V + j]; },
              [&](int i, int j, float x) { DVN[i * V + j] = x; });
  __syncthreads();
  // dQg = dO S^T, dW = -dVn S^T, dKG = Vn dS'^T, dAqk = Tril(dO Vn^T), dgamma
  wg_mm<C, K>(V, [&](int i, int kk) { return DO[i * V + kk]; }, [&](int kk, int j) { return S[j * V + kk]; },
              [&](int i, int j, float x) { DQG[i * K + j] = x; });
  wg_mm<C, K>(V, [&](int i, int kk) { return DVN[i * V + kk]; }, [&](int kk, int j) { return S[j * V + kk]; },
              [&](int i, int j, float x) { DW[i * K + j] = -x; });
  wg_mm<C, K>(V, [&](int i, int kk) { return VN[i * V + kk]; }, [&](int kk, int j) { return DS[j * V + kk]; },
              [&](int i, int j, float x) { DKG[i * K + j] = x; });
  wg_mm<C, C>(V, [&](int i, int kk) { return DO[i * V + kk]; }, [&](int kk, int j) { return VN[j * V + kk]; },
              [&](int i, int j, float x) { DAQK[i * C + j] = j <= i ? x : 0.f; });
  if (tid < K) {
    float acc = 0.f;
    for (int v = 0; v < V; ++v) acc += S[tid * V + v] * DS[tid * V + v];
    DGAM[tid] = acc;
  }
  __syncthreads();
  // dA = dW Kb^T + dVn Vb^T;  dKb = A^T dW;  dVb = A^T dVn
  wg_mm<C, C>(K + V,
              [&](int i, int kk) { return kk < K ? DW[i * K + kk] : DVN[i * V + kk - K]; },
              [&](int kk, int j) { return kk < K ? KB[j * K + kk] : VB[j * V + kk - K]; },
              [&](int i, int j, float x) { DA[i * C + j] = x; });
  wg_mm<C, K>(C, [&](int i, int kk) { return A[kk * C + i]; }, [&](int kk, int j) { return DW[kk * K + j]; },
              [&](int i, int j, float x) { DKB[i * K + j] = x; });
  wg_mm<C, V>(C, [&](int i, int kk) { return A[kk * C + i]; }, [&](int kk, int j) { return DVN[kk * V + j]; },
              [&](int i, int j, float x) { DVB[i * V + j] = x; });
  __syncthreads();
  // dL = -StrictTril(A^T dA A^T)
  wg_mm<C, C>(C, [&](int i, int kk) { return A[kk * C + i]; }, [&](int kk, int j) { return DA[kk * C + j]; },
              [&](int i, int j, float x) { T1[i * C + j] = x; });
  __syncthreads();
  wg_mm<C, C>(C, [&](int i, int kk) { return T1[i * C + kk]; }, [&](int kk, int j) { return A[j * C + kk]; },
              [&](int i, int j, float x) { DL[i * C + j] = j < i ? -x : 0.f; });
  __syncthreads();

  // per element: thread -> channel d, rows i = tid / K + (256 / K) m
  {
    const int d = tid % K;
    constexpr int RS = kBT / K;
    const float Gl = G[(C - 1) * K + d];
    for (int i = tid / K; i < C; i += RS) {
      const float Gi = G[i * K + d], qi = QN[i * K + d], ki = KN[i * K + d], bi = BETA[i];
      float sAq = 0.f, sMq = 0.f;  // query side: keys j <= i
      for (int j = 0; j <= i; ++j) {
        const float kE = KN[j * K + d] * __expf(Gi - G[j * K + d]);
        sAq += DAQK[i * C + j] * kE;
        sMq += bi * DL[i * C + j] * kE;
      }
      float sAk = 0.f, sMk = 0.f;  // key side: queries r >= i
      for (int r = i; r < C; ++r) {
        const float E = __expf(G[r * K + d] - Gi);
        sAk += DAQK[r * C + i] * QN[r * K + d] * E;
        sMk += BETA[r] * DL[r * C + i] * KN[r * K + d] * E;
      }
      const float eg = __expf(Gi);
      const float dqg = DQG[i * K + d], dkb = DKB[i * K + d], dkg = DKG[i * K + d];
      DQN[i * K + d] = s * eg * dqg + s * sAq;
      DKN[i * K + d] = dkb * bi * eg + dkg * __expf(Gl - Gi) + s * sAk + sMq + sMk;
      float dG = dqg * QG[i * K + d] + dkb * KB[i * K + d] - dkg * KG[i * K + d] + qi * s * sAq - ki * s * sAk +
                 ki * sMq - ki * sMk;
      if (i == C - 1) {
        float dGl = DGAM[d] * GAM[d];
        for (int r = 0; r < C; ++r) dGl += DKG[r * K + d] * KG[r * K + d];
        dG += dGl;
      }
      DG[i * K + d] = dG;
    }
  }
  // dbeta and dv: thread -> row
  if (tid < C) {
    const int i = tid;
    float db = 0.f;
    if (i < it.len) {
      const size_t vrow = ((size_t)(it.tok0 + i) * H + it.h) * V;
      for (int v = 0; v < V; ++v) {
        const float dvb = DVB[i * V + v];
        db += dvb * ldx(a.v, vrow + v, qf32);
        a.dv[vrow + v] = BETA[i] * dvb;
      }
      for (int d = 0; d < K; ++d) db += DKB[i * K + d] * KN[i * K + d] * __expf(G[i * K + d]);
      for (int j = 0; j < i; ++j) db += DL[i * C + j] * Mm[i * C + j];
      a.dbeta[(size_t)(it.tok0 + i) * H + it.h] = db;
    }
  }
  __syncthreads();
  // L2-norm backward: row dot products q^ . dq^ and k^ . dk^
  if (tid < 2 * C) {
    const int r = tid % C;
    const float* X = tid < C ? QN : KN;
    const float* D = tid < C ? DQN : DKN;
    float acc = 0.f;
    for (int d = 0; d < K; ++d) acc += X[r * K + d] * D[r * K + d];
    sDot[tid] = acc;
  }
  __syncthreads();
  for (int e = tid; e < C * K; e += kBT) {
    const int r = e / K, d = e % K;
    if (r >= it.len) continue;
    const size_t idx = ((size_t)(it.tok0 + r) * H + it.h) * K + d;
    float gq = DQN[e], gk = DKN[e];
    if (a.l2norm) {
      const float nq = sl[o.nq + r], nk = sl[o.nk + r];
      gq = nq > a.l2eps ? (gq - QN[e] * sDot[r]) / nq : gq / a.l2eps;
      gk = nk > a.l2eps ? (gk - KN[e] * sDot[C + r]) / nk : gk / a.l2eps;
    }
    a.dq[idx] = gq;
    a.dk[idx] = gk;
  }
  // dg = reverse cumsum of dG over the chunk
  if (tid < K) {
    const int d = tid;
    float run = 0.f;
    for (int r = C - 1; r >= 0; --r) {
      run += DG[r * K + d];
      if (r < it.len) a.dg[((size_t)(it.tok0 + r) * H + it.h) * K + d] = run;
    }
  }
}

// stages: bit 0 prep, bit 1 chunk-start states, bit 2 state gradients, bit 3 chunk gradients
template <int K>
hipError_t launch_k(const BwdArgs& a, int nitems, int stages, hipStream_t s) {
  const int nvb = K / 16;
  if ((stages & 1) && nitems > 0) hipLaunchKernelGGL(bwd_prep_kernel<K>, dim3(nitems), dim3(kBT), 0, s, a);
  if (a.nunits > 0) {
    if ((stages & 2) && nitems > 0)
      hipLaunchKernelGGL(bwd_states_fwd_kernel<K>, dim3(a.nunits * nvb), dim3(kBT), 0, s, a);
    if (stages & 4) hipLaunchKernelGGL(bwd_states_bwd_kernel<K>, dim3(a.nunits * nvb), dim3(kBT), 0, s, a);
  }
  if ((stages & 8) && nitems > 0) hipLaunchKernelGGL(bwd_chunk_kernel<K>, dim3(nitems), dim3(kBT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int K, int nitems, int stages, hipStream_t s) {
  return K == 128 ? launch_k<128>(a, nitems, stages, s) : launch_k<64>(a, nitems, stages, s);
}

}  // namespace kda
