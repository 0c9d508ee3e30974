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
// Four stages:
//   prep        per (chunk, head): the chunk terms above, from the inputs
//   states_fwd  per (sequence, head, 16 columns): chunk-start states, in order
//   states_bwd  per (sequence, head, 16 columns): dS' per chunk, in reverse; dh0
//   chunk       per (chunk, head): every other gradient. With bf16 q/k/v one
//               fused launch (products on bf16 MFMA, then the elementwise and
//               gated-sum rules, the item on chip); with fp32 two launches (fp32
//               products through the slab, then the rules)
// The chunk terms and states live in a per-(chunk, head) fp32 slab of the
// workspace. prep and the fp32 elementwise kernel are latency-bound chains of
// phases and run 16 waves per workgroup (one workgroup per CU by LDS); the fp32
// product kernel runs 4 waves with its operand slices double-buffered; the two
// state passes run 8 waves, 4 on the per-chunk MFMA chain and 4 that load and
// stage the chunk operands ahead of it. Loads are issued before stores
// throughout: on this GPU a memory-counter wait also waits for every earlier
// store.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int kBT = 256;  // threads per workgroup (the state passes run 2 kBT)
constexpr int kBW = 1024;  // threads of the per-chunk rebuild and elementwise kernels
constexpr int kNWW = kBW / 64;
constexpr int C = kChunk;

__device__ __forceinline__ float ldx(const void* p, size_t i, int f32) {
  return f32 ? reinterpret_cast<const float*>(p)[i] : to_f32(reinterpret_cast<const bf16*>(p)[i]);
}

struct ItemB {
  int p, h, len;
  int64_t tok0;
};

// NE elements per thread of a [C, W] row block of tensor x at (chunk it, head h):
// element e = threadIdx.x + NT m is row e / W, column e % W. Rows past the chunk
// end read row 0's address (always valid: a chunk holds at least one token) and
// become 0. All loads are issued before any result is used.
template <typename TX, int NE, int NT, int W>
__device__ __forceinline__ void load_rows(const void* x, const ItemB& it, int H, float* out) {
  const TX* p = reinterpret_cast<const TX*>(x);
  TX raw[NE];
#pragma unroll
  for (int m = 0; m < NE; ++m) {
    const int e = (int)threadIdx.x + NT * m, r = e / W, d = e % W;
    const int rr = r < it.len ? r : 0;
    raw[m] = p[((size_t)(it.tok0 + rr) * H + it.h) * W + d];
  }
#pragma unroll
  for (int m = 0; m < NE; ++m) {
    const int r = ((int)threadIdx.x + NT * m) / W;
    out[m] = r < it.len ? to_f32(raw[m]) : 0.f;
  }
}

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

__device__ __forceinline__ bf16x4 to_bf16x4(floatx4 x) { return __builtin_convertvector(x, bf16x4); }

// fp32 16x16x4 MFMA step: lane (g, i) = (l / 16, l % 16) gives A[i][g] and
// B[g][i] of a 4-deep slice; the accumulator lane holds rows 4 g + r, column i
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// out(i, j) = sum_kk A(i, kk) B(kk, j) for an M x N result over KD (a multiple
// of 16), with A(i, kk) = A[i * lda + kk] (TA: A[kk * lda + i]) and B(kk, j) =
// B[kk * ldb + j] (TB: B[j * ldb + kk]). 16-deep slices of both operands pass
// through registers into LDS (smem: 16 (M + 4) + 16 (N + 4) floats), loaded
// along the contiguous index; the next slice's loads are in flight while the
// current slice is multiplied. Each thread accumulates 4 rows x M N / 1024
// columns. Ends with a barrier, before the epilogue calls.
template <int M, int N, bool TA, bool TB, typename FO>
__device__ __forceinline__ void lds_mm(int KD, const float* A, int lda, const float* B, int ldb, float* smem,
                                       FO fo) {
  constexpr int KS = 16;
  constexpr int NC = M * N / (kBT * 4);
  constexpr int NCG = N / NC;
  constexpr int SA = M + 4, SB = N + 4;
  constexpr int LA = M * KS / kBT, LB = N * KS / kBT;  // slice elements per thread
  static_assert(NC % 4 == 0 && (M / 4) * NCG == kBT, "thread tiling");
  static_assert(LA * kBT == M * KS && LB * kBT == N * KS, "slice split");
  float* sa = smem;
  float* sb = smem + KS * SA;
  const int tid = threadIdx.x;
  const int rg = tid / NCG, cg = tid % NCG;
  float acc[4][NC];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[r][c] = 0.f;
  float ra[LA], rb[LB];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int m = 0; m < LA; ++m) {
      const int e = tid + kBT * m;
      ra[m] = TA ? A[(size_t)(k0 + e / M) * lda + e % M] : A[(size_t)(e / KS) * lda + k0 + e % KS];
    }
#pragma unroll
    for (int m = 0; m < LB; ++m) {
      const int e = tid + kBT * m;
      rb[m] = TB ? B[(size_t)(e / KS) * ldb + k0 + e % KS] : B[(size_t)(k0 + e / N) * ldb + e % N];
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < KD; k0 += KS) {
#pragma unroll
    for (int m = 0; m < LA; ++m) {
      const int e = tid + kBT * m;
      if (TA) sa[(e / M) * SA + e % M] = ra[m];
      else sa[(e % KS) * SA + e / KS] = ra[m];
    }
#pragma unroll
    for (int m = 0; m < LB; ++m) {
      const int e = tid + kBT * m;
      if (TB) sb[(e % KS) * SB + e / KS] = rb[m];
      else sb[(e / N) * SB + e % N] = rb[m];
    }
    __syncthreads();
    if (k0 + KS < KD) fetch(k0 + KS);  // in flight during the products below
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const floatx4 a4 = *reinterpret_cast<const floatx4*>(sa + kk * SA + 4 * rg);
      float b[NC];
#pragma unroll
      for (int c = 0; c < NC; c += 4) {
        const floatx4 b4 = *reinterpret_cast<const floatx4*>(sb + kk * SB + NC * cg + c);
        b[c] = b4[0]; b[c + 1] = b4[1]; b[c + 2] = b4[2]; b[c + 3] = b4[3];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[r][c] += a4[r] * b[c];
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) fo(4 * rg + r, NC * cg + c, acc[r][c]);
}

// ---------------------------------------------------------------- prep
template <int K>
__global__ __launch_bounds__(kBW) void bwd_prep_kernel(BwdArgs a) {
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

  // rows of q, k, g, v (rows past the chunk end are zero tokens), all loads in
  // flight together: no store is issued in between, since every memory-counter
  // wait would also wait for earlier stores
  constexpr int NE = C * K / kBW;
  float qv[NE], kv[NE], gv[NE], vv[NE];
  if (qf32) {
    load_rows<float, NE, kBW, K>(a.q, it, H, qv);
    load_rows<float, NE, kBW, K>(a.k, it, H, kv);
    load_rows<float, NE, kBW, V>(a.v, it, H, vv);
  } else {
    load_rows<bf16, NE, kBW, K>(a.q, it, H, qv);
    load_rows<bf16, NE, kBW, K>(a.k, it, H, kv);
    load_rows<bf16, NE, kBW, V>(a.v, it, H, vv);
  }
  if (a.g_f32) load_rows<float, NE, kBW, K>(a.g, it, H, gv);
  else load_rows<bf16, NE, kBW, K>(a.g, it, H, gv);
  if (tid < C) sB[tid] = tid < it.len ? ldx(a.beta, (size_t)(it.tok0 + tid) * H + it.h, a.beta_f32) : 0.f;
#pragma unroll
  for (int m = 0; m < NE; ++m) {
    const int e = tid + kBW * m, r = e / K, d = e % K;
    sQ[r * KP + d] = qv[m];
    sK[r * KP + d] = kv[m];
    sG[r * KP + d] = gv[m];
  }
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
  for (int e = tid; e < C * K; e += kBW) {
    const int r = e / K, d = e % K;
    const float G = sG[r * KP + d], Gl = sG[(C - 1) * KP + d];
    const float qn = sQ[r * KP + d], kn = sK[r * KP + d];
    const float eg = __expf(G);
    if (qf32) sl[o.qg + e] = a.scale * qn * eg;
    const float kgv = kn * __expf(Gl - G);
    sl[o.kg + e] = kgv;
    // bf16 inputs: a bf16 copy for the bf16 state-gradient pass (its MFMA
    // operand type), in the second half of the Vb array
    if (!qf32) reinterpret_cast<bf16*>(sl + o.vb)[K * C + e] = (bf16)kgv;
    sl[o.kb + e] = sB[r] * kn * eg;
  }
  // Vb for the fp32 product kernel (the bf16 one rebuilds it from v and beta)
  if (qf32) {
#pragma unroll
    for (int m = 0; m < NE; ++m) {
      const int e = tid + kBW * m;
      sl[o.vb + e] = sB[e / V] * vv[m];
    }
  }
  // with bf16 inputs only the bf16 state-gradient pass reads Qg, as a bf16 MFMA
  // operand with the chunk row contiguous: stored so, Qg^T [K][C] in bf16 in the
  // first half of its slab array (the same fp32 value, rounded once)
  if (!qf32) {
    bf16* qgt = reinterpret_cast<bf16*>(sl + o.qg);
    for (int e = tid; e < C * K; e += kBW) {
      const int d = e / C, r = e % C;
      qgt[e] = (bf16)(a.scale * sQ[r * KP + d] * __expf(sG[r * KP + d]));
    }
  }
  if (tid < K) sl[o.gam + tid] = __expf(sG[(C - 1) * KP + tid]);
  if (tid < C) sl[o.beta + tid] = sB[tid];

  // relation tiles (query block ib, key block jb <= ib) on fp32 MFMA with the
  // key block's first row as reference: q_i exp(G_i - rho) <= |q_i| for i in
  // block ib >= jb, k_j exp(rho - G_j) spans at most 15 steps of decay
  {
    const int lane = tid & 63, gq = lane >> 4, xi = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int t = w; t < 10; t += kNWW) {
      // t -> (ib, jb) over the 10 causal block pairs
      const int ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
      const int jb = t - ib * (ib + 1) / 2;
      floatx4 accQ = zero4(), accK = zero4();
      const int i = 16 * ib + xi, j = 16 * jb + xi;
#pragma unroll 4
      for (int k0 = 0; k0 < K; k0 += 4) {
        const int d = k0 + gq;
        const float rho = sG[(16 * jb) * KP + d];
        const float ei = __expf(sG[i * KP + d] - rho);
        const float kj = sK[j * KP + d] * __expf(rho - sG[j * KP + d]);
        accQ = mfma4(sQ[i * KP + d] * ei, kj, accQ);
        accK = mfma4(sK[i * KP + d] * ei, kj, accK);
      }
      floatx4 aqv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 16 * ib + 4 * gq + r, jj = 16 * jb + xi;
        const float aq = jj <= ii ? a.scale * accQ[r] : 0.f;
        const float mv = jj < ii ? accK[r] : 0.f;
        if (qf32) sl[o.aqk + ii * C + jj] = aq;   // bf16 inputs read only the bf16 Aqk^T below
        sl[o.m + ii * C + jj] = mv;
        sL[ii * CP + jj] = sB[ii] * mv;
        aqv[r] = aq;
      }
      // bf16 inputs: Aqk^T [C][C] in bf16 for the bf16 state-gradient pass, in
      // the array of dQg (which only fp32 inputs use): lane (g, i) holds rows
      // 16 ib + 4 g .. + 3 of column 16 jb + i
      if (!qf32)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(sl + o.dqg) + (16 * jb + xi) * C + 16 * ib + 4 * gq) =
            to_bf16x4(aqv);
    }
    // the blocks above the diagonal are zero
    for (int e = tid; e < C * C; e += kBW) {
      const int ii = e / C, jj = e % C;
      if (jj / 16 > ii / 16) {
        if (qf32) sl[o.aqk + e] = 0.f;
        sl[o.m + e] = 0.f;
        sL[ii * CP + jj] = 0.f;
        if (!qf32) reinterpret_cast<bf16*>(sl + o.dqg)[jj * C + ii] = bf16(0.f);
      }
    }
  }
  __syncthreads();

  // the q rows are no longer needed: their LDS holds Vb for the U product below
#pragma unroll
  for (int m = 0; m < NE; ++m) {
    const int e = tid + kBW * m;
    sQ[(e / V) * KP + e % V] = sB[e / V] * vv[m];
  }
  // A = (I + L)^-1, blocked: wave w < 4 inverts diagonal block w by forward
  // substitution (lane xi -> column xi; the four lane groups compute the same
  // values), then its block column below the diagonal on fp32 MFMA:
  //   A_ib,w = -D_ib sum_{kb=w}^{ib-1} L_ib,kb A_kb,w,  D_ib = A_ib,ib
  // with the reduction index of step s at lane group g taken as 4 g + s, so an
  // accumulator tile (lane (g, i) holds rows 4 g + r) is itself the B operand.
  {
    const int lane = tid & 63, gq = lane >> 4, xi = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (w < 4) {
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == xi) ? 1.f : 0.f;
      const float* Lb = sL + (16 * w) * CP + 16 * w;
#pragma unroll
      for (int j = 0; j < 15; ++j)
#pragma unroll
        for (int i = j + 1; i < 16; ++i) x[i] -= Lb[i * CP + j] * x[j];
      if (gq == 0)
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[(16 * w + i) * CP + 16 * w + xi] = x[i];
    }
    for (int e = tid; e < C * C; e += kBW) {  // blocks above the diagonal are zero
      const int i = e / C, j = e % C;
      if (j / 16 > i / 16) sA[i * CP + j] = 0.f;
    }
    __syncthreads();
    if (w < 4) {
      floatx4 Dw, Ab[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) Dw[q] = sA[(16 * w + 4 * gq + q) * CP + 16 * w + xi];
#pragma unroll
      for (int ib = 1; ib < 4; ++ib) {
        Ab[ib] = zero4();
        if (ib > w) {
          floatx4 P = zero4();
#pragma unroll
          for (int kb = 0; kb < 3; ++kb) {
            if (kb >= w && kb < ib) {
              floatx4 La;
#pragma unroll
              for (int q = 0; q < 4; ++q) La[q] = sL[(16 * ib + xi) * CP + 16 * kb + 4 * gq + q];
              P = mma16_f32(P, La, kb == w ? Dw : Ab[kb]);
            }
          }
          floatx4 Da;
#pragma unroll
          for (int q = 0; q < 4; ++q) Da[q] = sA[(16 * ib + xi) * CP + 16 * ib + 4 * gq + q];
          Ab[ib] = -mma16_f32(zero4(), Da, P);
        }
      }
#pragma unroll
      for (int ib = 1; ib < 4; ++ib)
        if (ib > w)
#pragma unroll
          for (int r = 0; r < 4; ++r) sA[(16 * ib + 4 * gq + r) * CP + 16 * w + xi] = Ab[ib][r];
    }
    __syncthreads();
  }
  for (int e = tid; e < C * C; e += kBW) sl[o.a + e] = sA[(e / C) * CP + e % C];

  // W = A Kb, U = A Vb on fp32 MFMA: output tile (row block ib, 16 channels ct),
  // reduction over the key rows j < 16 (ib + 1) (A is lower triangular)
  {
    const int lane = tid & 63, gq = lane >> 4, xi = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int NCT = K / 16;
    for (int t = w; t < 4 * NCT; t += kNWW) {
      const int ib = t / NCT, ct = t % NCT;
      const int d = 16 * ct + xi;
      floatx4 accW = zero4(), accU = zero4();
      for (int k0 = 0; k0 < 16 * (ib + 1); k0 += 4) {
        const int j = k0 + gq;
        const float aij = sA[(16 * ib + xi) * CP + j];
        accW = mfma4(aij, sB[j] * sK[j * KP + d] * __expf(sG[j * KP + d]), accW);
        accU = mfma4(aij, sQ[j * KP + d], accU);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 16 * ib + 4 * gq + r;
        sl[o.w + ii * K + d] = accW[r];
        sl[o.u + ii * V + d] = accU[r];
      }
      // bf16 inputs: also W^T [K][C] in bf16 for the bf16 state-gradient pass, in
      // the slab array of Vb (which only fp32 inputs use)
      if (!qf32)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(sl + o.vb) + d * C + 16 * ib + 4 * gq) = to_bf16x4(accW);
    }
  }
}

// 16 bytes per lane from global memory straight into LDS (lane l writes the
// LDS base + 16 l; the base must be wave-uniform). The host pass, which only
// emits the launch stub, does not accept the 16-byte form of the builtin.
#if defined(__HIP_DEVICE_COMPILE__)
#define KDA_LDS_DMA16(gptr, ldsptr) __builtin_amdgcn_global_load_lds((gptr), (ldsptr), 16, 0, 0)
#else
#define KDA_LDS_DMA16(gptr, ldsptr) ((void)0)
#endif

// ---------------------------------------------------------- chunk-start states
// One workgroup (8 waves) per (sequence, head, 16-column block) walks the
// chunks in order. Compute wave w (0..3) keeps state rows [16 TPW w,
// 16 TPW (w + 1)) of the block as fp32 MFMA accumulators (16x16x4: lane (g, i) =
// (l / 16, l % 16) holds rows 4 g + r, column i of a 16 x 16 tile; an A operand
// lane holds row i, reduction index g of a 4-deep slice, a B operand lane
// reduction index g, column i). Loader waves 4..7 bring the next chunk's
// operands into the other of two LDS buffers and copy the chunk-start state to
// the slab, so the compute waves only run the two products of each chunk. Two
// barriers per chunk: A (operands and start state published) and B (V_new
// published, start state read).

template <int K>
__global__ __launch_bounds__(2 * kBT) void bwd_states_fwd_kernel(BwdArgs a) {
  constexpr int V = K, KP = K + 4, NVB = V / 16, TPW = K / 64, NF = C * K / 4 / kBT;
  // two LDS buffers of the chunk operands: loader waves fill one while the
  // compute waves multiply from the other
  __shared__ __attribute__((aligned(16))) float sW[2][C * KP], sKG[2][C * KP];
  __shared__ __attribute__((aligned(16))) float sU[2][C * 20];
  // the start state and V_new transposed (column-major, rows padded by 4), so
  // that a lane reads 4 consecutive reduction indices at once
  constexpr int SP = K + 4, VP = C + 4;
  __shared__ __attribute__((aligned(16))) float sST[16 * SP], sVnT[16 * VP];
  // gamma padded to 1 KB: one direct-to-LDS instruction fills it
  __shared__ __attribute__((aligned(16))) float sGam[2][256];
  const int tid = threadIdx.x;
  const int lane = tid & 63, gq = lane >> 4, xi = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the NVB workgroups of one (sequence, head) get ids congruent modulo 8: with
  // round-robin dispatch over the 8 XCDs they share one L2 for the chunk operands
  const int bid = (int)blockIdx.x, slot = bid >> 3;
  const int u = (slot / NVB) * 8 + (bid & 7), vb = slot % NVB;
  if (u >= a.nunits) return;
  const int seq = u / a.H, h = u % a.H;
  const BwdSlab& o = a.sl;
  int p0, nch;
  seq_chunks(a, seq, p0, nch);
  const int col = 16 * vb + xi;

  if (w < 4) {
    // ---------------------------------------------------------- compute waves
    // wave w: V_new rows 16 w .. 16 w + 15, state rows 16 (TPW w + t) ..
    floatx4 S[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (TPW * w + t) + 4 * gq + r;
        S[t][r] = a.init ? a.init[((size_t)u * K + row) * V + col] : 0.f;
      }
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      *reinterpret_cast<floatx4*>(sST + xi * SP + 16 * (TPW * w + t) + 4 * gq) = S[t];
    // The reduction index of 16-deep slice k0 is ordered k0 + 4 g + s (lane group
    // g, MFMA step s), so each lane's operands for the 4 steps are 4 consecutive
    // floats: one 16-byte LDS read instead of four, all issued before the MFMAs.
    for (int cc = 0; cc < nch; ++cc) {
      const int b = cc & 1;
      __syncthreads();  // A: operands of chunk cc and its start state published
      // Vn = U - W S (four independent accumulator chains, one per step s)
      {
        floatx4 Wa[K / 16], Sb[K / 16];
#pragma unroll
        for (int q = 0; q < K / 16; ++q) {
          Wa[q] = *reinterpret_cast<const floatx4*>(&sW[b][(16 * w + xi) * KP + 16 * q + 4 * gq]);
          Sb[q] = *reinterpret_cast<const floatx4*>(sST + xi * SP + 16 * q + 4 * gq);
        }
        floatx4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int q = 0; q < K / 16; ++q)
#pragma unroll
          for (int st = 0; st < 4; ++st) acc[st] = mfma4(Wa[q][st], Sb[q][st], acc[st]);
        const floatx4 ws = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        floatx4 vn;
#pragma unroll
        for (int r = 0; r < 4; ++r) vn[r] = sU[b][(16 * w + 4 * gq + r) * 20 + xi] - ws[r];
        *reinterpret_cast<floatx4*>(sVnT + xi * VP + 16 * w + 4 * gq) = vn;
      }
      __syncthreads();  // B: Vn published; the start state has been read
      // S = Diag(gamma) S + KG^T Vn (two accumulator chains per tile)
      floatx4 Vb[C / 16];
#pragma unroll
      for (int q = 0; q < C / 16; ++q) Vb[q] = *reinterpret_cast<const floatx4*>(sVnT + xi * VP + 16 * q + 4 * gq);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int rt = TPW * w + t;
        float Ka[C / 16][4];
#pragma unroll
        for (int q = 0; q < C / 16; ++q)
#pragma unroll
          for (int st = 0; st < 4; ++st) Ka[q][st] = sKG[b][(16 * q + 4 * gq + st) * KP + 16 * rt + xi];
#pragma unroll
        for (int r = 0; r < 4; ++r) S[t][r] *= sGam[b][16 * rt + 4 * gq + r];
        floatx4 acc2 = zero4();
#pragma unroll
        for (int q = 0; q < C / 16; ++q) {
          S[t] = mfma4(Ka[q][0], Vb[q][0], S[t]);
          acc2 = mfma4(Ka[q][1], Vb[q][1], acc2);
          S[t] = mfma4(Ka[q][2], Vb[q][2], S[t]);
          acc2 = mfma4(Ka[q][3], Vb[q][3], acc2);
        }
        S[t] += acc2;
        *reinterpret_cast<floatx4*>(sST + xi * SP + 16 * rt + 4 * gq) = S[t];
      }
    }
  } else {
    // ----------------------------------------------------------- loader waves
    // The chunk operands go from the slab straight into LDS
    // (global_load_lds_dwordx4: lane l of one instruction writes the 16 bytes at
    // the LDS base + 16 l), with no register round trip and no LDS write
    // instructions. One instruction fills 1 KB of a padded LDS array; a lane
    // whose 16 bytes fall on a row's pad loads the row's first 16 bytes there
    // (never read). The four loader waves split each array's instructions; the
    // last one is issued by several waves (same bytes, same data), so every wave
    // issues the same count and one memory-counter wait per barrier is exact
    // (a wave's vector-memory loads and stores retire in issue order on this
    // counter). W and U of chunk c (read before barrier B(c)) are loaded after
    // B(c - 2), into the buffer chunk c - 2 has finished with; KG and gamma
    // (read after B(c)) after A(c - 1). Chunk indices are clamped, so the
    // loads are unconditional.
    // Thread lt also copies K / 16 entries of the chunk-start state to the
    // checkpoint as runs of four columns (rows lt / 4 + 64 m, columns
    // 4 (lt % 4) .. + 3 of the block): one 8- or 16-byte store per run rather
    // than four element stores, which cost the CU's vector-memory path as much
    // as full ones.
    const int lt = tid - kBT, ll = lt & 63, lw = __builtin_amdgcn_readfirstlane(lt >> 6);
    constexpr int NSR = K / 64;                       // state runs per thread
    constexpr int NIA = C * KP / 256, NJA = (NIA + 3) / 4;  // 1 KB pieces of W / KG; per wave
    constexpr int NIU = C * 20 / 256, NJU = (NIU + 3) / 4;  // of the U block
    constexpr int NKG = NJA + 1, NWU = NJA + NJU;     // DMA instructions per wave and group
    // a barrier's wait leaves the instructions issued after its group in flight
    constexpr int NW = NKG + NSR + NWU;
    static_assert(C * KP % 256 == 0 && C * 20 % 256 == 0 && K <= 256, "LDS arrays must be whole 1 KB pieces");
    static_assert(NW < 64, "vector-memory count is 6 bits");
    // s_waitcnt immediates: vector-memory count n (bits 3:0 and 15:14), LDS
    // count 0 (bits 11:8), export count at its maximum
    constexpr int kWaitW = (NW & 15) | ((NW >> 4) << 14) | (7 << 4);
    constexpr int kWaitWU = (NWU & 15) | ((NWU >> 4) << 14) | (7 << 4);
    constexpr int kWait0 = 7 << 4;
    // The loader's barriers are bare: the waits each one needs are the explicit
    // ones before it, while a fenced barrier would also wait for the transfers
    // of later chunks still in flight. The empty asm statements keep the
    // compiler from moving memory accesses across the barrier.
    auto barrier = [] {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    int offA[NJA], offU[NJU];
#pragma unroll
    for (int j = 0; j < NJA; ++j) {
      const int x = 256 * min(lw + 4 * j, NIA - 1) + 4 * ll;  // float index in the padded array
      const int r = x / KP, c = x % KP;
      offA[j] = r * K + (c < K ? c : 0);
    }
#pragma unroll
    for (int j = 0; j < NJU; ++j) {
      const int x = 256 * min(lw + 4 * j, NIU - 1) + 4 * ll;
      const int r = x / 20, c = x % 20;
      offU[j] = r * V + 16 * vb + (c < 16 ? c : 0);
    }
    const int offG = ll < K / 4 ? 4 * ll : 0;  // lanes past gamma fill the array's unused tail
    auto issue_wu = [&](int cc, int b) {
      cc = cc < nch - 1 ? cc : nch - 1;
      const float* sl = slab_of(a, p0 + cc, h);
#pragma unroll
      for (int j = 0; j < NJA; ++j)
        KDA_LDS_DMA16(sl + o.w + offA[j], &sW[b][256 * min(lw + 4 * j, NIA - 1)]);
#pragma unroll
      for (int j = 0; j < NJU; ++j)
        KDA_LDS_DMA16(sl + o.u + offU[j], &sU[b][256 * min(lw + 4 * j, NIU - 1)]);
    };
    auto issue_kg = [&](int cc, int b) {
      cc = cc < nch - 1 ? cc : nch - 1;
      const float* sl = slab_of(a, p0 + cc, h);
#pragma unroll
      for (int j = 0; j < NJA; ++j)
        KDA_LDS_DMA16(sl + o.kg + offA[j], &sKG[b][256 * min(lw + 4 * j, NIA - 1)]);
      KDA_LDS_DMA16(sl + o.gam + offG, &sGam[b][0]);
    };
    if (nch > 0) {
      issue_wu(0, 0);
      issue_kg(0, 0);
      issue_wu(1, 1);
      __builtin_amdgcn_s_waitcnt(kWaitWU);  // chunk 0 has landed
      for (int cc = 0; cc < nch; ++cc) {
        const int b = cc & 1;
        barrier();  // A
        issue_kg(cc + 1, b ^ 1);
        // sST is column-major (column c at c * SP): the 4 reads of a run hit 16
        // rows x 4 column groups of distinct banks
        floatx4 rS[NSR];
#pragma unroll
        for (int m = 0; m < NSR; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) rS[m][c] = sST[(4 * (lt & 3) + c) * SP + (lt >> 2) + 64 * m];
        __builtin_amdgcn_s_waitcnt(kWaitW);  // KG and gamma of chunk cc have landed
        barrier();  // B
        float* sl = slab_of(a, p0 + cc, h);
        // with bf16 q/k/v the product kernel reads S as bf16 (its MFMA operand
        // type), so it is stored rounded, in the first half of its slab array
        if (a.bf16_qkv) {
#pragma unroll
          for (int m = 0; m < NSR; ++m)
            *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(sl + o.S) + ((lt >> 2) + 64 * m) * V + 16 * vb +
                                       4 * (lt & 3)) = to_bf16x4(rS[m]);
        } else {
#pragma unroll
          for (int m = 0; m < NSR; ++m)
            *reinterpret_cast<floatx4*>(sl + o.S + ((lt >> 2) + 64 * m) * V + 16 * vb + 4 * (lt & 3)) = rS[m];
        }
        issue_wu(cc + 2, b);
        __builtin_amdgcn_s_waitcnt(kWaitW);  // W and U of chunk cc + 1 have landed
      }
      __builtin_amdgcn_s_waitcnt(kWait0);  // no transfer outlives the wave
    }
  }
}

// ------------------------------------------------------------ state gradients
// Same layout as above, chunks in reverse: compute wave w (0..3) keeps rows of
// dS (the gradient of the state at the current chunk boundary) as
// accumulators. Three barriers per chunk: A (chunk operands and dS' published),
// B (dVn published), C (the update is done). Loader waves 4..7 copy dS' to the
// slab and stage the previous chunk's operands in two groups: KG, Aqk, dO and
// gamma after B (dO and gamma into the other of two buffers), Qg and W after
// C; each group's next loads are issued as soon as it is staged.
template <int K>
__global__ __launch_bounds__(2 * kBT) void bwd_states_bwd_kernel(BwdArgs a) {
  constexpr int V = K, KP = K + 4, CP = C + 4, NVB = V / 16, TPW = K / 64, NF = C * K / 4 / kBT;
  constexpr int NA = C * C / 4 / kBT;
  __shared__ __attribute__((aligned(16))) float sKG[C * KP], sQG[C * KP], sW[C * KP], sAq[C * CP];
  // dO, dVn and dS' transposed (column-major, rows padded by 4): with the
  // reduction index of 16-deep slice k0 ordered k0 + 4 g + s (lane group g,
  // MFMA step s), a lane reads its 4 steps' operands as one 16-byte load
  constexpr int SP = K + 4, VP = C + 4;
  __shared__ __attribute__((aligned(16))) float sdOT[2][16 * VP], sdVnT[16 * VP], sdST[16 * SP];
  __shared__ float sGam[2][K];
  const int tid = threadIdx.x;
  const int lane = tid & 63, gq = lane >> 4, xi = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the NVB workgroups of one (sequence, head) get ids congruent modulo 8: with
  // round-robin dispatch over the 8 XCDs they share one L2 for the chunk operands
  const int bid = (int)blockIdx.x, slot = bid >> 3;
  const int u = (slot / NVB) * 8 + (bid & 7), vb = slot % NVB;
  if (u >= a.nunits) return;
  const int seq = u / a.H, h = u % a.H;
  const BwdSlab& o = a.sl;
  int p0, nch;
  seq_chunks(a, seq, p0, nch);
  const int col = 16 * vb + xi;

  if (w < 4) {
    // ---------------------------------------------------------- compute waves
    floatx4 dS[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (TPW * w + t) + 4 * gq + r;
        dS[t][r] = a.d_final ? a.d_final[((size_t)u * K + row) * V + col] : 0.f;
      }
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      *reinterpret_cast<floatx4*>(sdST + xi * SP + 16 * (TPW * w + t) + 4 * gq) = dS[t];
    for (int cc = nch - 1; cc >= 0; --cc) {
      const int b = cc & 1;
      __syncthreads();  // A
      floatx4 Ob[C / 16];
#pragma unroll
      for (int q = 0; q < C / 16; ++q) Ob[q] = *reinterpret_cast<const floatx4*>(&sdOT[b][xi * VP + 16 * q + 4 * gq]);
      // dVn rows 16 w .. 16 w + 15 = Aqk^T dO + KG dS' (one accumulator chain per step s)
      {
        floatx4 Ka[K / 16], Sb[K / 16];
#pragma unroll
        for (int q = 0; q < K / 16; ++q) {
          Ka[q] = *reinterpret_cast<const floatx4*>(sKG + (16 * w + xi) * KP + 16 * q + 4 * gq);
          Sb[q] = *reinterpret_cast<const floatx4*>(sdST + xi * SP + 16 * q + 4 * gq);
        }
        floatx4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int q = 0; q < C / 16; ++q)
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc[st] = mfma4(sAq[(16 * q + 4 * gq + st) * CP + 16 * w + xi], Ob[q][st], acc[st]);
#pragma unroll
        for (int q = 0; q < K / 16; ++q)
#pragma unroll
          for (int st = 0; st < 4; ++st) acc[st] = mfma4(Ka[q][st], Sb[q][st], acc[st]);
        const floatx4 dv = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        *reinterpret_cast<floatx4*>(sdVnT + xi * VP + 16 * w + 4 * gq) = dv;
      }
      __syncthreads();  // B
      // dS = Diag(gamma) dS' + Qg^T dO - W^T dVn
      floatx4 Vb[C / 16];
#pragma unroll
      for (int q = 0; q < C / 16; ++q) Vb[q] = *reinterpret_cast<const floatx4*>(sdVnT + xi * VP + 16 * q + 4 * gq);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int rt = TPW * w + t;
#pragma unroll
        for (int r = 0; r < 4; ++r) dS[t][r] *= sGam[b][16 * rt + 4 * gq + r];
        floatx4 acc2 = zero4();
#pragma unroll
        for (int q = 0; q < C / 16; ++q)
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int k = 16 * q + 4 * gq + st;
            dS[t] = mfma4(sQG[k * KP + 16 * rt + xi], Ob[q][st], dS[t]);
            acc2 = mfma4(-sW[k * KP + 16 * rt + xi], Vb[q][st], acc2);
          }
        dS[t] += acc2;
        *reinterpret_cast<floatx4*>(sdST + xi * SP + 16 * rt + 4 * gq) = dS[t];
      }
      __syncthreads();  // C
    }
    if (a.dh0) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * (TPW * w + t) + 4 * gq + r;
          a.dh0[((size_t)u * K + row) * V + col] = dS[t][r];
        }
    }
  } else {
    // ----------------------------------------------------------- loader waves
    const int lt = tid - kBT;
    constexpr int NSC = K / 16;
    const int qf32 = !a.bf16_qkv;
    // dO block of the chunk as raw bits (fp32: four words; bf16: two words),
    // converted when it is staged
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    struct G1 {
      floatx4 kg[NF], aq[NA];
      u32x4 o32;
      u32x2 o16;
      bool ok;
      float g;
    };
    floatx4 rQG[NF], rW[NF];
    // loads are unconditional: the chunk index is clamped to 0
    auto fetch1 = [&](G1& r1, int cc) {
      cc = cc > 0 ? cc : 0;
      const float* sl = slab_of(a, p0 + cc, h);
#pragma unroll
      for (int m = 0; m < NF; ++m) r1.kg[m] = *reinterpret_cast<const floatx4*>(sl + o.kg + 4 * (lt + kBT * m));
#pragma unroll
      for (int m = 0; m < NA; ++m) r1.aq[m] = *reinterpret_cast<const floatx4*>(sl + o.aqk + 4 * (lt + kBT * m));
      const ItemB it = chunk_of(a, p0 + cc, h);
      const int r = lt >> 2, c0 = 16 * vb + 4 * (lt & 3);
      r1.ok = r < it.len;
      const size_t at = ((size_t)(it.tok0 + (r1.ok ? r : 0)) * a.H + h) * V + c0;  // row 0 is always valid
      r1.o32 = u32x4{0u, 0u, 0u, 0u};
      r1.o16 = u32x2{0u, 0u};
      if (qf32) r1.o32 = *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(a.d_o) + at);
      else r1.o16 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const bf16*>(a.d_o) + at);
      r1.g = sl[o.gam + (lt < K ? lt : 0)];
    };
    auto fetch2 = [&](int cc) {
      cc = cc > 0 ? cc : 0;
      const float* sl = slab_of(a, p0 + cc, h);
#pragma unroll
      for (int m = 0; m < NF; ++m) {
        rQG[m] = *reinterpret_cast<const floatx4*>(sl + o.qg + 4 * (lt + kBT * m));
        rW[m] = *reinterpret_cast<const floatx4*>(sl + o.w + 4 * (lt + kBT * m));
      }
    };
    auto stage1 = [&](const G1& r1, int b) {
#pragma unroll
      for (int m = 0; m < NF; ++m) {
        const int e = 4 * (lt + kBT * m), r = e / K, d = e % K;
        *reinterpret_cast<floatx4*>(sKG + r * KP + d) = r1.kg[m];
      }
#pragma unroll
      for (int m = 0; m < NA; ++m) {
        const int e = 4 * (lt + kBT * m);
        *reinterpret_cast<floatx4*>(sAq + (e / C) * CP + e % C) = r1.aq[m];
      }
      float dov[4];
      if (qf32) {
#pragma unroll
        for (int c = 0; c < 4; ++c) dov[c] = __uint_as_float(r1.o32[c]);
      } else {
        dov[0] = __uint_as_float(r1.o16[0] << 16);
        dov[1] = __uint_as_float(r1.o16[0] & 0xffff0000u);
        dov[2] = __uint_as_float(r1.o16[1] << 16);
        dov[3] = __uint_as_float(r1.o16[1] & 0xffff0000u);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) sdOT[b][(4 * (lt & 3) + c) * VP + (lt >> 2)] = r1.ok ? dov[c] : 0.f;
      if (lt < K) sGam[b][lt] = r1.g;
    };
    auto stage2 = [&]() {
#pragma unroll
      for (int m = 0; m < NF; ++m) {
        const int e = 4 * (lt + kBT * m), r = e / K, d = e % K;
        *reinterpret_cast<floatx4*>(sQG + r * KP + d) = rQG[m];
        *reinterpret_cast<floatx4*>(sW + r * KP + d) = rW[m];
      }
    };
    // group 1 has two register sets: set cur holds chunk cc - 1 at step cc and
    // is refilled with chunk cc - 3 once staged (two chunks of latency)
    auto step = [&](int cc, G1& cur) {
      __syncthreads();  // A
      float rS[NSC];
#pragma unroll
      for (int m = 0; m < NSC; ++m) rS[m] = sdST[(lt & 15) * SP + (lt >> 4) + 16 * m];
      __syncthreads();  // B
      float* sl = slab_of(a, p0 + cc, h);
#pragma unroll
      for (int m = 0; m < NSC; ++m) sl[o.dS + ((lt >> 4) + 16 * m) * V + 16 * vb + (lt & 15)] = rS[m];  // gradient of the chunk-end state
      if (cc > 0) stage1(cur, (cc - 1) & 1);
      fetch1(cur, cc - 3);
      __syncthreads();  // C
      if (cc > 0) stage2();
      fetch2(cc - 2);
    };
    if (nch > 0) {
      G1 X, Y;  // X: chunks of the parity of nch - 1, Y: the other parity
      fetch1(X, nch - 1);
      fetch2(nch - 1);
      fetch1(Y, nch - 2);
      stage1(X, (nch - 1) & 1);
      stage2();
      fetch1(X, nch - 3);
      fetch2(nch - 2);
      // step cc stages chunk cc - 1: from Y when cc = nch - 1, nch - 3, ..., from X otherwise
      for (int cc = nch - 1; cc >= 0; cc -= 2) {
        step(cc, Y);
        if (cc - 1 >= 0) step(cc - 1, X);
      }
    }
  }
}

// State gradients for bf16 q/k/v: the same recurrence, barriers and loader
// schedule as bwd_states_bwd_kernel, with the products on
// v_mfma_f32_16x16x32_bf16 (operands rounded to bf16, the input compute dtype,
// accumulation and the state dS in fp32). Every operand sits in LDS with its
// reduction index contiguous (rows padded by 8 elements): KG [c][k], Aqk^T
// [c][j], Qg^T [k][j], W^T [k][j], and dO^T, dVn^T, dS'^T [column][reduction];
// lane (g, i) supplies reduction indices 32 s + 8 g .. + 7 of row i, one 16-byte
// read per operand and step. A 16 x 16 result tile keeps the MFMA's layout (rows
// 4 g + r, column i), so dVn and dS leave as 8-byte transposed writes.
template <int K>
__global__ __launch_bounds__(2 * kBT) void bwd_states_bwd_bf16_kernel(BwdArgs a) {
  constexpr int V = K, NVB = V / 16, TPW = K / 64, NF = C * K / 4 / kBT;
  constexpr int PK = K + 8, PC = C + 8;  // bf16 row pitches
  __shared__ __attribute__((aligned(16))) bf16 sKG[C * PK], sAqT[C * PC], sQGT[K * PC], sWT[K * PC];
  __shared__ __attribute__((aligned(16))) bf16 sdOT[2][16 * PC], sdVnT[16 * PC], sdST[16 * PK];
  __shared__ float sGam[2][K];
  const int tid = threadIdx.x;
  const int lane = tid & 63, gq = lane >> 4, xi = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the NVB workgroups of one (sequence, head) get ids congruent modulo 8: with
  // round-robin dispatch over the 8 XCDs they share one L2 for the chunk operands
  const int bid = (int)blockIdx.x, slot = bid >> 3;
  const int u = (slot / NVB) * 8 + (bid & 7), vb = slot % NVB;
  if (u >= a.nunits) return;
  const int seq = u / a.H, h = u % a.H;
  const BwdSlab& o = a.sl;
  int p0, nch;
  seq_chunks(a, seq, p0, nch);
  const int col = 16 * vb + xi;

  if (w < 4) {
    // ---------------------------------------------------------- compute waves
    floatx4 dS[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (TPW * w + t) + 4 * gq + r;
        dS[t][r] = a.d_final ? a.d_final[((size_t)u * K + row) * V + col] : 0.f;
      }
      *reinterpret_cast<bf16x4*>(sdST + xi * PK + 16 * (TPW * w + t) + 4 * gq) = to_bf16x4(dS[t]);
    }
    for (int cc = nch - 1; cc >= 0; --cc) {
      const int b = cc & 1;
      __syncthreads();  // A
      // dVn rows 16 w .. 16 w + 15 = Aqk^T dO + KG dS'
      {
        floatx4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
        for (int s = 0; s < C; s += 32) {
          const bf16x8 fa = *reinterpret_cast<const bf16x8*>(sAqT + (16 * w + xi) * PC + s + 8 * gq);
          const bf16x8 fb = *reinterpret_cast<const bf16x8*>(&sdOT[b][xi * PC + s + 8 * gq]);
          acc0 = mma32(acc0, fa, fb);
        }
#pragma unroll
        for (int s = 0; s < K; s += 32) {
          const bf16x8 fa = *reinterpret_cast<const bf16x8*>(sKG + (16 * w + xi) * PK + s + 8 * gq);
          const bf16x8 fb = *reinterpret_cast<const bf16x8*>(sdST + xi * PK + s + 8 * gq);
          acc1 = mma32(acc1, fa, fb);
        }
        *reinterpret_cast<bf16x4*>(sdVnT + xi * PC + 16 * w + 4 * gq) = to_bf16x4(acc0 + acc1);
      }
      __syncthreads();  // B
      // dS = Diag(gamma) dS' + Qg^T dO - W^T dVn
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int rt = TPW * w + t;
#pragma unroll
        for (int r = 0; r < 4; ++r) dS[t][r] *= sGam[b][16 * rt + 4 * gq + r];
        floatx4 acc2 = zero4();
#pragma unroll
        for (int s = 0; s < C; s += 32) {
          const bf16x8 fq = *reinterpret_cast<const bf16x8*>(sQGT + (16 * rt + xi) * PC + s + 8 * gq);
          const bf16x8 fo = *reinterpret_cast<const bf16x8*>(&sdOT[b][xi * PC + s + 8 * gq]);
          const bf16x8 fw = *reinterpret_cast<const bf16x8*>(sWT + (16 * rt + xi) * PC + s + 8 * gq);
          const bf16x8 fv = *reinterpret_cast<const bf16x8*>(sdVnT + xi * PC + s + 8 * gq);
          dS[t] = mma32(dS[t], fq, fo);
          acc2 = mma32(acc2, fw, fv);
        }
        dS[t] -= acc2;
        *reinterpret_cast<bf16x4*>(sdST + xi * PK + 16 * rt + 4 * gq) = to_bf16x4(dS[t]);
      }
      __syncthreads();  // C
    }
    if (a.dh0) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * (TPW * w + t) + 4 * gq + r;
          a.dh0[((size_t)u * K + row) * V + col] = dS[t][r];
        }
    }
  } else {
    // ----------------------------------------------------------- loader waves
    const int lt = tid - kBT;
    constexpr int NSR = K / 64;   // runs of the dS' copy per thread
    // KG [C][K], Aqk^T [C][C], Qg^T and W^T [K][C] come from the slab already
    // in bf16 (the chunk-term kernel writes them so for bf16 inputs) and are
    // copied to LDS as 16-byte pieces: piece q = lt + 256 m of an [R][S] matrix
    // is row q / (S / 8), columns 8 (q % (S / 8)) .. + 7
    constexpr int NQP = K * C / 8 / kBT, NAP = C * C / 8 / kBT;
    static_assert(NQP * kBT == K * C / 8 && NAP * kBT == C * C / 8, "piece split");
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    struct G1 {
      u32x4 kg[NQP], aq[NAP];
      u32x2 o16;
      bool ok;
      float g;
    };
    u32x4 rQG[NQP], rW[NQP];
    // loads are unconditional: the chunk index is clamped to 0
    auto fetch1 = [&](G1& r1, int cc) {
      cc = cc > 0 ? cc : 0;
      const float* sl = slab_of(a, p0 + cc, h);
      const bf16* kgb = reinterpret_cast<const bf16*>(sl + o.vb) + K * C;
      const bf16* aqt = reinterpret_cast<const bf16*>(sl + o.dqg);
#pragma unroll
      for (int m = 0; m < NQP; ++m) r1.kg[m] = *reinterpret_cast<const u32x4*>(kgb + 8 * (lt + kBT * m));
#pragma unroll
      for (int m = 0; m < NAP; ++m) r1.aq[m] = *reinterpret_cast<const u32x4*>(aqt + 8 * (lt + kBT * m));
      const ItemB it = chunk_of(a, p0 + cc, h);
      const int r = lt >> 2, c0 = 16 * vb + 4 * (lt & 3);
      r1.ok = r < it.len;
      const size_t at = ((size_t)(it.tok0 + (r1.ok ? r : 0)) * a.H + h) * V + c0;  // row 0 is always valid
      r1.o16 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const bf16*>(a.d_o) + at);
      r1.g = sl[o.gam + (lt < K ? lt : 0)];
    };
    auto fetch2 = [&](int cc) {
      cc = cc > 0 ? cc : 0;
      const float* sl = slab_of(a, p0 + cc, h);
      const bf16* qgt = reinterpret_cast<const bf16*>(sl + o.qg);
      const bf16* wt = reinterpret_cast<const bf16*>(sl + o.vb);
#pragma unroll
      for (int m = 0; m < NQP; ++m) {
        rQG[m] = *reinterpret_cast<const u32x4*>(qgt + 8 * (lt + kBT * m));
        rW[m] = *reinterpret_cast<const u32x4*>(wt + 8 * (lt + kBT * m));
      }
    };
    auto stage1 = [&](const G1& r1, int b) {
#pragma unroll
      for (int m = 0; m < NQP; ++m) {
        const int q = lt + kBT * m;
        *reinterpret_cast<u32x4*>(sKG + (q / (K / 8)) * PK + 8 * (q % (K / 8))) = r1.kg[m];
      }
#pragma unroll
      for (int m = 0; m < NAP; ++m) {
        const int q = lt + kBT * m;
        *reinterpret_cast<u32x4*>(sAqT + (q / (C / 8)) * PC + 8 * (q % (C / 8))) = r1.aq[m];
      }
      const bf16x4 dob = r1.ok ? __builtin_bit_cast(bf16x4, r1.o16) : bf16x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; ++c) sdOT[b][(4 * (lt & 3) + c) * PC + (lt >> 2)] = dob[c];
      if (lt < K) sGam[b][lt] = r1.g;
    };
    auto stage2 = [&]() {
#pragma unroll
      for (int m = 0; m < NQP; ++m) {
        const int q = lt + kBT * m, k = q / (C / 8), j0 = 8 * (q % (C / 8));
        *reinterpret_cast<u32x4*>(sQGT + k * PC + j0) = rQG[m];
        *reinterpret_cast<u32x4*>(sWT + k * PC + j0) = rW[m];
      }
    };
    // group 1 has two register sets: set cur holds chunk cc - 1 at step cc and
    // is refilled with chunk cc - 3 once staged (two chunks of latency)
    auto step = [&](int cc, G1& cur) {
      __syncthreads();  // A
      // the gradient of the chunk-end state, as the recurrence used it (bf16),
      // to the slab as runs of four columns (rows lt / 4 + 64 m), one 8-byte
      // store per run
      bf16x4 rS[NSR];
#pragma unroll
      for (int m = 0; m < NSR; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) rS[m][c] = sdST[(4 * (lt & 3) + c) * PK + (lt >> 2) + 64 * m];
      __syncthreads();  // B
      float* sl = slab_of(a, p0 + cc, h);
#pragma unroll
      for (int m = 0; m < NSR; ++m)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(sl + o.dS) + ((lt >> 2) + 64 * m) * V + 16 * vb +
                                   4 * (lt & 3)) = rS[m];
      if (cc > 0) stage1(cur, (cc - 1) & 1);
      fetch1(cur, cc - 3);
      __syncthreads();  // C
      if (cc > 0) stage2();
      fetch2(cc - 2);
    };
    if (nch > 0) {
      G1 X, Y;  // X: chunks of the parity of nch - 1, Y: the other parity
      fetch1(X, nch - 1);
      fetch2(nch - 1);
      fetch1(Y, nch - 2);
      stage1(X, (nch - 1) & 1);
      stage2();
      fetch1(X, nch - 3);
      fetch2(nch - 2);
      // step cc stages chunk cc - 1: from Y when cc = nch - 1, nch - 3, ..., from X otherwise
      for (int cc = nch - 1; cc >= 0; cc -= 2) {
        step(cc, Y);
        if (cc - 1 >= 0) step(cc - 1, X);
      }
    }
  }
}

// ------------------------------------------------------------ chunk gradients
// pointers to the slab arrays of one (chunk, head)
struct SlabPtrs {
  float *QG, *KG, *W, *KB, *U, *VB, *AQK, *A, *Mm, *BETA, *GAM, *S, *DS, *DO, *VN, *DVN, *DVB, *DQG,
      *DW, *DKG, *DKB, *DAQK, *DA, *T1, *DL, *DGAM;
};
__device__ __forceinline__ SlabPtrs slab_ptrs(float* sl, const BwdSlab& o) {
  SlabPtrs P;
  P.QG = sl + o.qg; P.KG = sl + o.kg; P.W = sl + o.w;
  P.KB = sl + o.kb; P.U = sl + o.u; P.VB = sl + o.vb; P.AQK = sl + o.aqk; P.A = sl + o.a; P.Mm = sl + o.m;
  P.BETA = sl + o.beta; P.GAM = sl + o.gam; P.S = sl + o.S; P.DS = sl + o.dS; P.DO = sl + o.dO; P.VN = sl + o.vn;
  P.DVN = sl + o.dvn; P.DVB = sl + o.dvb; P.DQG = sl + o.dqg; P.DW = sl + o.dw; P.DKG = sl + o.dkg;
  P.DKB = sl + o.dkb; P.DAQK = sl + o.daqk;
  P.DA = sl + o.da; P.T1 = sl + o.t1; P.DL = sl + o.dl; P.DGAM = sl + o.dgam;
  return P;
}

// the matrix products of the chunk reverse step
template <int K>
__global__ __launch_bounds__(kBT) void bwd_chunk_mm_kernel(BwdArgs a) {
  constexpr int V = K;
  __shared__ __attribute__((aligned(16))) float smem[16 * (C + 4) + 16 * (K + 4)];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= items_in_use(a)) return;
  const ItemB it = chunk_of(a, (int)blockIdx.x / a.H, (int)blockIdx.x % a.H);
  const SlabPtrs P = slab_ptrs(slab_of(a, it.p, it.h), a.sl);
  const int qf32 = !a.bf16_qkv;

  {
    // dO of the chunk into the slab: all loads first (typed), then the stores
    constexpr int NE = C * V / kBT;
    float dov[NE];
    if (qf32) load_rows<float, NE, kBT, V>(a.d_o, it, a.H, dov);
    else load_rows<bf16, NE, kBT, V>(a.d_o, it, a.H, dov);
#pragma unroll
    for (int m = 0; m < NE; ++m) P.DO[tid + kBT * m] = dov[m];
  }
  if (tid < K) {
    float acc = 0.f;
#pragma unroll 16
    for (int v = 0; v < V; ++v) acc += P.S[tid * V + v] * P.DS[tid * V + v];
    P.DGAM[tid] = acc;
  }
  __syncthreads();
  // Vn = U - W S;  dVn = Aqk^T dO + KG dS'
  lds_mm<C, V, false, false>(K, P.W, K, P.S, V, smem,
                             [&](int i, int j, float x) { P.VN[i * V + j] = P.U[i * V + j] - x; });
  lds_mm<C, V, true, false>(C, P.AQK, C, P.DO, V, smem, [&](int i, int j, float x) { P.DVN[i * V + j] = x; });
  lds_mm<C, V, false, false>(K, P.KG, K, P.DS, V, smem, [&](int i, int j, float x) { P.DVN[i * V + j] += x; });
  __syncthreads();
  // dQg = dO S^T, dW = -dVn S^T, dKG = Vn dS'^T, dAqk = Tril(dO Vn^T)
  lds_mm<C, K, false, true>(V, P.DO, V, P.S, V, smem, [&](int i, int j, float x) { P.DQG[i * K + j] = x; });
  lds_mm<C, K, false, true>(V, P.DVN, V, P.S, V, smem, [&](int i, int j, float x) { P.DW[i * K + j] = -x; });
  lds_mm<C, K, false, true>(V, P.VN, V, P.DS, V, smem, [&](int i, int j, float x) { P.DKG[i * K + j] = x; });
  lds_mm<C, C, false, true>(V, P.DO, V, P.VN, V, smem,
                            [&](int i, int j, float x) { P.DAQK[i * C + j] = j <= i ? x : 0.f; });
  __syncthreads();
  // dA = dW Kb^T + dVn Vb^T;  dKb = A^T dW;  dVb = A^T dVn
  lds_mm<C, C, false, true>(K, P.DW, K, P.KB, K, smem, [&](int i, int j, float x) { P.DA[i * C + j] = x; });
  lds_mm<C, C, false, true>(V, P.DVN, V, P.VB, V, smem, [&](int i, int j, float x) { P.DA[i * C + j] += x; });
  lds_mm<C, K, true, false>(C, P.A, C, P.DW, K, smem, [&](int i, int j, float x) { P.DKB[i * K + j] = x; });
  lds_mm<C, V, true, false>(C, P.A, C, P.DVN, V, smem, [&](int i, int j, float x) { P.DVB[i * V + j] = x; });
  __syncthreads();
  // dL = -StrictTril(A^T dA A^T)
  lds_mm<C, C, true, false>(C, P.A, C, P.DA, C, smem, [&](int i, int j, float x) { P.T1[i * C + j] = x; });
  __syncthreads();
  lds_mm<C, C, false, true>(C, P.T1, C, P.A, C, smem,
                            [&](int i, int j, float x) { P.DL[i * C + j] = j < i ? -x : 0.f; });
}

// The four gated sums of the chunk reverse step (per row i, channel d; P = dAqk,
// dM = Diag(beta) dL, E_ij = exp(G_i - G_j))
//   query side  sum_{j<=i} P_ij k_j E_ij,   sum_{j<i} dM_ij k_j E_ij
//   key side    sum_{r>=i} P_ri q_r E_ri,   sum_{r>i} dM_ri k_r E_ri
// as fp32 MFMA products over 16-row blocks with one reference per block (the
// rebasing of "KDA Doesn't Care About the Future", section "The rebasing
// trick"): with rho_b = G of the first row of block b, a key j of block b
// carries exp(rho_b - G_j) (at most 15 steps of decay) and the query row
// exp(G_i - rho_b) <= 1 for i >= 16 b; the key side uses the reference of row
// i's own block the same way. For the 16 x 16 tile (row block ib, channel
// d = 16 ct + xi) of lane (gq, xi): qa, qm, ka, km hold rows 16 ib + 4 gq + r.
// LDS operands in fp32: G, k^, q^ as [C][K]; P and dM as [C][C + 4].
template <int K>
__device__ __forceinline__ void gated_sums(const float* sG, const float* sKN, const float* sQN, const float* sP,
                                           const float* sDM, int ib, int d, int gq, int xi, floatx4& qa,
                                           floatx4& qm, floatx4& ka, floatx4& km) {
  constexpr int CP = C + 4;
  qa = zero4(); qm = zero4(); ka = zero4(); km = zero4();
  // query side: key blocks b <= ib
  for (int b = 0; b <= ib; ++b) {
    const float rho = sG[(16 * b) * K + d];
    floatx4 accA = zero4(), accM = zero4();
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4) {
      const int j = 16 * b + k0 + gq;
      const float kf = sKN[j * K + d] * __expf(rho - sG[j * K + d]);
      accA = mfma4(sP[(16 * ib + xi) * CP + j], kf, accA);
      accM = mfma4(sDM[(16 * ib + xi) * CP + j], kf, accM);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = __expf(sG[(16 * ib + 4 * gq + r) * K + d] - rho);
      qa[r] += e * accA[r];
      qm[r] += e * accM[r];
    }
  }
  // key side: query blocks b >= ib, reference of block ib
  {
    const float rho = sG[(16 * ib) * K + d];
    for (int b = ib; b < 4; ++b) {
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const int r = 16 * b + k0 + gq;
        const float e = __expf(sG[r * K + d] - rho);
        ka = mfma4(sP[r * CP + 16 * ib + xi], sQN[r * K + d] * e, ka);
        km = mfma4(sDM[r * CP + 16 * ib + xi], sKN[r * K + d] * e, km);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float f = __expf(rho - sG[(16 * ib + 4 * gq + r) * K + d]);
      ka[r] *= f;
      km[r] *= f;
    }
  }
}

// the elementwise rules of element (row i, channel d): the gradients of the
// normalised q and k and of G (before the reverse cumsum), from dQg, dKb, dKG
// and the four gated sums; Qg = s q e^G, Kb = beta k e^G and KG = k e^(Gl - G)
// are rebuilt from the staged rows
template <int K>
__device__ __forceinline__ void elem_rules(const float* sG, const float* sQN, const float* sKN, const float* sBeta,
                                           const float* sDGl, int i, int d, float s, float dqg, float dkb, float dkg,
                                           float qa, float qm, float ka, float km, float& gqn, float& gkn,
                                           float& dG) {
  const float Gi = sG[i * K + d], qi = sQN[i * K + d], ki = sKN[i * K + d], bi = sBeta[i];
  const float Gl = sG[(C - 1) * K + d];
  const float eg = __expf(Gi), egl = __expf(Gl - Gi);
  gqn = s * eg * dqg + s * qa;
  gkn = dkb * bi * eg + dkg * egl + s * ka + qm + km;
  dG = dqg * (s * qi * eg) + dkb * (bi * ki * eg) - dkg * (ki * egl) + qi * s * qa - ki * s * ka + ki * qm - ki * km;
  if (i == C - 1) dG += sDGl[d];
}

// ----------------------------- chunk gradients, fused, on MFMA (bf16 input)
// With bf16 q, k, v (and dO) the products above run on v_mfma_f32_16x16x32_bf16:
// every operand is rounded to bf16 (the input compute dtype, as in the forward's
// bf16 path) and every product accumulates in fp32. One workgroup (8 waves) per
// (chunk, head) keeps all operands and intermediates of the item on chip, reads
// each slab array once and writes only the gradients: Vn, dVn, dW, dA and T1
// stay in LDS, and dQg, dKb, dKG, dAqk, dL stay in registers for the
// elementwise phase that follows the products in the same workgroup.
//
// An operand matrix sits in LDS with its reduction index contiguous: the
// A operand as [output row][reduction], the B operand as [output column]
// [reduction], rows padded by 8 elements (16 bytes) so that the 16 rows read by
// one b128 access fall into distinct banks. Lane (g, i) supplies reduction
// indices 32 s + 8 g .. + 7 of row i in step s, for both operands. Products
// that leave their result as an A operand, or in global memory, are issued with
// the operands swapped (lane (g, i) then holds row i, columns 4 g .. 4 g + 3 of
// the result); the others keep the MFMA's own layout (rows 4 g .. 4 g + 3,
// column i), which stores transposed with one 8-byte write per lane.
//
// Phases (operands staged from registers loaded one or more phases earlier):
//   1  Vn = U - W S                               (W, S^T)
//   2  dVn = Aqk^T dO + KG dS'                    (Aqk^T, dO^T, KG, dS'^T)
//   3  dKG = Vn dS'^T;  dgamma = rowsum(S * dS')  (dS')
//   4  dQg = dO S^T, dW = -dVn S^T, dAqk = Tril(dO Vn^T)   (dO, S)
//   5  dA = dW Kb^T + dVn Vb^T, dKb = A^T dW, dVb = A^T dVn (Kb, Vb, A^T)
//   6  T1 = A^T dA                                (A staged for phase 7)
//   7  dL = -StrictTril(T1 A^T)
//   then the elementwise phase: gated sums and rules per tile of the C x K
//   tiling, dq, dk, dg, dv, dbeta
constexpr int kMT = 512;  // threads of the fused kernel

// output tiles of an M x N product over 8 waves: each wave a BM x BN block of
// 16 x 16 tiles
template <int M, int N>
struct MTiles {
  static constexpr int TM = M / 16, TN = N / 16, TPW = TM * TN / 8;
  static constexpr int BM = TPW >= 4 ? 2 : 1, BN = TPW / BM, WC = TN / BN;
  static_assert(BM * BN == TPW && (TM / BM) * WC == 8, "8 waves of whole tile blocks");
  __device__ static int r0(int w) { return 16 * BM * (w / WC); }
  __device__ static int c0(int w) { return 16 * BN * (w % WC); }
};

// acc[bm][bn] += sum over R reduction indices of A-row x B-row, for the wave's
// tile block at (r0, c0); SWAP issues the MFMA with the operands exchanged
template <int BM, int BN, int R, bool SWAP>
__device__ __forceinline__ void mfma_rows(floatx4 (&acc)[BM][BN], const bf16* A, int lda, const bf16* B, int ldb,
                                          int r0, int c0, int lane) {
  const int g = lane >> 4, i = lane & 15;
#pragma unroll
  for (int s = 0; s < R; s += 32) {
    bf16x8 fa[BM], fb[BN];
#pragma unroll
    for (int bm = 0; bm < BM; ++bm) fa[bm] = *reinterpret_cast<const bf16x8*>(A + (r0 + 16 * bm + i) * lda + s + 8 * g);
#pragma unroll
    for (int bn = 0; bn < BN; ++bn) fb[bn] = *reinterpret_cast<const bf16x8*>(B + (c0 + 16 * bn + i) * ldb + s + 8 * g);
#pragma unroll
    for (int bm = 0; bm < BM; ++bm)
#pragma unroll
      for (int bn = 0; bn < BN; ++bn)
        acc[bm][bn] = SWAP ? mma32(acc[bm][bn], fb[bn], fa[bm]) : mma32(acc[bm][bn], fa[bm], fb[bn]);
  }
}

template <int BM, int BN>
__device__ __forceinline__ void zero_acc(floatx4 (&acc)[BM][BN]) {
#pragma unroll
  for (int bm = 0; bm < BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < BN; ++bn) acc[bm][bn] = zero4();
}


// fp32 [ROWS][COLS] matrix (row-major, global) <-> registers, 4 consecutive
// elements per access; thread t takes groups t, t + kMT, ...
template <int ROWS, int COLS>
struct NatStage {
  static constexpr int N = ROWS * COLS / 4 / kMT;
  static_assert(N >= 1 && N * 4 * kMT == ROWS * COLS, "whole groups per thread");
  floatx4 v[N];
  __device__ void load(const float* src) {
#pragma unroll
    for (int m = 0; m < N; ++m) {
      const int e = (int)threadIdx.x + kMT * m, row = e / (COLS / 4), c = 4 * (e % (COLS / 4));
      v[m] = *reinterpret_cast<const floatx4*>(src + row * COLS + c);
    }
  }
  // bf16 [ROWS][COLS + 8] in LDS
  __device__ void store(bf16* dst) const {
#pragma unroll
    for (int m = 0; m < N; ++m) {
      const int e = (int)threadIdx.x + kMT * m, row = e / (COLS / 4), c = 4 * (e % (COLS / 4));
      *reinterpret_cast<bf16x4*>(dst + row * (COLS + 8) + c) = to_bf16x4(v[m]);
    }
  }
};

// bf16 [ROWS][COLS] matrix as 16-byte pieces: piece q = t + kMT m is row
// q / (COLS / 8), columns 8 (q % (COLS / 8)) .. + 7; copied to LDS with rows
// padded to COLS + 8
template <int ROWS, int COLS>
struct PieceStage {
  static constexpr int N = ROWS * COLS / 8 / kMT;
  static_assert(N >= 1 && N * 8 * kMT == ROWS * COLS, "whole pieces per thread");
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v[N];
  __device__ void load(const bf16* src) {
#pragma unroll
    for (int m = 0; m < N; ++m) v[m] = *reinterpret_cast<const u32x4*>(src + 8 * ((int)threadIdx.x + kMT * m));
  }
  __device__ void store(bf16* dst) const {
#pragma unroll
    for (int m = 0; m < N; ++m) {
      const int q = (int)threadIdx.x + kMT * m;
      *reinterpret_cast<u32x4*>(dst + (q / (COLS / 8)) * (COLS + 8) + 8 * (q % (COLS / 8))) = v[m];
    }
  }
};

// fp32 [ROWS][COLS] matrix in 4 x 4 blocks: block b = t + kMT m holds rows
// 4 (b / (COLS / 4)) + r, columns 4 (b % (COLS / 4)) .. + 3 in v[m][r]; stored
// to LDS either as is or transposed ([COLS][ROWS + 8])
template <int ROWS, int COLS>
struct BlkStage {
  static constexpr int NB = (ROWS / 4) * (COLS / 4);
  static constexpr int N = (NB + kMT - 1) / kMT;
  floatx4 v[N][4];
  __device__ static bool has(int m) { return NB % kMT == 0 || (int)threadIdx.x + kMT * m < NB; }
  __device__ static int brow(int m) { return 4 * (((int)threadIdx.x + kMT * m) / (COLS / 4)); }
  __device__ static int bcol(int m) { return 4 * (((int)threadIdx.x + kMT * m) % (COLS / 4)); }
  __device__ void load(const float* src) {
#pragma unroll
    for (int m = 0; m < N; ++m)
      if (has(m)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[m][r] = *reinterpret_cast<const floatx4*>(src + (brow(m) + r) * COLS + bcol(m));
      }
  }
  // the same blocks from a bf16 [ROWS][COLS] matrix, widened
  __device__ void load(const bf16* src) {
#pragma unroll
    for (int m = 0; m < N; ++m)
      if (has(m)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[m][r] = load4_f32(src + (brow(m) + r) * COLS + bcol(m));
      }
  }
  __device__ void store(bf16* dst) const {
#pragma unroll
    for (int m = 0; m < N; ++m)
      if (has(m)) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<bf16x4*>(dst + (brow(m) + r) * (COLS + 8) + bcol(m)) = to_bf16x4(v[m][r]);
      }
  }
  __device__ void store_t(bf16* dst) const {
#pragma unroll
    for (int m = 0; m < N; ++m)
      if (has(m)) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<bf16x4*>(dst + (bcol(m) + c) * (ROWS + 8) + brow(m)) =
              to_bf16x4(floatx4{v[m][0][c], v[m][1][c], v[m][2][c], v[m][3][c]});
      }
  }
};

template <int K>
__global__ __launch_bounds__(kMT) void bwd_chunk_fused_kernel(BwdArgs a) {
  constexpr int V = K;
  constexpr int PK = K + 8, PC = C + 8;      // LDS row pitches of the bf16 operands (elements)
  constexpr int CK = C * PK, KK = K * PK, KC = K * PC, CCS = C * PC;  // matrix sizes (elements)
  // LDS plan of the product phases (bf16 elements): Vn, dVn, dVn^T stay from
  // their phase to their last use; the operand area Q is re-laid out per phase;
  // dA^T, T1 and A reuse the space of Vn and dVn once those are dead
  constexpr int oVn = 0, odVn = CK, odVnT = 2 * CK, oQ = 2 * CK + KC;
  constexpr int oW = oQ, oST = oQ + CK;                                        // phase 1
  constexpr int oAqT = oQ, odOT = oQ + CCS, oKG = odOT + KC, odST = oKG + CK;  // phase 2
  constexpr int odS = oQ;                                                      // phase 3
  constexpr int odW = oQ, odWT = oQ + CK, odO = odWT + KC, oS = odO + CK;      // phase 4
  constexpr int oKb = odO, oVb = oKb + CK, oAT = oVb + CK;                     // phase 5
  constexpr int odAT = 0, oT1 = CCS, oA = 2 * CCS;                             // phases 5-7
  constexpr int kMM = (oS + KK > oAT + CCS ? oS + KK : oAT + CCS) > odST + KK
                          ? (oS + KK > oAT + CCS ? oS + KK : oAT + CCS)
                          : odST + KK;
  static_assert(oA + CCS <= odVnT + KC, "LDS plan");
  static_assert(oT1 + CCS <= oQ && odAT + CCS <= odVn, "phase 5-7 results over dead matrices");
  // the elementwise phase lays the same memory out as fp32: G, k^, q^ [C][K],
  // dAqk and Diag(beta) dL [C][C + 4], per channel tile row dots, 16-row block
  // totals of dG and the per wave row partial column sums of dKG * KG
  using TCV = MTiles<C, V>;   // C x V and C x K results (K == V)
  using TCC = MTiles<C, C>;
  constexpr int CP = C + 4, NCT = K / 16;
  constexpr int WRV = 8 / TCV::WC;            // wave rows of the C x K tiling
  constexpr int fG = 0, fKN = C * K, fQN = 2 * C * K, fP = 3 * C * K, fDM = fP + C * CP, fDotP = fDM + C * CP,
                fBT = fDotP + NCT * 2 * C, fDGlP = fBT + 4 * K, kEF = fDGlP + WRV * K;
  constexpr int kBytes = (2 * kMM > 4 * kEF ? 2 * kMM : 4 * kEF);
  __shared__ __attribute__((aligned(16))) char lds[kBytes];
  bf16* smem = reinterpret_cast<bf16*>(lds);
  float* sF = reinterpret_cast<float*>(lds);
  // dbeta partial sums per row: dVb . v per wave column of the C x V tiling,
  // dKb . (k^ e^G) likewise, and dL . M per wave column of the C x C tiling
  constexpr int kDbSlots = 2 * TCV::WC + TCC::WC;
  __shared__ float sBeta[C], sDot[2 * C], sDGl[K], sDgam[K], sDbP[kDbSlots * C];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i = lane & 15;
  if ((int)blockIdx.x >= items_in_use(a)) return;
  const ItemB it = chunk_of(a, (int)blockIdx.x / a.H, (int)blockIdx.x % a.H);
  float* sl = slab_of(a, it.p, it.h);
  const BwdSlab& o = a.sl;
  const SlabPtrs P = slab_ptrs(sl, o);
  const int H = a.H;
  const int r0v = TCV::r0(w), c0v = TCV::c0(w), r0c = TCC::r0(w), c0c = TCC::c0(w);

  floatx4 acc[TCV::BM][TCV::BN];
  floatx4 acc2[TCC::BM][TCC::BN];
  // results kept in registers for the elementwise phase, in the MFMA's own
  // layout (lane (g, i): rows 4 g + r, column i of each 16 x 16 tile), which is
  // the layout of its tiles: dQg, dKb, dKG over the C x K tiling; dAqk and dL
  // with rows i, columns 4 g + r over the C x C tiling
  floatx4 kQG[TCV::BM][TCV::BN], kKB[TCV::BM][TCV::BN], kKG[TCV::BM][TCV::BN];
  floatx4 kAQ[TCC::BM][TCC::BN], kDL[TCC::BM][TCC::BN];

  // ---- loads of phase 1, and the state S (kept in registers until phase 4)
  NatStage<C, K> rW;
  BlkStage<K, V> rS;
  rW.load(P.W);
  rS.load(reinterpret_cast<const bf16*>(P.S));
  floatx4 rU[TCV::BM][TCV::BN];
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCV::BN; ++bn)
      rU[bm][bn] = *reinterpret_cast<const floatx4*>(P.U + (r0v + 16 * bm + i) * V + c0v + 16 * bn + 4 * g);

  // loads of phase 2, issued with those of phase 1: Aqk, dO (bf16 rows of the
  // chunk; rows past its end are zeroed where they are staged), KG, dS'
  // Aqk^T and KG come from their bf16 copies in the slab (the chunk-term kernel
  // writes them for the state-gradient pass): the same values this kernel would
  // round to bf16 itself
  PieceStage<C, C> rAq;
  rAq.load(reinterpret_cast<const bf16*>(P.DQG));
  constexpr int NDO = (C / 4) * (V / 4), PDO = (NDO + kMT - 1) / kMT;
  bf16x4 rdO[PDO][4];
  auto do_has = [&](int m) { return NDO % kMT == 0 || tid + kMT * m < NDO; };
  auto do_row = [&](int m) { return 4 * ((tid + kMT * m) / (V / 4)); };
  auto do_col = [&](int m) { return 4 * ((tid + kMT * m) % (V / 4)); };
  auto do_val = [&](int m, int r) { return do_row(m) + r < it.len ? rdO[m][r] : bf16x4{0, 0, 0, 0}; };
  {
    const bf16* dO = reinterpret_cast<const bf16*>(a.d_o);
#pragma unroll
    for (int m = 0; m < PDO; ++m)
      if (do_has(m)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = do_row(m) + r, rr = row < it.len ? row : 0;
          rdO[m][r] = *reinterpret_cast<const bf16x4*>(dO + ((size_t)(it.tok0 + rr) * H + it.h) * V + do_col(m));
        }
      }
  }
  PieceStage<C, K> rKG;
  rKG.load(reinterpret_cast<const bf16*>(P.VB) + K * C);
  BlkStage<K, V> rdS;
  rdS.load(reinterpret_cast<const bf16*>(P.DS));

  // ---- phase 1: Vn = U - W S
  rW.store(smem + oW);
  rS.store_t(smem + oST);
  __syncthreads();
  zero_acc(acc);
  mfma_rows<TCV::BM, TCV::BN, K, true>(acc, smem + oW, PK, smem + oST, PK, r0v, c0v, lane);
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCV::BN; ++bn)
      *reinterpret_cast<bf16x4*>(smem + oVn + (r0v + 16 * bm + i) * PK + c0v + 16 * bn + 4 * g) =
          to_bf16x4(rU[bm][bn] - acc[bm][bn]);
  __syncthreads();

  // ---- phase 2: dVn = Aqk^T dO + KG dS'
  rAq.store(smem + oAqT);
#pragma unroll
  for (int m = 0; m < PDO; ++m)
    if (do_has(m)) {
      const bf16x4 d0 = do_val(m, 0), d1 = do_val(m, 1), d2 = do_val(m, 2), d3 = do_val(m, 3);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<bf16x4*>(smem + odOT + (do_col(m) + c) * PC + do_row(m)) = bf16x4{d0[c], d1[c], d2[c], d3[c]};
    }
  rKG.store(smem + oKG);
  rdS.store_t(smem + odST);
  // loads of phase 5: Kb, and Vb = beta v rebuilt from the inputs as the
  // chunk-term kernel builds it (rows past the chunk end are zero), and A
  NatStage<C, K> rKb, rVb;
  rKb.load(P.KB);
  {
    const bf16* vin = reinterpret_cast<const bf16*>(a.v);
#pragma unroll
    for (int m = 0; m < NatStage<C, V>::N; ++m) {
      const int e = tid + kMT * m, row = e / (V / 4), c = 4 * (e % (V / 4)), rr = row < it.len ? row : 0;
      const floatx4 vv = widen4(*reinterpret_cast<const bf16x4*>(vin + ((size_t)(it.tok0 + rr) * H + it.h) * V + c));
      rVb.v[m] = row < it.len ? P.BETA[row] * vv : zero4();
    }
  }
  BlkStage<C, C> rA;
  rA.load(P.A);
  __syncthreads();
  zero_acc(acc);
  mfma_rows<TCV::BM, TCV::BN, C, false>(acc, smem + oAqT, PC, smem + odOT, PC, r0v, c0v, lane);
  mfma_rows<TCV::BM, TCV::BN, K, false>(acc, smem + oKG, PK, smem + odST, PK, r0v, c0v, lane);
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCV::BN; ++bn) {
      const int R0 = r0v + 16 * bm, C0 = c0v + 16 * bn;
      const bf16x4 y = to_bf16x4(acc[bm][bn]);
      *reinterpret_cast<bf16x4*>(smem + odVnT + (C0 + i) * PC + R0 + 4 * g) = y;
#pragma unroll
      for (int r = 0; r < 4; ++r) smem[odVn + (R0 + 4 * g + r) * PK + C0 + i] = y[r];
    }
  __syncthreads();

  // ---- phase 3: dKG = Vn dS'^T (kept), dgamma = rowsum(S * dS')
  rdS.store(smem + odS);
#pragma unroll
  for (int m = 0; m < BlkStage<K, V>::N; ++m) {
    floatx4 part = zero4();
    if (BlkStage<K, V>::has(m)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const floatx4 pr = rS.v[m][r] * rdS.v[m][r];
        part[r] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
      }
    }
    // the V / 4 lanes of one block row are consecutive (V / 4 divides 64)
#pragma unroll
    for (int off = 1; off < V / 4; off <<= 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[r] += __shfl_xor(part[r], off, 64);
    if (BlkStage<K, V>::has(m) && BlkStage<K, V>::bcol(m) == 0)
      *reinterpret_cast<floatx4*>(sDgam + BlkStage<K, V>::brow(m)) = part;
  }
  __syncthreads();
  zero_acc(kKG);
  mfma_rows<TCV::BM, TCV::BN, V, false>(kKG, smem + oVn, PK, smem + odS, PK, r0v, c0v, lane);
  __syncthreads();

  // ---- phase 4: dQg = dO S^T (kept), dW = -dVn S^T, dAqk = Tril(dO Vn^T) (kept)
#pragma unroll
  for (int m = 0; m < PDO; ++m)
    if (do_has(m)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) *reinterpret_cast<bf16x4*>(smem + odO + (do_row(m) + r) * PK + do_col(m)) = do_val(m, r);
    }
  rS.store(smem + oS);
  // v in the C x V tiling's layout, for the dbeta term of dVb in phase 5, and
  // beta of the tiling's rows, for dv
  float vt[TCV::BM][TCV::BN][4], bta[TCV::BM][4];
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
    for (int r = 0; r < 4; ++r) bta[bm][r] = P.BETA[r0v + 16 * bm + 4 * g + r];
  {
    const bf16* vin = reinterpret_cast<const bf16*>(a.v);
#pragma unroll
    for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
      for (int bn = 0; bn < TCV::BN; ++bn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0v + 16 * bm + 4 * g + r, rr = row < it.len ? row : 0;
          const float x = to_f32(vin[((size_t)(it.tok0 + rr) * H + it.h) * V + c0v + 16 * bn + i]);
          vt[bm][bn][r] = row < it.len ? x : 0.f;
        }
  }
  __syncthreads();
  zero_acc(kQG);
  mfma_rows<TCV::BM, TCV::BN, V, false>(kQG, smem + odO, PK, smem + oS, PK, r0v, c0v, lane);
  zero_acc(acc);
  mfma_rows<TCV::BM, TCV::BN, V, false>(acc, smem + odVn, PK, smem + oS, PK, r0v, c0v, lane);
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCV::BN; ++bn) {
      const int R0 = r0v + 16 * bm, C0 = c0v + 16 * bn;
      const bf16x4 y = to_bf16x4(-acc[bm][bn]);
      *reinterpret_cast<bf16x4*>(smem + odWT + (C0 + i) * PC + R0 + 4 * g) = y;
#pragma unroll
      for (int r = 0; r < 4; ++r) smem[odW + (R0 + 4 * g + r) * PK + C0 + i] = y[r];
    }
  zero_acc(kAQ);
  mfma_rows<TCC::BM, TCC::BN, V, true>(kAQ, smem + odO, PK, smem + oVn, PK, r0c, c0c, lane);
#pragma unroll
  for (int bm = 0; bm < TCC::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCC::BN; ++bn) {
      const int row = r0c + 16 * bm + i, col = c0c + 16 * bn + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) kAQ[bm][bn][r] = col + r <= row ? kAQ[bm][bn][r] : 0.f;
    }
  __syncthreads();

  // ---- phase 5: dA = dW Kb^T + dVn Vb^T (kept as dA^T), dKb = A^T dW (kept),
  // dVb = A^T dVn -> dv = beta dVb and the dbeta term dVb . v
  rKb.store(smem + oKb);
  rVb.store(smem + oVb);
  rA.store_t(smem + oAT);
  __syncthreads();
  zero_acc(acc2);
  mfma_rows<TCC::BM, TCC::BN, K, false>(acc2, smem + odW, PK, smem + oKb, PK, r0c, c0c, lane);
  mfma_rows<TCC::BM, TCC::BN, V, false>(acc2, smem + odVn, PK, smem + oVb, PK, r0c, c0c, lane);
#pragma unroll
  for (int bm = 0; bm < TCC::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCC::BN; ++bn)
      *reinterpret_cast<bf16x4*>(smem + odAT + (c0c + 16 * bn + i) * PC + r0c + 16 * bm + 4 * g) =
          to_bf16x4(acc2[bm][bn]);
  zero_acc(kKB);
  mfma_rows<TCV::BM, TCV::BN, C, false>(kKB, smem + oAT, PC, smem + odWT, PC, r0v, c0v, lane);
  zero_acc(acc);
  mfma_rows<TCV::BM, TCV::BN, C, false>(acc, smem + oAT, PC, smem + odVnT, PC, r0v, c0v, lane);
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm) {
    floatx4 part = zero4();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0v + 16 * bm + 4 * g + r;
      const float b = bta[bm][r];
#pragma unroll
      for (int bn = 0; bn < TCV::BN; ++bn) {
        part[r] += acc[bm][bn][r] * vt[bm][bn][r];
        if (row < it.len) a.dv[((size_t)(it.tok0 + row) * H + it.h) * V + c0v + 16 * bn + i] = b * acc[bm][bn][r];
      }
    }
    // over the 16 columns of each tile (lanes i of one group g)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[r] += __shfl_xor(part[r], off, 64);
    if (i == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) sDbP[(w % TCV::WC) * C + r0v + 16 * bm + 4 * g + r] = part[r];
  }
  __syncthreads();

  // ---- phase 6: T1 = A^T dA (A staged for phase 7 over dead dVn / dVn^T);
  // loads of the elementwise phase: q, k, g rows (zero past the chunk end) and
  // the row norms
  constexpr int N4 = C * K / 4 / kMT;
  static_assert(N4 >= 1 && N4 * 4 * kMT == C * K, "staging split");
  floatx4 rq4[N4], rk4[N4], rg4[N4];
  float qinv[N4], kinv[N4];
  {
    auto in_idx = [&](int m) {
      const int e = tid + kMT * m, row = e / (K / 4), c = 4 * (e % (K / 4)), rr = row < it.len ? row : 0;
      return ((size_t)(it.tok0 + rr) * H + it.h) * K + c;
    };
#pragma unroll
    for (int m = 0; m < N4; ++m) {
      rq4[m] = load4_f32(reinterpret_cast<const bf16*>(a.q) + in_idx(m));
      rk4[m] = load4_f32(reinterpret_cast<const bf16*>(a.k) + in_idx(m));
    }
    if (a.g_f32) {
#pragma unroll
      for (int m = 0; m < N4; ++m) rg4[m] = load4_f32(reinterpret_cast<const float*>(a.g) + in_idx(m));
    } else {
#pragma unroll
      for (int m = 0; m < N4; ++m) rg4[m] = load4_f32(reinterpret_cast<const bf16*>(a.g) + in_idx(m));
    }
#pragma unroll
    for (int m = 0; m < N4; ++m) {
      const int row = (tid + kMT * m) / (K / 4);
      qinv[m] = a.l2norm ? sl[o.nq + row] : 1.f;   // row norms; inverted when staged
      kinv[m] = a.l2norm ? sl[o.nk + row] : 1.f;
    }
  }
  // and the elementwise phase's slab operands: M and beta over the C x C
  // tiling, KG over the C x K tiling, beta of row tid, gamma of channel tid - K
  floatx4 rMm[TCC::BM][TCC::BN];
  float bdl[TCC::BM], rKGt[TCV::BM][TCV::BN][4];
#pragma unroll
  for (int bm = 0; bm < TCC::BM; ++bm) {
    bdl[bm] = P.BETA[r0c + 16 * bm + i];
#pragma unroll
    for (int bn = 0; bn < TCC::BN; ++bn)
      rMm[bm][bn] = *reinterpret_cast<const floatx4*>(P.Mm + (r0c + 16 * bm + i) * C + c0c + 16 * bn + 4 * g);
  }
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCV::BN; ++bn)
#pragma unroll
      for (int r = 0; r < 4; ++r) rKGt[bm][bn][r] = P.KG[(r0v + 16 * bm + 4 * g + r) * K + c0v + 16 * bn + i];
  const float rbeta0 = tid < C ? P.BETA[tid] : 0.f;
  const float rgam = tid >= K && tid < 2 * K ? P.GAM[tid - K] : 0.f;
  rA.store(smem + oA);
  zero_acc(acc2);
  mfma_rows<TCC::BM, TCC::BN, C, true>(acc2, smem + oAT, PC, smem + odAT, PC, r0c, c0c, lane);
#pragma unroll
  for (int bm = 0; bm < TCC::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCC::BN; ++bn)
      *reinterpret_cast<bf16x4*>(smem + oT1 + (r0c + 16 * bm + i) * PC + c0c + 16 * bn + 4 * g) =
          to_bf16x4(acc2[bm][bn]);
  __syncthreads();

  // ---- phase 7: dL = -StrictTril(T1 A^T) (kept)
  zero_acc(kDL);
  mfma_rows<TCC::BM, TCC::BN, C, true>(kDL, smem + oT1, PC, smem + oA, PC, r0c, c0c, lane);
#pragma unroll
  for (int bm = 0; bm < TCC::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCC::BN; ++bn) {
      const int row = r0c + 16 * bm + i, col = c0c + 16 * bn + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) kDL[bm][bn][r] = col + r < row ? -kDL[bm][bn][r] : 0.f;
    }
  __syncthreads();

  // ---- elementwise phase (the LDS now holds the fp32 layout)
  float* sG = sF + fG;
  float* sKN = sF + fKN;
  float* sQN = sF + fQN;
  float* sP = sF + fP;
  float* sDM = sF + fDM;
  float* sDotP = sF + fDotP;   // [NCT][2 C]
  float* sBT = sF + fBT;       // [4][K]
  float* sDGlP = sF + fDGlP;   // [WRV][K]
#pragma unroll
  for (int m = 0; m < N4; ++m) {
    const int e = tid + kMT * m, row = e / (K / 4);
    const bool in = row < it.len;
    const float qi = 1.f / fmaxf(qinv[m], a.l2eps), ki = 1.f / fmaxf(kinv[m], a.l2eps);
    reinterpret_cast<floatx4*>(sQN)[e] = in ? (a.l2norm ? rq4[m] * qi : rq4[m]) : zero4();
    reinterpret_cast<floatx4*>(sKN)[e] = in ? (a.l2norm ? rk4[m] * ki : rk4[m]) : zero4();
    reinterpret_cast<floatx4*>(sG)[e] = in ? rg4[m] : zero4();
  }
  if (tid < C) sBeta[tid] = rbeta0;
  // dAqk and Diag(beta) dL (rows i, columns 4 g + r of each tile); the dbeta
  // term dL . M over the lane's columns, then the tile's lane groups
#pragma unroll
  for (int bm = 0; bm < TCC::BM; ++bm) {
    const int row = r0c + 16 * bm + i;
    const float b = bdl[bm];
    float part = 0.f;
#pragma unroll
    for (int bn = 0; bn < TCC::BN; ++bn) {
      const int col = c0c + 16 * bn + 4 * g;
      const floatx4 mm = rMm[bm][bn];
      *reinterpret_cast<floatx4*>(sP + row * CP + col) = kAQ[bm][bn];
      *reinterpret_cast<floatx4*>(sDM + row * CP + col) = b * kDL[bm][bn];
#pragma unroll
      for (int r = 0; r < 4; ++r) part += kDL[bm][bn][r] * mm[r];
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (g == 0) sDbP[(2 * TCV::WC + w % TCC::WC) * C + row] = part;
  }
  // column sums of dKG * KG over the wave's rows (for the gradient of the last
  // row's cumulative gate), per wave row of the C x K tiling
#pragma unroll
  for (int bn = 0; bn < TCV::BN; ++bn) {
    const int col = c0v + 16 * bn + i;
    float part = 0.f;
#pragma unroll
    for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
      for (int r = 0; r < 4; ++r) part += kKG[bm][bn][r] * rKGt[bm][bn][r];
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (g == 0) sDGlP[(w / TCV::WC) * K + col] = part;
  }
  __syncthreads();
  // gate cumsum in place, sequential over the rows of each channel (bitwise the
  // chunk-term kernel's G); the last row's gate gradient from its parts
  if (tid < K) {
    float run = 0.f;
    for (int r = 0; r < C; ++r) {
      run += sG[r * K + tid];
      sG[r * K + tid] = run;
    }
  } else if (tid < 2 * K) {
    const int d = tid - K;
    float acc1 = sDgam[d] * rgam;
#pragma unroll
    for (int q = 0; q < WRV; ++q) acc1 += sDGlP[q * K + d];
    sDGl[d] = acc1;
  }
  __syncthreads();

  // tiles of the C x K tiling (the wave's own): the gated sums, the elementwise
  // rules; dq, dk leave here (with the L2 flag as the gradients of the
  // normalised rows, completed below); the within-tile reverse sums of dG stay
  // in registers; the dbeta term dKb . (k^ e^G)
  const float s = a.scale;
  float sfx[TCV::BM][TCV::BN][4];
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm) {
    floatx4 dbk = zero4();
#pragma unroll
    for (int bn = 0; bn < TCV::BN; ++bn) {
      const int ib = (r0v >> 4) + bm, ct = (c0v >> 4) + bn, d = 16 * ct + i;
      floatx4 qa, qm, ka, km;
      gated_sums<K>(sG, sKN, sQN, sP, sDM, ib, d, g, i, qa, qm, ka, km);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ib + 4 * g + r;
        const float qi = sQN[row * K + d], ki = sKN[row * K + d];
        float gqn, gkn;
        elem_rules<K>(sG, sQN, sKN, sBeta, sDGl, row, d, s, kQG[bm][bn][r], kKB[bm][bn][r], kKG[bm][bn][r], qa[r],
                      qm[r], ka[r], km[r], gqn, gkn, sfx[bm][bn][r]);
        dbk[r] += kKB[bm][bn][r] * ki * __expf(sG[row * K + d]);
        if (row < it.len) {
          const size_t idx = ((size_t)(it.tok0 + row) * H + it.h) * K + d;
          a.dq[idx] = gqn;
          a.dk[idx] = gkn;
        }
        if (a.l2norm) {
          float pq = qi * gqn, pk = ki * gkn;
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) {
            pq += __shfl_xor(pq, off, 64);
            pk += __shfl_xor(pk, off, 64);
          }
          if (i == 0) {
            sDotP[ct * 2 * C + row] = pq;
            sDotP[ct * 2 * C + C + row] = pk;
          }
        }
      }
      // dg: reverse sums within the lane's 4 rows, then over the later lane
      // groups of the tile; the later 16-row blocks are added below
#pragma unroll
      for (int r = 2; r >= 0; --r) sfx[bm][bn][r] += sfx[bm][bn][r + 1];
      float tot[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[q] = __shfl(sfx[bm][bn][0], 16 * q + i, 64);
      float later = 0.f;
#pragma unroll
      for (int q = 3; q >= 1; --q) later += q > g ? tot[q] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) sfx[bm][bn][r] += later;
      if (g == 0) sBT[ib * K + d] = ((tot[3] + tot[2]) + tot[1]) + tot[0];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) dbk[r] += __shfl_xor(dbk[r], off, 64);
    if (i == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) sDbP[(TCV::WC + w % TCV::WC) * C + r0v + 16 * bm + 4 * g + r] = dbk[r];
  }
  __syncthreads();
#pragma unroll
  for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
    for (int bn = 0; bn < TCV::BN; ++bn) {
      const int ib = (r0v >> 4) + bm, d = c0v + 16 * bn + i;
      float after = 0.f;
#pragma unroll
      for (int b = 3; b >= 1; --b) after += b > ib ? sBT[b * K + d] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ib + 4 * g + r;
        if (row < it.len) a.dg[((size_t)(it.tok0 + row) * H + it.h) * K + d] = sfx[bm][bn][r] + after;
      }
    }
  if (tid < C && tid < it.len) {
    float db = 0.f;
#pragma unroll
    for (int q = 0; q < kDbSlots; ++q) db += sDbP[q * C + tid];
    a.dbeta[(size_t)(it.tok0 + tid) * H + it.h] = db;
  }
  // L2-norm backward: dq = (dq^ - q^ (q^ . dq^)) / |q| (dq^ / eps where the norm
  // is clamped), likewise dk; each lane completes the elements it stored
  if (a.l2norm) {
    if (tid < 2 * C) {
      float acc1 = 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc1 += sDotP[ct * 2 * C + tid];
      sDot[tid] = acc1;
    }
    __syncthreads();
#pragma unroll
    for (int bm = 0; bm < TCV::BM; ++bm)
#pragma unroll
      for (int bn = 0; bn < TCV::BN; ++bn) {
        const int ib = (r0v >> 4) + bm, d = c0v + 16 * bn + i;
        float gqv[4], gkv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * ib + 4 * g + r;
          const size_t idx = ((size_t)(it.tok0 + (row < it.len ? row : 0)) * H + it.h) * K + d;
          gqv[r] = a.dq[idx];
          gkv[r] = a.dk[idx];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * ib + 4 * g + r;
          if (row < it.len) {
            const size_t idx = ((size_t)(it.tok0 + row) * H + it.h) * K + d;
            const float nq = sl[o.nq + row], nk = sl[o.nk + row];
            a.dq[idx] = nq > a.l2eps ? (gqv[r] - sQN[row * K + d] * sDot[row]) / nq : gqv[r] / a.l2eps;
            a.dk[idx] = nk > a.l2eps ? (gkv[r] - sKN[row * K + d] * sDot[C + row]) / nk : gkv[r] / a.l2eps;
          }
        }
      }
  }
}

// the elementwise and gated-sum rules (gated_sums, elem_rules), the L2-norm
// backward and the reverse cumsum, for fp32 q/k/v (bf16 input runs them inside
// bwd_chunk_fused_kernel)
template <int K>
__global__ __launch_bounds__(kBW) void bwd_chunk_elem_kernel(BwdArgs a) {
  constexpr int V = K;
  constexpr int CP = C + 4;
  constexpr int NCT = K / 16;  // 16-channel column tiles
  __shared__ __attribute__((aligned(16))) float sG[C * K], sKN[C * K], sQN[C * K];
  __shared__ float sP[C * CP], sDM[C * CP];  // dAqk and dM = Diag(beta) dL
  __shared__ float sBeta[C], sDot[2 * C], sDGl[K];
  __shared__ float sDotP[NCT * 2 * C];  // per channel tile row dots q^ . dq^, k^ . dk^
  __shared__ float sBT[4 * K];          // 16-row block totals of dG
  const int tid = threadIdx.x;
  const int lane = tid & 63, gq = lane >> 4, xi = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if ((int)blockIdx.x >= items_in_use(a)) return;
  const ItemB it = chunk_of(a, (int)blockIdx.x / a.H, (int)blockIdx.x % a.H);
  const BwdSlab& o = a.sl;
  float* sl = slab_of(a, it.p, it.h);
  const SlabPtrs P = slab_ptrs(sl, o);
  const int H = a.H;
  const int qf32 = !a.bf16_qkv;
  const float s = a.scale;

  // staging: every load of the thread first, then the LDS stores. q^, k^ and G
  // are rebuilt from the inputs with the same operations, in the same order, as
  // the chunk-term kernel builds them (normalised with its stored row norms;
  // the gate cumsum sequential over the rows of a channel), so they are
  // bitwise its values; rows past the chunk end are zero tokens.
  constexpr int N4 = C * K / 4 / kBW, NPP = C * C / kBW;
  static_assert(N4 * 4 * kBW == C * K && NPP * kBW == C * C, "staging split");
  floatx4 rk4[N4], rq4[N4], rg4[N4];
  float rp[NPP], rl[NPP], rbeta[NPP];
  auto in_idx = [&](int m) {
    const int e = tid + kBW * m, row = e / (K / 4), c = 4 * (e % (K / 4)), rr = row < it.len ? row : 0;
    return ((size_t)(it.tok0 + rr) * H + it.h) * K + c;
  };
  if (qf32) {
#pragma unroll
    for (int m = 0; m < N4; ++m) {
      rq4[m] = load4_f32(reinterpret_cast<const float*>(a.q) + in_idx(m));
      rk4[m] = load4_f32(reinterpret_cast<const float*>(a.k) + in_idx(m));
    }
  } else {
#pragma unroll
    for (int m = 0; m < N4; ++m) {
      rq4[m] = load4_f32(reinterpret_cast<const bf16*>(a.q) + in_idx(m));
      rk4[m] = load4_f32(reinterpret_cast<const bf16*>(a.k) + in_idx(m));
    }
  }
  if (a.g_f32) {
#pragma unroll
    for (int m = 0; m < N4; ++m) rg4[m] = load4_f32(reinterpret_cast<const float*>(a.g) + in_idx(m));
  } else {
#pragma unroll
    for (int m = 0; m < N4; ++m) rg4[m] = load4_f32(reinterpret_cast<const bf16*>(a.g) + in_idx(m));
  }
#pragma unroll
  for (int m = 0; m < NPP; ++m) {
    const int e = tid + kBW * m;
    rp[m] = P.DAQK[e];
    rl[m] = P.DL[e];
    rbeta[m] = P.BETA[e / C];
  }
  const float rb = tid < C ? P.BETA[tid] : 0.f;
  float qinv[N4], kinv[N4];
#pragma unroll
  for (int m = 0; m < N4; ++m) {
    const int row = (tid + kBW * m) / (K / 4);
    qinv[m] = a.l2norm ? 1.f / fmaxf(sl[o.nq + row], a.l2eps) : 1.f;
    kinv[m] = a.l2norm ? 1.f / fmaxf(sl[o.nk + row], a.l2eps) : 1.f;
  }
#pragma unroll
  for (int m = 0; m < N4; ++m) {
    const int e = tid + kBW * m, row = e / (K / 4);
    const bool in = row < it.len;
    reinterpret_cast<floatx4*>(sQN)[e] = in ? (a.l2norm ? rq4[m] * qinv[m] : rq4[m]) : zero4();
    reinterpret_cast<floatx4*>(sKN)[e] = in ? (a.l2norm ? rk4[m] * kinv[m] : rk4[m]) : zero4();
    reinterpret_cast<floatx4*>(sG)[e] = in ? rg4[m] : zero4();
  }
#pragma unroll
  for (int m = 0; m < NPP; ++m) {
    const int e = tid + kBW * m;
    sP[(e / C) * CP + e % C] = rp[m];
    sDM[(e / C) * CP + e % C] = rbeta[m] * rl[m];
  }
  if (tid < C) sBeta[tid] = rb;
  // gradient of the last row's cumulative gate through KG and gamma
  if (tid < K) {
    float acc = P.DGAM[tid] * P.GAM[tid];
#pragma unroll 16
    for (int r = 0; r < C; ++r) acc += P.DKG[r * K + tid] * P.KG[r * K + tid];
    sDGl[tid] = acc;
  }
  __syncthreads();
  // gate cumsum in place, sequential over the rows of each channel
  if (tid < K) {
    float run = 0.f;
    for (int r = 0; r < C; ++r) {
      run += sG[r * K + tid];
      sG[r * K + tid] = run;
    }
  }
  __syncthreads();

  // output tiles (row block ib, channel tile ct): wave w takes tiles w, w + 16, ...
  // The per-element gradients each tile needs are loaded up front, so that no
  // load waits behind an earlier tile's stores.
  constexpr int TPWE = 4 * NCT / kNWW;
  static_assert(TPWE >= 1 && TPWE * kNWW == 4 * NCT, "tile split");
  float pdqg[TPWE][4], pdkb[TPWE][4], pdkg[TPWE][4];
#pragma unroll
  for (int t = 0; t < TPWE; ++t) {
    const int tile = w + kNWW * t, ib = tile / NCT, d = 16 * (tile % NCT) + xi;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ib + 4 * gq + r;
      pdqg[t][r] = P.DQG[i * K + d];
      pdkb[t][r] = P.DKB[i * K + d];
      pdkg[t][r] = P.DKG[i * K + d];
    }
  }
  // dq and dk leave from each tile (with the L2 flag as the gradients of the
  // normalised rows, completed below); the within-tile reverse sums of dG stay
  // in registers for dg
  float sfx[TPWE][4];
#pragma unroll
  for (int t = 0; t < TPWE; ++t) {
    const int tile = w + kNWW * t;
    const int ib = tile / NCT, ct = tile % NCT;
    const int d = 16 * ct + xi;
    floatx4 qa, qm, ka, km;
    gated_sums<K>(sG, sKN, sQN, sP, sDM, ib, d, gq, xi, qa, qm, ka, km);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ib + 4 * gq + r;
      const float qi = sQN[i * K + d], ki = sKN[i * K + d];
      float gqn, gkn;
      elem_rules<K>(sG, sQN, sKN, sBeta, sDGl, i, d, s, pdqg[t][r], pdkb[t][r], pdkg[t][r], qa[r], qm[r], ka[r],
                    km[r], gqn, gkn, sfx[t][r]);
      if (i < it.len) {
        const size_t idx = ((size_t)(it.tok0 + i) * H + it.h) * K + d;
        a.dq[idx] = gqn;
        a.dk[idx] = gkn;
      }
      if (a.l2norm) {
        // row dots over the tile's 16 columns (lane shuffles), one slot per
        // (channel tile, row)
        float pq = qi * gqn, pk = ki * gkn;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          pq += __shfl_xor(pq, off, 64);
          pk += __shfl_xor(pk, off, 64);
        }
        if (xi == 0) {
          sDotP[ct * 2 * C + i] = pq;
          sDotP[ct * 2 * C + C + i] = pk;
        }
      }
    }
    // dg = reverse cumsum of dG over the chunk rows: within the lane's 4 rows,
    // then over the later lane groups of the tile (shuffles); the later 16-row
    // blocks are added below from their totals, each in a fixed order
#pragma unroll
    for (int r = 2; r >= 0; --r) sfx[t][r] += sfx[t][r + 1];
    float tot[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[q] = __shfl(sfx[t][0], 16 * q + xi, 64);
    float later = 0.f;
#pragma unroll
    for (int q = 3; q >= 1; --q) later += q > gq ? tot[q] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) sfx[t][r] += later;
    if (gq == 0) sBT[ib * K + d] = ((tot[3] + tot[2]) + tot[1]) + tot[0];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TPWE; ++t) {
    const int tile = w + kNWW * t, ib = tile / NCT, d = 16 * (tile % NCT) + xi;
    float after = 0.f;
#pragma unroll
    for (int b = 3; b >= 1; --b) after += b > ib ? sBT[b * K + d] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * ib + 4 * gq + r;
      if (row < it.len) a.dg[((size_t)(it.tok0 + row) * H + it.h) * K + d] = sfx[t][r] + after;
    }
  }
  // dbeta and dv: TPR consecutive threads per row, each over a share of the channels
  {
    constexpr int TPR = kBW / C;
    const int i = tid / TPR, part = tid % TPR;
    float db = 0.f;
    if (i < it.len) {
      constexpr int NV = V / TPR, NK = K / TPR, NJ = C / TPR;
      const size_t vrow = ((size_t)(it.tok0 + i) * H + it.h) * V;
      const int v0 = part * NV, d0 = part * NK;
      // loads first (no store in between), then the sums, then the dv stores
      float dvb[NV], vv[NV], dkb[NK], dl[NJ], mm[NJ];
#pragma unroll
      for (int c = 0; c < NV; ++c) dvb[c] = P.DVB[i * V + v0 + c];
      if (qf32) {
#pragma unroll
        for (int c = 0; c < NV; ++c) vv[c] = reinterpret_cast<const float*>(a.v)[vrow + v0 + c];
      } else {
#pragma unroll
        for (int c = 0; c < NV; ++c) vv[c] = to_f32(reinterpret_cast<const bf16*>(a.v)[vrow + v0 + c]);
      }
#pragma unroll
      for (int c = 0; c < NK; ++c) dkb[c] = P.DKB[i * K + d0 + c];
#pragma unroll
      for (int c = 0; c < NJ; ++c) {
        const int j = part + TPR * c;
        dl[c] = P.DL[i * C + j];
        mm[c] = P.Mm[i * C + j];
      }
#pragma unroll
      for (int c = 0; c < NV; ++c) db += dvb[c] * vv[c];
#pragma unroll
      for (int c = 0; c < NK; ++c) db += dkb[c] * sKN[i * K + d0 + c] * __expf(sG[i * K + d0 + c]);
#pragma unroll
      for (int c = 0; c < NJ; ++c) db += (part + TPR * c < i) ? dl[c] * mm[c] : 0.f;
#pragma unroll
      for (int c = 0; c < NV; ++c) a.dv[vrow + v0 + c] = sBeta[i] * dvb[c];
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) db += __shfl_xor(db, off, 64);
    if (part == 0 && i < it.len) a.dbeta[(size_t)(it.tok0 + i) * H + it.h] = db;
  }
  __syncthreads();
  // L2-norm backward: dq = (dq^ - q^ (q^ . dq^)) / |q| (dq^ / eps where the norm
  // is clamped), likewise dk. The row dots are summed over the channel tiles in
  // a fixed order; each lane then completes the dq, dk elements it stored.
  if (a.l2norm) {
    if (tid < 2 * C) {
      float acc = 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc += sDotP[ct * 2 * C + tid];
      sDot[tid] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPWE; ++t) {
      const int tile = w + kNWW * t, ib = tile / NCT, d = 16 * (tile % NCT) + xi;
      float gqv[4], gkv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ib + 4 * gq + r;
        const size_t idx = ((size_t)(it.tok0 + (row < it.len ? row : 0)) * H + it.h) * K + d;
        gqv[r] = a.dq[idx];
        gkv[r] = a.dk[idx];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ib + 4 * gq + r;
        if (row < it.len) {
          const size_t idx = ((size_t)(it.tok0 + row) * H + it.h) * K + d;
          const float nq = sl[o.nq + row], nk = sl[o.nk + row];
          a.dq[idx] = nq > a.l2eps ? (gqv[r] - sQN[row * K + d] * sDot[row]) / nq : gqv[r] / a.l2eps;
          a.dk[idx] = nk > a.l2eps ? (gkv[r] - sKN[row * K + d] * sDot[C + row]) / nk : gkv[r] / a.l2eps;
        }
      }
    }
  }
}

// stages: bit 0 prep, bit 1 chunk-start states, bit 2 state gradients, bit 3 chunk gradients
template <int K>
hipError_t launch_k(const BwdArgs& a, int nitems, int stages, hipStream_t s) {
  const int nvb = K / 16;
  const unsigned sgrid = (unsigned)((a.nunits + 7) / 8 * 8 * nvb);  // see the XCD mapping above
  if ((stages & 1) && nitems > 0) hipLaunchKernelGGL(bwd_prep_kernel<K>, dim3(nitems), dim3(kBW), 0, s, a);
  if (a.nunits > 0) {
    if ((stages & 2) && nitems > 0)
      hipLaunchKernelGGL(bwd_states_fwd_kernel<K>, dim3(sgrid), dim3(2 * kBT), 0, s, a);
    if (stages & 4) {
      if (a.bf16_qkv) hipLaunchKernelGGL(bwd_states_bwd_bf16_kernel<K>, dim3(sgrid), dim3(2 * kBT), 0, s, a);
      else hipLaunchKernelGGL(bwd_states_bwd_kernel<K>, dim3(sgrid), dim3(2 * kBT), 0, s, a);
    }
  }
  if ((stages & 8) && nitems > 0) {
    if (a.bf16_qkv) {
      hipLaunchKernelGGL(bwd_chunk_fused_kernel<K>, dim3(nitems), dim3(kMT), 0, s, a);
    } else {
      hipLaunchKernelGGL(bwd_chunk_mm_kernel<K>, dim3(nitems), dim3(kBT), 0, s, a);
      hipLaunchKernelGGL(bwd_chunk_elem_kernel<K>, dim3(nitems), dim3(kBW), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int K, int nitems, int stages, hipStream_t s) {
  return K == 128 ? launch_k<128>(a, nitems, stages, s) : launch_k<64>(a, nitems, stages, s);
}

}  // namespace kda
