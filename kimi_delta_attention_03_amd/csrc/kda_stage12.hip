// Stage 1+2 of the chunkwise KDA forward on gfx950: one workgroup (4 waves)
// per (chunk, head). Everything a chunk needs stays in LDS; the outputs are
// written once, as MFMA fragments, into the chunk's workspace record.
//
// What it computes for a chunk of C = 64 tokens (Tokamax "chunk_kda_fwd
// design doc", sections 4.1.2-4.1.4 and 9.1.3-9.1.5, Paper Eq. 6-7):
//   G    = log2(e) * inclusive cumsum of g over the chunk (per key channel)
//   Aqk  = scale * Tril(sum_d q_i k_j 2^(G_i - G_j))            (diagonal kept)
//   L    = StrictTril(beta_i * sum_d k_i k_j 2^(G_i - G_j))
//   A    = (I + L)^-1                                           (fp32)
//   W    = A (beta * k * 2^G),  U = A (beta * v)
//   qg   = scale * q * 2^G,     kg = k * 2^(G_last - G),  gamma = 2^G_last
//
// Relation tiles use the rebasing of "KDA Doesn't Care About the Future",
// section "The rebasing trick": 2^(G_i - G_j) = 2^(G_i - r) 2^(r - G_j) with
// one reference r per 16-row query block, r = G of the block's FIRST row.
// For a key j in an earlier block both factors are <= 1; for a key in the
// query's own block the key factor spans at most 15 steps (<= 2^108 at the
// g >= -5 bound, section "What's the catch?"), so nothing overflows, and r
// never depends on a later token: every output row is a function of tokens
// up to that row only (section "Decisions Decisions").
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// block-wide LDS synchronisation without waiting for global memory traffic
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float ld_scalar(const void* p, size_t idx, int is_f32) {
  return is_f32 ? reinterpret_cast<const float*>(p)[idx]
                : (float)reinterpret_cast<const bf16*>(p)[idx];
}

template <typename T>
__device__ __forceinline__ float sumsq16(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {  // two bf16 per word: the high half is the bf16 bit pattern
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
      s += lo * lo + hi * hi;
    } else {
      const float x = __uint_as_float(w[i]);
      s += x * x;
    }
  }
  return s;
}

// 8 phys-ordered values of row `row` at 32-block kb from an LDS row of T
template <typename T, int STRIDE>
__device__ __forceinline__ floatx8 lds_row8(const T* base, int row, int c0) {
  floatx4 a = load4_f32(base + row * STRIDE + c0);
  floatx4 b = load4_f32(base + row * STRIDE + c0 + 16);
  return stackf(a, b);
}
__device__ __forceinline__ floatx4 ldsf4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

template <typename T>
__device__ __forceinline__ void store_frag8(char* base, size_t frag_elem_index, const floatx8& x) {
  typename Vec<T>::x8 y;
  cvt8(x, y);
  *reinterpret_cast<typename Vec<T>::x8*>(reinterpret_cast<T*>(base) + frag_elem_index) = y;
}

template <typename T, int K>
__global__ __launch_bounds__(kThreads, 1) void stage12_kernel(Stage12Args a) {
  constexpr int C = kChunk;
  constexpr int V = K;
  constexpr int NKB = K / 32;          // 32-wide channel blocks
  constexpr int GS = K + 4;            // sG row stride (floats)
  constexpr int KS = (sizeof(T) == 2) ? K + 8 : K + 4;  // sK / sV row stride (elements)
  constexpr int AS = C + 4;            // sA row stride (floats)
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = K / EPC;         // 16-byte chunks per row
  constexpr int NCH = C * CPR / kThreads;  // chunks per thread for a C x K tile
  constexpr int TPC = kThreads / K;    // threads per channel in the cumsum
  constexpr int RPS = C / TPC;         // rows per cumsum segment
  static_assert(NCH * kThreads == C * CPR, "tile split");

  __shared__ __attribute__((aligned(16))) float sG[C * GS];   // G, later V (as T)
  __shared__ __attribute__((aligned(16))) T sK[C * KS];
  __shared__ __attribute__((aligned(16))) float sA[C * AS];   // scratch, L, then A
  __shared__ float sB[C], sQn[C], sKn[C];
  T* sV = reinterpret_cast<T*>(sG);
  static_assert(sizeof(T) * C * KS <= sizeof(float) * C * GS, "sV fits in sG");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: conditions on it must compile to scalar branches,
  // because an MFMA placed under an EXEC mask still executes for all lanes
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4;
  const int xi = lane & 15;
  const int H = a.H;
  const int p = blockIdx.x / H;
  const int h = blockIdx.x - p * H;

  int64_t tok0;
  int len;
  if (a.varlen) {
    const int2 ct = reinterpret_cast<const int2*>(a.ws + a.off_chunk_tab)[p];
    tok0 = ct.x;
    len = ct.y;
    if (len <= 0) return;  // unused chunk slot
  } else {
    tok0 = (int64_t)p * C;
    len = C;
  }
  char* rec = a.ws + a.meta_bytes + ((size_t)h * a.ncp + p) * a.rec_bytes;
  const T* qg_ = reinterpret_cast<const T*>(a.q);
  const T* kg_ = reinterpret_cast<const T*>(a.k);
  const T* vg_ = reinterpret_cast<const T*>(a.v);
  auto rowK = [&](int i) -> size_t { return ((size_t)(tok0 + i) * H + h) * K; };
  auto rowV = [&](int i) -> size_t { return ((size_t)(tok0 + i) * H + h) * V; };

  // ---------------- phase 1: beta, gate cumsum, k -> LDS, norms, v prefetch
  if (tid < C) sB[tid] = tid < len ? ld_scalar(a.beta, (size_t)(tok0 + tid) * H + h, a.beta_f32) : 0.f;

  float loc[RPS];
  {
    const int c = tid % K;
    const int seg = tid / K;
    float run = 0.f;
#pragma unroll
    for (int r = 0; r < RPS; ++r) {
      const int i = seg * RPS + r;
      const float gv = i < len ? ld_scalar(a.g, rowK(i) + c, a.g_f32) : 0.f;
      run += gv;
      loc[r] = run;
    }
    sA[seg * K + c] = run;  // segment totals (sA is free until the relations)
  }

  // k and v tiles, 16 bytes per thread and chunk; kept as vector values (not
  // arrays) so they stay in registers until they are written to LDS
  typedef uint32_t rawv __attribute__((ext_vector_type(4 * NCH)));
  rawv kraw, vraw;
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    const int ci = tid + m * kThreads;
    const int row = ci / CPR, col = (ci % CPR) * EPC;
    uint4 kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (row < len) {
      kk = *reinterpret_cast<const uint4*>(kg_ + rowK(row) + col);
      vv = *reinterpret_cast<const uint4*>(vg_ + rowV(row) + col);
    }
    kraw[4 * m] = kk.x; kraw[4 * m + 1] = kk.y; kraw[4 * m + 2] = kk.z; kraw[4 * m + 3] = kk.w;
    vraw[4 * m] = vv.x; vraw[4 * m + 1] = vv.y; vraw[4 * m + 2] = vv.z; vraw[4 * m + 3] = vv.w;
  }
  auto part = [](const rawv& r, int m) { return uint4{r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]}; };
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    const int ci = tid + m * kThreads;
    const int row = ci / CPR, col = (ci % CPR) * EPC;
    *reinterpret_cast<uint4*>(sK + row * KS + col) = part(kraw, m);
  }
  if (a.l2norm) {
    // rows are owned by CPR consecutive lanes: reduce the squares across them
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int ci = tid + m * kThreads;
      const int row = ci / CPR, col = (ci % CPR) * EPC;
      float sk = sumsq16<T>(part(kraw, m));
      uint4 qr = {0u, 0u, 0u, 0u};
      if (row < len) qr = *reinterpret_cast<const uint4*>(qg_ + rowK(row) + col);
      float sq = sumsq16<T>(qr);
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) {
        sk += __shfl_xor(sk, o, 64);
        sq += __shfl_xor(sq, o, 64);
      }
      if (col == 0) {
        sKn[row] = 1.f / fmaxf(sqrtf(sk), a.l2eps);
        sQn[row] = 1.f / fmaxf(sqrtf(sq), a.l2eps);
      }
    }
  } else if (tid < C) {
    sKn[tid] = 1.f;
    sQn[tid] = 1.f;
  }
  lds_sync();
  {
    const int c = tid % K;
    const int seg = tid / K;
    float carry = 0.f;
    for (int s = 0; s < seg; ++s) carry += sA[s * K + c];
#pragma unroll
    for (int r = 0; r < RPS; ++r) sG[(seg * RPS + r) * GS + c] = (carry + loc[r]) * kLog2e;
  }
  lds_sync();

  // ---------------- phase 2: relation tiles for query block w (this wave)
  // Aqk^T and L^T tiles (keys j x queries i) = Khat_j . (Qhat_i | Khat'_i):
  //   Qhat_i = q_i 2^(G_i - r), Khat'_i = k_i 2^(G_i - r), Khat_j = k_j 2^(r - G_j),
  //   r = G of row 16 w.
  const int irow = 16 * w + xi;
  {
    const float qn = sQn[irow];
    const float kni = sKn[irow];
    floatx4 accQ[4], accL[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) { accQ[bj] = zero4(); accL[bj] = zero4(); }
    const T* qrow = qg_ + rowK(irow < len ? irow : 0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int c0 = 32 * kb + 4 * gq;
      const floatx8 Gi = stackf(ldsf4(sG + irow * GS + c0), ldsf4(sG + irow * GS + c0 + 16));
      const floatx8 Gr = stackf(ldsf4(sG + (16 * w) * GS + c0), ldsf4(sG + (16 * w) * GS + c0 + 16));
      floatx8 qv = stackf(load4_f32(qrow + c0), load4_f32(qrow + c0 + 16));
      if (irow >= len) qv = floatx8{0, 0, 0, 0, 0, 0, 0, 0};
      const floatx8 kv = lds_row8<T, KS>(sK, irow, c0);
      floatx8 qh, kh, qgv;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float e = exp2_fast(Gi[t] - Gr[t]);
        qh[t] = qv[t] * qn * e;
        kh[t] = kv[t] * kni * e;
        qgv[t] = a.scale * qv[t] * qn * exp2_fast(Gi[t]);
      }
      store_frag8<T>(rec + a.off_qg, ((size_t)(w * NKB + kb) * 64 + lane) * 8, qgv);
      typename Vec<T>::x8 qhT, khT;
      cvt8(qh, qhT);
      cvt8(kh, khT);
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        if (bj <= w) {
          const int j = 16 * bj + xi;
          const floatx8 Gj = stackf(ldsf4(sG + j * GS + c0), ldsf4(sG + j * GS + c0 + 16));
          const floatx8 kj = lds_row8<T, KS>(sK, j, c0);
          const float knj = sKn[j];
          floatx8 kk;
#pragma unroll
          for (int t = 0; t < 8; ++t) kk[t] = kj[t] * knj * exp2_fast(Gr[t] - Gj[t]);
          typename Vec<T>::x8 kkT;
          cvt8(kk, kkT);
          accQ[bj] = mma32(accQ[bj], kkT, qhT);
          accL[bj] = mma32(accL[bj], kkT, khT);
        }
      }
    }
    // epilogue: lane (gq, xi) holds, per tile bj, row irow and columns 16 bj + 4 gq + r
    const float bi = sB[irow];
    floatx4 aq[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      floatx4 lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool diag = (bj == w);
        const int jc = 4 * gq + r;
        aq[bj][r] = (bj < w || (diag && jc <= xi)) ? a.scale * accQ[bj][r] : 0.f;
        lv[r] = (bj < w || (diag && jc < xi)) ? bi * accL[bj][r] : 0.f;
      }
      if (bj <= w) *reinterpret_cast<floatx4*>(sA + irow * AS + 16 * bj + 4 * gq) = lv;
    }
    if (w == 0 || w == 2)  // blocks (0,1) and (2,3) are read as zeros later
      *reinterpret_cast<floatx4*>(sA + irow * AS + 16 * (w + 1) + 4 * gq) = zero4();
    // Aqk fragments of query block w: kb' = 0 from tiles (0, 1), kb' = 1 from (2, 3)
    store_frag8<T>(rec + a.off_aq, ((size_t)(w * 2 + 0) * 64 + lane) * 8, stackf(aq[0], aq[1]));
    if (w >= 2)
      store_frag8<T>(rec + a.off_aq, ((size_t)(w * 2 + 1) * 64 + lane) * 8, stackf(aq[2], aq[3]));
  }

  // ---------------- phase 3: gated keys kg^T and gamma (only G, k needed)
  {
    constexpr int TPW = K / 64;  // 16-channel row tiles per wave
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int rt = w * TPW + m;
      const int ch = 16 * rt + xi;
      const float Glast = sG[(C - 1) * GS + ch];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        floatx8 x;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int j = 32 * kb + (t < 4 ? 4 * gq + t : 16 + 4 * gq + t - 4);
          x[t] = to_f32(sK[j * KS + ch]) * sKn[j] * exp2_fast(Glast - sG[j * GS + ch]);
        }
        store_frag8<T>(rec + a.off_kg, ((size_t)(rt * 2 + kb) * 64 + lane) * 8, x);
      }
    }
    if (tid < K) reinterpret_cast<float*>(rec + a.off_gam)[tid] = exp2_fast(sG[(C - 1) * GS + tid]);
  }
  lds_sync();

  // ---------------- phase 4: A = (I + L)^-1 in fp32
  // 4a: diagonal 16x16 blocks by forward substitution, wave w -> block w,
  //     lane column xi (lanes of the other groups compute the same values)
  {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == xi) ? 1.f : 0.f;
    const float* Lb = sA + (16 * w) * AS + 16 * w;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
#pragma unroll
      for (int i = j + 1; i < 16; ++i) x[i] -= Lb[i * AS + j] * x[j];
    }
    if (gq == 0) {
      float* Db = sA + (16 * w) * AS + 16 * w;
#pragma unroll
      for (int i = 0; i < 16; ++i) Db[i * AS + xi] = x[i];
    }
  }
  lds_sync();
  // 4b: block column w below the diagonal:
  //     A_{ib,w} = -D_ib * sum_{kb=w}^{ib-1} L_{ib,kb} A_{kb,w}
  floatx4 Ab[4];
  {
    floatx4 Dw;
#pragma unroll
    for (int s = 0; s < 4; ++s) Dw[s] = sA[(16 * w + 4 * gq + s) * AS + 16 * w + xi];
#pragma unroll
    for (int ib = 1; ib < 4; ++ib) {
      Ab[ib] = zero4();
      if (ib > w) {
        floatx4 P = zero4();
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) {
          if (kb >= w && kb < ib) {
            const floatx4 La = ldsf4(sA + (16 * ib + xi) * AS + 16 * kb + 4 * gq);
            const floatx4 Bk = (kb == w) ? Dw : Ab[kb];
            P = mma16_f32(P, La, Bk);
          }
        }
        const floatx4 Da = ldsf4(sA + (16 * ib + xi) * AS + 16 * ib + 4 * gq);
        const floatx4 R = mma16_f32(zero4(), Da, P);
        Ab[ib] = -R;
      }
    }
  }
  lds_sync();
#pragma unroll
  for (int ib = 1; ib < 4; ++ib) {
    if (ib > w) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sA[(16 * ib + 4 * gq + r) * AS + 16 * w + xi] = Ab[ib][r];
    }
  }
  lds_sync();

  // ---------------- phase 5a: W^T tiles = (beta k 2^G)^T A^T
  // A fragments (rt, kb) for the causal pairs: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
  typename Vec<T>::x8 Af[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb <= rt / 2) {
        const int c0 = 32 * kb + 4 * gq;
        const floatx8 x = stackf(ldsf4(sA + (16 * rt + xi) * AS + c0),
                                 ldsf4(sA + (16 * rt + xi) * AS + c0 + 16));
        cvt8(x, Af[rt][kb]);
      }
    }
  }
  {
    const int kbp = w % NKB;             // W fragment column block of this wave
    constexpr int RSTEP = 4 / NKB;       // rt stride between this wave's row tiles
    const int rt0 = w / NKB;
    typename Vec<T>::x8 BKf[2][2];       // [ct 2kbp / 2kbp+1][kb]
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ch = 16 * (2 * kbp + cc) + xi;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        floatx8 x;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int j = 32 * kb + (t < 4 ? 4 * gq + t : 16 + 4 * gq + t - 4);
          x[t] = sB[j] * to_f32(sK[j * KS + ch]) * sKn[j] * exp2_fast(sG[j * GS + ch]);
        }
        cvt8(x, BKf[cc][kb]);
      }
    }
    // rt runs over compile-time values (a register array indexed by a runtime
    // value becomes a compare/select chain); the wave-uniform guard picks the
    // row tiles of this wave
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if ((rt - rt0) % RSTEP != 0) continue;
      floatx4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb <= rt / 2) {
          acc0 = mma32(acc0, BKf[0][kb], Af[rt][kb]);
          acc1 = mma32(acc1, BKf[1][kb], Af[rt][kb]);
        }
      }
      store_frag8<T>(rec + a.off_w, ((size_t)(rt * NKB + kbp) * 64 + lane) * 8, stackf(acc0, acc1));
    }
  }
  lds_sync();  // G and k are dead: reuse sG for v

  // ---------------- phase 5b/5c: U tiles = A (beta v), accumulator layout
#pragma unroll
  for (int m = 0; m < NCH; ++m) {
    const int ci = tid + m * kThreads;
    const int row = ci / CPR, col = (ci % CPR) * EPC;
    *reinterpret_cast<uint4*>(sV + row * KS + col) = part(vraw, m);
  }
  lds_sync();
  {
    constexpr int NVB = V / 16;
#pragma unroll
    for (int vb = w; vb < NVB; vb += 4) {
      typename Vec<T>::x8 BV[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        floatx8 x;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int j = 32 * kb + (t < 4 ? 4 * gq + t : 16 + 4 * gq + t - 4);
          x[t] = sB[j] * to_f32(sV[j * KS + 16 * vb + xi]);
        }
        cvt8(x, BV[kb]);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        floatx4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb <= rt / 2) acc = mma32(acc, Af[rt][kb], BV[kb]);
        typename Vec<T>::x4 y;
        cvt4(acc, y);
        *reinterpret_cast<typename Vec<T>::x4*>(reinterpret_cast<T*>(rec + a.off_u) +
                                                ((size_t)(vb * 4 + rt) * 64 + lane) * 4) = y;
      }
    }
  }
}

}  // namespace

hipError_t launch_stage12(const Stage12Args& a, int K, int bf16, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  dim3 grid(nblocks), block(kThreads);
  if (bf16) {
    if (K == 128) hipLaunchKernelGGL((stage12_kernel<kda::bf16, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage12_kernel<kda::bf16, 64>), grid, block, 0, s, a);
  } else {
    if (K == 128) hipLaunchKernelGGL((stage12_kernel<float, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage12_kernel<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kda
