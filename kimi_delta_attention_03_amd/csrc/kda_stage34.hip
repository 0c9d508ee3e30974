// Stage 3+4 of the chunkwise KDA forward on gfx950: the ordered recurrence
// over chunks and the output (Tokamax "chunk_kda_fwd design doc", sections
// 4.3.2-4.3.3 and 9.1.6, Paper Eq. 8-9). Per chunk, with chunk-start state S:
//   V_new = U - W S
//   O     = qg S + Aqk V_new          (written to o, cast to the input dtype)
//   S     = Diag(gamma) S + kg^T V_new
//
// The V columns of S evolve independently (every product above is linear in
// S's columns), so one workgroup owns a 16-column block of S for one
// (sequence, head) and walks that sequence's chunks in order. The K x 16
// fp32 state block lives in MFMA accumulators spread over the 4 waves; each
// chunk exchanges only the state block and V_new (as MFMA B fragments)
// through LDS. The chunk operands are read as ready-made MFMA fragments from
// the stage-1+2 record, one chunk ahead of use.
//
// Workgroup ids are mapped so that the V/16 workgroups of one (sequence,
// head) get ids congruent modulo 8: with round-robin dispatch over the 8
// XCDs they share one L2, which then serves the repeated reads of W, qg, kg
// and Aqk. Variable-length sequences are visited longest first.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename T, int K>
struct ChunkFrags {
  static constexpr int NKB = K / 32;
  static constexpr int TPW = K / 64;
  typename Vec<T>::x8 w[NKB];      // W rows of this wave's 16-row block
  typename Vec<T>::x8 qg[NKB];     // qg rows of this wave's block
  typename Vec<T>::x8 aq[2];       // Aqk rows of this wave's block
  typename Vec<T>::x8 kg[TPW][2];  // kg^T rows for this wave's state tiles
  typename Vec<T>::x4 u;           // U, accumulator layout
  floatx4 gam[TPW];                // gamma for this lane's state rows
};

template <typename T, int K>
__device__ __forceinline__ void load_frags(ChunkFrags<T, K>& f, const char* rec, const Stage34Args& a,
                                           int w, int lane, int vb, int gq) {
  constexpr int NKB = K / 32;
  constexpr int TPW = K / 64;
  typedef typename Vec<T>::x8 F8;
  typedef typename Vec<T>::x4 F4;
  const F8* W = reinterpret_cast<const F8*>(rec + a.off_w);
  const F8* QG = reinterpret_cast<const F8*>(rec + a.off_qg);
  const F8* AQ = reinterpret_cast<const F8*>(rec + a.off_aq);
  const F8* KG = reinterpret_cast<const F8*>(rec + a.off_kg);
  const F4* U = reinterpret_cast<const F4*>(rec + a.off_u);
  const float* G = reinterpret_cast<const float*>(rec + a.off_gam);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    f.w[kb] = W[(w * NKB + kb) * 64 + lane];
    f.qg[kb] = QG[(w * NKB + kb) * 64 + lane];
  }
  f.aq[0] = AQ[(w * 2 + 0) * 64 + lane];
  if (w >= 2) f.aq[1] = AQ[(w * 2 + 1) * 64 + lane];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int rt = w * TPW + m;
    f.kg[m][0] = KG[(rt * 2 + 0) * 64 + lane];
    f.kg[m][1] = KG[(rt * 2 + 1) * 64 + lane];
    f.gam[m] = *reinterpret_cast<const floatx4*>(G + 16 * rt + 4 * gq);
  }
  f.u = U[(vb * 4 + w) * 64 + lane];
}

template <typename T, int K>
__global__ __launch_bounds__(kThreads) void stage34_kernel(Stage34Args a) {
  constexpr int C = kChunk;
  constexpr int V = K;
  constexpr int NKB = K / 32;
  constexpr int NVB = V / 16;
  constexpr int TPW = K / 64;      // 16-row state tiles per wave
  constexpr int NST = K / 16;      // state tiles
  typedef typename Vec<T>::x4 F4;

  __shared__ F4 sS[NST][64];       // state block as B-operand halves
  __shared__ F4 sVn[4][64];        // V_new block as B-operand halves

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: conditions on it must compile to scalar branches,
  // because an MFMA placed under an EXEC mask still executes for all lanes
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4;
  const int xi = lane & 15;

  // XCD-aware id mapping: ids u*? with equal id % 8 share an XCD
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int u = (slot / NVB) * 8 + xcd;
  const int vb = slot % NVB;
  if (u >= a.nunits) return;
  const int H = a.H;
  int seq = u / H;
  const int h = u - seq * H;

  size_t p0;
  int nch;
  const int2* ctab = reinterpret_cast<const int2*>(a.ws + a.off_chunk_tab);
  if (a.varlen) {
    seq = reinterpret_cast<const int*>(a.ws + a.off_order)[seq];
    const int2 st = reinterpret_cast<const int2*>(a.ws + a.off_seq_tab)[seq];
    p0 = (size_t)st.x;
    nch = st.y;
  } else {
    p0 = (size_t)seq * a.nt;
    nch = a.nt;
  }
  const char* rec0 = a.ws + a.meta_bytes + ((size_t)h * a.ncp + p0) * a.rec_bytes;
  const size_t state_base = ((size_t)seq * H + h) * K * V + 16 * vb + xi;

  // state tiles of this wave: rows 16 * (w * TPW + m) + 4 gq + r, column 16 vb + xi
  floatx4 S[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int rt = w * TPW + m;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[m][r] = a.init ? a.init[state_base + (size_t)(16 * rt + 4 * gq + r) * V] : 0.f;
    F4 y;
    cvt4(S[m], y);
    sS[rt][lane] = y;
  }
  lds_sync();

  T* out = reinterpret_cast<T*>(a.o);
  ChunkFrags<T, K> F[2];
  if (nch > 0) load_frags<T, K>(F[0], rec0, a, w, lane, vb, gq);

  auto step = [&](ChunkFrags<T, K>& f, int c) {
    int64_t tok0;
    int len;
    if (a.varlen) {
      const int2 ct = ctab[p0 + c];
      tok0 = ct.x;
      len = ct.y;
    } else {
      tok0 = (int64_t)(p0 + c) * C;
      len = C;
    }
    // V_new and the inter-chunk read for rows 16 w .. 16 w + 15
    floatx4 accV = zero4(), accO = zero4();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const typename Vec<T>::x8 Sb = stack8<T>(sS[2 * kb][lane], sS[2 * kb + 1][lane]);
      accV = mma32(accV, f.w[kb], Sb);
      accO = mma32(accO, f.qg[kb], Sb);
    }
    const floatx4 vn = widen4(f.u) - accV;
    F4 vnT;
    cvt4(vn, vnT);
    sVn[w][lane] = vnT;
    lds_sync();
    const typename Vec<T>::x8 Vb0 = stack8<T>(sVn[0][lane], sVn[1][lane]);
    const typename Vec<T>::x8 Vb1 = stack8<T>(sVn[2][lane], sVn[3][lane]);
    // intra-chunk contribution, causal: row block w only reads V_new blocks <= w
    accO = mma32(accO, f.aq[0], Vb0);
    if (w >= 2) accO = mma32(accO, f.aq[1], Vb1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * w + 4 * gq + r;
      if (row < len) {
        T y;
        if constexpr (sizeof(T) == 2) y = (T)accO[r]; else y = accO[r];
        out[((size_t)(tok0 + row) * H + h) * V + 16 * vb + xi] = y;
      }
    }
    // state update for this wave's tiles
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      S[m] = S[m] * f.gam[m];
      S[m] = mma32(S[m], f.kg[m][0], Vb0);
      S[m] = mma32(S[m], f.kg[m][1], Vb1);
      F4 y;
      cvt4(S[m], y);
      sS[w * TPW + m][lane] = y;
    }
    lds_sync();
  };

  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) load_frags<T, K>(F[1], rec0 + (size_t)(c + 1) * a.rec_bytes, a, w, lane, vb, gq);
    step(F[0], c);
    if (c + 1 >= nch) break;
    if (c + 2 < nch) load_frags<T, K>(F[0], rec0 + (size_t)(c + 2) * a.rec_bytes, a, w, lane, vb, gq);
    step(F[1], c + 1);
  }

  if (a.final_state) {
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int rt = w * TPW + m;
#pragma unroll
      for (int r = 0; r < 4; ++r) a.final_state[state_base + (size_t)(16 * rt + 4 * gq + r) * V] = S[m][r];
    }
  }
}

}  // namespace

hipError_t launch_stage34(const Stage34Args& a, int K, int bf16, hipStream_t s) {
  if (a.nunits <= 0) return hipSuccess;
  const int nvb = K / 16;
  const int units8 = (a.nunits + 7) / 8;
  dim3 grid(units8 * 8 * nvb), block(kThreads);
  if (bf16) {
    if (K == 128) hipLaunchKernelGGL((stage34_kernel<kda::bf16, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage34_kernel<kda::bf16, 64>), grid, block, 0, s, a);
  } else {
    if (K == 128) hipLaunchKernelGGL((stage34_kernel<float, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage34_kernel<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kda
