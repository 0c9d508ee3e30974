// Stage 3+4 of the chunkwise KDA forward on gfx950: the ordered recurrence
// over chunks and the output (Tokamax "chunk_kda_fwd design doc", sections
// 4.3.2-4.3.3 and 9.1.6, Paper Eq. 8-9). Per chunk, with chunk-start state S:
//   V_new = U - W S
//   O     = qg S + Aqk V_new          (written to o, cast to the input dtype)
//   S     = Diag(gamma) S + kg^T V_new
//
// The V columns of S evolve independently (every product above is linear in
// S's columns), so one workgroup owns a 16-column block of S for one
// (sequence, head) and walks that sequence's chunks in order.
//
// The workgroup has 12 waves in three roles. Only V_new and the state update
// form the chain that is serial over chunks; the output is taken off it:
//   V waves 0..3      - wave r computes V_new for chunk rows 16 r .. 16 r + 15
//   state waves 4..7  - hold the K x 16 fp32 state block in MFMA accumulators
//                       (K / 64 tiles of 16 rows each) and apply the update
//   output waves 8..11 - wave 8 + r computes O for rows 16 r .. 16 r + 15 one
//                       chunk behind, from the previous chunk's S and V_new
// Every chunk step has two barriers: B1 publishes V_new, B2 the new state,
// both as MFMA B-operand halves in LDS; S and V_new are double-buffered so
// the output waves can read chunk c - 1's copies while chunk c is in flight.
// Each role issues its loads for a chunk NB - 1 steps ahead through a ring of
// NB register buffers, in the window where its own work is off the chain:
// state waves before B1 (while V_new is computed), V waves after B1 (while
// the state is updated), output waves before B1. A full vector-memory queue
// then stalls a wave that has nothing on the chain.
//
// Workgroup ids are mapped so that the V/16 workgroups of one (sequence,
// head) get ids congruent modulo 8: with round-robin dispatch over the 8
// XCDs they share one L2, which then serves the repeated reads of W, qg, kg
// and Aqk. Variable-length sequences are visited longest first.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int kThreads34 = 768;

__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// operands of one chunk for a V wave
template <typename T, int K>
struct VFrags {
  static constexpr int NKB = K / 32;
  typename Vec<T>::x8 w[NKB];   // W rows of this wave's 16-row block
  typename Vec<T>::x4 u;        // U, accumulator layout
};

// operands of one chunk for an output wave
template <typename T, int K>
struct OFrags {
  static constexpr int NKB = K / 32;
  typename Vec<T>::x8 qg[NKB];  // qg rows of this wave's block
  typename Vec<T>::x8 aq[2];    // Aqk rows of this wave's block
};

// operands of one chunk for a state wave
template <typename T, int K>
struct StateFrags {
  static constexpr int TPW = K / 64;
  typename Vec<T>::x8 kg[TPW][2];  // kg^T rows of this wave's state tiles
  float gam;                       // gamma of channel 16 TPW s + lane % (16 TPW)
};

// Fragment loads go through a buffer resource covering one record: a uniform
// descriptor and a single per-lane offset register shared by every load.
__device__ __forceinline__ void bload(bf16x8& d, __amdgpu_buffer_rsrc_t r, int lane_off, int soff) {
  d = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, soff, 0));
}
__device__ __forceinline__ void bload(floatx8& d, __amdgpu_buffer_rsrc_t r, int lane_off, int soff) {
  const floatx4 a = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, 2 * lane_off, soff, 0));
  const floatx4 b = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, 2 * lane_off + 16, soff, 0));
  d = stackf(a, b);
}
__device__ __forceinline__ void bload4(bf16x4& d, __amdgpu_buffer_rsrc_t r, int lane_off, int soff) {
  d = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, lane_off / 2, soff, 0));
}
__device__ __forceinline__ void bload4(floatx4& d, __amdgpu_buffer_rsrc_t r, int lane_off, int soff) {
  d = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, soff, 0));
}

// lane_off = 16 * lane; frag8 fragments are 64 * 8 elements, accumulator-layout
// fragments 64 * 4 elements. Every lane-byte loaded here passes the CU's
// vector-memory path, whose rate bounds a chunk step, so nothing is loaded
// twice: gamma comes as one float per lane and is spread by lane shuffles.
template <typename T, int K>
__device__ __forceinline__ void load_v(VFrags<T, K>& f, __amdgpu_buffer_rsrc_t rs, const Stage34Args& a, int r,
                                       int lane_off, int vb) {
  constexpr int NKB = K / 32;
  constexpr int F8B = 512 * (int)sizeof(T);  // bytes of one frag8 fragment
  constexpr int F4B = 256 * (int)sizeof(T);  // bytes of one accumulator fragment
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) bload(f.w[kb], rs, lane_off, (int)a.off_w + (r * NKB + kb) * F8B);
  bload4(f.u, rs, lane_off, (int)a.off_u + (vb * 4 + r) * F4B);
}

template <typename T, int K>
__device__ __forceinline__ void load_o(OFrags<T, K>& f, __amdgpu_buffer_rsrc_t rs, const Stage34Args& a, int r,
                                       int lane_off) {
  constexpr int NKB = K / 32;
  constexpr int F8B = 512 * (int)sizeof(T);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) bload(f.qg[kb], rs, lane_off, (int)a.off_qg + (r * NKB + kb) * F8B);
  // every wave issues both Aqk loads (no branch around a load keeps the
  // compiler's memory-counter waits exact); rows < 32 have no second block and
  // point that load past the end of the record, where it reads zeros without
  // touching memory
  bload(f.aq[0], rs, lane_off, (int)a.off_aq + aq_frag(r, 0) * F8B);
  bload(f.aq[1], rs, lane_off, r >= 2 ? (int)a.off_aq + aq_frag(r, 1) * F8B : (int)a.rec_bytes);
}

template <typename T, int K>
__device__ __forceinline__ void load_state(StateFrags<T, K>& f, __amdgpu_buffer_rsrc_t rs, const Stage34Args& a,
                                           int s, int lane_off, int gam_off) {
  constexpr int TPW = K / 64;
  constexpr int F8B = 512 * (int)sizeof(T);
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int rt = s * TPW + m;
    bload(f.kg[m][0], rs, lane_off, (int)a.off_kg + (rt * 2 + 0) * F8B);
    bload(f.kg[m][1], rs, lane_off, (int)a.off_kg + (rt * 2 + 1) * F8B);
  }
  f.gam = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        rs, gam_off, (int)a.off_gam + 64 * TPW * s, 0));
}

template <typename T, int K, int NB>
__global__ __launch_bounds__(kThreads34) void stage34_kernel(Stage34Args a) {
  constexpr int C = kChunk;
  constexpr int V = K;
  constexpr int NKB = K / 32;
  constexpr int NVB = V / 16;
  constexpr int TPW = K / 64;      // 16-row state tiles per state wave
  constexpr int NST = K / 16;      // state tiles
  typedef typename Vec<T>::x4 F4;
  typedef typename Vec<T>::x8 F8;

  __shared__ F4 sS[2][NST][64];    // state block as B-operand halves, by chunk parity
  __shared__ F4 sVn[2][4][64];     // V_new block as B-operand halves, by chunk parity

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: conditions on it must compile to scalar branches,
  // because an MFMA placed under an EXEC mask still executes for all lanes
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = w >> 2;         // 0: V waves, 1: state waves, 2: output waves
  const int r0 = w & 3;
  const int gq = lane >> 4;
  const int xi = lane & 15;

  // XCD-aware id mapping: ids with equal id % 8 run on the same XCD
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int u = (slot / NVB) * 8 + xcd;
  const int vb = slot % NVB;
  if (u >= a.nunits) return;
  const int H = a.H;
  int seq = u / H;
  const int h = u - seq * H;

  // chunk c of this sequence starts at token tfirst + 64 c; every chunk but the
  // last is full, the last holds lastlen tokens
  size_t p0;
  int nch;
  int64_t tfirst;
  int lastlen = kChunk;
  if (a.varlen) {
    const int2* ctab = reinterpret_cast<const int2*>(a.ws + a.off_chunk_tab);
    seq = reinterpret_cast<const int*>(a.ws + a.off_order)[seq];
    const int2 st = reinterpret_cast<const int2*>(a.ws + a.off_seq_tab)[seq];
    p0 = (size_t)st.x;
    nch = st.y;
    tfirst = nch > 0 ? (int64_t)ctab[p0].x : 0;
    if (nch > 0) lastlen = ctab[p0 + nch - 1].y;
  } else {
    p0 = (size_t)seq * a.nt;
    nch = a.nt;
    tfirst = (int64_t)p0 * kChunk;
  }
  const int last = nch - 1;
  const size_t state_base = ((size_t)seq * H + h) * K * V + 16 * vb + xi;
  // buffer resource over exactly one record (chunk cc of this sequence, head h;
  // records are chunk-major): offsets past the record read zeros
  auto rec_rsrc = [&](int c) {
    const int cc = c < last ? c : last;  // prefetches past the end re-read the last chunk
    const char* base = a.ws + a.meta_bytes + (((size_t)p0 + cc) * H + h) * a.rec_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)a.rec_bytes, 0x00020000);
  };
  const int lane_off = 16 * lane;

  if (nch <= 0) {  // empty sequence: final state = initial state (uniform branch, no barriers)
    if (role == 1 && a.final_state) {
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const int rt = (r0)*TPW + m;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const size_t i = state_base + (size_t)(16 * rt + 4 * gq + r) * V;
          a.final_state[i] = a.init ? a.init[i] : 0.f;
        }
      }
    }
    return;
  }
  // whole ring passes with a single exit: steps past the last chunk only issue
  // their (clamped) loads. An exit inside a pass, or a separate tail, would
  // make the memory-counter waits at the top of a pass cover the ring. Every
  // role passes 1 + 2 (npass NB + 1) barriers.
  const int npass = (nch + NB - 1) / NB;

  if (role == 1) {
    // ------------------------------------------------------------ state waves
    const int s = r0;
    floatx4 S[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int rt = s * TPW + m;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[m][r] = a.init ? a.init[state_base + (size_t)(16 * rt + 4 * gq + r) * V] : 0.f;
      F4 y;
      cvt4(S[m], y);
      sS[0][rt][lane] = y;
    }
    StateFrags<T, K> F[NB];
    const int gam_off = 4 * (lane % (16 * TPW));
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) {
      load_state<T, K>(F[i], rec_rsrc(i), a, s, lane_off, gam_off);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();  // initial state published
    auto step = [&](StateFrags<T, K>& f, StateFrags<T, K>& next, int c) {
      load_state<T, K>(next, rec_rsrc(c + NB - 1), a, s, lane_off, gam_off);
      lds_sync();  // B1: V_new of chunk c published
      if (c < nch) {  // uniform: every role skips the same steps, barriers included
        const F8 Vb0 = stack8<T>(sVn[c & 1][0][lane], sVn[c & 1][1][lane]);
        const F8 Vb1 = stack8<T>(sVn[c & 1][2][lane], sVn[c & 1][3][lane]);
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
          floatx4 gm;
#pragma unroll
          for (int r = 0; r < 4; ++r) gm[r] = __shfl(f.gam, 16 * m + 4 * gq + r, 64);
          S[m] = S[m] * gm;
          S[m] = mma32(S[m], f.kg[m][0], Vb0);
          S[m] = mma32(S[m], f.kg[m][1], Vb1);
          F4 y;
          cvt4(S[m], y);
          sS[(c + 1) & 1][s * TPW + m][lane] = y;
        }
      }
      lds_sync();  // B2: state after chunk c published
    };
    for (int p = 0; p < npass; ++p) {
#pragma unroll
      for (int j = 0; j < NB; ++j) step(F[j], F[(j + NB - 1) % NB], p * NB + j);
    }
    lds_sync();  // the output waves' last chunk
    lds_sync();
    if (a.final_state) {
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const int rt = s * TPW + m;
#pragma unroll
        for (int r = 0; r < 4; ++r) a.final_state[state_base + (size_t)(16 * rt + 4 * gq + r) * V] = S[m][r];
      }
    }
  } else if (role == 0) {
    // ---------------------------------------------------------------- V waves
    VFrags<T, K> F[NB];
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) {
      load_v<T, K>(F[i], rec_rsrc(i), a, r0, lane_off, vb);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();  // initial state published
    auto step = [&](VFrags<T, K>& f, VFrags<T, K>& next, int c) {
      if (c < nch) {
        floatx4 accV = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          accV = mma32(accV, f.w[kb], stack8<T>(sS[c & 1][2 * kb][lane], sS[c & 1][2 * kb + 1][lane]));
        const floatx4 vn = widen4(f.u) - accV;
        F4 vnT;
        cvt4(vn, vnT);
        sVn[c & 1][r0][lane] = vnT;
      }
      lds_sync();  // B1: V_new of chunk c published
      load_v<T, K>(next, rec_rsrc(c + NB - 1), a, r0, lane_off, vb);
      lds_sync();  // B2
    };
    for (int p = 0; p < npass; ++p) {
#pragma unroll
      for (int j = 0; j < NB; ++j) step(F[j], F[(j + NB - 1) % NB], p * NB + j);
    }
    lds_sync();  // the output waves' last chunk
    lds_sync();
  } else {
    // ----------------------------------------------------------- output waves
    // chunk d is written in the step after its own: its chunk-start state and
    // V_new stay in the other parity's LDS buffers until the step after that
    T* out = reinterpret_cast<T*>(a.o);
    T* sink = reinterpret_cast<T*>(const_cast<char*>(a.ws) + a.off_sink);
    OFrags<T, K> F[NB];
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) {
      load_o<T, K>(F[i], rec_rsrc(i), a, r0, lane_off);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();  // initial state published
    lds_sync();  // step of chunk 0: nothing to write yet
    lds_sync();
    auto step = [&](OFrags<T, K>& f, OFrags<T, K>& next, int d) {
      // before B1: take S_d (overwritten in this step's second half) and issue loads
      F8 Sb[NKB];
      if (d < nch) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) Sb[kb] = stack8<T>(sS[d & 1][2 * kb][lane], sS[d & 1][2 * kb + 1][lane]);
      }
      load_o<T, K>(next, rec_rsrc(d + NB - 1), a, r0, lane_off);
      lds_sync();  // B1
      const int64_t tok0 = tfirst + (int64_t)d * C;
      const int len = d < nch - 1 ? C : (d == nch - 1 ? lastlen : 0);
      // accO is built transposed (operands swapped): lane (g, i) then holds chunk
      // row 16 r0 + i at the four consecutive columns 16 vb + 4 g .. + 3, which
      // leaves as one vector store per lane
      floatx4 accO = zero4();
      if (d < nch) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) accO = mma32(accO, Sb[kb], f.qg[kb]);
        // intra-chunk part, causal: row block r0 reads V_new blocks <= r0
        accO = mma32(accO, stack8<T>(sVn[d & 1][0][lane], sVn[d & 1][1][lane]), f.aq[0]);
        if (r0 >= 2) accO = mma32(accO, stack8<T>(sVn[d & 1][2][lane], sVn[d & 1][3][lane]), f.aq[1]);
      }
      // rows past the end of a short chunk, and every row of a step past the
      // last chunk, store into the sink: the store is never under a branch
      const int row = 16 * r0 + xi;
      F4 y;
      cvt4(accO, y);
      T* dst = row < len ? out + ((size_t)(tok0 + row) * H + h) * V + 16 * vb + 4 * gq : sink;
      *reinterpret_cast<F4*>(dst) = y;
      lds_sync();  // B2
    };
    for (int p = 0; p < npass; ++p) {
#pragma unroll
      for (int j = 0; j < NB; ++j) step(F[j], F[(j + NB - 1) % NB], p * NB + j);
    }
  }
}

}  // namespace

hipError_t launch_stage34(const Stage34Args& a, int K, int bf16, hipStream_t s) {
  if (a.nunits <= 0) return hipSuccess;
  const int nvb = K / 16;
  const int units8 = (a.nunits + 7) / 8;
  dim3 grid(units8 * 8 * nvb), block(kThreads34);
  if (bf16) {
    if (K == 128) hipLaunchKernelGGL((stage34_kernel<kda::bf16, 128, 4>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage34_kernel<kda::bf16, 64, 4>), grid, block, 0, s, a);
  } else {
    if (K == 128) hipLaunchKernelGGL((stage34_kernel<float, 128, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stage34_kernel<float, 64, 4>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kda
