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
// The workgroup has 8 waves in two roles:
//   row waves 0..3   - wave r computes V_new and O for chunk rows 16 r .. 16 r + 15
//   state waves 4..7 - hold the K x 16 fp32 state block in MFMA accumulators
//                      (K / 64 tiles of 16 rows each) and apply the update.
// Per chunk the row waves publish V_new and the state waves publish the new
// state (both as MFMA B-operand halves) through LDS; both roles pass the
// same two barriers per chunk. The chunk operands are read as ready-made MFMA
// fragments from the stage-1+2 record through a ring of NB register buffers,
// NB - 1 chunks ahead of use.
//
// Workgroup ids are mapped so that the V/16 workgroups of one (sequence,
// head) get ids congruent modulo 8: with round-robin dispatch over the 8
// XCDs they share one L2, which then serves the repeated reads of W, qg, kg
// and Aqk. Variable-length sequences are visited longest first.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int kThreads34 = 512;

__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// operands of one chunk for a row wave
template <typename T, int K>
struct RowFrags {
  static constexpr int NKB = K / 32;
  typename Vec<T>::x8 w[NKB];   // W rows of this wave's 16-row block
  typename Vec<T>::x8 qg[NKB];  // qg rows of this wave's block
  typename Vec<T>::x8 aq[2];    // Aqk rows of this wave's block
  typename Vec<T>::x4 u;        // U, accumulator layout
};

// operands of one chunk for a state wave
template <typename T, int K>
struct StateFrags {
  static constexpr int TPW = K / 64;
  typename Vec<T>::x8 kg[TPW][2];  // kg^T rows of this wave's state tiles
  float gam;                       // gamma of channel 16 TPW s + lane % (16 TPW)
};

// Fragment loads go through a buffer resource covering one record: a uniform
// descriptor and a single per-lane offset register shared by every load. With 64-bit per-lane
// addresses instead, the register allocator reuses address registers that are
// still the destination of in-flight loads and the prefetch ring stalls.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
template <typename T, int K, bool OUT>
__device__ __forceinline__ void load_row(RowFrags<T, K>& f, __amdgpu_buffer_rsrc_t rs, int soff,
                                         const Stage34Args& a, int r, int lane_off, int vb) {
  constexpr int NKB = K / 32;
  constexpr int F8B = 512 * (int)sizeof(T);  // bytes of one frag8 fragment
  constexpr int F4B = 256 * (int)sizeof(T);  // bytes of one accumulator fragment
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    bload(f.w[kb], rs, lane_off, soff + (int)a.off_w + (r * NKB + kb) * F8B);
    if constexpr (OUT) bload(f.qg[kb], rs, lane_off, soff + (int)a.off_qg + (r * NKB + kb) * F8B);
  }
  // every wave issues both Aqk loads (no branch around a load keeps the
  // compiler's memory-counter waits exact); rows < 32 have no second block and
  // point that load past the end of the record, where it reads zeros without
  // touching memory. Without an output (OUT false) qg and Aqk are not needed.
  if constexpr (OUT) {
    bload(f.aq[0], rs, lane_off, soff + (int)a.off_aq + aq_frag(r, 0) * F8B);
    bload(f.aq[1], rs, lane_off, r >= 2 ? soff + (int)a.off_aq + aq_frag(r, 1) * F8B : (int)a.rec_bytes);
  }
  bload4(f.u, rs, lane_off, soff + (int)a.off_u + (vb * 4 + r) * F4B);
}

template <typename T, int K>
__device__ __forceinline__ void load_state(StateFrags<T, K>& f, __amdgpu_buffer_rsrc_t rs, int soff,
                                           const Stage34Args& a, int s, int lane_off, int gam_off) {
  constexpr int TPW = K / 64;
  constexpr int F8B = 512 * (int)sizeof(T);
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int rt = s * TPW + m;
    bload(f.kg[m][0], rs, lane_off, soff + (int)a.off_kg + (rt * 2 + 0) * F8B);
    bload(f.kg[m][1], rs, lane_off, soff + (int)a.off_kg + (rt * 2 + 1) * F8B);
  }
  f.gam = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        rs, gam_off, soff + (int)a.off_gam + 64 * TPW * s, 0));
}

// OUT false: no output o (affine summaries, final state only); the row waves
// then load neither qg nor Aqk and skip the output products.
template <typename T, int K, int NB, bool OUT>
__global__ __launch_bounds__(kThreads34) void stage34_kernel(Stage34Args a) {
  constexpr int C = kChunk;
  constexpr int V = K;
  constexpr int NKB = K / 32;
  constexpr int NVB = V / 16;
  constexpr int TPW = K / 64;      // 16-row state tiles per state wave
  constexpr int NST = K / 16;      // state tiles
  typedef typename Vec<T>::x4 F4;
  typedef typename Vec<T>::x8 F8;

  __shared__ F4 sS[NST][64];       // state block as B-operand halves
  __shared__ F4 sVn[4][64];        // V_new block as B-operand halves

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: conditions on it must compile to scalar branches,
  // because an MFMA placed under an EXEC mask still executes for all lanes
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    tfirst = (int64_t)seq * a.row_T + a.seg_t0;
  }
  const int last = nch - 1;
  const size_t state_base = ((size_t)seq * H + h) * K * V + 16 * vb + xi;
  // buffer resource over exactly one record (chunk cc of this sequence, head h;
  // records are chunk-major): offsets past the record read zeros
  auto rec_rsrc = [&](int cc) {
    const char* base = a.ws + a.meta_bytes + (((size_t)p0 + cc) * H + h) * a.rec_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)a.rec_bytes, 0x00020000);
  };
  const int lane_off = 16 * lane;

  if (w >= 4) {
    // ------------------------------------------------------------ state waves
    const int s = w - 4;
    floatx4 S[TPW];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int rt = s * TPW + m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // identity start: state row 16 rt + 4 gq + r, column 16 vb + xi
        const float id = (16 * rt + 4 * gq + r == 16 * vb + xi) ? 1.f : 0.f;
        S[m][r] = a.init_identity ? id : a.init ? a.init[state_base + (size_t)(16 * rt + 4 * gq + r) * V] : 0.f;
      }
      F4 y;
      cvt4(S[m], y);
      sS[rt][lane] = y;
    }
    if (nch > 0) {
      StateFrags<T, K> F[NB];
      // prefetches are unconditional (chunk index clamped to the last chunk): with
      // no branch around the loads the memory-counter waits stay exact
      auto issue = [&](StateFrags<T, K>& f, int c) {
        const int cc = c < last ? c : last;
        load_state<T, K>(f, rec_rsrc(cc), 0, a, s, lane_off, 4 * (lane % (16 * TPW)));
      };
      // the prologue loads stay in chunk order (no scheduling across the barriers):
      // the memory-counter wait at the top of each ring pass is computed from
      // the worst case over the loop entry and the back edge
#pragma unroll
      for (int i = 0; i < NB - 1; ++i) {
        issue(F[i], i);
        __builtin_amdgcn_sched_barrier(0);
      }
      lds_sync();  // initial state published
      auto step = [&](StateFrags<T, K>& f, StateFrags<T, K>& next, int c) {
        issue(next, c + NB - 1);
        if (c < nch) {  // uniform: both roles skip the same steps, barriers included
          lds_sync();   // V_new of chunk c published
          const F8 Vb0 = stack8<T>(sVn[0][lane], sVn[1][lane]);
          const F8 Vb1 = stack8<T>(sVn[2][lane], sVn[3][lane]);
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
            sS[s * TPW + m][lane] = y;
          }
          lds_sync();  // state after chunk c published
        }
      };
      // whole ring passes with a single exit: steps past the last chunk only
      // issue their (clamped) loads. An exit inside a pass, or a separate tail,
      // would make the memory-counter waits at the top of a pass cover the ring.
      const int npass = (nch + NB - 1) / NB;
      for (int p = 0; p < npass; ++p) {
#pragma unroll
        for (int j = 0; j < NB; ++j) step(F[j], F[(j + NB - 1) % NB], p * NB + j);
      }
    }
    if (a.final_state) {
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const int rt = s * TPW + m;
#pragma unroll
        for (int r = 0; r < 4; ++r) a.final_state[state_base + (size_t)(16 * rt + 4 * gq + r) * V] = S[m][r];
      }
    }
  } else {
    // -------------------------------------------------------------- row waves
    if (nch <= 0) return;
    const int r0 = w;  // chunk rows 16 r0 .. 16 r0 + 15
    T* out = reinterpret_cast<T*>(a.o);
    T* sink = reinterpret_cast<T*>(const_cast<char*>(a.ws) + a.off_sink);
    RowFrags<T, K> F[NB];
    auto issue = [&](RowFrags<T, K>& f, int c) {
      const int cc = c < last ? c : last;
      load_row<T, K, OUT>(f, rec_rsrc(cc), 0, a, r0, lane_off, vb);
    };
    // prologue loads in chunk order (see the state waves)
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) {
      issue(F[i], i);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_sync();  // initial state published
    auto step = [&](RowFrags<T, K>& f, RowFrags<T, K>& next, int c) {
      const int64_t tok0 = tfirst + (int64_t)c * C;
      const int len = c < nch - 1 ? C : (c == nch - 1 ? lastlen : 0);
      // critical part first: V_new = U - W S feeds the state waves
      F8 Sb[NKB];
      if (c < nch) {  // uniform, as in the state waves
        floatx4 accV = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          Sb[kb] = stack8<T>(sS[2 * kb][lane], sS[2 * kb + 1][lane]);
          accV = mma32(accV, f.w[kb], Sb[kb]);
        }
        const floatx4 vn = (a.zero_u ? zero4() : widen4(f.u)) - accV;
        F4 vnT;
        cvt4(vn, vnT);
        sVn[r0][lane] = vnT;
        lds_sync();  // V_new of chunk c published
      }
      // the next loads are issued while the state waves apply the update; a
      // full vector-memory queue then stalls this wave, not the chain
      issue(next, c + NB - 1);
      // accO is built transposed (operands swapped): lane (g, i) then holds chunk
      // row 16 r0 + i at the four consecutive columns 16 vb + 4 g .. + 3, which
      // leaves as one vector store per lane
      floatx4 accO = zero4();
      if (c < nch) {
        if constexpr (OUT) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) accO = mma32(accO, Sb[kb], f.qg[kb]);
          const F8 Vb0 = stack8<T>(sVn[0][lane], sVn[1][lane]);
          const F8 Vb1 = stack8<T>(sVn[2][lane], sVn[3][lane]);
          // intra-chunk part, causal: row block r0 reads V_new blocks <= r0
          accO = mma32(accO, Vb0, f.aq[0]);
          if (r0 >= 2) accO = mma32(accO, Vb1, f.aq[1]);
        }
        lds_sync();  // state after chunk c published
      }
      if constexpr (OUT) {
        // rows past the end of a short chunk, and every row of a step past the
        // last chunk, store into the sink: the store is never under a branch
        const int row = 16 * r0 + xi;
        F4 y;
        cvt4(accO, y);
        T* dst = (row < len && out) ? out + ((size_t)(tok0 + row) * H + h) * V + 16 * vb + 4 * gq : sink;
        *reinterpret_cast<F4*>(dst) = y;
      }
    };
    // whole ring passes with a single exit (see the state waves)
    const int npass = (nch + NB - 1) / NB;
    for (int p = 0; p < npass; ++p) {
#pragma unroll
      for (int j = 0; j < NB; ++j) step(F[j], F[(j + NB - 1) % NB], p * NB + j);
    }
  }
}

// S_out[:, j] = M S0[:, j] + N[:, j]; block = (pair u, 64 columns), wave w
// handles rows w, w + 4, ...; each lane keeps its column of S0 in registers.
template <int K>
__global__ __launch_bounds__(256) void affine_apply_kernel(const float* M, const float* N, const float* S0,
                                                            float* S_out) {
  constexpr int V = K;
  constexpr int NCB = V / 64;
  const int u = blockIdx.x / NCB;
  const int j = (blockIdx.x % NCB) * 64 + (threadIdx.x & 63);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t base = (size_t)u * K * V;
  float s0[K];
#pragma unroll
  for (int l = 0; l < K; ++l) s0[l] = S0[base + (size_t)l * V + j];
  for (int i = w; i < K; i += 4) {
    const float* mrow = M + (size_t)u * K * K + (size_t)i * K;
    float acc = N[base + (size_t)i * V + j];
#pragma unroll
    for (int l = 0; l < K; ++l) acc += mrow[l] * s0[l];
    S_out[base + (size_t)i * V + j] = acc;
  }
}

}  // namespace

hipError_t launch_affine_apply(const float* M, const float* N, const float* S0, float* S_out, int nunits, int K,
                               hipStream_t s) {
  if (nunits <= 0) return hipSuccess;
  const dim3 grid((unsigned)(nunits * (K / 64))), block(256);
  if (K == 128) hipLaunchKernelGGL(affine_apply_kernel<128>, grid, block, 0, s, M, N, S0, S_out);
  else hipLaunchKernelGGL(affine_apply_kernel<64>, grid, block, 0, s, M, N, S0, S_out);
  return hipGetLastError();
}

hipError_t launch_stage34(const Stage34Args& a, int K, int bf16, hipStream_t s) {
  if (a.nunits <= 0) return hipSuccess;
  const int nvb = K / 16;
  const int units8 = (a.nunits + 7) / 8;
  dim3 grid(units8 * 8 * nvb), block(kThreads34);
  if (a.o) {
    if (bf16) {
      if (K == 128) hipLaunchKernelGGL((stage34_kernel<kda::bf16, 128, 4, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((stage34_kernel<kda::bf16, 64, 4, true>), grid, block, 0, s, a);
    } else {
      if (K == 128) hipLaunchKernelGGL((stage34_kernel<float, 128, 2, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((stage34_kernel<float, 64, 4, true>), grid, block, 0, s, a);
    }
  } else {
    if (bf16) {
      if (K == 128) hipLaunchKernelGGL((stage34_kernel<kda::bf16, 128, 4, false>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((stage34_kernel<kda::bf16, 64, 4, false>), grid, block, 0, s, a);
    } else {
      if (K == 128) hipLaunchKernelGGL((stage34_kernel<float, 128, 2, false>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((stage34_kernel<float, 64, 4, false>), grid, block, 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace kda
