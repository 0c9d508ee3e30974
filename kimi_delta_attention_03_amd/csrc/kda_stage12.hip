// Stage 1+2 of the chunkwise KDA forward on gfx950. Workgroups (4 waves) are
// persistent: each loops over (chunk, head) items, keeps everything an item
// needs in LDS and writes the outputs once, as MFMA fragments, into the item's
// workspace record. The raw inputs of the next item are loaded into registers
// as soon as the current item has consumed them.
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
//
// Inputs are read with buffer loads whose descriptor covers exactly the valid
// rows of the chunk: rows past the end of a short (variable-length) chunk read
// as zeros, so no load sits behind a branch.
#include <atomic>

#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// block-wide LDS synchronisation without waiting for global memory traffic
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 4 consecutive elements of T as a raw register value
template <typename T> struct Raw4;
template <> struct Raw4<bf16> { typedef u32x2 type; };
template <> struct Raw4<float> { typedef u32x4 type; };

template <typename T>
__device__ __forceinline__ typename Raw4<T>::type bload4(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (sizeof(T) == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ floatx4 bf16pair4(uint32_t a, uint32_t b) {
  return floatx4{__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u),
                 __uint_as_float(b << 16), __uint_as_float(b & 0xffff0000u)};
}
template <typename T>
__device__ __forceinline__ floatx4 unpack4(const typename Raw4<T>::type& x) {
  if constexpr (sizeof(T) == 2) return bf16pair4(x[0], x[1]);
  else return floatx4{__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3])};
}

// squares of the elements in a 16-byte chunk of T
template <typename T>
__device__ __forceinline__ float sumsq16(const u32x4& u) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {  // two bf16 per word: the high half is the bf16 bit pattern
      const float lo = __uint_as_float(u[i] << 16), hi = __uint_as_float(u[i] & 0xffff0000u);
      s += lo * lo + hi * hi;
    } else {
      const float x = __uint_as_float(u[i]);
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

// descriptor over rows [0, len) of a [tokens, H, rowbytes] tensor, starting at
// (token tok0, head h)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* p, int64_t tok0, int h, int H,
                                                            int rowbytes, int len) {
  const char* base = reinterpret_cast<const char*>(p) + ((size_t)tok0 * H + h) * (size_t)rowbytes;
  const int n = len > 0 ? (len - 1) * H * rowbytes + rowbytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, n, 0x00020000);
}

// GATE: g holds raw gate values and phase 1 applies the activation of the
// Tokamax "chunk_kda_fwd design doc", section 9.1.3, with x = raw + dt_bias and
// lambda = exp(A_log_h): g = -lambda softplus(x) (mode 1) or
// g = lower_bound * sigmoid(lambda x) (mode 2). Rows past the end of a short
// chunk keep g = 0 (identity decay), as for pre-activated gates.
template <typename T, int K, bool GF32, bool GATE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1)))
void stage12_kernel(Stage12Args a) {
  constexpr int C = kChunk;
  constexpr int V = K;
  constexpr int E = (int)sizeof(T);
  constexpr int NKB = K / 32;          // 32-wide channel blocks
  constexpr int GS = K + 4;            // sG row stride (floats)
  constexpr int KS = (E == 2) ? K + 8 : K + 4;  // sK / sV row stride (elements)
  constexpr int AS = C + 4;            // sA row stride (floats)
  constexpr int EPC = 16 / E;          // elements per 16-byte chunk
  constexpr int CPR = K / EPC;         // 16-byte chunks per row
  constexpr int NCH = C * CPR / kThreads;  // chunks per thread for a C x K tile
  constexpr int kRowStep = kThreads / CPR; // rows between a thread's chunks
  constexpr int CPT = K / 16;          // gate channels per thread in the cumsum
  constexpr int SEG = 16;              // row segments of the cumsum
  constexpr int RPS = C / SEG;         // rows per segment
  constexpr int GB = CPT * (GF32 ? 4 : 2);       // gate bytes per thread and row
  constexpr int GL = GB / 16 > 0 ? GB / 16 : 1;  // 16-byte gate loads per row (8-byte if GB == 8)
  constexpr bool kPrefetch = true;      // fp32 runs one wave per SIMD and has the registers too
  static_assert(NCH * kThreads == C * CPR, "tile split");
  static_assert(kThreads % CPR == 0, "rows per step");

  __shared__ __attribute__((aligned(16))) float sG[C * GS];   // G, later V (as T)
  __shared__ __attribute__((aligned(16))) T sK[C * KS];
  __shared__ __attribute__((aligned(16))) float sA[C * AS];   // scratch, L, then A
  __shared__ float sB[C], sKn[C];
  T* sV = reinterpret_cast<T*>(sG);
  static_assert(sizeof(T) * C * KS <= sizeof(float) * C * GS, "sV fits in sG");
  static_assert(SEG * K <= C * AS, "cumsum totals fit in sA");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar: conditions on it must compile to scalar branches,
  // because an MFMA placed under an EXEC mask still executes for all lanes
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4;
  const int xi = lane & 15;
  const int H = a.H;
  const int nitems = (a.varlen ? *reinterpret_cast<const int*>(a.ws) : (int)a.ncp) * H;
  if ((int)blockIdx.x >= nitems) return;

  // per-thread constant byte offsets inside one (chunk, head) row block
  const int RBK = K * E, RBV = V * E, RBG = K * (GF32 ? 4 : 2), RBB = a.beta_f32 ? 4 : 2;
  const int kv_row = tid / CPR, kv_col = (tid % CPR) * EPC;
  const int off_k0 = kv_row * H * RBK + kv_col * E;
  const int off_v0 = kv_row * H * RBV + kv_col * E;
  const int kstep = kRowStep * H * RBK, vstep = kRowStep * H * RBV;
  const int cg = tid % 16, seg = tid / 16;
  const int off_g0 = seg * RPS * H * RBG + cg * CPT * (GF32 ? 4 : 2);
  const int irow = 16 * w + xi;
  const int off_q0 = irow * H * RBK + 4 * gq * E;
  const int off_b = (tid & 63) * H * RBB;

  struct Item { int p, h, len; int64_t tok0; };
  const int2* ctab = reinterpret_cast<const int2*>(a.ws + a.off_chunk_tab);
  auto item_of = [&](int it) {
    Item r;
    r.p = it / H;
    r.h = it - r.p * H;
    if (a.varlen) {
      const int2 ct = ctab[r.p];
      r.tok0 = ct.x;
      r.len = ct.y;
    } else {
      const int row = r.p / a.nt_seg;
      r.tok0 = (int64_t)row * a.row_T + a.seg_t0 + (int64_t)(r.p - row * a.nt_seg) * C;
      r.len = C;
    }
    return r;
  };

  // raw inputs of one item, as loaded
  struct RawIn {
    u32x4 k[NCH], v[NCH];
    u32x4 g[RPS][GL];
    typename Raw4<T>::type q[NKB][2];
    uint32_t b;
    float gbias[GATE ? CPT : 1];  // dt_bias of this thread's gate channels (GATE only)
    float alog;                   // A_log of the item's head (GATE only)
  };
  // the raw inputs are loaded in three groups, each as soon as the previous
  // item has consumed its registers: k, g, beta (phase 1), q (phase 2), v (phase 5)
  auto issue_q = [&](RawIn& r, const Item& it) {
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(a.q, it.tok0, it.h, H, RBK, it.len);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      r.q[kb][0] = bload4<T>(rq, off_q0 + 32 * kb * E);
      r.q[kb][1] = bload4<T>(rq, off_q0 + (32 * kb + 16) * E);
    }
  };
  auto issue_kgb = [&](RawIn& r, const Item& it) {
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(a.k, it.tok0, it.h, H, RBK, it.len);
    const __amdgpu_buffer_rsrc_t rg = rows_rsrc(a.g, it.tok0, it.h, H, RBG, it.len);
    const __amdgpu_buffer_rsrc_t rb = rows_rsrc(a.beta, it.tok0, it.h, H, RBB, it.len);
#pragma unroll
    for (int m = 0; m < NCH; ++m) r.k[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_k0 + m * kstep, 0, 0);
#pragma unroll
    for (int rr = 0; rr < RPS; ++rr) {
#pragma unroll
      for (int l = 0; l < GL; ++l) {
        if constexpr (GB >= 16) {
          r.g[rr][l] = __builtin_amdgcn_raw_buffer_load_b128(rg, off_g0 + rr * H * RBG + 16 * l, 0, 0);
        } else {
          const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rg, off_g0 + rr * H * RBG, 0, 0);
          r.g[rr][l] = u32x4{x[0], x[1], 0u, 0u};
        }
      }
    }
    r.b = a.beta_f32 ? __builtin_amdgcn_raw_buffer_load_b32(rb, off_b, 0, 0)
                     : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, off_b, 0, 0);
    if constexpr (GATE) {
      r.alog = a.A_log[it.h];
#pragma unroll
      for (int c = 0; c < CPT; ++c) r.gbias[c] = a.dt_bias ? a.dt_bias[(size_t)it.h * K + cg * CPT + c] : 0.f;
    }
  };
  auto issue_v = [&](RawIn& r, const Item& it) {
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(a.v, it.tok0, it.h, H, RBV, it.len);
#pragma unroll
    for (int m = 0; m < NCH; ++m) r.v[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, off_v0 + m * vstep, 0, 0);
  };

  RawIn R;
  if constexpr (kPrefetch) {
    const Item it0 = item_of(blockIdx.x);
    issue_kgb(R, it0);
    issue_q(R, it0);
    issue_v(R, it0);
  }

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const Item it = item_of(item);
    const int nxt = item + (int)gridDim.x < nitems ? item + (int)gridDim.x : nitems - 1;
    const Item nx = item_of(nxt);
    if constexpr (!kPrefetch) {
      issue_kgb(R, it);
      issue_q(R, it);
      issue_v(R, it);
    }
    const int p = it.p, h = it.h;
    char* rec = a.ws + a.meta_bytes + ((size_t)p * H + h) * a.rec_bytes;  // chunk-major

    // ---------------- phase 1: beta, k -> LDS, k norms, gate cumsum
    if (tid < C) {
      const uint32_t bw = R.b;
      sB[tid] = a.beta_f32 ? __uint_as_float(bw) : __uint_as_float(bw << 16);
    }
#pragma unroll
    for (int m = 0; m < NCH; ++m)
      *reinterpret_cast<u32x4*>(sK + (kv_row + m * kRowStep) * KS + kv_col) = R.k[m];
    if (a.l2norm) {
      // rows are owned by CPR consecutive lanes: reduce the squares across them
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        float sk = sumsq16<T>(R.k[m]);
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) sk += __shfl_xor(sk, o, 64);
        if (kv_col == 0) sKn[kv_row + m * kRowStep] = 1.f / fmaxf(sqrtf(sk), a.l2eps);
      }
    } else if (tid < C) {
      sKn[tid] = 1.f;
    }
    // inclusive cumsum over rows: thread (cg, seg) sums its CPT channels over the
    // RPS rows of segment seg. The four segments of a wave sit in its four
    // 16-lane rows (seg % 4 == gq), so their exclusive prefix is a scan across
    // lane rows (permlane swaps); the rows go to sG with that prefix included
    // and the wave's total to sA. After the barrier, the totals of the earlier
    // waves are added and the result is converted to log2 units.
    {
      float lam = 0.f;
      if constexpr (GATE) lam = __expf(R.alog);
      auto gate = [&](int rr, int c) {
        float gv;
        if constexpr (GF32) gv = __uint_as_float(R.g[rr][c / 4][c % 4]);
        else gv = (c & 1) ? __uint_as_float(R.g[rr][c / 8][(c % 8) / 2] & 0xffff0000u)
                          : __uint_as_float(R.g[rr][c / 8][(c % 8) / 2] << 16);
        if constexpr (GATE) {
          const float x = gv + R.gbias[c];
          // hardware exp2 / log2 based exp and log: the activations only need
          // fp32 relative accuracy where the decay is not ~1 anyway
          if (a.gate_mode == 1) {
            const float sp = fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)));  // softplus, stable form
            gv = -lam * sp;
          } else {
            gv = a.gate_lb / (1.f + __expf(-lam * x));  // lower_bound * sigmoid
          }
          if (seg * RPS + rr >= it.len) gv = 0.f;
        }
        return gv;
      };
      auto put_row = [&](int rr, int c, floatx4 x) {
        *reinterpret_cast<floatx4*>(sG + (seg * RPS + rr) * GS + cg * CPT + c) = x;
      };
      // segment totals; with the activation the rows (without the prefix) are
      // stored on the way, so that it is evaluated once
      float run[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) run[c] = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPS; ++rr) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) run[c] += gate(rr, c);
        if constexpr (GATE) {
#pragma unroll
          for (int c = 0; c < CPT; c += 4) put_row(rr, c, floatx4{run[c], run[c + 1], run[c + 2], run[c + 3]});
        }
      }
      // exclusive prefix over lane rows r = 0..3 of the totals x_r:
      // permlane16_swap(x, x) gives {x0, x0, x2, x2} and {x1, x1, x3, x3} by row,
      // permlane32_swap(P, P) of the pair sums P gives {P01 x4} and {P23 x4}
      float pre[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const unsigned xu = __float_as_uint(run[c]);
        const auto a16 = __builtin_amdgcn_permlane16_swap(xu, xu, false, false);
        const float lo = __uint_as_float(a16[0]), hi = __uint_as_float(a16[1]);
        const unsigned Pu = __float_as_uint(lo + hi);
        const auto a32 = __builtin_amdgcn_permlane32_swap(Pu, Pu, false, false);
        const float P01 = __uint_as_float(a32[0]), P23 = __uint_as_float(a32[1]);
        pre[c] = ((gq & 1) ? lo : 0.f) + ((gq & 2) ? P01 : 0.f);
        run[c] = P01 + P23;  // this wave's total
      }
      if (gq == 0) {
#pragma unroll
        for (int c = 0; c < CPT; c += 4)
          *reinterpret_cast<floatx4*>(sA + w * K + cg * CPT + c) = floatx4{run[c], run[c + 1], run[c + 2], run[c + 3]};
      }
      if constexpr (GATE) {
#pragma unroll
        for (int rr = 0; rr < RPS; ++rr) {
#pragma unroll
          for (int c = 0; c < CPT; c += 4) {
            const floatx4 p4{pre[c], pre[c + 1], pre[c + 2], pre[c + 3]};
            put_row(rr, c, ldsf4(sG + (seg * RPS + rr) * GS + cg * CPT + c) + p4);
          }
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < RPS; ++rr) {
#pragma unroll
          for (int c = 0; c < CPT; ++c) pre[c] += gate(rr, c);
#pragma unroll
          for (int c = 0; c < CPT; c += 4) put_row(rr, c, floatx4{pre[c], pre[c + 1], pre[c + 2], pre[c + 3]});
        }
      }
    }
    // k, g and beta of this item are consumed: start loading the next item's
    if constexpr (kPrefetch) issue_kgb(R, nx);
    lds_sync();
    {
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        floatx4 carry = zero4();
#pragma unroll
        for (int s = 0; s < 3; ++s)
          if (s < w) carry += ldsf4(sA + s * K + cg * CPT + c);
#pragma unroll
        for (int rr = 0; rr < RPS; ++rr) {
          float* gp = sG + (seg * RPS + rr) * GS + cg * CPT + c;
          *reinterpret_cast<floatx4*>(gp) = (carry + ldsf4(gp)) * kLog2e;
        }
      }
    }
    lds_sync();

    // ---------------- phase 2: relation tiles for query block w (this wave)
    // Aqk^T and L^T tiles (keys j x queries i) = Khat_j . (Qhat_i | Khat'_i):
    //   Qhat_i = q_i 2^(G_i - r), Khat'_i = k_i 2^(G_i - r), Khat_j = k_j 2^(r - G_j),
    //   r = G of row 16 w.
    {
      const float kni = sKn[irow];
      // q of row irow: this lane holds channels 32 kb + 4 gq + {0..3, 16..19}; the
      // row's L2 norm sums the squares over the 4 lane groups of the row
      float qn = 1.f;
      if (a.l2norm) {
        float qss = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const floatx8 x = stackf(unpack4<T>(R.q[kb][0]), unpack4<T>(R.q[kb][1]));
#pragma unroll
          for (int t = 0; t < 8; ++t) qss += x[t] * x[t];
        }
        qss += __shfl_xor(qss, 16, 64);
        qss += __shfl_xor(qss, 32, 64);
        qn = 1.f / fmaxf(sqrtf(qss), a.l2eps);
      }
      floatx4 accQ[4], accL[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) { accQ[bj] = zero4(); accL[bj] = zero4(); }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int c0 = 32 * kb + 4 * gq;
        const floatx8 Gi = stackf(ldsf4(sG + irow * GS + c0), ldsf4(sG + irow * GS + c0 + 16));
        const floatx8 Gr = stackf(ldsf4(sG + (16 * w) * GS + c0), ldsf4(sG + (16 * w) * GS + c0 + 16));
        const floatx8 qv = stackf(unpack4<T>(R.q[kb][0]), unpack4<T>(R.q[kb][1]));
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
      store_frag8<T>(rec + a.off_aq, ((size_t)aq_frag(w, 0) * 64 + lane) * 8, stackf(aq[0], aq[1]));
      if (w >= 2)
        store_frag8<T>(rec + a.off_aq, ((size_t)aq_frag(w, 1) * 64 + lane) * 8, stackf(aq[2], aq[3]));
    }

    // q of this item is consumed: start loading the next item's
    if constexpr (kPrefetch) issue_q(R, nx);

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
    for (int m = 0; m < NCH; ++m)
      *reinterpret_cast<u32x4*>(sV + (kv_row + m * kRowStep) * KS + kv_col) = R.v[m];
    if constexpr (kPrefetch) issue_v(R, nx);
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

    lds_sync();  // LDS is reused by the next item
  }
}

}  // namespace

template <typename T, int K, bool GF32, bool GATE>
static hipError_t launch12g(const Stage12Args& a, int nitems, hipStream_t s) {
  // resident workgroups per CU (the same for every MI355X), computed once;
  // concurrent first calls compute the same value
  static std::atomic<int> occ_cache{-1};
  int occ = occ_cache.load(std::memory_order_relaxed);
  if (occ < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stage12_kernel<T, K, GF32, GATE>, kThreads, 0) != hipSuccess ||
        n < 1)
      n = 1;
    occ = n;
    occ_cache.store(n, std::memory_order_relaxed);
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus < 1)
    cus = 256;
  const int grid = nitems < occ * cus ? nitems : occ * cus;
  hipLaunchKernelGGL((stage12_kernel<T, K, GF32, GATE>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, int K, bool GF32>
static hipError_t launch12(const Stage12Args& a, int nitems, hipStream_t s) {
  return a.gate_mode ? launch12g<T, K, GF32, true>(a, nitems, s) : launch12g<T, K, GF32, false>(a, nitems, s);
}

hipError_t launch_stage12(const Stage12Args& a, int K, int bf16, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  if (bf16) {
    if (K == 128) return a.g_f32 ? launch12<kda::bf16, 128, true>(a, nblocks, s) : launch12<kda::bf16, 128, false>(a, nblocks, s);
    return a.g_f32 ? launch12<kda::bf16, 64, true>(a, nblocks, s) : launch12<kda::bf16, 64, false>(a, nblocks, s);
  }
  if (K == 128) return a.g_f32 ? launch12<float, 128, true>(a, nblocks, s) : launch12<float, 128, false>(a, nblocks, s);
  return a.g_f32 ? launch12<float, 64, true>(a, nblocks, s) : launch12<float, 64, false>(a, nblocks, s);
}

}  // namespace kda
