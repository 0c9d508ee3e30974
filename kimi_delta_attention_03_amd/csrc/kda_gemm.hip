// bf16 GEMM with fp32 accumulation on gfx950 MFMA, for the plain projections
// of the KDA layer ("KDAChunkwise" docs, sections "From the hidden states to
// causal Q, K, and V" and "Returning to the model dimension": the input
// projections of the hidden states and the output projection back to the
// model dimension).
//
//   C[m, n] = sum_k A[m, k] B[n, k]      A [M, K] (row stride lda), B [N, K]
//                                         (row stride ldb), C [M, N] (ldc)
//
// Both operands are K-contiguous, as the layer stores them (activations
// [tokens, features], Linear weights [out, in]), so every lane loads 16
// contiguous bytes of one row for an MFMA operand.
//
// Tiling: a workgroup of 4 waves computes a 256 x 256 tile of C; wave (wm, wn)
// owns the 128 x 128 quadrant and keeps it in 16 accumulators of
// v_mfma_f32_32x32x16_bf16 (4 x 4 tiles of 32 x 32). K advances in slices of
// 64 through a double-buffered LDS stage (2 x 64 KB): while slice kt is
// multiplied out of one buffer, slice kt + 1 (already in registers) is written
// to the other and slice kt + 2 is loaded from global memory into the freed
// registers, so every load has a whole slice of MFMAs to arrive. One barrier
// per slice, placed so that the next slice's first fragments are read while
// the current slice's last MFMAs run.
//
// LDS layout: a slice is [256 rows][8 chunks of 8 bf16] with the chunk index
// XOR-ed with (row / 2) % 8, so the 16-byte operand reads of consecutive rows
// at one k offset spread over all banks. LDS has 64 banks of 4 bytes and
// serves a 16-byte access for 16 lanes at a time: row r starts in bank
// 32 (r % 2), so the 16 rows read by 16 lanes at one k offset (and the 2 rows
// x 8 chunks written by 16 lanes) fall in 16 distinct 4-bank groups.
//
// Workgroup-to-tile mapping: the workgroups of one XCD (ids congruent mod 8)
// take blocks of 8 x 4 tiles, so each A slice is read by 4 and each B slice by
// 8 workgroups sharing that XCD's L2.
//
// Output: fp32 C is stored straight from the accumulators (each store
// instruction covers 128 contiguous bytes of two rows). bf16 C is computed
// transposed (B as the first MFMA operand, so a lane holds runs of four columns
// of one row), staged through LDS and written back as 16-byte pieces of whole
// rows: 32 store instructions per lane instead of 256 two-byte ones.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "kda_device.h"
#include "kda_kernels.h"
#include "kda_gemm.h"

namespace kda {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8, kGroupN = 4;   // tiles per XCD block

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ floatx4 zero4f() { return floatx4{0.f, 0.f, 0.f, 0.f}; }
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

template <typename TC>
__device__ __forceinline__ void store_out(TC* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<bf16>(bf16* p, float v) { *p = (bf16)v; }
// KTAIL: K is not a multiple of 64 and the chunks past K are zeroed by selects
// (without it the loop carries no select between a load and its LDS write)
// sum of x over the D / 8 consecutive lanes of a (row, head) group (D = 64 or
// 128), on data-parallel-primitive moves inside a 16-lane row: swaps of lane
// pairs and pairs of pairs within each quad, then the mirror within each half
// row (pairs quad 0 with 1, 2 with 3) and, for 16 lanes, the mirror within the
// row (pairs the halves); every lane of the group ends with the group's sum
__device__ __forceinline__ float head_sum(float x, int d) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  if (d == 128)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

// NORM: the output-gate epilogue (bf16 C only, see kda_gemm.h)
template <typename TC, bool KTAIL, bool NORM = false>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_nt_kernel(GemmArgs a) {
  // LDS buffer b: A slice at smem[b][0, 32 KB), B slice at smem[b][32 KB, 64 KB)
  __shared__ __attribute__((aligned(16))) char smem[2][(kBM + kBN) * kBK * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  // bf16 C is computed transposed (B as the first MFMA operand) and staged
  // through LDS for row-contiguous stores; fp32 C keeps A first (see the end)
  constexpr bool kTr = sizeof(TC) == 2;

  // tile of this workgroup (XCD-aware blocks of kGroupM x kGroupN tiles)
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int blk = (slot / (kGroupM * kGroupN)) * 8 + xcd;
  const int j = slot % (kGroupM * kGroupN);
  const int nbn = (a.ntn + kGroupN - 1) / kGroupN;
  // the tile indices are uniform; the integer division runs on the vector ALU,
  // so they are moved to scalar registers explicitly (otherwise the buffer
  // resources built from them may be taken as per-lane values)
  const int tm = __builtin_amdgcn_readfirstlane((blk / nbn) * kGroupM + j % kGroupM);
  const int tn = __builtin_amdgcn_readfirstlane((blk % nbn) * kGroupN + j / kGroupM);
  if (tm >= a.ntm || tn >= a.ntn) return;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

  const bf16* A = static_cast<const bf16*>(a.A);
  const bf16* B = static_cast<const bf16*>(a.B);

  // Loads of one K slice go through buffer resources over the tile's rows of A
  // and B (rows past M or N lie outside the resource and read as zero, with no
  // branch): thread tid loads row tid / 8 + 32 i, 16-byte chunk tid % 8, of
  // both slices. K past the end is zeroed by a select.
  const int64_t rowsA = a.M - m0 < kBM ? a.M - m0 : kBM, rowsB = a.N - n0 < kBN ? a.N - n0 : kBN;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(A + m0 * a.lda), (short)0, (int)(rowsA * a.lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16*>(B + n0 * a.ldb), (short)0, (int)(rowsB * a.ldb * 2), 0x00020000);
  const int lrow = tid >> 3, lch = tid & 7;
  const int voffA = (int)((lrow * a.lda + lch * 8) * 2), voffB = (int)((lrow * a.ldb + lch * 8) * 2);
  const int strA = (int)(32 * a.lda * 2), strB = (int)(32 * a.ldb * 2);
  u32x4 ra[8], rb[8];
  // half h of a slice: rows lrow + 32 i for i in [4 h, 4 h + 4)
  auto load_half = [&](int64_t k0, int h) {
    const int ko = (int)(k0 * 2);
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) {
      ra[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsA, voffA, ko + i * strA, 0));
      rb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsB, voffB, ko + i * strB, 0));
    }
    if constexpr (KTAIL) {
      const bool kin = k0 + lch * 8 < a.K;
#pragma unroll
      for (int i = 4 * h; i < 4 * h + 4; ++i) {
        ra[i] = kin ? ra[i] : u32x4{0, 0, 0, 0};
        rb[i] = kin ? rb[i] : u32x4{0, 0, 0, 0};
      }
    }
  };
  // LDS byte offsets of this thread's chunks (row lrow + 32 i): the XOR key
  // (row / 2) % 8 is the same for every i
  const int soff = lrow * 128 + ((lch ^ ((lrow >> 1) & 7)) << 4);
  auto store_half = [&](int buf, int h) {
    char* base = smem[buf] + soff;
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) {
      *reinterpret_cast<u32x4*>(base + i * 32 * 128) = ra[i];
      *reinterpret_cast<u32x4*>(base + kBM * kBK * 2 + i * 32 * 128) = rb[i];
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = zero16();

  // operand reads: lane l supplies row (l % 32) of a 32-row tile and the 8
  // k values 8 (l / 32) .. + 7 of the current 16-wide k step. The XOR key of
  // rows wm 128 + 32 x + orow is (orow / 2) % 8 for every x, and chunk 2 s + og
  // XOR-ed with it is 2 s XOR (og ^ key): a lane's fragment addresses differ
  // across x, y and buffers only by constants.
  const int orow = lane & 31, og = lane >> 5;
  const int kx = og ^ ((orow >> 1) & 7);
  int ofa[4], ofb[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    ofa[st] = (wm * 128 + orow) * 128 + (((2 * st) ^ kx) << 4);
    ofb[st] = kBM * kBK * 2 + (wn * 128 + orow) * 128 + (((2 * st) ^ kx) << 4);
  }
  auto read_frags = [&](int buf, int s, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
    const char* base = smem[buf];
#pragma unroll
    for (int x = 0; x < 4; ++x) fa[x] = *reinterpret_cast<const bf16x8*>(base + ofa[s] + x * 32 * 128);
#pragma unroll
    for (int y = 0; y < 4; ++y) fb[y] = *reinterpret_cast<const bf16x8*>(base + ofb[s] + y * 32 * 128);
  };
  auto mma = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4]) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
        acc[x][y] = kTr ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[y], fa[x], acc[x][y], 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
  };

  // Pipeline over K slices of 64: slice kt is multiplied out of LDS buffer
  // kt % 2. At the start of that, slice kt + 1 (loaded into registers during
  // slice kt - 1) is written to the other buffer, each register being reloaded
  // with slice kt + 2 right after its write, so a load has a whole slice of
  // MFMAs to arrive. The one barrier of a slice sits before the MFMAs of its
  // last 16-wide k step: by then every wave has read all of this slice's
  // fragments and written the next slice, so the next slice's first fragments
  // are read while those MFMAs run.
  constexpr int MFMA = 0x008, VMEM_RD = 0x020, DS_RD = 0x100, DS_WR = 0x200;
  bf16x8 f0a[4], f0b[4], f1a[4], f1b[4];
  const int nk = (int)((a.K + kBK - 1) / kBK);
  load_half(0, 0);
  load_half(0, 1);
  store_half(0, 0);
  store_half(0, 1);
  load_half(nk > 1 ? kBK : 0, 0);
  load_half(nk > 1 ? kBK : 0, 1);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  read_frags(0, 0, f0a, f0b);
  int kt = 0;
  for (; kt + 1 < nk; ++kt) {
    const int buf = kt & 1;
    const int64_t kl = (int64_t)(kt + 2 < nk ? kt + 2 : nk - 1) * kBK;
    // k steps 0 and 1: the fragments of the following step are read first,
    // then half of the next slice goes to LDS, each register reloaded from
    // global memory right after its write
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st == 0) {
        mma(f0a, f0b);
        read_frags(buf, 1, f1a, f1b);
      } else {
        mma(f1a, f1b);
        read_frags(buf, 2, f0a, f0b);
      }
      store_half(buf ^ 1, st);
      load_half(kl, st);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(DS_RD, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(DS_WR, 1, 0);
        __builtin_amdgcn_sched_group_barrier(VMEM_RD, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // k step 2
    mma(f0a, f0b);
    read_frags(buf, 3, f1a, f1b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(DS_RD, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(MFMA, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    // every wave has read this slice's fragments and written the next slice:
    // the barrier, then the next slice's first fragments are read under the
    // MFMAs of k step 3 (global loads stay in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    read_frags(buf ^ 1, 0, f0a, f0b);
    mma(f1a, f1b);
    __builtin_amdgcn_sched_group_barrier(DS_RD, 8, 0);
    __builtin_amdgcn_sched_group_barrier(MFMA, 16, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    const int buf = kt & 1;
    read_frags(buf, 1, f1a, f1b);
    mma(f0a, f0b);
    read_frags(buf, 2, f0a, f0b);
    mma(f1a, f1b);
    read_frags(buf, 3, f1a, f1b);
    mma(f0a, f0b);
    mma(f1a, f1b);
  }

  TC* C = static_cast<TC*>(a.C);
  if constexpr (!kTr) {
    // fp32 C: accumulator element r of lane l is row 8 (r / 4) + 4 (l / 32) +
    // r % 4, column l % 32; one store instruction covers 128 contiguous bytes of
    // each of two rows
    const bool full = m0 + kBM <= a.M && n0 + kBN <= a.N;   // uniform
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int64_t col = n0 + wn * 128 + y * 32 + orow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * 128 + x * 32 + 8 * (r >> 2) + 4 * og + (r & 3);
          if (full || (row < a.M && col < a.N)) store_out<TC>(C + row * a.ldc + col, acc[x][y][r]);
        }
      }
    return;
  } else {
    // bf16 C, computed transposed: element r of lane l is row l % 32, column
    // 8 (r / 4) + 4 (l / 32) + r % 4 of the 32 x 32 tile, i.e. four consecutive
    // columns of one row per group r / 4.
    if (a.vec_out) {
      // Each wave stages its 128 x 128 quadrant through its own 32 KB of LDS
      // (rows of 256 bytes, 16-byte chunks XOR-swizzled by row) and writes it
      // back in 16-byte pieces of whole rows: one store instruction covers four
      // complete rows. Pieces of partial tiles that cross M or N are written
      // element by element.
      const bool full = m0 + kBM <= a.M && n0 + kBN <= a.N;   // uniform
      char* q = &smem[0][0] + w * 32768;
      // every wave has read its last operand fragments before any staging write
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int rw = x * 32 + orow;
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int byte = (32 * y + 8 * g + 4 * og) * 2;
            const floatx16& c = acc[x][y];
            char* dst = q + rw * 256 + (((byte >> 4) ^ (rw & 15)) << 4) + (byte & 15);
            if constexpr (NORM) {
              // the gate factor sigmoid(G) in (0, 1), staged as fp16 (2^-11 relative)
              half4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (_Float16)(1.f / (1.f + __expf(-c[4 * g + e])));
              *reinterpret_cast<half4*>(dst) = o;
            } else {
              bf16x4 o;
              o[0] = (bf16)c[4 * g]; o[1] = (bf16)c[4 * g + 1]; o[2] = (bf16)c[4 * g + 2]; o[3] = (bf16)c[4 * g + 3];
              *reinterpret_cast<bf16x4*>(dst) = o;
            }
          }
      }
      // the quadrant region is this wave's own: an LDS wait orders the reads
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (NORM) {
        // 32 row pieces of 8 columns per lane, piece i at row 4 i + lane / 16;
        // the D / 8 lanes of a (row, head) are consecutive, so the head's sum of
        // squares is a reduction over them (N is a multiple of D: a head lies
        // wholly inside or past N). o is read in groups of 4 pieces, each group
        // loaded while the one before it is normalised and stored.
        constexpr int GP = 4, NG = 32 / GP;
        floatx4 ob[2][GP][2];
        auto load_o = [&](int gi, floatx4 (&dst)[GP][2]) {
#pragma unroll
          for (int i3 = 0; i3 < GP; ++i3) {
            const int rw = 4 * (gi * GP + i3) + (lane >> 4), ch = lane & 15;
            const int64_t row = m0 + wm * 128 + rw, col = n0 + wn * 128 + ch * 8;
            dst[i3][0] = zero4f();
            dst[i3][1] = zero4f();
            if (row < a.M && col < a.N) {
              dst[i3][0] = *reinterpret_cast<const floatx4*>(a.norm_o + row * a.ldo + col);
              dst[i3][1] = *reinterpret_cast<const floatx4*>(a.norm_o + row * a.ldo + col + 4);
            }
          }
        };
        load_o(0, ob[0]);
        // a lane's 8 channels are the same in every piece: n0 and wn 128 are
        // multiples of D, so the channel of column 8 ch + e is (8 ch + e) % D
        const int d0 = (8 * (lane & 15)) % a.norm_d;
        float nw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) nw[e] = a.norm_w[d0 + e];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          if (gi + 1 < NG) load_o(gi + 1, ob[(gi + 1) & 1]);
#pragma unroll
          for (int i3 = 0; i3 < GP; ++i3) {
            const int rw = 4 * (gi * GP + i3) + (lane >> 4), ch = lane & 15;
            const int64_t row = m0 + wm * 128 + rw, col = n0 + wn * 128 + ch * 8;
            const half8 gt = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(
                                                           q + rw * 256 + ((ch ^ (rw & 15)) << 4)));
            float ov[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { ov[e] = ob[gi & 1][i3][0][e]; ov[4 + e] = ob[gi & 1][i3][1][e]; }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += ov[e] * ov[e];
            const float inv = 1.f / sqrtf(head_sum(ss, a.norm_d) / (float)a.norm_d + a.norm_eps);
            bf16x8 yv;
#pragma unroll
            for (int e = 0; e < 8; ++e) yv[e] = (bf16)(ov[e] * inv * nw[e] * (float)gt[e]);
            if (row < a.M && col < a.N) *reinterpret_cast<bf16x8*>(C + row * a.ldc + col) = yv;
          }
        }
        return;
      }
#pragma unroll
      for (int i0 = 0; i0 < 32; i0 += 8) {
        u32x4 rv[8];
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) {
          const int rw = 4 * (i0 + i2) + (lane >> 4), ch = lane & 15;
          rv[i2] = *reinterpret_cast<const u32x4*>(q + rw * 256 + ((ch ^ (rw & 15)) << 4));
        }
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) {
          const int rw = 4 * (i0 + i2) + (lane >> 4), ch = lane & 15;
          const int64_t row = m0 + wm * 128 + rw, col = n0 + wn * 128 + ch * 8;
          if (full || (row < a.M && col + 8 <= a.N)) {
            *reinterpret_cast<u32x4*>(C + row * a.ldc + col) = rv[i2];
          } else if (row < a.M) {
            const bf16* e = reinterpret_cast<const bf16*>(&rv[i2]);
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (col + k < a.N) C[row * a.ldc + col + k] = e[k];
          }
        }
      }
      return;
    }
    // C rows not 16-byte aligned: element stores
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int64_t row = m0 + wm * 128 + x * 32 + orow;
      if (row >= a.M) continue;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = n0 + wn * 128 + y * 32 + 8 * g + 4 * og;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < a.N) store_out<TC>(C + row * a.ldc + col + e, acc[x][y][4 * g + e]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K <= 128 (the layer's rank-r up-projections): the whole K of a tile is one
// pass of 8 k steps, so the product is cheap and the kernel is bound by its
// output writes and, with the output-gate epilogue, by reading o. The 256 x 256
// pipeline above holds one workgroup per CU, and all of them reach their
// epilogue at once: HBM then takes the stores of every tile in a burst and
// idles during the products and the next tile's first loads.
//
// Here a workgroup of 4 waves keeps the B tile of one 128-column block in LDS
// (32 KB, loaded once) and walks row tiles of 128 rows; two or three such
// workgroups share a CU, so one's loads and stores overlap another's products.
// Wave w computes rows 32 w .. 32 w + 31 against the 128 columns as 4 tiles of
// v_mfma_f32_32x32x16_bf16. The A fragments of a row tile (8 x 16 bytes per
// lane) come straight from global memory into registers, the next tile's
// issued before this tile's epilogue.
//
// Every global access of the epilogue covers whole 128-byte lines:
// - fp32 C keeps A as the first MFMA operand (element r of lane l is row
//   8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of a tile), so one store
//   instruction writes 128 contiguous bytes of each of two rows;
// - bf16 C takes B first (lane l holds row l % 32 at runs of four columns).
//   With the output-gate epilogue, sigmoid of the product is staged per wave in
//   LDS (fp16, 8 KB) and the rows are then processed as pieces: lanes 0-31 hold
//   columns 4 (l % 32) .. + 3 of one row and lanes 32-63 of the next, so o is
//   read as 512 contiguous bytes per row (issued before the products) and y
//   written as 256; a head's sum of squares is a reduction over D / 4 lanes.
//
// B in LDS: row r (column n0 + r of C) holds 16 chunks of 8 bf16, chunk ch at
// byte 256 r + 16 (ch ^ (r % 16)): the 16 lanes of one read phase take rows
// r .. r + 15 at one chunk and hit 16 distinct 4-bank groups. The gate stage
// uses the same row format (128 fp16 per row).
//
// Workgroup mapping: id b runs on XCD b % 8; the workgroups of XCD x take the
// row tiles congruent to x mod 8 for every column block, so each A tile is
// read from HBM once and then served by that XCD's L2.
constexpr int kSBM = 128, kSBN = 128;

// sum of x over the n consecutive lanes of an aligned group (n = 16 or 32):
// lane pair and pair-of-pair swaps, the mirror within each 8 lanes and within
// each 16 (each step leaves every lane with its group's partial sum), then the
// other 16-lane half for n = 32
__device__ __forceinline__ float group_sum(float x, int n) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  if (n == 32) x += __shfl_xor(x, 16, 64);
  return x;
}

template <typename TC, bool NORM>
__global__ __launch_bounds__(kGemmThreads, NORM ? 2 : 3) void gemm_smallk_kernel(GemmArgs a, int cpw) {
  constexpr bool kTr = sizeof(TC) == 2;   // B as the first operand
  __shared__ __attribute__((aligned(16))) char sB[kSBN * 256];
  __shared__ __attribute__((aligned(16))) char sG[NORM ? 4 * 32 * 256 : 16];   // gate stage, 8 KB per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int x = bid & 7, sl = bid >> 3;
  const int cb = __builtin_amdgcn_readfirstlane(sl % a.ntn);
  const int sub = __builtin_amdgcn_readfirstlane(sl / a.ntn);
  const int64_t n0 = (int64_t)cb * kSBN;
  const bf16* A = static_cast<const bf16*>(a.A);
  const bf16* B = static_cast<const bf16*>(a.B);
  const int kch = (int)(a.K / 8);  // 16-byte chunks of K (K is a multiple of 8)

  // B tile of this column block, zero past N and past K
  for (int e = tid; e < kSBN * 16; e += kGemmThreads) {
    const int r = e >> 4, ch = e & 15;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n0 + r < a.N && ch < kch) v = *reinterpret_cast<const u32x4*>(B + (n0 + r) * a.ldb + ch * 8);
    *reinterpret_cast<u32x4*>(sB + r * 256 + ((ch ^ (r & 15)) << 4)) = v;
  }
  __syncthreads();

  const int64_t step = 8 * (int64_t)cpw;
  int64_t tm = x + 8 * (int64_t)sub;
  if (tm >= a.ntm) return;

  const int orow = lane & 31, og = lane >> 5;
  const int key = orow & 15;
  // A fragments of row tile t: lane l reads row 32 w + l % 32, chunk 2 s + l / 32
  // for k step s, through a buffer resource over the tile's rows (rows past M
  // read as zero); chunks past K are zeroed by a select
  bf16x8 fa[8];
  auto load_a = [&](int64_t t) {
    const int64_t m0 = t * kSBM;
    const int64_t rows = a.M - m0 < kSBM ? a.M - m0 : kSBM;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(A + m0 * a.lda), (short)0, (int)(rows * a.lda * 2), 0x00020000);
    const int voff = (int)(((32 * w + orow) * a.lda + og * 8) * 2);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 32 * s, 0));
      fa[s] = __builtin_bit_cast(bf16x8, 2 * s + og < kch ? v : u32x4{0u, 0u, 0u, 0u});
    }
  };
  load_a(tm);
  TC* C = static_cast<TC*>(a.C);
  // output-gate epilogue: this lane's four columns n0 + 4 (l % 32) .. + 3 and their weights
  const int pc = 4 * orow;
  const bool pcol = n0 + pc < a.N;
  floatx4 nw = zero4f();
  if constexpr (NORM) {
#pragma unroll
    for (int e = 0; e < 4; ++e) nw[e] = a.norm_w[(pc + e) % a.norm_d];
  }
  char* gst = sG + (NORM ? w * 32 * 256 : 0);

  for (; tm < a.ntm; tm += step) {
    const int64_t r0 = tm * kSBM + 32 * w;   // first row of this wave
    // o for the epilogue, issued ahead of the products: piece i is row
    // r0 + 2 i + l / 32 at columns n0 + 4 (l % 32) .. + 3. o and C go through
    // buffer resources over the wave's 32 rows (rows past M lie outside them:
    // loads read zero, stores are dropped); a lane whose columns lie past N
    // points its offset past the end too
    floatx4 ov[16];
    __amdgpu_buffer_rsrc_t rc;
    int coff = 0;
    if constexpr (NORM) {
      const int64_t left = a.M - r0, nrow = left < 0 ? 0 : (left < 32 ? left : 32);
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.norm_o + r0 * a.ldo + n0), (short)0, (int)(nrow * a.ldo * 4), 0x00020000);
      rc = __builtin_amdgcn_make_buffer_rsrc(C + r0 * a.ldc + n0, (short)0, (int)(nrow * a.ldc * 2), 0x00020000);
      const int ooff = pcol ? (int)((og * a.ldo + pc) * 4) : 0x40000000;
      coff = pcol ? (int)((og * a.ldc + pc) * 2) : 0x40000000;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        ov[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(ro, ooff, (int)(2 * i * a.ldo * 4), 0));
    }
    floatx16 acc[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[y] = zero16();
    // B fragments one k step ahead of the products (two register sets; left
    // to itself the compiler hoists all 32 reads and the registers overflow)
    auto read_b = [&](int s, bf16x8 (&fb)[4]) {
#pragma unroll
      for (int y = 0; y < 4; ++y)
        fb[y] = *reinterpret_cast<const bf16x8*>(sB + y * 32 * 256 + orow * 256 + (((2 * s + og) ^ key) << 4));
    };
    bf16x8 fb[2][4];
    read_b(0, fb[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) read_b(s + 1, fb[(s + 1) & 1]);
#pragma unroll
      for (int y = 0; y < 4; ++y)
        acc[y] = kTr ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s & 1][y], fa[s], acc[y], 0, 0, 0)
                     : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s], fb[s & 1][y], acc[y], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next row tile's A fragments (the last tile reloads its own)
    load_a(tm + step < a.ntm ? tm + step : tm);

    if constexpr (NORM) {
      // stage sigmoid(G) for this wave's 32 rows: lane l writes row l % 32 at
      // columns 32 y + 8 q + 4 (l / 32) .. + 3, 8 bytes into chunk 4 y + q
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          half4 gv;
#pragma unroll
          for (int e = 0; e < 4; ++e) gv[e] = (_Float16)(1.f / (1.f + __expf(-acc[y][4 * q + e])));
          *reinterpret_cast<half4*>(gst + orow * 256 + (((4 * y + q) ^ key) << 4) + 8 * og) = gv;
        }
      // the stage is this wave's own: an LDS wait orders its reads after the writes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int dl = a.norm_d / 4;   // lanes per head
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rw = 2 * i + og;
        const half4 gv = *reinterpret_cast<const half4*>(gst + rw * 256 + (((orow >> 1) ^ (rw & 15)) << 4) +
                                                         8 * (orow & 1));
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += ov[i][e] * ov[i][e];
        const float inv = 1.f / sqrtf(group_sum(ss, dl) / (float)a.norm_d + a.norm_eps);
        bf16x4 yv;
#pragma unroll
        for (int e = 0; e < 4; ++e) yv[e] = (bf16)(ov[i][e] * inv * nw[e] * (float)gv[e]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, yv), rc, coff, (int)(2 * i * a.ldc * 2), 0);
      }
    } else if constexpr (kTr) {
      // bf16 C without the gate: runs of four columns of row r0 + l % 32
      const int64_t row = r0 + orow;
      if (row < a.M) {
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t col = n0 + 32 * y + 8 * q + 4 * og;
            if (a.vec4 && col + 4 <= a.N) {
              bf16x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (bf16)acc[y][4 * q + e];
              *reinterpret_cast<bf16x4*>(C + row * a.ldc + col) = o;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < a.N) store_out<TC>(C + row * a.ldc + col + e, acc[y][4 * q + e]);
            }
          }
      }
    } else {
      // fp32 C: element r of tile y is row r0 + 8 (r / 4) + 4 (l / 32) + r % 4,
      // column n0 + 32 y + l % 32
      const bool full = r0 + 32 <= a.M && n0 + kSBN <= a.N;   // uniform
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int64_t col = n0 + 32 * y + orow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = r0 + 8 * (r >> 2) + 4 * og + (r & 3);
          if (full || (row < a.M && col < a.N)) store_out<TC>(C + row * a.ldc + col, acc[y][r]);
        }
      }
    }
  }
}

// resident workgroups per CU of one instantiation, computed once per process
template <typename TC, bool NORM>
static int smallk_occupancy() {
  static std::atomic<int> occ_cache{-1};
  int occ = occ_cache.load(std::memory_order_relaxed);
  if (occ < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_smallk_kernel<TC, NORM>, kGemmThreads, 0) !=
            hipSuccess || n < 1)
      n = 1;
    occ = n;
    occ_cache.store(n, std::memory_order_relaxed);
  }
  return occ;
}

template <typename TC, bool NORM>
static hipError_t launch_smallk(GemmArgs a, hipStream_t s) {
  a.ntm = (int)((a.M + kSBM - 1) / kSBM);
  a.ntn = (int)((a.N + kSBN - 1) / kSBN);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  // resident workgroups per XCD, split evenly over the column blocks
  const int per_xcd = smallk_occupancy<TC, NORM>() * cus / 8;
  int cpw = per_xcd / a.ntn;
  if (cpw < 1) cpw = 1;
  const int64_t row_groups = ((int64_t)a.ntm + 7) / 8;   // row tiles per XCD and column block
  if (cpw > row_groups) cpw = (int)row_groups;
  const dim3 grid((unsigned)(8 * (int64_t)a.ntn * cpw)), block(kGemmThreads);
  hipLaunchKernelGGL((gemm_smallk_kernel<TC, NORM>), grid, block, 0, s, a, cpw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a0, int out_f32, hipStream_t s) {
  GemmArgs a = a0;
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  a.ntm = (int)((a.M + kBM - 1) / kBM);
  a.ntn = (int)((a.N + kBN - 1) / kBN);
  // bf16 C is written in 16-byte row pieces: every row start 16-byte aligned
  a.vec_out = !out_f32 && a.ldc % 8 == 0 && reinterpret_cast<uintptr_t>(a.C) % 16 == 0;
  const int nbm = (a.ntm + kGroupM - 1) / kGroupM, nbn = (a.ntn + kGroupN - 1) / kGroupN;
  const int nblk8 = (nbm * nbn + 7) / 8 * 8;   // blocks, padded to whole rounds of 8 XCDs
  const dim3 grid((unsigned)(nblk8 * kGroupM * kGroupN)), block(kGemmThreads);
  const bool ktail = a.K % kBK != 0;
  const bool smallk = a.K <= kSBN;
  if (a.norm_o) {
    if (out_f32 || !a.vec_out || !a.norm_w || !(a.norm_d == 64 || a.norm_d == 128) || a.N % a.norm_d ||
        a.ldo % 8 || reinterpret_cast<uintptr_t>(a.norm_o) % 16)
      return hipErrorInvalidValue;
    if (smallk) return launch_smallk<bf16, true>(a, s);
    if (ktail) hipLaunchKernelGGL((gemm_bf16_nt_kernel<bf16, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_bf16_nt_kernel<bf16, false, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (smallk) {
    a.vec4 = a.ldc % 4 == 0 && reinterpret_cast<uintptr_t>(a.C) % (out_f32 ? 16 : 8) == 0;
    return out_f32 ? launch_smallk<float, false>(a, s) : launch_smallk<bf16, false>(a, s);
  }
  if (out_f32) {
    if (ktail) hipLaunchKernelGGL((gemm_bf16_nt_kernel<float, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_bf16_nt_kernel<float, false>), grid, block, 0, s, a);
  } else {
    if (ktail) hipLaunchKernelGGL((gemm_bf16_nt_kernel<bf16, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_bf16_nt_kernel<bf16, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace kda
