// Chunk map for packed variable-length input (Tokamax "chunk_kda_fwd design
// doc", sections 3.5 and 9.1.7): every sequence is cut into 64-token chunks
// from its own start, so no chunk spans two sequences, and the physical
// chunks of all sequences are numbered consecutively. One workgroup builds,
// without any host round trip:
//   chunk table [slot]  = (first token, valid length), length 0 for unused slots
//   sequence table [n]  = (first chunk slot, chunk count)
//   order [rank]        = sequence ids, longest first (ties by id)
//   header word 0       = number of chunk slots in use
// cu_seqlens is read defensively: each boundary is clamped into [0, T] and
// made non-decreasing, so malformed input cannot address memory outside the
// inputs or the workspace.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int kMapThreads = 1024;
constexpr int kSortMax = 4096;

__device__ __forceinline__ int block_scan_max(int x, int* s) {
  const int t = threadIdx.x;
  s[t] = x;
  __syncthreads();
  for (int o = 1; o < kMapThreads; o <<= 1) {
    const int y = t >= o ? s[t - o] : INT_MIN;
    __syncthreads();
    if (y > s[t]) s[t] = y;
    __syncthreads();
  }
  const int r = s[t];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_scan_sum(int x, int* s) {
  const int t = threadIdx.x;
  s[t] = x;
  __syncthreads();
  for (int o = 1; o < kMapThreads; o <<= 1) {
    const int y = t >= o ? s[t - o] : 0;
    __syncthreads();
    s[t] += y;
    __syncthreads();
  }
  const int r = s[t];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kMapThreads) void varlen_map_kernel(const int32_t* cu, int nseq, int64_t T,
                                                                 char* ws, size_t ncp, size_t off_ct,
                                                                 size_t off_st, size_t off_ord) {
  __shared__ int s_scan[kMapThreads];
  __shared__ int s_nch[kSortMax];
  int2* ctab = reinterpret_cast<int2*>(ws + off_ct);
  int2* stab = reinterpret_cast<int2*>(ws + off_st);
  int* order = reinterpret_cast<int*>(ws + off_ord);
  const int t = threadIdx.x;
  const int TT = (int)T;
  int prev_end = min(max((int)cu[0], 0), TT);  // e_{-1}
  int chunk_carry = 0;
  for (int base = 0; base < nseq; base += kMapThreads) {
    const int n = base + t;
    const int raw = n < nseq ? min(max((int)cu[n + 1], 0), TT) : INT_MIN;
    const int mx = block_scan_max(raw, s_scan);
    const int end = n < nseq ? max(mx, prev_end) : prev_end;
    // start of n = end of n-1 (the previous lane, or the carry at the tile start)
    s_scan[t] = end;
    __syncthreads();
    const int start = t == 0 ? prev_end : s_scan[t - 1];
    __syncthreads();
    const int len = n < nseq ? end - start : 0;
    const int nch = (len + kChunk - 1) / kChunk;
    const int incl = block_scan_sum(nch, s_scan);
    const int first = chunk_carry + incl - nch;
    if (n < nseq) {
      stab[n] = make_int2(first, nch);
      if (nseq <= kSortMax) s_nch[n] = nch;
      for (int c = 0; c < nch; ++c) {
        const size_t slot = (size_t)first + c;
        if (slot < ncp) ctab[slot] = make_int2(start + c * kChunk, min(kChunk, len - c * kChunk));
      }
    }
    // carries for the next tile: last lane's end and the tile's chunk total
    if (t == kMapThreads - 1) {
      s_scan[0] = end;
      s_scan[1] = chunk_carry + incl;
    }
    __syncthreads();
    prev_end = s_scan[0];
    chunk_carry = s_scan[1];
    __syncthreads();
  }
  for (size_t slot = (size_t)chunk_carry + t; slot < ncp; slot += kMapThreads) ctab[slot] = make_int2(0, 0);
  // header word 0: chunk slots in use (<= ncp by construction; clamped for safety)
  if (t == 0) reinterpret_cast<int*>(ws)[0] = min(chunk_carry, (int)ncp);
  if (nseq <= kSortMax) {
    __syncthreads();
    for (int n = t; n < nseq; n += kMapThreads) {
      const int mine = s_nch[n];
      int rank = 0;
      for (int m = 0; m < nseq; ++m) {
        const int other = s_nch[m];
        rank += (other > mine) || (other == mine && m < n);
      }
      order[rank] = n;
    }
  } else {
    for (int n = t; n < nseq; n += kMapThreads) order[n] = n;
  }
}

}  // namespace

hipError_t launch_varlen_map(const int32_t* cu, int nseq, int64_t T, char* ws, size_t ncp,
                             size_t off_chunk_tab, size_t off_seq_tab, size_t off_order, hipStream_t s) {
  hipLaunchKernelGGL(varlen_map_kernel, dim3(1), dim3(kMapThreads), 0, s, cu, nseq, T, ws, ncp, off_chunk_tab,
                     off_seq_tab, off_order);
  return hipGetLastError();
}

}  // namespace kda
