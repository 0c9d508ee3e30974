// kda_validate_inputs: the value preconditions of the fast path, checked on
// the GPU (Tokamax "chunk_kda_fwd design doc", section 5.3 "Required Runtime
// Invariants": gates inside the lower bound, beta in [0, 1], and section 3.5:
// cu_seqlens non-decreasing from 0 to the packed length).
//
// One launch of a fixed grid: every workgroup reduces a grid-stride share of
// g and beta (min, max over the finite entries, count of non-finite ones)
// and of cu_seqlens (first index that breaks the invariants) into one
// partial record in the caller's scratch; the host copies the partials back,
// synchronises the stream and finishes the reduction.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "kda.h"
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int kValBlocks = 256;
constexpr int kValThreads = 256;

struct ValidatePartial {
  float gmin, gmax, bmin, bmax;
  unsigned long long g_nonfinite, b_nonfinite;
  long long cu_bad;     // first bad index of cu_seqlens, or INT64_MAX
  long long pad;
};
static_assert(sizeof(ValidatePartial) * kValBlocks <= KDA_VALIDATE_SCRATCH_BYTES, "scratch too small");

__device__ __forceinline__ float as_f32(const bf16* p, int64_t i) { return (float)p[i]; }
__device__ __forceinline__ float as_f32(const float* p, int64_t i) { return p[i]; }

template <typename Op, typename X>
__device__ X block_reduce(X x, X* s, Op op) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = op(x, __shfl_xor(x, o, 64));
  if (lane == 0) s[w] = x;
  __syncthreads();
  X r = s[0];
#pragma unroll
  for (int i = 1; i < kValThreads / 64; ++i) r = op(r, s[i]);
  __syncthreads();
  return r;
}

template <typename TG, typename TB>
__global__ __launch_bounds__(kValThreads) void validate_kernel(const TG* g, int64_t ng, const TB* beta, int64_t nb,
                                                               const int32_t* cu, int nseq, int64_t T,
                                                               ValidatePartial* out) {
  __shared__ float sf[kValThreads / 64];
  __shared__ unsigned long long su[kValThreads / 64];
  __shared__ long long sl[kValThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kValThreads;
  const int64_t i0 = (int64_t)blockIdx.x * kValThreads + threadIdx.x;
  float gmin = INFINITY, gmax = -INFINITY, bmin = INFINITY, bmax = -INFINITY;
  unsigned long long gnf = 0, bnf = 0;
  for (int64_t i = i0; i < ng; i += stride) {
    const float x = as_f32(g, i);
    if (isfinite(x)) {
      gmin = fminf(gmin, x);
      gmax = fmaxf(gmax, x);
    } else {
      ++gnf;
    }
  }
  for (int64_t i = i0; i < nb; i += stride) {
    const float x = as_f32(beta, i);
    if (isfinite(x)) {
      bmin = fminf(bmin, x);
      bmax = fmaxf(bmax, x);
    } else {
      ++bnf;
    }
  }
  long long bad = INT64_MAX;
  if (cu) {
    for (int64_t i = i0; i <= (int64_t)nseq; i += stride) {
      const int32_t c = cu[i];
      const bool wrong = (i == 0 && c != 0) || (i > 0 && c < cu[i - 1]) || (i == nseq && (int64_t)c != T);
      if (wrong && i < bad) bad = i;
    }
  }
  auto fmin_op = [](float a, float b) { return fminf(a, b); };
  auto fmax_op = [](float a, float b) { return fmaxf(a, b); };
  auto add_op = [](unsigned long long a, unsigned long long b) { return a + b; };
  auto min_op = [](long long a, long long b) { return a < b ? a : b; };
  ValidatePartial r;
  r.gmin = block_reduce(gmin, sf, fmin_op);
  r.gmax = block_reduce(gmax, sf, fmax_op);
  r.bmin = block_reduce(bmin, sf, fmin_op);
  r.bmax = block_reduce(bmax, sf, fmax_op);
  r.g_nonfinite = block_reduce(gnf, su, add_op);
  r.b_nonfinite = block_reduce(bnf, su, add_op);
  r.cu_bad = block_reduce(bad, sl, min_op);
  r.pad = 0;
  if (threadIdx.x == 0) out[blockIdx.x] = r;
}

template <typename TG>
hipError_t launch_val(const void* g, int64_t ng, const void* beta, int64_t nb, int b_f32, const int32_t* cu, int nseq,
                      int64_t T, ValidatePartial* out, hipStream_t s) {
  if (b_f32)
    hipLaunchKernelGGL((validate_kernel<TG, float>), dim3(kValBlocks), dim3(kValThreads), 0, s,
                       static_cast<const TG*>(g), ng, static_cast<const float*>(beta), nb, cu, nseq, T, out);
  else
    hipLaunchKernelGGL((validate_kernel<TG, bf16>), dim3(kValBlocks), dim3(kValThreads), 0, s,
                       static_cast<const TG*>(g), ng, static_cast<const bf16*>(beta), nb, cu, nseq, T, out);
  return hipGetLastError();
}

}  // namespace
}  // namespace kda

extern "C" kda_status kda_validate_inputs(const kda_fwd_params* p, const void* g, const void* beta,
                                          const int32_t* cu_seqlens, void* scratch, size_t scratch_bytes,
                                          hipStream_t stream, kda_input_report* report) {
  using namespace kda;
  clear_msg();
  if (!p || !report) return fail_msg(KDA_ERR_INVALID_ARG, "params and report must be non-NULL");
  report->failed = -1;
  if (p->B < 0 || p->T < 0 || p->H <= 0 || p->K <= 0 || p->num_seqs < 0)
    return fail_msg(KDA_ERR_INVALID_ARG, "need B >= 0, T >= 0, H > 0, K > 0, num_seqs >= 0");
  for (int32_t d : {p->g_dtype, p->beta_dtype})
    if (d != KDA_DTYPE_F32 && d != KDA_DTYPE_BF16) return fail_msg(KDA_ERR_INVALID_ARG, "unknown dtype %d", d);
  if (p->num_seqs > 0 && !cu_seqlens) return fail_msg(KDA_ERR_INVALID_ARG, "num_seqs > 0 needs cu_seqlens");
  if (p->num_seqs == 0 && cu_seqlens) return fail_msg(KDA_ERR_INVALID_ARG, "cu_seqlens given but num_seqs == 0");
  const int64_t ng = p->B * p->T * p->H * (int64_t)p->K;
  const int64_t nb = p->B * p->T * p->H;
  const size_t ge = p->g_dtype == KDA_DTYPE_BF16 ? 2 : 4, be = p->beta_dtype == KDA_DTYPE_BF16 ? 2 : 4;
  if (ng > 0 && (!g || !beta)) return fail_msg(KDA_ERR_INVALID_ARG, "g and beta must be non-NULL");
  if ((g && reinterpret_cast<uintptr_t>(g) % ge) || (beta && reinterpret_cast<uintptr_t>(beta) % be) ||
      (cu_seqlens && reinterpret_cast<uintptr_t>(cu_seqlens) % 4))
    return fail_msg(KDA_ERR_INVALID_ARG, "g, beta and cu_seqlens must be aligned to their element size");
  if (!scratch || reinterpret_cast<uintptr_t>(scratch) % 16 || scratch_bytes < KDA_VALIDATE_SCRATCH_BYTES)
    return fail_msg(KDA_ERR_WORKSPACE, "scratch must be a 16-byte aligned device buffer of >= %d bytes",
                    KDA_VALIDATE_SCRATCH_BYTES);
  auto* parts = static_cast<ValidatePartial*>(scratch);
  const int b_f32 = p->beta_dtype == KDA_DTYPE_F32;
  const hipError_t e =
      p->g_dtype == KDA_DTYPE_F32
          ? launch_val<float>(g, ng, beta, nb, b_f32, cu_seqlens, p->num_seqs, p->T, parts, stream)
          : launch_val<bf16>(g, ng, beta, nb, b_f32, cu_seqlens, p->num_seqs, p->T, parts, stream);
  if (e != hipSuccess) return fail_msg(KDA_ERR_HIP, "validate launch: %s", hipGetErrorString(e));
  std::vector<ValidatePartial> host(kValBlocks);
  if (hipMemcpyAsync(host.data(), parts, sizeof(ValidatePartial) * kValBlocks, hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail_msg(KDA_ERR_HIP, "validate: copy back or synchronisation failed");
  kda_input_report r{INFINITY, -INFINITY, INFINITY, -INFINITY, 0, 0, -1, 0};
  long long bad = INT64_MAX;
  for (const ValidatePartial& v : host) {
    r.g_min = fminf(r.g_min, v.gmin);
    r.g_max = fmaxf(r.g_max, v.gmax);
    r.beta_min = fminf(r.beta_min, v.bmin);
    r.beta_max = fmaxf(r.beta_max, v.bmax);
    r.g_nonfinite += (int64_t)v.g_nonfinite;
    r.beta_nonfinite += (int64_t)v.b_nonfinite;
    if (v.cu_bad < bad) bad = v.cu_bad;
  }
  r.cu_first_bad = bad == INT64_MAX ? -1 : (int64_t)bad;
  if (r.g_nonfinite) r.failed = 1;
  else if (ng > 0 && (r.g_min < -5.f || r.g_max > 0.f)) r.failed = 2;
  else if (r.beta_nonfinite) r.failed = 3;
  else if (nb > 0 && (r.beta_min < 0.f || r.beta_max > 1.f)) r.failed = 4;
  else if (r.cu_first_bad >= 0) r.failed = 5;
  *report = r;
  switch (r.failed) {
    case 1: return fail_msg(KDA_ERR_INVALID_ARG, "g has %lld non-finite entries", (long long)r.g_nonfinite);
    case 2:
      return fail_msg(KDA_ERR_INVALID_ARG, "g must lie in [-5, 0] (found min %g, max %g)", (double)r.g_min,
                      (double)r.g_max);
    case 3: return fail_msg(KDA_ERR_INVALID_ARG, "beta has %lld non-finite entries", (long long)r.beta_nonfinite);
    case 4:
      return fail_msg(KDA_ERR_INVALID_ARG, "beta must lie in [0, 1] (found min %g, max %g)", (double)r.beta_min,
                      (double)r.beta_max);
    case 5:
      return fail_msg(KDA_ERR_INVALID_ARG,
                      "cu_seqlens breaks cu[0] == 0, non-decreasing, cu[num_seqs] == T at index %lld",
                      (long long)r.cu_first_bad);
    default: break;
  }
  return KDA_OK;
}
