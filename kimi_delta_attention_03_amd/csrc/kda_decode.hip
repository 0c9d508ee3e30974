// One decode step of the KDA token recurrence on gfx950 ("KDA Doesn't Care
// About the Future", section "Chunkwise KDA in Broad Strokes", steps (0)-(5);
// Tokamax "chunk_kda_fwd design doc", section 9.1.2, Paper Eq. 1):
//   S_bar = Diag(exp g) S                 decay
//   e     = v - S_bar^T k                 prediction error
//   S     = S_bar + beta k e^T            delta-rule write
//   o     = scale * S^T q                 read after the write
// Every column of S evolves on its own (each line above is column-wise), so
// lane j of a wave owns column j of one (sequence, head) state: the column
// stays in registers and both dot products over K are lane-local; the K
// values of q, k and exp(g), the same for every lane, are read from LDS.
// The state is read once and written once, coalesced across lanes.
#include "kda_device.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, typename TG, typename TB, int K>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  constexpr int V = K;
  constexpr int NVB = V / 64;
  const int lane = threadIdx.x;
  const int u = blockIdx.x / NVB;             // (sequence, head)
  const int j = (blockIdx.x % NVB) * 64 + lane;  // state column
  const T* q = reinterpret_cast<const T*>(a.q) + (size_t)u * K;
  const T* k = reinterpret_cast<const T*>(a.k) + (size_t)u * K;
  const TG* g = reinterpret_cast<const TG*>(a.g) + (size_t)u * K;
  const float beta = to_f32(reinterpret_cast<const TB*>(a.beta)[u]);
  const float vj = to_f32(reinterpret_cast<const T*>(a.v)[(size_t)u * V + j]);
  float* S = a.state + (size_t)u * K * V + j;

  // q, k and the decay factors of this head, shared by the wave through LDS
  // (broadcast reads), with the optional L2 norms folded in
  __shared__ float sq[K], sk[K], sa[K];
  float qs = 0.f, ks = 0.f;
  for (int i = lane; i < K; i += 64) {
    const float qi = to_f32(q[i]), ki = to_f32(k[i]);
    sq[i] = qi;
    sk[i] = ki;
    sa[i] = exp2f(kLog2e * to_f32(g[i]));
    qs += qi * qi;
    ks += ki * ki;
  }
  float qn = 1.f, kn = 1.f;
  if (a.l2norm) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      qs += __shfl_xor(qs, off, 64);
      ks += __shfl_xor(ks, off, 64);
    }
    qn = 1.f / fmaxf(sqrtf(qs), a.l2eps);
    kn = 1.f / fmaxf(sqrtf(ks), a.l2eps);
  }
  __syncthreads();

  float s[K];
#pragma unroll
  for (int i = 0; i < K; ++i) s[i] = S[(size_t)i * V];
  float e = vj;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    s[i] *= sa[i];
    e -= kn * sk[i] * s[i];
  }
  const float be = beta * e;
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    s[i] += be * kn * sk[i];
    o += qn * sq[i] * s[i];
    S[(size_t)i * V] = s[i];
  }
  o *= a.scale;
  if constexpr (sizeof(T) == 2) reinterpret_cast<bf16*>(a.o)[(size_t)u * V + j] = (bf16)o;
  else reinterpret_cast<float*>(a.o)[(size_t)u * V + j] = o;
}

template <typename T, int K>
hipError_t launch_t(const DecodeArgs& a, int g_f32, int b_f32, hipStream_t s) {
  const dim3 grid((unsigned)(a.nunits * (K / 64))), block(64);
  if (g_f32) {
    if (b_f32) hipLaunchKernelGGL((decode_kernel<T, float, float, K>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<T, float, bf16, K>), grid, block, 0, s, a);
  } else {
    if (b_f32) hipLaunchKernelGGL((decode_kernel<T, bf16, float, K>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<T, bf16, bf16, K>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int K, int bf16_qkv, int g_f32, int b_f32, hipStream_t s) {
  if (a.nunits <= 0) return hipSuccess;
  if (bf16_qkv) return K == 128 ? launch_t<kda::bf16, 128>(a, g_f32, b_f32, s) : launch_t<kda::bf16, 64>(a, g_f32, b_f32, s);
  return K == 128 ? launch_t<float, 128>(a, g_f32, b_f32, s) : launch_t<float, 64>(a, g_f32, b_f32, s);
}

}  // namespace kda
