// The scale folded into the RMSNorm in front of the layer: the folded norm
// weight gamma' = fp16(gamma / s), and the norm itself, which then yields the
// activation X' = X diag(s)^-1 of the W4A16 product directly (the fold is
// done offline; at run time only the norm runs). Both are HBM-bound.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

// gamma'[k] = fp16(float32(gamma[k]) / s[k]): a correctly rounded float32
// division, then one rounding to fp16
__global__ __launch_bounds__(256) void fold_norm_weight_kernel(const uint16_t* __restrict__ gamma,
                                                               const float* __restrict__ s, int K,
                                                               uint16_t* __restrict__ out) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  out[k] = __half_as_ushort(__float2half_rn(h2f(gamma[k]) / s[k]));
}

// One workgroup of 256 threads per row; the row stays in registers between
// the square sum and the scaling (CH chunks of 8 values per thread, so
// K <= 2048 CH). r = 1 / sqrt(sum(x^2) / K + eps) in float32 (tree sum:
// wavefront shuffles, then the 4 wavefront sums in LDS in a fixed order);
// y = fp16(x * r * gamma) with float32 products.
template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ gamma, int K,
                                                      float eps, uint16_t* __restrict__ Y) {
  __shared__ float wsum[4];
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* xr = X + row * K;
  u32x4 v[CH];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = 8 * (tid + 256 * c);
    v[c] = k < K ? *reinterpret_cast<const u32x4*>(xr + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = h2f((uint16_t)(v[c][i] & 0xffffu));
      const float b = h2f((uint16_t)(v[c][i] >> 16));
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float r = 1.0f / sqrtf(tot / (float)K + eps);
  uint16_t* yr = Y + row * K;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = 8 * (tid + 256 * c);
    if (k < K) {
      const u32x4 g = *reinterpret_cast<const u32x4*>(gamma + k);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = h2f((uint16_t)(v[c][i] & 0xffffu)) * r * h2f((uint16_t)(g[i] & 0xffffu));
        const float b = h2f((uint16_t)(v[c][i] >> 16)) * r * h2f((uint16_t)(g[i] >> 16));
        o[i] = (uint32_t)__half_as_ushort(__float2half_rn(a)) |
               ((uint32_t)__half_as_ushort(__float2half_rn(b)) << 16);
      }
      *reinterpret_cast<u32x4*>(yr + k) = o;
    }
  }
}

}  // namespace

hipError_t launch_fold_norm_weight(const __half* gamma, const float* s, int K, __half* out,
                                   hipStream_t st) {
  hipLaunchKernelGGL(fold_norm_weight_kernel, dim3((K + 255) / 256), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(gamma), s, K,
                     reinterpret_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const __half* X, const __half* gamma, int M, int K, float eps, __half* Y,
                          hipStream_t st) {
  const int ch = (K + 2047) / 2048;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  const uint16_t* g = reinterpret_cast<const uint16_t*>(gamma);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
#define AWQ_RN(C) \
  hipLaunchKernelGGL((rmsnorm_kernel<C>), dim3((unsigned)M), dim3(256), 0, st, x, g, K, eps, y)
  switch (ch) {
    case 1: AWQ_RN(1); break;
    case 2: AWQ_RN(2); break;
    case 3: AWQ_RN(3); break;
    case 4: AWQ_RN(4); break;
    case 5: AWQ_RN(5); break;
    case 6: AWQ_RN(6); break;
    case 7: AWQ_RN(7); break;
    case 8: AWQ_RN(8); break;
    default: return hipErrorNotSupported;
  }
#undef AWQ_RN
  return hipGetLastError();
}

}  // namespace awq
