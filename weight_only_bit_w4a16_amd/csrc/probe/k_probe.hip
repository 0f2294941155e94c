// Measurement probes for the benchmark (not part of libawq's product ABI):
// the practical ceilings the kernels are compared with, and the shader clock.
//
//   awq_probe_stream_read   reads a buffer once with 16-byte nontemporal loads
//                           (contiguous, the pattern of the M = 1 decode
//                           kernel) and writes one word per workgroup: the
//                           HBM streaming-read rate a kernel can reach
//   awq_probe_mfma          a loop of independent fp16 32x32x16 MFMAs from
//                           registers on random-valued operands: the matrix
//                           cores' rate at the clock they hold under load
//   awq_probe_clock         one wavefront spins for a fixed number of 100 MHz
//                           real-time ticks and reports the shader-clock
//                           ticks that passed: the shader clock at that moment
//
// Every kernel has a bounded loop and writes only inside the buffers it is
// given; the launchers check the sizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// workgroup b reads 16-byte items b*256 + t + j*stride (stride = grid*256),
// sixteen loads in flight per thread: of the patterns measured on MI355X
// (1-16 loads per thread, 1024-16384 workgroups of 256-1024 threads, with
// and without the nontemporal hint) this one, at 2048 workgroups, streams
// fastest
constexpr int kStreamUnroll = 16;
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0, 0, 0, 0};
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];  // every component: 16-byte loads stay
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  // keep the loads alive: one word per workgroup, from lane 0 of wave 0
  uint32_t a = (acc.x ^ acc.y) ^ (acc.z ^ acc.w);
  a = __reduce_xor_sync(0xffffffffffffffffull, a);
  if (threadIdx.x == 0) out[blockIdx.x] = a;
}

// iters x 8 independent MFMAs per wavefront; operands from the seed buffer
__global__ __launch_bounds__(256) void mfma_kernel(const u32x4* __restrict__ seed, int iters,
                                                   float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  u32x4 a = seed[lane], b = seed[64 + lane];
  floatx16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// out[2 slot] = shader-clock ticks, out[2 slot + 1] = real-time ticks
__global__ void clock_kernel(unsigned long long* __restrict__ out, int slot, int rt_ticks) {
  if (threadIdx.x != 0) return;
  const unsigned long long r0 = wall_clock64();
  const unsigned long long c0 = clock64();
  unsigned long long r1 = r0;
  for (int it = 0; it < (1 << 22) && r1 - r0 < (unsigned long long)rt_ticks; ++it)
    r1 = wall_clock64();
  const unsigned long long c1 = clock64();
  out[2 * slot] = c1 - c0;
  out[2 * slot + 1] = r1 - r0;
}

}  // namespace

extern "C" {

// src: n16 16-byte items (device); out: at least `grid` uint32 (device)
int awq_probe_stream_read(const void* src, size_t n16, int grid, void* out, void* stream) {
  if (!src || !out || n16 == 0 || grid <= 0) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, n16, (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// seed: 128 16-byte items (device); out: 4 grid floats (device)
int awq_probe_mfma(const void* seed, int grid, int iters, void* out, void* stream) {
  if (!seed || !out || grid <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)seed, iters, (float*)out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// out: 2 (slot + 1) uint64 (device)
int awq_probe_clock(void* out, int slot, int rt_ticks, void* stream) {
  if (!out || slot < 0 || rt_ticks <= 0) return 1;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (unsigned long long*)out, slot, rt_ticks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
