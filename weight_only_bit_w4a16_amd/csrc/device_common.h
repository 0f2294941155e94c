// Device helpers shared by the HIP kernels of libawq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A value in an SGPR (in_sgpr) or a VGPR (in_vgpr) that the compiler cannot
// see through: the empty asm emits no instruction, so the register is
// written by the compiler's own move. Used to give three-operand VALU
// instructions their constants in registers, since a VOP3 encoding takes no
// literal on gfx950.
__device__ __forceinline__ uint32_t in_sgpr(uint32_t c) {
  asm("" : "=s"(c) : "0"(c));
  return c;
}
__device__ __forceinline__ uint32_t in_vgpr(uint32_t c) {
  asm("" : "=v"(c) : "0"(c));
  return c;
}

// fp16 bit pattern of 1024.0: OR-ing a code c << e (e + bits <= 10) into its
// mantissa gives the fp16 value 1024 + c * 2^e exactly.
constexpr uint32_t kMagic2 = 0x64006400u;

// The unpack constants in registers, made once per kernel outside its loops
// (the empty asm is not moved out of a loop by the compiler, so a mask made
// at its use would cost one scalar move per use): the fp16 magic number in a
// VGPR and the nibble / 3-bit masks in SGPRs, so that (w & mask) | magic is
// one v_and_or_b32 (see and_or). Fields a kernel does not use cost nothing.
struct UnpackRegs {
  uint32_t magic;     // kMagic2
  uint32_t lo4, hi4;  // int4: codes 0, 4 (0x000F000F) and 1, 5 (0x00F000F0) of a word
  uint32_t m3[5];     // int3: the five pair masks of a 10-code word
};
__device__ __forceinline__ UnpackRegs unpack_regs() {
  UnpackRegs r;
  r.magic = in_vgpr(kMagic2);
  r.lo4 = in_sgpr(0x000F000Fu);
  r.hi4 = in_sgpr(0x00F000F0u);
  r.m3[0] = in_sgpr(0x001C0007u);
  r.m3[1] = in_sgpr(0x00E00038u);
  r.m3[2] = in_sgpr(0x0007000Eu);
  r.m3[3] = in_sgpr(0x00380070u);
  r.m3[4] = in_sgpr(0x00070380u);
  return r;
}

// Grid of one quantization group (asymmetric round-to-nearest, the range
// always containing 0, "number of levels" read as 2^b - 1 steps). All
// operations are single IEEE float32 roundings: the library is compiled with
// -ffp-contract=off and float division is correctly rounded.
struct GroupGrid {
  float delta;
  float rdelta;  // approximate 1 / delta (v_rcp_f32), used only to pick codes fast
  int z;
};

__device__ __forceinline__ GroupGrid group_grid(float wmin, float wmax, int qmax) {
  const float lo = fminf(wmin, 0.0f);
  const float hi = fmaxf(wmax, 0.0f);
  const float r = hi - lo;
  GroupGrid g;
  if (r == 0.0f) {
    g.delta = 1.0f;
    g.z = 0;
  } else {
    g.delta = r / (float)qmax;
    g.z = (int)rintf(-lo / g.delta);
  }
  g.rdelta = __builtin_amdgcn_rcpf(g.delta);
  return g;
}

// Symmetric grid of one group (the zero_point=false option of the AWQ
// config): delta = max|W'| / (2^(b-1) - 1), codes rint(W' / delta) in
// [-(2^(b-1) - 1), 2^(b-1) - 1] stored with the offset z = 2^(b-1); an
// all-zero group gets delta = 1.
__device__ __forceinline__ GroupGrid group_grid_sym(float amax, int half) {
  GroupGrid g;
  g.delta = amax == 0.0f ? 1.0f : amax / (float)(half - 1);
  g.z = half;
  g.rdelta = __builtin_amdgcn_rcpf(g.delta);
  return g;
}

// the grid of a group from its min and max, symmetric or asymmetric
template <bool SYM, int BITS>
__device__ __forceinline__ GroupGrid grid_of(float wmin, float wmax) {
  if constexpr (SYM)
    return group_grid_sym(fmaxf(__builtin_fabsf(wmin), __builtin_fabsf(wmax)), 1 << (BITS - 1));
  else
    return group_grid(wmin, wmax, (1 << BITS) - 1);
}

// q = clamp(rint(wp / delta) + z, 0, qmax) with wp / delta the correctly
// rounded fp32 quotient. |wp / delta| <= qmax, and wp * rdelta is within
// 2 ulp of the exact quotient, so it rounds to the same integer unless it
// lies within a few ulp of a half-integer; only those (rare) lanes pay for
// the IEEE division.
__device__ __forceinline__ int quant_code(float wp, GroupGrid g, int qmax) {
  const float t = wp * g.rdelta;
  float qf = rintf(t);
  if (__builtin_fabsf(__builtin_amdgcn_fractf(t) - 0.5f) < 0x1p-16f) qf = rintf(wp / g.delta);
  const int q = (int)qf + g.z;
  return q < 0 ? 0 : (q > qmax ? qmax : q);
}

// int3 packing: the 16 lanes of one 128-code block (an aligned 16-lane
// segment) each hold 8 consecutive codes as 24 bits (lane i: codes
// 8i .. 8i+7); lane w < 13 gets word w of the block, codes 10w .. 10w+9 at
// bits 3 (k - 10w) (the last word holds codes 120 .. 127); lanes 13 .. 15 get 0.
__device__ __forceinline__ uint32_t int3_block_word(uint32_t packed24, int w) {
  const int t1 = (10 * w) >> 3;
  const uint32_t lo24 = __shfl(packed24, t1 < 15 ? t1 : 15, 16);
  const uint32_t hi24 = __shfl(packed24, t1 + 1 < 15 ? t1 + 1 : 15, 16);
  const uint64_t both = (uint64_t)lo24 | ((uint64_t)(t1 + 1 < 16 ? hi24 : 0u) << 24);
  const int first = 10 * w - 8 * t1;
  const int count = w < 12 ? 10 : (w == 12 ? 8 : 0);
  const uint32_t word = (uint32_t)(both >> (3 * first));
  return word & (count >= 10 ? 0x3fffffffu : ((1u << (3 * count)) - 1u));
}

// min and max over a workgroup of NT threads (NT / 64 wavefronts): wavefront
// shuffles, then the wavefront results through LDS (red holds 2 NT / 64
// floats); every thread gets the result
template <int NT>
__device__ __forceinline__ void block_minmax(float& mn, float& mx, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[wave] = mn;
    red[NT / 64 + wave] = mx;
  }
  __syncthreads();
  mn = red[0];
  mx = red[NT / 64];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) {
    mn = fminf(mn, red[w]);
    mx = fmaxf(mx, red[NT / 64 + w]);
  }
}

__device__ __forceinline__ float h2f(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// Group parameters of row n, group g, for a row of ng groups. Plain storage
// (CS = false): float32 steps and uint8 zero points, [N][ng] each. Compact
// storage (CS = true): fp16 steps [N][ng] and 4-bit zero points, 8 per
// uint32 word in group order, [N][ceil(ng / 8)].
template <bool CS>
__device__ __forceinline__ float group_scale(const void* S, size_t n, int ng, int g) {
  if constexpr (CS)
    return h2f(static_cast<const uint16_t*>(S)[n * ng + g]);
  else
    return static_cast<const float*>(S)[n * ng + g];
}
template <bool CS>
__device__ __forceinline__ uint32_t group_zero(const void* Z, size_t n, int ng, int g) {
  if constexpr (CS)
    return (static_cast<const uint32_t*>(Z)[n * ((ng + 7) >> 3) + (g >> 3)] >> (4 * (g & 7))) &
           15u;
  else
    return static_cast<const uint8_t*>(Z)[n * ng + g];
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

}  // namespace awq
