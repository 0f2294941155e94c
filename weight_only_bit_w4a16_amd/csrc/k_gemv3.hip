// Decode kernel for 3-bit weights (W3A16), M <= 4 activation rows.
//
// Layout reminder: a group of 128 codes is 13 words of 10 codes (bits 30-31
// and the last word's slots 8-9 are zero), so a group never shares a word
// with its neighbours. One lane owns one (row, group) item: it loads the 13
// words and the group's step and zero point, unpacks with the fp16
// magic-number trick and accumulates with v_dot2_f32_f16.
//
// Unpacking. For a word w with codes c0..c9 (c_i at bits 3i), five AND-OR
// operations (plus two shifts) give five fp16 pairs with every code inside
// the fp16 mantissa of 1024:
//   p0 = (w      & 0x001C0007) | M -> (1024 +   c0, 1024 +  4 c6)
//   p1 = (w      & 0x00E00038) | M -> (1024 + 8 c1, 1024 + 32 c7)
//   p2 = (w >> 8 & 0x0007000E) | M -> (1024 + 2 c3, 1024 +    c8)
//   p3 = (w >> 8 & 0x00380070) | M -> (1024 +16 c4, 1024 +  8 c9)
//   p4 = (w << 1 & 0x00070380) | M -> (1024 +128 c2, 1024 +   c5)
// The activation pairs are stored pre-divided by those powers of two, so
//   dot2(p, x') = 1024 (x'_a + x'_b) + x''_a c_a + x''_b c_b,  x'' = 2^e x',
// and per group  sum x'' (c - z) = sum dot2 - C - z S,  C = 1024 sum x',
// S = sum x'', with C and S computed once per call.
//
// Rows are processed in passes of RB rows per workgroup (RB * groups items
// fill the workgroup); the per-item partial sums go to LDS and each row is
// added up in a fixed order, so the result is bitwise reproducible. The next
// pass's weights are loaded while the current pass is reduced, and the first
// pass's while the activations are prepared.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int IPT = 4;     // items per thread per pass: rows_per_pass * groups <= 256 * IPT
constexpr int WSTR = 8;    // LDS dwords per word of activation pairs (5 used, 16 B aligned)
constexpr int GSTR = 13 * WSTR;

// code slot of the lo / hi half of pair t of a word, and its power-of-two weight
__device__ __constant__ int kPairLo[5] = {0, 1, 3, 4, 2};
__device__ __constant__ int kPairHi[5] = {6, 7, 8, 9, 5};

// (a & m) | o as one v_and_or_b32: m in an SGPR and o in a VGPR (from
// unpack_regs), since a VOP3 instruction takes no literal on gfx950 and with
// both constants visible the compiler would emit an AND and an OR. The
// instruction is the compiler's own, not inline asm: only then does it keep
// the wait states gfx950 requires between a VALU write and an MFMA reading
// the result (it does not track writes made by inline asm, and an MFMA
// issued right after such a write can read the register's old value).
__device__ __forceinline__ uint32_t and_or3(uint32_t a, uint32_t m, uint32_t o) {
  return (a & m) | o;
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)__half_as_ushort(__float2half_rn(a)) |
         ((uint32_t)__half_as_ushort(__float2half_rn(b)) << 16);
}

}  // namespace

template <int MR, bool CS>
__global__ __launch_bounds__(256) void gemv_w3_kernel(const uint16_t* __restrict__ X,
                                                      const uint32_t* __restrict__ Q,
                                                      const void* __restrict__ S,
                                                      const void* __restrict__ Z,
                                                      uint16_t* __restrict__ Y, int M, int N,
                                                      int K, int wpr, int RB, int gshift) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int ng = K >> 7;                  // 128-code blocks per row
  const int ngr = max(1, ng >> gshift);  // groups per row (scale / zero-point stride)
  u32x4* xp4 = reinterpret_cast<u32x4*>(smem);                                  // [MR][ng][13][8]
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem);
  float2* cs = reinterpret_cast<float2*>(smem + (size_t)MR * ng * GSTR * 4);     // [MR][ng]
  float2* wsum = cs + MR * ng;                                                  // [MR][ng][13]
  float* part = reinterpret_cast<float*>(wsum + MR * ng * 13);                  // [RB][MR][ng]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nrb = (N + RB - 1) / RB;

  uint32_t wv[IPT][13];
  float dl[IPT];
  uint32_t zl[IPT];
  auto load_pass = [&](int rb) {
    const int items = min(RB, N - rb * RB) * ng;
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int it = min(tid + 256 * u, items - 1);
      const int r = it / ng, g = it % ng;
      const size_t n = (size_t)rb * RB + r;
      const uint32_t* qg = Q + n * wpr + 13 * g;
#pragma unroll
      for (int k = 0; k < 13; ++k) wv[u][k] = ld_nt(qg + k);
      dl[u] = group_scale<CS>(S, n, ngr, g >> gshift);
      zl[u] = group_zero<CS>(Z, n, ngr, g >> gshift);
    }
  };
  // the first pass's weights are in flight while the activations are prepared
  if ((int)blockIdx.x < nrb) load_pass(blockIdx.x);

  // ---- activation pairs, pre-divided by the unpacking weights --------------
  // one thread per (row m, group g, word w): 10 activations -> 5 pairs
  for (int i = tid; i < M * ng * 13; i += 256) {
    const int w = i % 13;
    const int mg = i / 13;  // m * ng + g
    const int m = mg / ng, g = mg % ng;
    const uint16_t* xg = X + (size_t)m * K + g * 128 + 10 * w;
    float xv[10];
#pragma unroll
    for (int c = 0; c < 10; ++c) xv[c] = (10 * w + c < 128) ? h2f(xg[c]) : 0.f;
    // pairs (c0,c6)/(1,1/4) (c1,c7)/(1/8,1/32) (c3,c8)/(1/2,1) (c4,c9)/(1/16,1/8) (c2,c5)/(1/128,1)
    const float a0 = xv[0], b0 = xv[6] * 0.25f;
    const float a1 = xv[1] * 0.125f, b1 = xv[7] * 0.03125f;
    const float a2 = xv[3] * 0.5f, b2 = xv[8];
    const float a3 = xv[4] * 0.0625f, b3 = xv[9] * 0.125f;
    const float a4 = xv[2] * 0.0078125f, b4 = xv[5];
    const uint32_t p0 = pack2(a0, b0), p1 = pack2(a1, b1), p2 = pack2(a2, b2), p3 = pack2(a3, b3),
                   p4 = pack2(a4, b4);
    uint32_t* dst = xp + (size_t)mg * GSTR + w * WSTR;
    *reinterpret_cast<u32x4*>(dst) = u32x4{p0, p1, p2, p3};
    dst[4] = p4;
    // sums of the stored (rounded) pair values x' and of x'' = 2^e x'
    float c = 0.f, sx = 0.f;
    const uint32_t pp[5] = {p0, p1, p2, p3, p4};
    const float wl[5] = {1.f, 8.f, 2.f, 16.f, 128.f}, wh[5] = {4.f, 32.f, 1.f, 8.f, 1.f};
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      const float lo = h2f((uint16_t)(pp[t] & 0xffffu)), hi = h2f((uint16_t)(pp[t] >> 16));
      c += lo + hi;
      sx += lo * wl[t] + hi * wh[t];
    }
    wsum[i] = make_float2(c, sx);
  }
  __syncthreads();
  for (int i = tid; i < M * ng; i += 256) {
    float c = 0.f, sx = 0.f;
#pragma unroll
    for (int w = 0; w < 13; ++w) {
      const float2 v = wsum[i * 13 + w];
      c += v.x;
      sx += v.y;
    }
    cs[i] = make_float2(1024.f * c, sx);
  }
  __syncthreads();

  const UnpackRegs ur = unpack_regs();
  for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
    const int items = min(RB, N - rb * RB) * ng;
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int it = tid + 256 * u;
      if (it < items) {
        const int r = it / ng, g = it % ng;
        float acc[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll
        for (int k = 0; k < 13; ++k) {
          const uint32_t w = wv[u][k];
          const uint32_t t8 = w >> 8, u1 = w << 1;
          const uint32_t pr[5] = {and_or3(w, ur.m3[0], ur.magic), and_or3(w, ur.m3[1], ur.magic),
                                  and_or3(t8, ur.m3[2], ur.magic), and_or3(t8, ur.m3[3], ur.magic),
                                  and_or3(u1, ur.m3[4], ur.magic)};
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            if (m < M) {
              const size_t base = ((size_t)m * ng + g) * 13 + k;  // in units of WSTR dwords
              const u32x4 x4 = xp4[base * 2];
              const uint32_t x5 = xp[base * WSTR + 4];
              acc[m] = dot2(pr[0], x4[0], acc[m]);
              acc[m] = dot2(pr[1], x4[1], acc[m]);
              acc[m] = dot2(pr[2], x4[2], acc[m]);
              acc[m] = dot2(pr[3], x4[3], acc[m]);
              acc[m] = dot2(pr[4], x5, acc[m]);
            }
          }
        }
        const float zf = (float)zl[u];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < M) {
            const float2 c = cs[m * ng + g];
            part[(r * MR + m) * ng + g] = dl[u] * (acc[m] - __builtin_fmaf(zf, c.y, c.x));
          }
        }
      }
    }
    // next pass's weights in flight during the row sums
    if (rb + (int)gridDim.x < nrb) load_pass(rb + gridDim.x);
    __syncthreads();
    // row sums in a fixed order: wavefront `wave` adds up rows wave, wave+4, ...
    for (int rm = wave; rm < RB * M; rm += 4) {
      const int r = rm / M, m = rm % M;
      const size_t n = (size_t)rb * RB + r;
      if (n < (size_t)N) {
        const float* pr = part + (size_t)(r * MR + m) * ng;
        float v = 0.f;
        for (int g = lane; g < ng; g += 64) v += pr[g];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(v));
      }
    }
    __syncthreads();
  }
}

namespace {
int cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}
}  // namespace

template <bool CS>
hipError_t launch_gemv_w3_t(const __half* X, const uint32_t* q, const void* scales,
                            const void* zeros, int M, int N, int K, int group, __half* Y,
                            hipStream_t st) {
  if (M > kGemvW3MaxM) return hipErrorNotSupported;
  const int gshift = group_shift(group);
  const int ng = K / 128;
  const int RB = (256 * IPT) / ng;  // rows per pass
  if (RB < 1) return hipErrorNotSupported;
  const int wpr = words_per_row(K, 3, group);
  const int mr = M == 1 ? 1 : (M == 2 ? 2 : 4);
  const size_t lds = (size_t)mr * ng * GSTR * 4 + (size_t)mr * ng * 8 + (size_t)mr * ng * 13 * 8 +
                     (size_t)RB * mr * ng * 4;
  if (lds > 64 * 1024) return hipErrorNotSupported;
  const int nrb = (N + RB - 1) / RB;
  const dim3 grid((unsigned)min(nrb, 4 * cus())), block(256);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  if (mr == 1)
    hipLaunchKernelGGL((gemv_w3_kernel<1, CS>), grid, block, lds, st, x, q, scales, zeros, y, M, N, K,
                       wpr, RB, gshift);
  else if (mr == 2)
    hipLaunchKernelGGL((gemv_w3_kernel<2, CS>), grid, block, lds, st, x, q, scales, zeros, y, M, N, K,
                       wpr, RB, gshift);
  else
    hipLaunchKernelGGL((gemv_w3_kernel<4, CS>), grid, block, lds, st, x, q, scales, zeros, y, M, N, K,
                       wpr, RB, gshift);
  return hipGetLastError();
}

hipError_t launch_gemv_w3(const __half* X, const uint32_t* q, const void* scales,
                          const void* zeros, int M, int N, int K, int group, __half* Y,
                          hipStream_t st, bool cs) {
  return cs ? launch_gemv_w3_t<true>(X, q, scales, zeros, M, N, K, group, Y, st)
            : launch_gemv_w3_t<false>(X, q, scales, zeros, M, N, K, group, Y, st);
}

}  // namespace awq
