// Quantize-and-pack, activation statistic, scale candidates and the fold of
// diag(s)^-1 into the activation. These are the HBM-bound "offline" kernels
// that feed the W4A16 product.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

// ---------------------------------------------------------------------------
// Round-to-nearest quantize-and-pack.
// One thread owns 8 consecutive codes of one group; the TPG = group/8
// threads of a group sit in one wavefront and reduce min/max with shuffles.
// int4: each thread writes its own packed word. int3: each thread folds its
// 8 codes into 24 bits; within each 128-code block (16 threads, 13 words),
// thread w gathers the 24-bit pieces that cover codes 10w..10w+9 from its
// neighbours and writes word w.
// ---------------------------------------------------------------------------
// The packed codes, steps and zero points go out with nontemporal stores: a
// packed matrix is read later (by the products), not by the next kernel, and
// with ordinary stores its lines were written back to HBM while the next
// kernel ran (the decode launches right after a pack of the 8192x28672 layer
// took 24.2 instead of 22.3 us; same bits, same pack time).
template <int BITS, int TPG, bool SYM>
__global__ __launch_bounds__(256) void quant_pack_kernel(const uint16_t* __restrict__ W,
                                                         const float* __restrict__ s, int N, int K,
                                                         uint32_t* __restrict__ Q,
                                                         float* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros, int wpr) {
  constexpr int G = TPG * 8;
  constexpr int QMAX = (1 << BITS) - 1;
  const int ng = K / G;
  // grid: x walks the K/8 threads of a row, y the rows (strided past 65535)
  const int tr = blockIdx.x * 256 + threadIdx.x;
  // threads past the row end form whole groups (K and 256 threads are
  // multiples of the group); they work on the last group so every lane
  // joins the shuffles, and store nothing
  const bool active = tr < K / 8;
  const int tt = active ? tr : K / 8 - TPG + (tr % TPG);
  const int j = tt % TPG;
  const int g = tt / TPG;
  const int k0 = 8 * tt;
  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = 1.0f;
  if (s != nullptr) {
    const float4 s0 = *reinterpret_cast<const float4*>(s + k0);
    const float4 s1 = *reinterpret_cast<const float4*>(s + k0 + 4);
    sv[0] = s0.x, sv[1] = s0.y, sv[2] = s0.z, sv[3] = s0.w;
    sv[4] = s1.x, sv[5] = s1.y, sv[6] = s1.z, sv[7] = s1.w;
  }
  // rows blockIdx.y, + gridDim.y, ...; the next row's load is issued before
  // the current row is processed
  uint4 raw = *reinterpret_cast<const uint4*>(W + (size_t)blockIdx.y * K + k0);
  for (int nr = blockIdx.y; nr < N; nr += gridDim.y) {
    const size_t n = (size_t)nr;
    const int nx = min(nr + (int)gridDim.y, N - 1);
    const uint4 next = *reinterpret_cast<const uint4*>(W + (size_t)nx * K + k0);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    raw = next;
    float wp[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wp[2 * i] = h2f((uint16_t)(rw[i] & 0xffffu));
      wp[2 * i + 1] = h2f((uint16_t)(rw[i] >> 16));
    }
    // s == 1 multiplies exactly, so plain RTN takes the same path
#pragma unroll
    for (int i = 0; i < 8; ++i) wp[i] = wp[i] * sv[i];
    float mn = wp[0], mx = wp[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn = fminf(mn, wp[i]);
      mx = fmaxf(mx, wp[i]);
    }
#pragma unroll
    for (int off = 1; off < TPG; off <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, off, TPG));
      mx = fmaxf(mx, __shfl_xor(mx, off, TPG));
    }
    const GroupGrid gg = grid_of<SYM, BITS>(mn, mx);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= (uint32_t)quant_code(wp[i], gg, QMAX) << (BITS * i);

    uint32_t* qrow = Q + n * wpr;
    if (BITS == 4) {
      if (active) __builtin_nontemporal_store(packed, qrow + g * (G / 8) + j);
    } else {
      const int jb = j & 15;                         // lane in the 128-code block
      const int blk = g * (G / 128) + (j >> 4);      // block of the row
      const uint32_t word = int3_block_word(packed, jb);
      if (active) {
        if (jb < 13) {
          __builtin_nontemporal_store(word, qrow + 13 * blk + jb);
        } else if (blk == K / 128 - 1 && 13 * blk + jb < wpr) {
          __builtin_nontemporal_store(0u, qrow + 13 * blk + jb);  // row padding to 16 bytes
        }
      }
    }
    if (active && j == 0) {
      __builtin_nontemporal_store(gg.delta, scales + n * ng + g);
      __builtin_nontemporal_store((uint8_t)gg.z, zeros + n * ng + g);
    }
  }
}

// ---------------------------------------------------------------------------
// Per-output-channel groups (a group of the whole row, K a multiple of 128):
// one workgroup of 512 threads per row, the row held in registers (CH chunks
// of 8 codes per thread, K <= 4096 CH) between the row-wide min / max and the
// quantization. Chunk c of thread t covers codes 8 (t + 512 c) .. + 7, so the
// 16 threads of a 128-code block are one aligned 16-lane segment, as the
// int3 word gather needs.
// ---------------------------------------------------------------------------
template <int BITS, int CH, bool SYM>
__global__ __launch_bounds__(512) void quant_pack_row_kernel(const uint16_t* __restrict__ W,
                                                             const float* __restrict__ s, int K,
                                                             uint32_t* __restrict__ Q,
                                                             float* __restrict__ scales,
                                                             uint8_t* __restrict__ zeros,
                                                             int wpr) {
  constexpr int QMAX = (1 << BITS) - 1;
  __shared__ float red[16];
  const size_t n = blockIdx.x;
  const int t = threadIdx.x;
  u32x4 raw[CH];
  float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k0 = 8 * (t + 512 * c);
    raw[c] = k0 < K ? *reinterpret_cast<const u32x4*>(W + n * K + k0) : u32x4{0u, 0u, 0u, 0u};
    if (k0 < K) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sv = s != nullptr ? s[k0 + i] : 1.0f;
        const float wp = h2f((uint16_t)(raw[c][i >> 1] >> (16 * (i & 1)))) * sv;
        mn = fminf(mn, wp);
        mx = fmaxf(mx, wp);
      }
    }
  }
  block_minmax<512>(mn, mx, red);
  const GroupGrid gg = grid_of<SYM, BITS>(mn, mx);
  uint32_t* qrow = Q + n * wpr;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k0 = 8 * (t + 512 * c);
    if (8 * 512 * c >= K) break;  // uniform: no thread has this chunk
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sv = s != nullptr && k0 < K ? s[k0 + i] : 1.0f;
      const float wp = h2f((uint16_t)(raw[c][i >> 1] >> (16 * (i & 1)))) * sv;
      packed |= (uint32_t)quant_code(wp, gg, QMAX) << (BITS * i);
    }
    if (BITS == 4) {
      if (k0 < K) qrow[k0 >> 3] = packed;
    } else {
      // blocks are whole 16-lane segments, all inside or all past the row
      const int jb = t & 15, blk = k0 >> 7;
      const uint32_t word = int3_block_word(packed, jb);
      if (k0 < K) {
        if (jb < 13)
          __builtin_nontemporal_store(word, qrow + 13 * blk + jb);
        else if (blk == K / 128 - 1 && 13 * blk + jb < wpr)
          __builtin_nontemporal_store(0u, qrow + 13 * blk + jb);  // row padding to 16 bytes
      }
    }
  }
  if (BITS == 4 && t < wpr - K / 8) qrow[K / 8 + t] = 0u;  // int4 rows are whole 16 B
  if (t == 0) {
    scales[n] = gg.delta;
    zeros[n] = (uint8_t)gg.z;
  }
}

hipError_t launch_quant_pack_row(const __half* W, const float* s, int N, int K, int bits,
                                 bool zero_point, uint32_t* q, float* scales, uint8_t* zeros,
                                 hipStream_t st) {
  const int ch = (K + 4095) / 4096;
  if (ch > kRowMaxChunks) return hipErrorNotSupported;
  const int wpr = words_per_row(K, bits, K);
  const uint16_t* w = reinterpret_cast<const uint16_t*>(W);
#define AWQ_QR(B, C, SY)                                                                       \
  hipLaunchKernelGGL((quant_pack_row_kernel<B, C, SY>), dim3((unsigned)N), dim3(512), 0, st, w, \
                     s, K, q, scales, zeros, wpr)
#define AWQ_QR2(C)                    \
  do {                                \
    if (bits == 4 && zero_point)      \
      AWQ_QR(4, C, false);            \
    else if (bits == 4)               \
      AWQ_QR(4, C, true);             \
    else if (zero_point)              \
      AWQ_QR(3, C, false);            \
    else                              \
      AWQ_QR(3, C, true);             \
  } while (0)
  switch (ch) {
    case 1: AWQ_QR2(1); break;
    case 2: AWQ_QR2(2); break;
    case 3: AWQ_QR2(3); break;
    case 4: AWQ_QR2(4); break;
    case 5: AWQ_QR2(5); break;
    case 6: AWQ_QR2(6); break;
    case 7: AWQ_QR2(7); break;
    default: AWQ_QR2(8); break;
  }
#undef AWQ_QR2
#undef AWQ_QR
  return hipGetLastError();
}

hipError_t launch_quant_pack(const __half* W, const float* s, int N, int K, int bits, int group,
                             bool zero_point, uint32_t* q, float* scales, uint8_t* zeros,
                             hipStream_t st) {
  if (row_group(group))
    return launch_quant_pack_row(W, s, N, K, bits, zero_point, q, scales, zeros, st);
  const int wpr = words_per_row(K, bits, group);
  // about 4 rows per thread
  const int gy = (N + 3) / 4 < 65535 ? (N + 3) / 4 : 65535;
  const dim3 grid((unsigned)((K / 8 + 255) / 256), (unsigned)gy);
  const uint16_t* w = reinterpret_cast<const uint16_t*>(W);
#define AWQ_QP1(B, T, SY)                                                                    \
  hipLaunchKernelGGL((quant_pack_kernel<B, T, SY>), grid, dim3(256), 0, st, w, s, N, K, q, \
                     scales, zeros, wpr)
#define AWQ_QP(B, T)      \
  do {                    \
    if (zero_point)       \
      AWQ_QP1(B, T, false); \
    else                  \
      AWQ_QP1(B, T, true);  \
  } while (0)
  if (bits == 4) {
    if (group == 128) AWQ_QP(4, 16);
    else if (group == 256) AWQ_QP(4, 32);
    else AWQ_QP(4, 64);
  } else {
    if (group == 128) AWQ_QP(3, 16);
    else if (group == 256) AWQ_QP(3, 32);
    else AWQ_QP(3, 64);
  }
#undef AWQ_QP
#undef AWQ_QP1
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compact group parameters: steps rounded to fp16, zero points as 4-bit
// fields, 8 per uint32 word in group order; one thread per zero-point word.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void compact_params_kernel(const float* __restrict__ S,
                                                             const uint8_t* __restrict__ Z, int N,
                                                             int ng, uint16_t* __restrict__ S16,
                                                             uint32_t* __restrict__ Z4) {
  const int zw = (ng + 7) >> 3;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)N * zw) return;
  const size_t n = (size_t)(i / zw);
  const int w = (int)(i % zw);
  uint32_t word = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int g = 8 * w + u;
    if (g < ng) {
      word |= ((uint32_t)Z[n * ng + g] & 15u) << (4 * u);
      S16[n * ng + g] = __half_as_ushort(__float2half_rn(S[n * ng + g]));
    }
  }
  Z4[i] = word;
}

hipError_t launch_compact_params(const float* scales, const uint8_t* zeros, int N, int ng,
                                 uint16_t* scales16, uint32_t* zeros4, hipStream_t st) {
  const long items = (long)N * ((ng + 7) / 8);
  hipLaunchKernelGGL(compact_params_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                     st, scales, zeros, N, ng, scales16, zeros4);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// X' = fp16(float32(X) / s), 8 elements per thread, the quotient correctly
// rounded to fp32 and then to fp16. x * (1/s) with the hardware reciprocal is
// within 2 ulp (fp32) of the correctly rounded quotient, so it rounds to the
// same fp16 unless its 13 dropped mantissa bits lie within a few ulp of the
// fp16 midpoint, or the result is an fp16 subnormal; those lanes divide.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fold_one(float x, float sv, float rs) {
  float t = x * rs;
  const uint32_t low = __float_as_uint(t) & 0x1fffu;
  const uint32_t dist = low > 0x1000u ? low - 0x1000u : 0x1000u - low;
  if (dist <= 8u || __builtin_fabsf(t) < 0x1p-14f) t = x / sv;
  return (uint32_t)__half_as_ushort(__float2half_rn(t));
}

__global__ __launch_bounds__(256) void fold_kernel(const uint16_t* __restrict__ X,
                                                   const float* __restrict__ s, int M, int K,
                                                   uint16_t* __restrict__ Y) {
  const int k = 8 * (blockIdx.x * 256 + threadIdx.x);
  if (k >= K) return;
  const float4 s0 = *reinterpret_cast<const float4*>(s + k);
  const float4 s1 = *reinterpret_cast<const float4*>(s + k + 4);
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float rs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rs[i] = __builtin_amdgcn_rcpf(sv[i]);
  // rows blockIdx.y, + gridDim.y, ...; the next row's load is issued first
  uint4 raw = *reinterpret_cast<const uint4*>(X + (size_t)blockIdx.y * K + k);
  for (int mr = blockIdx.y; mr < M; mr += gridDim.y) {
    const size_t e = (size_t)mr * K + k;
    const int mx = min(mr + (int)gridDim.y, M - 1);
    const uint4 next = *reinterpret_cast<const uint4*>(X + (size_t)mx * K + k);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    raw = next;
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      out[p] = fold_one(h2f((uint16_t)(rw[p] & 0xffffu)), sv[2 * p], rs[2 * p]) |
               (fold_one(h2f((uint16_t)(rw[p] >> 16)), sv[2 * p + 1], rs[2 * p + 1]) << 16);
    *reinterpret_cast<uint4*>(Y + e) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

hipError_t launch_fold(const __half* X, const float* s, int M, int K, __half* Y, hipStream_t st) {
  const int gy = (M + 3) / 4 < 65535 ? (M + 3) / 4 : 65535;  // about 4 rows per thread
  const dim3 grid((unsigned)((K / 8 + 255) / 256), (unsigned)gy);
  hipLaunchKernelGGL(fold_kernel, grid, dim3(256), 0, st, reinterpret_cast<const uint16_t*>(X), s,
                     M, K, reinterpret_cast<uint16_t*>(Y));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// m[k] = sum_t |x[t,k]| / T in float64. The fp16 sum is exact in float64
// for T < 8192, so the split over 16 token slices does not change the result.
// Block = 64 columns x 16 token slices (one wavefront per slice); each
// thread keeps 8 independent loads in flight.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void act_stats_kernel(const uint16_t* __restrict__ X, int T,
                                                         int K, double* __restrict__ m) {
  __shared__ double part[16][64];
  const int c = threadIdx.x & 63;
  const int slice = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + c;
  double acc = 0.0;
  if (k < K) {
    const uint16_t* xc = X + k;
    int t = slice;
    for (; t + 16 * 7 < T; t += 16 * 8) {
      uint16_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = xc[(size_t)(t + 16 * u) * K];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += fabs((double)h2f(v[u]));
    }
    for (; t < T; t += 16) acc += fabs((double)h2f(xc[(size_t)t * K]));
  }
  part[slice][c] = acc;
  __syncthreads();
  if (slice == 0 && k < K) {
    double sum = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += part[i][c];
    m[k] = sum / (double)T;
  }
}

hipError_t launch_act_stats(const __half* X, int T, int K, double* m, hipStream_t st) {
  hipLaunchKernelGGL(act_stats_kernel, dim3((K + 63) / 64), dim3(1024), 0, st,
                     reinterpret_cast<const uint16_t*>(X), T, K, m);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// s[a, k] = float32(pow(m[k], alpha[a])) with pow in float64; 1 where m == 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scale_candidates_kernel(const double* __restrict__ m, int K,
                                                               const float* __restrict__ alpha,
                                                               int n_alpha,
                                                               float* __restrict__ s) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)K * n_alpha) return;
  const int a = (int)(i / K);
  const int k = (int)(i % K);
  const double mk = m[k];
  s[i] = mk > 0.0 ? (float)pow(mk, (double)alpha[a]) : 1.0f;
}

hipError_t launch_scale_candidates(const double* m, int K, const float* alpha, int n_alpha,
                                   float* s, hipStream_t st) {
  const long total = (long)K * n_alpha;
  hipLaunchKernelGGL(scale_candidates_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     st, m, K, alpha, n_alpha, s);
  return hipGetLastError();
}

}  // namespace awq
