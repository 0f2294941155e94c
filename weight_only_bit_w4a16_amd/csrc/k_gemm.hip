// Prefill / batched W4A16 (and W3A16) product on the fp16 matrix cores, and
// the fp16 "A * B^T" contraction the scale search uses.
//
// One workgroup (4 wavefronts, 2 x 2) computes a 128 x 128 tile of
// Y = A B^T, A = X' [M, K] fp16 and B = dequant(Q) [N, K]. The K loop runs
// one 128-code group per step: the packed words, group steps and zero points
// of the next step are loaded into registers while the matrix cores work on
// the current step; then the tile is dequantized to fp16 (q - z) * delta in
// LDS and the activation tile is copied next to it. Each wavefront computes
// 64 x 64 with v_mfma_f32_32x32x16_f16.
//
// Code order in LDS. The packed words are unpacked with the fp16 magic-number
// trick, which yields codes in pairs that are not adjacent in k; the
// activation tile is stored with the same permutation of k, so the
// contraction (a sum over k) is unchanged:
//   int4, per 8-code word:  c0 c4 c2 c6 c1 c5 c3 c7
//   int3, per 10-code word: c0 c6 c1 c7 c3 c8 c4 c9 c2 c5
// (an int3 group is 13 words = 130 slots, of which the last 2 hold no code;
// their activation slots are zero). fp16 B tiles (the search) keep natural
// order.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128;
constexpr int NT = 256;

template <int BMODE>
struct Cfg;
template <>
struct Cfg<0> {  // fp16 B, natural order
  static constexpr int SLOTS = 128, STRIDE = 136;
};
template <>
struct Cfg<4> {
  static constexpr int SLOTS = 128, STRIDE = 136;
};
template <>
struct Cfg<3> {
  static constexpr int SLOTS = 144, STRIDE = 152;  // 130 used + zero pad to 9 x 16
};

__device__ __forceinline__ floatx16 mfma32(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t plo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t phi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}
__device__ __forceinline__ uint32_t hbits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 hv(uint32_t v) { return __builtin_bit_cast(h2, v); }

// ---- per-step register staging -------------------------------------------

template <int BMODE>
struct Stage;

// fp16 A and B, natural order: 8 x 16 B per thread for each operand
template <>
struct Stage<0> {
  u32x4 a[8], b[8];
};
// int4: A 8 x 16 B, B 2 x 16 B (8 words of one row) + delta + z
template <>
struct Stage<4> {
  u32x4 a[8];
  u32x4 b[2];
  float d;
  uint32_t z;
};
// int3: A 7 items x 5 dwords, B 7 words + delta/z per item
template <>
struct Stage<3> {
  uint32_t a[7][5];
  uint32_t b[7];
  float d[7];
  uint32_t z[7];
};

}  // namespace

template <int BMODE, int EPI>
__global__ __launch_bounds__(NT, 2) void gemm_kernel(const uint16_t* __restrict__ A,
                                                     const void* __restrict__ Bsrc,
                                                     const float* __restrict__ S,
                                                     const uint8_t* __restrict__ Z, int M, int N,
                                                     int K, int wpr, int gshift,
                                                     uint16_t* __restrict__ Y,
                                                     double* __restrict__ partial) {
  using C = Cfg<BMODE>;
  constexpr int STR = C::STRIDE;
  __shared__ __align__(16) uint16_t lds_a[BM * STR];
  __shared__ __align__(16) uint16_t lds_b[BN * STR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // tile order: when the tile count splits evenly over the 8 XCDs, give each
  // XCD a contiguous run of tiles that walk M for a fixed N tile, so the
  // weight tile is reused from that XCD's L2
  const int mt = (M + BM - 1) / BM;
  const int ntl = (N + BN - 1) / BN;
  const int total = mt * ntl;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int m0 = (t % mt) * BM;
  const int n0 = (t / mt) * BN;
  // fp16 B (the search) holds each error term as a hi and a lo fp16 part,
  // [N][2K] with chunk c = (hi of k-chunk c/2 | lo of k-chunk c/2): 2 steps
  // per 128-wide k-chunk, both against the same activation chunk
  const int nsteps = BMODE == 0 ? 2 * (K >> 7) : K >> 7;

  if (BMODE == 3) {
    // zero the slots 130..143 of every row once; they are never written again
    for (int i = tid; i < BM * 14; i += NT) {
      lds_a[(i / 14) * STR + 130 + i % 14] = 0;
      lds_b[(i / 14) * STR + 130 + i % 14] = 0;
    }
  }

  Stage<BMODE> st;
  auto load_step = [&](int ks) {
    const int k0 = BMODE == 0 ? (ks >> 1) << 7 : ks << 7;
    if constexpr (BMODE == 0 || BMODE == 4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = tid + NT * i;
        const int r = id >> 4, c8 = id & 15;
        const int m = m0 + r;
        if (m < M)
          st.a[i] = *reinterpret_cast<const u32x4*>(A + (size_t)m * K + k0 + 8 * c8);
        else
          st.a[i] = u32x4{0, 0, 0, 0};
      }
    }
    if constexpr (BMODE == 0) {
      const uint16_t* B = static_cast<const uint16_t*>(Bsrc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = tid + NT * i;
        const int r = id >> 4, c8 = id & 15;
        const int n = min(n0 + r, N - 1);
        st.b[i] = *reinterpret_cast<const u32x4*>(B + (size_t)n * 2 * K + (ks << 7) + 8 * c8);
      }
    } else if constexpr (BMODE == 4) {
      const uint32_t* Q = static_cast<const uint32_t*>(Bsrc);
      const int r = tid >> 1, h = tid & 1;
      const int n = min(n0 + r, N - 1);
      const uint32_t* p = Q + (size_t)n * wpr + ks * 16 + 8 * h;
      st.b[0] = ld_nt(reinterpret_cast<const u32x4*>(p));
      st.b[1] = ld_nt(reinterpret_cast<const u32x4*>(p + 4));
      const int ng = nsteps >> gshift;
      st.d = S[(size_t)n * ng + (ks >> gshift)];
      st.z = Z[(size_t)n * ng + (ks >> gshift)];
    } else {  // int3: items (row, word) over 128 rows x 13 words
      const uint32_t* Q = static_cast<const uint32_t*>(Bsrc);
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        const int id = tid + NT * i;
        if (id < BM * 13) {
          const int r = id / 13, j = id % 13;
          const int m = m0 + r;
          const int kx = k0 + 10 * j;
          if (m < M) {
            const uint32_t* px = reinterpret_cast<const uint32_t*>(A + (size_t)m * K + kx);
#pragma unroll
            for (int q = 0; q < 4; ++q) st.a[i][q] = px[q];
            st.a[i][4] = j < 12 ? px[4] : 0u;  // codes 128, 129 do not exist
          } else {
#pragma unroll
            for (int q = 0; q < 5; ++q) st.a[i][q] = 0u;
          }
          const int n = min(n0 + r, N - 1);
          st.b[i] = ld_nt(Q + (size_t)n * wpr + ks * 13 + j);
          st.d[i] = S[(size_t)n * nsteps + ks];
          st.z[i] = Z[(size_t)n * nsteps + ks];
        }
      }
    }
  };

  auto store_step = [&]() {
    if constexpr (BMODE == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = tid + NT * i;
        const int r = id >> 4, c8 = id & 15;
        *reinterpret_cast<u32x4*>(&lds_a[r * STR + 8 * c8]) = st.a[i];
        *reinterpret_cast<u32x4*>(&lds_b[r * STR + 8 * c8]) = st.b[i];
      }
    } else if constexpr (BMODE == 4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = tid + NT * i;
        const int r = id >> 4, c8 = id & 15;
        const u32x4 d = st.a[i];
        const u32x4 p = {plo(d[0], d[2]), plo(d[1], d[3]), phi(d[0], d[2]), phi(d[1], d[3])};
        *reinterpret_cast<u32x4*>(&lds_a[r * STR + 8 * c8]) = p;
      }
      const int r = tid >> 1, h = tid & 1;
      const h2 dh = {(_Float16)st.d, (_Float16)st.d};
      const h2 ze = hv((0xE400u + st.z) * 0x00010001u);       // -(1024 + z)
      const h2 zo = hv((0xD400u + 16u * st.z) * 0x00010001u);  // -(64 + z)
      const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
#pragma unroll
      for (int v = 0; v < 2; ++v) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w = st.b[v][q];
          const uint32_t w8 = w >> 8;
          const h2 e0 = (hv((w & 0x000F000Fu) | kMagic2) + ze) * dh;
          const h2 e1 = (hv((w8 & 0x000F000Fu) | kMagic2) + ze) * dh;
          const h2 o0 = __builtin_elementwise_fma(hv((w & 0x00F000F0u) | kMagic2), sixteenth, zo) * dh;
          const h2 o1 = __builtin_elementwise_fma(hv((w8 & 0x00F000F0u) | kMagic2), sixteenth, zo) * dh;
          const int word = 8 * h + 4 * v + q;
          *reinterpret_cast<u32x4*>(&lds_b[r * STR + 8 * word]) =
              u32x4{hbits(e0), hbits(e1), hbits(o0), hbits(o1)};
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        const int id = tid + NT * i;
        if (id < BM * 13) {
          const int r = id / 13, j = id % 13;
          const uint32_t* d = st.a[i];
          // (x0,x6) (x1,x7) (x3,x8) (x4,x9) (x2,x5) from d_i = (x[2i], x[2i+1])
          uint32_t* pa = reinterpret_cast<uint32_t*>(&lds_a[r * STR + 10 * j]);
          pa[0] = plo(d[0], d[3]);
          pa[1] = phi(d[0], d[3]);
          pa[2] = (d[1] >> 16) | (d[4] << 16);
          pa[3] = (d[2] & 0xffffu) | (d[4] & 0xffff0000u);
          pa[4] = (d[1] & 0xffffu) | (d[2] & 0xffff0000u);
          // codes: magic pairs with per-half power-of-two weights, made exact
          // integers c - z by one packed fma each, then scaled by delta
          const uint32_t w = st.b[i];
          const uint32_t t8 = w >> 8, u1 = w << 1;
          const uint32_t z = st.z[i];
          const h2 dh = {(_Float16)st.d[i], (_Float16)st.d[i]};
          const uint32_t raw[5] = {(w & 0x001C0007u) | kMagic2, (w & 0x00E00038u) | kMagic2,
                                   (t8 & 0x0007000Eu) | kMagic2, (t8 & 0x00380070u) | kMagic2,
                                   (u1 & 0x00070380u) | kMagic2};
          // per pair: (lo weight, hi weight) = (1,4) (8,32) (2,1) (16,8) (128,1)
          const h2 mul[5] = {{(_Float16)1.f, (_Float16)0.25f},
                             {(_Float16)0.125f, (_Float16)0.03125f},
                             {(_Float16)0.5f, (_Float16)1.f},
                             {(_Float16)0.0625f, (_Float16)0.125f},
                             {(_Float16)0.0078125f, (_Float16)1.f}};
          const float offl[5] = {1024.f, 128.f, 512.f, 64.f, 8.f};
          const float offh[5] = {256.f, 32.f, 1024.f, 128.f, 1024.f};
          uint32_t* pb = reinterpret_cast<uint32_t*>(&lds_b[r * STR + 10 * j]);
          const float zf = (float)z;
#pragma unroll
          for (int p = 0; p < 5; ++p) {
            const h2 add = {(_Float16)(-(offl[p] + zf)), (_Float16)(-(offh[p] + zf))};
            pb[p] = hbits(__builtin_elementwise_fma(hv(raw[p]), mul[p], add) * dh);
          }
        }
      }
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int lr = lane & 31;
  const int lk = (lane >> 5) * 8;
  load_step(0);
  for (int ks = 0; ks < nsteps; ++ks) {
    __syncthreads();  // previous step's MFMA reads are done
    store_step();
    __syncthreads();
    if (ks + 1 < nsteps) load_step(ks + 1);
    constexpr int NKS = C::SLOTS / 16;
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      const int ko = kk * 16 + lk;
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(&lds_a[(64 * wm + 32 * i + lr) * STR + ko]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(&lds_b[(64 * wn + 32 * j + lr) * STR + ko]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
    }
  }

  // D layout of the 32x32 MFMA: lane l holds column l % 32, rows
  // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15
  if constexpr (EPI == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + 64 * wn + 32 * j + lr;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(acc[i][j][v]));
        }
      }
  } else {
    __shared__ double wsum[4];
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + 64 * wn + 32 * j + lr;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const float e = acc[i][j][v];
          if (m < M && n < N) sq = __builtin_fmaf(e, e, sq);
        }
      }
    double ds = (double)sq;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ds += __shfl_xor(ds, off);
    if (lane == 0) wsum[wave] = ds;
    __syncthreads();
    if (tid == 0) partial[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

hipError_t launch_gemm(const __half* X, const uint32_t* q, const float* scales,
                       const uint8_t* zeros, int M, int N, int K, int bits, int group, __half* Y,
                       hipStream_t st) {
  if (bits == 3 && group != 128) return hipErrorNotSupported;
  int gshift = 0;
  while ((128 << gshift) < group) ++gshift;
  const int wpr = words_per_row(K, bits, group);
  const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  if (bits == 4)
    hipLaunchKernelGGL((gemm_kernel<4, 0>), dim3(tiles), dim3(NT), 0, st, x, q, scales, zeros, M,
                       N, K, wpr, gshift, y, nullptr);
  else
    hipLaunchKernelGGL((gemm_kernel<3, 0>), dim3(tiles), dim3(NT), 0, st, x, q, scales, zeros, M,
                       N, K, wpr, gshift, y, nullptr);
  return hipGetLastError();
}

// ||A (Bhi + Blo)^T||^2 as one float64 partial per workgroup tile; A is
// [M, K] fp16, B is [N, 2K] fp16 holding hi/lo parts per 128-wide k chunk
hipError_t launch_sqnorm_abt(const uint16_t* A, const uint16_t* B, int M, int N, int K,
                             double* partial, hipStream_t st) {
  const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  hipLaunchKernelGGL((gemm_kernel<0, 1>), dim3(tiles), dim3(NT), 0, st, A, B, nullptr, nullptr, M,
                     N, K, 0, 0, nullptr, partial);
  return hipGetLastError();
}

unsigned sqnorm_abt_tiles(int M, int N) {
  return (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

}  // namespace awq
