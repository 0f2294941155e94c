// Per-layer grid search over alpha for s = mean|x| ** alpha.
//
// The loss of a candidate s is ||Xcal D^T||_F^2 with D = W - Q(W s) / s
// (the fake-quant error of every weight), contracted on the fp16 matrix
// cores (float32 accumulation, float32 tile sums, float64 across tiles).
// Two evaluations, each well inside 1e-4 (relative) of an exact one at its
// sizes:
//  * scaled (T N >= 2^18): per column k, x_k D_nk = (x_k / s_k) *
//    (w_nk s_k - Q(W s)_nk), so the product is evaluated with activations
//    Xs = fp16(Xcal / s) (the fold kernel) and errors E = fp16(2^8 (W s -
//    Q(W s))), both of the same magnitude for every channel (the unscaled D
//    is tiny on channels with large s and loses its precision in fp16). The
//    2^8 keeps E clear of fp16 subnormals; the loss is divided by 2^16. The
//    rounding errors of both operands are random, so their effect on the
//    loss shrinks as 1/sqrt(T N): measured at most 6e-6 at T N = 2^20 on
//    the outlier-heavy layers, so below about 1.2e-5 at 2^18.
//  * hi/lo (small T N): Xcal as given (exact fp16) against D split into an
//    fp16 hi and lo part, contracted as one product over 2K.
// Then best = first index of the minimum loss and s_out = s_best. Layers
// that share one input (and so one s) are searched jointly: their losses are
// added per candidate, in layer order, before the argmin. Everything runs on
// the device; the host only enqueues.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

hipError_t launch_sqnorm_abt(const uint16_t* A, const uint16_t* B, int M, int N, int K, bool hilo,
                             double* partial, hipStream_t st);
unsigned sqnorm_abt_tiles(int M, int N);

namespace {

// Quantized exactly as the pack kernel does (same group grid, same
// rounding), one thread per 8 codes of a group. SCALED: E = fp16(2^8 (W s -
// (q - z) delta)), [N, K]. Otherwise D = W - (q - z) delta / s as hi = fp16(D)
// and lo = fp16(D - hi), [N, 2K]: 128-wide k chunk c -> hi at 256 c, lo at
// 256 c + 128.
template <int BITS, int TPG, bool SCALED, bool SYM>
__global__ __launch_bounds__(256) void fake_quant_error_kernel(const uint16_t* __restrict__ W,
                                                               const float* __restrict__ s, int N,
                                                               int K, uint16_t* __restrict__ E) {
  constexpr int G = TPG * 8;
  constexpr int QMAX = (1 << BITS) - 1;
  // grid: x walks the K/8 threads of a row, y the rows (strided past 65535);
  // threads past the row end work on the last group and store nothing
  const int tr = blockIdx.x * 256 + threadIdx.x;
  const bool active = tr < K / 8;
  const int tt = active ? tr : K / 8 - TPG + (tr % TPG);
  const int k0 = 8 * tt;
  const float4 s0 = *reinterpret_cast<const float4*>(s + k0);
  const float4 s1 = *reinterpret_cast<const float4*>(s + k0 + 4);
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
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
    float mn, mx;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float w = h2f((uint16_t)(i & 1 ? rw[i >> 1] >> 16 : rw[i >> 1] & 0xffffu));
      wp[i] = w * sv[i];
      mn = i == 0 ? wp[i] : fminf(mn, wp[i]);
      mx = i == 0 ? wp[i] : fmaxf(mx, wp[i]);
    }
#pragma unroll
    for (int off = 1; off < TPG; off <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, off, TPG));
      mx = fmaxf(mx, __shfl_xor(mx, off, TPG));
    }
    const GroupGrid gg = grid_of<SYM, BITS>(mn, mx);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t h[2], l[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * p + e;
        const int q = quant_code(wp[i], gg, QMAX);
        const float back = (float)(q - gg.z) * gg.delta;
        if constexpr (SCALED) {
          h[e] = __half_as_ushort(__float2half_rn((wp[i] - back) * 256.0f));
          l[e] = 0u;
        } else {
          // the codes are exact; D only feeds the loss, so the division by s
          // uses the hardware reciprocal (within 1 ulp)
          const float w = h2f((uint16_t)(e ? rw[p] >> 16 : rw[p] & 0xffffu));
          const float dv = w - back * __builtin_amdgcn_rcpf(sv[i]);
          const __half dh = __float2half_rn(dv);
          h[e] = __half_as_ushort(dh);
          l[e] = __half_as_ushort(__float2half_rn(dv - __half2float(dh)));
        }
      }
      hi[p] = h[0] | (h[1] << 16);
      lo[p] = l[0] | (l[1] << 16);
    }
    if (active) {
      if constexpr (SCALED) {
        *reinterpret_cast<uint4*>(E + n * K + k0) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      } else {
        uint16_t* row = E + n * 2 * K + 256 * (k0 >> 7) + (k0 & 127);
        *reinterpret_cast<uint4*>(row) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(row + 128) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
    }
  }
}

// The scaled form for NA candidate scales in one pass over W: E_a =
// fp16(2^8 (W s_a - (q - z) delta)) for s_a = s + a K, written to E + a N K.
// The codes and the bits of E_a are those of fake_quant_error_kernel (same
// group grid, same rounding, same operation order); W is read once for the
// NA candidates instead of once each. The tie test takes the exact division
// when t = wp / delta (approximated) lies within 2^-16 of a half-integer,
// written as |t - rint(t)| > 1/2 - 2^-16.
template <int BITS, int TPG, bool SYM, int NA>
__global__ __launch_bounds__(256) void fake_quant_error_multi_kernel(
    const uint16_t* __restrict__ W, const float* __restrict__ s, int N, int K,
    uint16_t* __restrict__ E) {
  constexpr int QMAX = (1 << BITS) - 1;
  const int tr = blockIdx.x * 256 + threadIdx.x;
  const bool active = tr < K / 8;
  const int tt = active ? tr : K / 8 - TPG + (tr % TPG);
  const int k0 = 8 * tt;
  float sv[NA][8];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const float4 s0 = *reinterpret_cast<const float4*>(s + (size_t)a * K + k0);
    const float4 s1 = *reinterpret_cast<const float4*>(s + (size_t)a * K + k0 + 4);
    sv[a][0] = s0.x; sv[a][1] = s0.y; sv[a][2] = s0.z; sv[a][3] = s0.w;
    sv[a][4] = s1.x; sv[a][5] = s1.y; sv[a][6] = s1.z; sv[a][7] = s1.w;
  }
  const size_t NK = (size_t)N * K;
  uint4 raw = *reinterpret_cast<const uint4*>(W + (size_t)blockIdx.y * K + k0);
  for (int nr = blockIdx.y; nr < N; nr += gridDim.y) {
    const size_t n = (size_t)nr;
    const int nx = min(nr + (int)gridDim.y, N - 1);
    const uint4 next = *reinterpret_cast<const uint4*>(W + (size_t)nx * K + k0);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    raw = next;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = h2f((uint16_t)(i & 1 ? rw[i >> 1] >> 16 : rw[i >> 1] & 0xffffu));
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      float wp[8];
      float mn, mx;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        wp[i] = w[i] * sv[a][i];
        mn = i == 0 ? wp[i] : fminf(mn, wp[i]);
        mx = i == 0 ? wp[i] : fmaxf(mx, wp[i]);
      }
#pragma unroll
      for (int off = 1; off < TPG; off <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, TPG));
        mx = fmaxf(mx, __shfl_xor(mx, off, TPG));
      }
      const GroupGrid gg = grid_of<SYM, BITS>(mn, mx);
      const float zf = (float)gg.z;
      uint32_t hv[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t h[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = 2 * p + e;
          const float t = wp[i] * gg.rdelta;
          float qf = rintf(t);
          if (__builtin_fabsf(t - qf) > 0.5f - 0x1p-16f) qf = rintf(wp[i] / gg.delta);
          // clamp(q, 0, QMAX) - z with q = qf + z
          const float qc = __builtin_amdgcn_fmed3f(qf, -zf, (float)QMAX - zf);
          const float back = qc * gg.delta;
          h[e] = __half_as_ushort(__float2half_rn((wp[i] - back) * 256.0f));
        }
        hv[p] = h[0] | (h[1] << 16);
      }
      if (active)
        // nontemporal: the planes (0.94 GB for a pair on 8192x28672) pass
        // through the caches once (the contraction that reads them then ran
        // 1-2% faster; same bits)
        __builtin_nontemporal_store(u32x4{hv[0], hv[1], hv[2], hv[3]},
                                    reinterpret_cast<u32x4*>(E + (size_t)a * NK + n * K + k0));
    }
  }
}

// The same for per-output-channel groups (the whole row): one workgroup of
// 512 threads per row, the row in registers between the row-wide min / max
// and the error terms (chunk c of thread t: codes 8 (t + 512 c) .. + 7).
template <int BITS, int CH, bool SCALED, bool SYM>
__global__ __launch_bounds__(512) void fake_quant_error_row_kernel(const uint16_t* __restrict__ W,
                                                                   const float* __restrict__ s,
                                                                   int K,
                                                                   uint16_t* __restrict__ E) {
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
        const float wp = h2f((uint16_t)(raw[c][i >> 1] >> (16 * (i & 1)))) * s[k0 + i];
        mn = fminf(mn, wp);
        mx = fmaxf(mx, wp);
      }
    }
  }
  block_minmax<512>(mn, mx, red);
  const GroupGrid gg = grid_of<SYM, BITS>(mn, mx);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k0 = 8 * (t + 512 * c);
    if (k0 >= K) continue;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t h[2], l[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * p + e;
        const float sv = s[k0 + i];
        const float w = h2f((uint16_t)(raw[c][p] >> (16 * e)));
        const float wp = w * sv;
        const int q = quant_code(wp, gg, QMAX);
        const float back = (float)(q - gg.z) * gg.delta;
        if constexpr (SCALED) {
          h[e] = __half_as_ushort(__float2half_rn((wp - back) * 256.0f));
          l[e] = 0u;
        } else {
          const float dv = w - back * __builtin_amdgcn_rcpf(sv);
          const __half dh = __float2half_rn(dv);
          h[e] = __half_as_ushort(dh);
          l[e] = __half_as_ushort(__float2half_rn(dv - __half2float(dh)));
        }
      }
      hi[p] = h[0] | (h[1] << 16);
      lo[p] = l[0] | (l[1] << 16);
    }
    if constexpr (SCALED) {
      *reinterpret_cast<uint4*>(E + n * K + k0) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    } else {
      uint16_t* row = E + n * 2 * K + 256 * (k0 >> 7) + (k0 & 127);
      *reinterpret_cast<uint4*>(row) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(row + 128) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
}

// loss[a] = sum of the tile partials of alpha a, in a fixed order
__global__ void reduce_loss_kernel(const double* __restrict__ partial, int tiles, double scale,
                                   double* __restrict__ loss) {
  __shared__ double buf[256];
  const int a = blockIdx.x;
  double acc = 0.0;
  for (int i = threadIdx.x; i < tiles; i += 256) acc += partial[(size_t)a * tiles + i];
  buf[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) buf[threadIdx.x] += buf[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[a] = buf[0] * scale;
}

// best = first index of the minimum (strict <), s_out = s_all[best]
__global__ void argmin_copy_kernel(const double* __restrict__ loss, int n_alpha,
                                   const float* __restrict__ s_all, int K, int* __restrict__ best,
                                   float* __restrict__ s_out) {
  int b = 0;
  for (int i = 1; i < n_alpha; ++i)
    if (loss[i] < loss[b]) b = i;
  if (blockIdx.x == 0 && threadIdx.x == 0) *best = b;
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < K; k += gridDim.x * blockDim.x)
    s_out[k] = s_all[(size_t)b * K + k];
}

// loss[a] = sum over layers l, in order, of lloss[l][a]
__global__ void sum_layers_kernel(const double* __restrict__ lloss, int n_layers, int n_alpha,
                                  double* __restrict__ loss) {
  const int a = blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= n_alpha) return;
  double v = 0.0;
  for (int l = 0; l < n_layers; ++l) v += lloss[(size_t)l * n_alpha + a];
  loss[a] = v;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// workspace: statistic, candidate scales, Xcal / s, the error term of the
// largest layer, the tile partials of the largest layer, per-layer losses
struct Layout {
  size_t m, s_all, xs, e, partial, lloss, total;
};

Layout layout(int maxN, int K, int T, int n_alpha, unsigned max_tiles, int n_layers) {
  Layout L;
  L.m = 0;
  L.s_all = L.m + align256((size_t)K * 8);
  L.xs = L.s_all + align256((size_t)n_alpha * K * 4);
  L.e = L.xs + align256((size_t)T * K * 2);
  L.partial = L.e + align256((size_t)maxN * K * 4);  // two E planes [2][N, K] or hi/lo D [N, 2K]
  L.lloss = L.partial + align256((size_t)n_alpha * max_tiles * 8);
  L.total = L.lloss + (n_layers > 1 ? align256((size_t)n_layers * n_alpha * 8) : 0);
  return L;
}

// the losses of every candidate scale for one layer W [N, K] -> loss[n_alpha]
hipError_t layer_losses(const __half* W, const __half* Xc, int N, int K, int T,
                        const float* s_all, int n_alpha, int bits, int group, bool zero_point,
                        uint16_t* Xs, uint16_t* E, double* partial, double* loss,
                        hipStream_t st) {
  const unsigned tiles = sqnorm_abt_tiles(T, N);
  const uint16_t* w = reinterpret_cast<const uint16_t*>(W);
  const int gy = (N + 3) / 4 < 65535 ? (N + 3) / 4 : 65535;  // about 4 rows per thread
  const dim3 fgrid((unsigned)((K / 8 + 255) / 256), (unsigned)gy);
  // the scaled single product's rounding effect on the loss shrinks as
  // 1/sqrt(T N); from 2^18 on it stays below about 1.2e-5
  const bool scaled = (long long)T * N >= (1LL << 18);
  hipError_t e;
  if (scaled && !row_group(group)) {
    // candidates in pairs: one pass over W writes both error terms (E holds
    // two [N, K] fp16 planes), then the fold and the contraction of each
    for (int a = 0; a < n_alpha; a += 2) {
      const int na = min(2, n_alpha - a);
      const float* s = s_all + (size_t)a * K;
#define AWQ_FM(B, TP, SY, NA)                                                              \
  hipLaunchKernelGGL((fake_quant_error_multi_kernel<B, TP, SY, NA>), fgrid, dim3(256), 0, st, \
                     w, s, N, K, E)
#define AWQ_FM2(B, TP)                         \
  do {                                         \
    if (na == 2 && zero_point)                 \
      AWQ_FM(B, TP, false, 2);                 \
    else if (na == 2)                          \
      AWQ_FM(B, TP, true, 2);                  \
    else if (zero_point)                       \
      AWQ_FM(B, TP, false, 1);                 \
    else                                       \
      AWQ_FM(B, TP, true, 1);                  \
  } while (0)
      if (bits == 4) {
        if (group == 128) AWQ_FM2(4, 16);
        else if (group == 256) AWQ_FM2(4, 32);
        else AWQ_FM2(4, 64);
      } else {
        if (group == 128) AWQ_FM2(3, 16);
        else if (group == 256) AWQ_FM2(3, 32);
        else AWQ_FM2(3, 64);
      }
#undef AWQ_FM2
#undef AWQ_FM
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      for (int b = 0; b < na; ++b) {
        e = launch_fold(Xc, s_all + (size_t)(a + b) * K, T, K, reinterpret_cast<__half*>(Xs), st);
        if (e != hipSuccess) return e;
        e = launch_sqnorm_abt(Xs, E + (size_t)b * N * K, T, N, K, false,
                              partial + (size_t)(a + b) * tiles, st);
        if (e != hipSuccess) return e;
      }
    }
    hipLaunchKernelGGL(reduce_loss_kernel, dim3(n_alpha), dim3(256), 0, st, partial, (int)tiles,
                       1.0 / 65536.0, loss);
    return hipGetLastError();
  }
  for (int a = 0; a < n_alpha; ++a) {
    const float* s = s_all + (size_t)a * K;
#define AWQ_FQ(B, TP, SC, SY)                                                                  \
  hipLaunchKernelGGL((fake_quant_error_kernel<B, TP, SC, SY>), fgrid, dim3(256), 0, st, w, s, N, \
                     K, E)
#define AWQ_FQ2(B, TP)                          \
  do {                                          \
    if (scaled && zero_point)                   \
      AWQ_FQ(B, TP, true, false);               \
    else if (scaled)                            \
      AWQ_FQ(B, TP, true, true);                \
    else if (zero_point)                        \
      AWQ_FQ(B, TP, false, false);              \
    else                                        \
      AWQ_FQ(B, TP, false, true);               \
  } while (0)
#define AWQ_FR(B, C, SC, SY)                                                                \
  hipLaunchKernelGGL((fake_quant_error_row_kernel<B, C, SC, SY>), dim3((unsigned)N), dim3(512), 0, \
                     st, w, s, K, E)
#define AWQ_FR2(B, C)                           \
  do {                                          \
    if (scaled && zero_point)                   \
      AWQ_FR(B, C, true, false);                \
    else if (scaled)                            \
      AWQ_FR(B, C, true, true);                 \
    else if (zero_point)                        \
      AWQ_FR(B, C, false, false);               \
    else                                        \
      AWQ_FR(B, C, false, true);                \
  } while (0)
#define AWQ_FR3(B)                              \
  do {                                          \
    switch ((K + 4095) / 4096) {                \
      case 1: AWQ_FR2(B, 1); break;             \
      case 2: AWQ_FR2(B, 2); break;             \
      case 3: AWQ_FR2(B, 3); break;             \
      case 4: AWQ_FR2(B, 4); break;             \
      case 5: AWQ_FR2(B, 5); break;             \
      case 6: AWQ_FR2(B, 6); break;             \
      case 7: AWQ_FR2(B, 7); break;             \
      default: AWQ_FR2(B, 8); break;            \
    }                                           \
  } while (0)
    if (row_group(group)) {  // per output channel
      if (bits == 4) AWQ_FR3(4);
      else AWQ_FR3(3);
    } else if (bits == 4) {
      if (group == 128) AWQ_FQ2(4, 16);
      else if (group == 256) AWQ_FQ2(4, 32);
      else AWQ_FQ2(4, 64);
    } else {
      if (group == 128) AWQ_FQ2(3, 16);
      else if (group == 256) AWQ_FQ2(3, 32);
      else AWQ_FQ2(3, 64);
    }
#undef AWQ_FR3
#undef AWQ_FR2
#undef AWQ_FR
#undef AWQ_FQ2
#undef AWQ_FQ
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (scaled) {
      e = launch_fold(Xc, s, T, K, reinterpret_cast<__half*>(Xs), st);
      if (e != hipSuccess) return e;
      e = launch_sqnorm_abt(Xs, E, T, N, K, false, partial + (size_t)a * tiles, st);
    } else {
      e = launch_sqnorm_abt(reinterpret_cast<const uint16_t*>(Xc), E, T, N, K, true,
                            partial + (size_t)a * tiles, st);
    }
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(reduce_loss_kernel, dim3(n_alpha), dim3(256), 0, st, partial, (int)tiles,
                     scaled ? 1.0 / 65536.0 : 1.0, loss);
  return hipGetLastError();
}

unsigned max_tiles_of(const int* N, int n_layers, int T) {
  unsigned t = 0;
  for (int l = 0; l < n_layers; ++l) t = t > sqnorm_abt_tiles(T, N[l]) ? t : sqnorm_abt_tiles(T, N[l]);
  return t;
}

int max_of(const int* N, int n_layers) {
  int v = 0;
  for (int l = 0; l < n_layers; ++l) v = v > N[l] ? v : N[l];
  return v;
}

}  // namespace

size_t search_workspace_bytes_joint(const int* N, int n_layers, int K, int T, int n_alpha) {
  const Layout L =
      layout(max_of(N, n_layers), K, T, n_alpha, max_tiles_of(N, n_layers, T), n_layers);
  // + the head the API layer keeps for the grid, the losses and the index
  return L.total + align256((size_t)n_alpha * 4) + align256((size_t)n_alpha * 8) + 256;
}

size_t search_workspace_bytes(int N, int K, int T, int n_alpha, int bits, int group) {
  (void)bits;
  (void)group;
  return search_workspace_bytes_joint(&N, 1, K, T, n_alpha);
}

hipError_t launch_search_joint(const __half* const* W, const int* N, int n_layers, const __half* Xc,
                               int K, int T, const float* alpha_dev, int n_alpha, int bits,
                               int group, bool zero_point, void* ws, double* loss_dev,
                               int* best_dev, float* s_out, hipStream_t st) {
  const Layout L =
      layout(max_of(N, n_layers), K, T, n_alpha, max_tiles_of(N, n_layers, T), n_layers);
  uint8_t* base = static_cast<uint8_t*>(ws);
  double* m = reinterpret_cast<double*>(base + L.m);
  float* s_all = reinterpret_cast<float*>(base + L.s_all);
  uint16_t* Xs = reinterpret_cast<uint16_t*>(base + L.xs);
  uint16_t* E = reinterpret_cast<uint16_t*>(base + L.e);
  double* partial = reinterpret_cast<double*>(base + L.partial);
  double* lloss = n_layers > 1 ? reinterpret_cast<double*>(base + L.lloss) : loss_dev;

  hipError_t e = launch_act_stats(Xc, T, K, m, st);
  if (e != hipSuccess) return e;
  e = launch_scale_candidates(m, K, alpha_dev, n_alpha, s_all, st);
  if (e != hipSuccess) return e;
  for (int l = 0; l < n_layers; ++l) {
    e = layer_losses(W[l], Xc, N[l], K, T, s_all, n_alpha, bits, group, zero_point, Xs, E, partial,
                     lloss + (size_t)l * n_alpha, st);
    if (e != hipSuccess) return e;
  }
  if (n_layers > 1) {
    hipLaunchKernelGGL(sum_layers_kernel, dim3((n_alpha + 63) / 64), dim3(64), 0, st, lloss,
                       n_layers, n_alpha, loss_dev);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(argmin_copy_kernel, dim3((K + 255) / 256), dim3(256), 0, st, loss_dev,
                     n_alpha, s_all, K, best_dev, s_out);
  return hipGetLastError();
}

hipError_t launch_search(const __half* W, const __half* Xc, int N, int K, int T,
                         const float* alpha_dev, int n_alpha, int bits, int group,
                         bool zero_point, void* ws, double* loss_dev, int* best_dev, float* s_out,
                         hipStream_t st) {
  return launch_search_joint(&W, &N, 1, Xc, K, T, alpha_dev, n_alpha, bits, group, zero_point, ws,
                             loss_dev, best_dev, s_out, st);
}

}  // namespace awq
