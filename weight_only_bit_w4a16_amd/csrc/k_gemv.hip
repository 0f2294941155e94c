// Decode kernels (M <= 16 activation rows): stream the packed weights once
// from HBM with 128-bit nontemporal loads, dequantize in registers and
// contract on the fp16 matrix cores (v_mfma_f32_16x16x32_f16).
//
// Work split. A workgroup (4 wavefronts) owns 16 output rows n; its 4
// wavefronts split K into 4 contiguous ranges of 128-code chunks and their
// partial sums are added in LDS in a fixed order (no atomics: the result is
// bitwise reproducible). Inside a wavefront, lane l = nl + 16*jj owns row
// n0 + nl and, for every chunk, the 32 consecutive codes 32*jj .. 32*jj+31
// (one 16-byte load). The four 16x16x32 MFMAs of a chunk therefore cover
// exactly one 128-code chunk of 16 rows, which never straddles a
// quantization group (group is a multiple of 128), so the group step is
// applied once per chunk to the fp32 MFMA result.
//
// Unpacking. For a packed word w with codes c0..c7 (c_i at bits 4i):
//   (w & 0x000F000F) | 0x64006400 = fp16 pair (1024 + c0, 1024 + c4)
//   (w & 0x00F000F0) | 0x64006400 = fp16 pair (1024 + 16 c1, 1024 + 16 c5)
// and the same on w >> 8 for (c2, c6), (c3, c7): 5 integer ops per 8 codes.
// The activation operand is permuted once per call to the same code order
// (the contraction is a sum, so any common permutation of k is exact).
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

__device__ __forceinline__ half8 as_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }

__device__ __forceinline__ floatx4 mfma16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(a), as_h8(b), c, 0, 0, 0);
}

// A operands in the code order of the unpacked weights, from the 32 fp16 activations
// x[0..31] of one lane's span held as 16 dwords d[i] = (x[2i], x[2i+1]).
// Operand (h, blk) dword p pairs x[8t + 2*sub + h] with x[8t + 2*sub + 4 + h],
// t = 2*blk + p/2, sub = p%2; h = 0 even slots, h = 1 odd slots.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

__device__ __forceinline__ void permute_x32(const uint32_t* d, u32x4& e1, u32x4& e2, u32x4& o1,
                                            u32x4& o2) {
  e1 = u32x4{pair_lo(d[0], d[2]), pair_lo(d[1], d[3]), pair_lo(d[4], d[6]), pair_lo(d[5], d[7])};
  e2 = u32x4{pair_lo(d[8], d[10]), pair_lo(d[9], d[11]), pair_lo(d[12], d[14]),
             pair_lo(d[13], d[15])};
  o1 = u32x4{pair_hi(d[0], d[2]), pair_hi(d[1], d[3]), pair_hi(d[4], d[6]), pair_hi(d[5], d[7])};
  o2 = u32x4{pair_hi(d[8], d[10]), pair_hi(d[9], d[11]), pair_hi(d[12], d[14]),
             pair_hi(d[13], d[15])};
}

__device__ __forceinline__ void load_x32(const uint16_t* p, uint32_t* d) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = q[i];
    d[4 * i] = v[0];
    d[4 * i + 1] = v[1];
    d[4 * i + 2] = v[2];
    d[4 * i + 3] = v[3];
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// The decode kernel. Two forms of the per-chunk arithmetic:
//
// OFFSET (M <= 4): the MFMAs multiply the raw fp16 values 1024 + c (even
// slots) and 1024 + 16 c (odd slots) with the activations; per chunk
//   sum_k x_k (c_k - z) = D_E + D_O / 16 - C - z * S,
//   C = 1024 * sum_even x + 64 * sum_odd x,  S = sum x,
// with C and S computed once per call, so no per-code zero-point
// subtraction is needed. The permuted activations, C and S live in LDS.
//
// EXACT (any M <= 16): every code becomes the exact fp16 integer c - z
// before the MFMA (one packed add or fma per 2 codes); the activation
// operands are read from global memory (L2-resident) and permuted in
// registers.
//
// Schedule. The grid is sized so that every workgroup is resident at once;
// workgroup b owns row blocks [b*rbw, b*rbw + rbw). Each wavefront walks its
// K range for each of those row blocks as one flat sequence of chunks, with
// a ring of PF 16-byte weight loads in flight that runs across row-block
// boundaries. The loop body has no divergent control flow, so the compiler
// can count outstanding loads exactly instead of draining them. A row block's
// partial sums go to LDS; after one barrier the 4 wavefront partials are
// added in a fixed order and stored.
// ---------------------------------------------------------------------------
enum { kOffset = 0, kExact = 1 };

// (a & m) | o as one v_and_or_b32: m in an SGPR and o in a VGPR (from
// unpack_regs), since a VOP3 instruction takes no literal on gfx950 and with
// both constants visible the compiler would emit an AND and an OR. The
// instruction is the compiler's own, not inline asm: only then does it keep
// the wait states gfx950 requires between a VALU write and an MFMA reading
// the result (it does not track writes made by inline asm, and an MFMA
// issued right after such a write can read the register's old value).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  return (a & m) | o;
}

template <int MODE, int MP, int PF, bool CS>
__global__ __launch_bounds__(256) void gemv_w4_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Q, const void* __restrict__ S,
    const void* __restrict__ Z, uint16_t* __restrict__ Y, int M, int N, int K, int gshift,
    int rbw) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int R = MODE == kOffset ? (MP < 4 ? MP : 4) : 4;
  const int nch = K >> 7;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wavefront
  const int c0 = (wave * nch) >> 2;
  const int c1 = ((wave + 1) * nch) >> 2;
  const int nc = c1 - c0;
  const int nl = lane & 15;
  const int jj = lane >> 4;
  const int nrb = (N + 15) >> 4;
  const int rb0 = blockIdx.x * rbw;
  const int nj = min(rbw, nrb - rb0);
  const int ngr = max(1, nch >> gshift);
  const int wpr = K >> 3;
  const int xr = min(nl, (MODE == kOffset ? MP : M) - 1);  // A-operand row of this lane

  const size_t xp_bytes = MODE == kOffset ? (size_t)nch * 256 * MP : 0;
  const size_t cs_bytes = MODE == kOffset ? (size_t)nch * MP * 8 : 0;
  const size_t part_bytes = (size_t)rbw * 4 * 64 * R * 4;
  u32x4* xp = reinterpret_cast<u32x4*>(smem);
  float2* cs = reinterpret_cast<float2*>(smem + xp_bytes);
  float* part = reinterpret_cast<float*>(smem + xp_bytes + cs_bytes);  // [rbw][4][64][R]
  // scales and zero points of the workgroup's rows, staged once: [rbw*16][ngr]
  float* sc = reinterpret_cast<float*>(smem + xp_bytes + cs_bytes + part_bytes);
  uint8_t* zz = reinterpret_cast<uint8_t*>(sc + (size_t)rbw * 16 * ngr);

  const uint32_t* qlane = Q + 4 * jj;
  const int F = nj * nc;

  // ---- weight prefetch ring -------------------------------------------------
  u32x4 wb[PF];
  int pj = 0, pc = c0;  // position of the next prefetch
  auto issue = [&](int slot) {
    const int j = min(pj, nj - 1);
    const int c = pj < nj ? pc : c1 - 1;
    const int n = min((rb0 + j) * 16 + nl, N - 1);
    wb[slot] = ld_nt(reinterpret_cast<const u32x4*>(qlane + (size_t)n * wpr + c * 16));
    if (++pc == c1) {
      pc = c0;
      ++pj;
    }
  };
  if (F > 0) {
#pragma unroll
    for (int i = 0; i < PF; ++i) issue(i);
  }

  // scales and zero points: whole rows, coalesced (a per-chunk load of 16
  // rows' values would touch 16 cache lines per instruction)
  // rows, 8 values per thread in flight at a time
  const int nsz = nj * 16 * ngr;
  for (int base = 0; base < nsz; base += 256 * 8) {
    float sv[8];
    uint8_t zv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = min(base + (int)threadIdx.x + 256 * u, nsz - 1);
      const int r = idx / ngr, g = idx - r * ngr;
      const size_t n = (size_t)min((rb0 + (r >> 4)) * 16 + (r & 15), N - 1);
      sv[u] = group_scale<CS>(S, n, ngr, g);
      zv[u] = (uint8_t)group_zero<CS>(Z, n, ngr, g);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + (int)threadIdx.x + 256 * u;
      if (idx < nsz) {
        sc[idx] = sv[u];
        zz[idx] = zv[u];
      }
    }
  }

  if constexpr (MODE == kOffset) {
    // permuted activations, C and S of this wavefront's chunks: one lane per
    // (chunk, row, jj); the 4 jj lanes of a (chunk, row) form a quad
    const int items = nc * M * 4;
    for (int t = lane; t < items; t += 64) {
      const int tj = t & 3;
      const int rest = t >> 2;
      const int tm = rest % M;
      const int tc = c0 + rest / M;
      uint32_t d[16];
      load_x32(X + (size_t)tm * K + tc * 128 + 32 * tj, d);
      u32x4 e1, e2, o1, o2;
      permute_x32(d, e1, e2, o1, o2);
      u32x4* dst = xp + ((size_t)(tc * 4 + tj) * 4) * MP + tm;
      dst[0] = e1;
      dst[MP] = e2;
      dst[2 * MP] = o1;
      dst[3 * MP] = o2;
      float se = 0.f, so = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        se += h2f((uint16_t)(d[i] & 0xffffu));
        so += h2f((uint16_t)(d[i] >> 16));
      }
      se += __shfl_xor(se, 1);
      so += __shfl_xor(so, 1);
      se += __shfl_xor(se, 2);
      so += __shfl_xor(so, 2);
      if (tj == 0) cs[tc * MP + tm] = make_float2(1024.f * se + 64.f * so, se + so);
    }
  }
  __syncthreads();

  const UnpackRegs ur = unpack_regs();
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint16_t* xlane = X + (size_t)xr * K + 32 * jj;
  floatx4 y = zero4;
  int cj = 0, cc = c0;  // position of the chunk being consumed
  for (int f0 = 0; f0 < F; f0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const bool valid = f0 + i < F;
      const u32x4 w = wb[i];
      issue(i);
      const int c = valid ? cc : c1 - 1;
      const int sidx = (min(cj, nj - 1) * 16 + nl) * ngr + (c >> gshift);
      const float d = valid ? sc[sidx] : 0.f;
      const uint32_t z = zz[sidx];
      u32x4 a0, a1, a2, a3;
      if constexpr (MODE == kOffset) {
        const u32x4* p = xp + ((size_t)(c * 4 + jj) * 4) * MP + xr;
        a0 = p[0];
        a1 = p[MP];
        a2 = p[2 * MP];
        a3 = p[3 * MP];
      } else {
        uint32_t dx[16];
        load_x32(xlane + c * 128, dx);
        permute_x32(dx, a0, a1, a2, a3);
      }
      uint32_t e[8], o[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t x = w[t];
        const uint32_t x8 = x >> 8;
        e[2 * t] = and_or(x, ur.lo4, ur.magic);      // (c0, c4)
        o[2 * t] = and_or(x, ur.hi4, ur.magic);      // (16 c1, 16 c5)
        e[2 * t + 1] = and_or(x8, ur.lo4, ur.magic);  // (c2, c6)
        o[2 * t + 1] = and_or(x8, ur.hi4, ur.magic);  // (16 c3, 16 c7)
      }
      if constexpr (MODE == kOffset) {
        const floatx4 de = mfma16(a1, u32x4{e[4], e[5], e[6], e[7]},
                                  mfma16(a0, u32x4{e[0], e[1], e[2], e[3]}, zero4));
        const floatx4 dd = mfma16(a3, u32x4{o[4], o[5], o[6], o[7]},
                                  mfma16(a2, u32x4{o[0], o[1], o[2], o[3]}, zero4));
        const float zf = (float)z;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float2 cv = cs[c * MP + min(4 * jj + r, MP - 1)];
          float t = __builtin_fmaf(dd[r], 0.0625f, de[r]) - cv.x;
          t = __builtin_fmaf(-zf, cv.y, t);
          y[r] = __builtin_fmaf(d, t, y[r]);
        }
      } else {
        // exact c - z: even slots (1024 + c) - (1024 + z), odd slots
        // (1024 + 16 c) / 16 - (64 + z)
        const h2 ze = __builtin_bit_cast(h2, (0xE400u + z) * 0x00010001u);
        const h2 zo = __builtin_bit_cast(h2, (0xD400u + 16u * z) * 0x00010001u);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          e[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, e[q]) + ze);
          o[q] = __builtin_bit_cast(
              uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, o[q]), sixteenth, zo));
        }
        floatx4 acc = mfma16(a0, u32x4{e[0], e[1], e[2], e[3]}, zero4);
        acc = mfma16(a1, u32x4{e[4], e[5], e[6], e[7]}, acc);
        acc = mfma16(a2, u32x4{o[0], o[1], o[2], o[3]}, acc);
        acc = mfma16(a3, u32x4{o[4], o[5], o[6], o[7]}, acc);
#pragma unroll
        for (int r = 0; r < R; ++r) y[r] = __builtin_fmaf(d, acc[r], y[r]);
      }
      if (valid && cc == c1 - 1) {  // row block done: park the partial in LDS
#pragma unroll
        for (int r = 0; r < R; ++r) part[((cj * 4 + wave) * 64 + lane) * R + r] = y[r];
        y = zero4;
      }
      if (++cc == c1) {
        cc = c0;
        ++cj;
      }
    }
  }
  if (nc == 0) {
    for (int j = 0; j < nj; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) part[((j * 4 + wave) * 64 + lane) * R + r] = 0.f;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nj * 64 * R; idx += 256) {
    const int j = idx / (64 * R);
    const int l = (idx / R) & 63;
    const int r = idx % R;
    const float* pp = part + (size_t)j * 4 * 64 * R + l * R + r;
    const float v = ((pp[0] + pp[64 * R]) + pp[2 * 64 * R]) + pp[3 * 64 * R];
    const int m = 4 * (l >> 4) + r;
    const int n = (rb0 + j) * 16 + (l & 15);
    if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(v));
  }
}

namespace {
int log2i(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

int cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}
}  // namespace


// Rows of the streaming decode kernels (one row per wavefront at a time).
// The dispatcher deals workgroup b to XCD b % 8. When the grid is a multiple
// of 8, XCD x takes the contiguous rows [x N / 8, (x + 1) N / 8) and its
// wavefronts interleave over them, so each XCD's L2 and address translation
// see one eighth of the matrix; otherwise (or if some wavefront would get
// more than 64 rows, or by_xcd is off) every wavefront interleaves over all
// N rows. A wavefront's rows are first, first + stride, ... (count of them,
// <= 64). Kernel traces (old and new mapping in one process, three boxes):
// 8192x28672 M = 1 22.1 -> 21.8, 25.3 -> 24.2 and 23.6 -> 23.8 us; int3
// 4096x11008 M = 2 9.6 -> 9.2-9.4; the others within 2%. The int4
// few-token kernel keeps the plain mapping (8192x28672 M = 2 28.8 -> 31.5
// us with it).
struct RowMap {
  int first, stride, count;
};
__device__ __forceinline__ RowMap row_map(int N, int per_wg, int idx, bool by_xcd = true) {
  const int G = gridDim.x;
  int first = blockIdx.x * per_wg + idx, stride = G * per_wg, end = N;
  if (by_xcd && (G & 7) == 0 && ((N + 7) >> 3) <= 64 * (G >> 3) * per_wg) {
    const int xc = blockIdx.x & 7;
    stride = (G >> 3) * per_wg;
    first = (int)(((long long)N * xc) >> 3) + (blockIdx.x >> 3) * per_wg + idx;
    end = (int)(((long long)N * (xc + 1)) >> 3);
  }
  return RowMap{first, stride, first < end ? (end - 1 - first) / stride + 1 : 0};
}

// ---------------------------------------------------------------------------
// M = 1: one row per wavefront at a time, read as contiguous 1 KB pieces.
//
// A 1 KB piece of a packed row holds 16 quantization groups (2048 codes).
// Lane l = j + 16*jj reads the 16 bytes at 64*j + 16*jj of the piece, i.e.
// quarter jj of group j, so one dwordx4 instruction covers the piece
// contiguously. In the 16x16x32 MFMA the 16 B-columns are then the 16 groups
// of the piece and the 16 A-rows are the activations of those same 16
// groups (lane (m, jj) holds the activations of quarter jj of group m), so
// the diagonal entry D[j][j] is the dot product of group j with its
// activations; the off-diagonal entries are not used. It sits in lane
// j + 16*(j/4), register j%4.
//
// Offset form: the B operands are the raw fp16 values 1024 + c (even code
// slots) and 1024 + 16 c (odd slots); the odd-slot activations are stored
// pre-multiplied by 1/16 (exact unless they fall below the fp16 normal
// range), so all four MFMAs of a piece accumulate into one D and, per group,
//   sum_k x'_k c_k - z * S = D - (C + z * S),
//   C = 1024 * sum_k x'_k,  S = sum_k x''_k,
// where x' is the stored operand and x'' = x' (even) or 16 x' (odd).
// The activation operands of all pieces depend only on k: they are prepared
// once per workgroup in LDS and shared by its 4 wavefronts, which stream
// different rows.
//
// DUAL (the gate and up projections of a gated MLP, which read the same
// activation): the ring walks items 2i (gate row n_i, from Q/S/Z) and 2i + 1
// (up row n_i, from Q2/S2/Z2); the gate sum waits in a register and the up
// item stores fp16(silu(g) * u), silu(g) = g / (1 + e^-g), in fp32.
//
// SEG = 2 (long rows): the two wavefronts 2r and 2r + 1 of a workgroup read
// the same rows, the first SP pieces and the rest; the second one's sums
// pass through LDS and the first one adds them and stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int SP, int RPF, bool FULL, bool DUAL, bool CS, int SEG = 1>
__global__ __launch_bounds__(256) void gemv_w4_m1_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Q, const void* __restrict__ S,
    const void* __restrict__ Z, const uint32_t* __restrict__ Q2, const void* __restrict__ S2,
    const void* __restrict__ Z2, uint16_t* __restrict__ Y, int N, int K, int gshift) {
  static_assert(SEG == 1 || (SEG == 2 && !DUAL), "row segments: plain product, 2 per row");
  constexpr int NP = SP * SEG;     // pieces of a row
  __shared__ u32x4 xs[NP][4][64];  // [piece][operand][lane]
  __shared__ float2 xcs[NP][16];   // (C, S) of group 16*piece + j
  __shared__ float segp[SEG > 1 ? 4 : 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int seg = SEG > 1 ? wave % SEG : 0;  // pieces seg*SP .. seg*SP + SP - 1
  const RowMap rm = row_map(N, 4 / SEG, wave / SEG);
  const int gw = rm.first;  // rows gw, gw + NW, ... of this wavefront
  const int NW = rm.stride;
  const int j = lane & 15;
  const int jj = lane >> 4;
  const int nch = K >> 7;  // groups of 128 codes per row; NP = ceil(nch / 16)
  const int ngr = max(1, nch >> gshift);
  const int wpr = K >> 3;
  const int cnt = rm.count;  // rows of this wavefront (<= 64)
  const int rdiag = j & 3;
  const bool diag = jj == (j >> 2);

  // this lane's group in every piece of its segment; without FULL the last
  // pieces may be partial or empty: their missing groups read a valid group
  // and get weight 0
  int goff[SP];
  bool gval[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    const int g = 16 * (seg * SP + s) + j;
    gval[s] = FULL || g < nch;
    goff[s] = FULL ? g : min(g, nch - 1);
  }

  // operand prep: thread (piece s, lane l) of the workgroup permutes the
  // activations of quarter l/16 of group 16 s + l%16. The activations are
  // loaded first; for long rows (SP >= 3) the prep runs after the first ring
  // loads are issued, so it overlaps their memory latency.
  constexpr bool kLatePrep = SP >= 3;
  constexpr int XI = (NP * 64 + 255) / 256;  // prep items per thread
  uint32_t xd[XI][16];
#pragma unroll
  for (int u = 0; u < XI; ++u) {
    const int t = min((int)threadIdx.x + 256 * u, NP * 64 - 1);
    const int g = min(16 * (t >> 6) + (t & 15), nch - 1);
    load_x32(X + g * 128 + 32 * ((t & 63) >> 4), xd[u]);
  }
  float cC[SP], cS[SP];
  auto prep = [&]() {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int t = (int)threadIdx.x + 256 * u;
      const int ps = t >> 6, pl = t & 63;
      uint32_t d[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) d[i] = xd[u][i];
      // odd slots: x / 16 rounded to fp16
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float od = h2f((uint16_t)(d[i] >> 16)) * 0.0625f;
        d[i] = (d[i] & 0xffffu) | ((uint32_t)__half_as_ushort(__float2half_rn(od)) << 16);
      }
      u32x4 o0, o1, o2, o3;
      permute_x32(d, o0, o1, o2, o3);
      float se = 0.f, so = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        se += h2f((uint16_t)(d[i] & 0xffffu));
        so += h2f((uint16_t)(d[i] >> 16));
      }
      se += __shfl_xor(se, 16);
      so += __shfl_xor(so, 16);
      se += __shfl_xor(se, 32);
      so += __shfl_xor(so, 32);
      if (t < NP * 64) {  // wave-uniform: NP * 64 is a multiple of 64
        xs[ps][0][pl] = o0;
        xs[ps][1][pl] = o1;
        xs[ps][2][pl] = o2;
        xs[ps][3][pl] = o3;
        if (pl < 16) xcs[ps][pl] = make_float2(1024.f * (se + so), se + 16.f * so);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      const float2 v = xcs[seg * SP + s][j];
      cC[s] = v.x;
      cS[s] = v.y;
    }
  };
  if constexpr (!kLatePrep) prep();

  // Ring of RPF rows x SP pieces. There are no prologue loads: the loop
  // starts RPF rows early with an empty ring, so every load of the ring is
  // issued at the end of an iteration and consumed one iteration later. (With
  // prologue loads the compiler merges the two loads feeding the loop phi
  // into one load at the top of the loop, which then waits for its data.)
  u32x4 wb[RPF][SP];
  float db[RPF][SP];
  uint32_t zb[RPF][SP];
#pragma unroll
  for (int r = 0; r < RPF; ++r)
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      wb[r][s] = u32x4{0, 0, 0, 0};
      db[r][s] = 0.f;
      zb[r][s] = 0u;
    }
  const int items = DUAL ? 2 * cnt : cnt;  // ring items (rows, or gate/up row pairs)
  const int last = max(items - 1, 0);
  const UnpackRegs ur = unpack_regs();
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t* qlane = Q + 16 * j + 4 * jj;
  const uint32_t* qlane2 = DUAL ? Q2 + 16 * j + 4 * jj : qlane;
  float outv = 0.f;
  float gsum = 0.f;  // DUAL: the gate sum of the current row
  for (int i0 = -RPF; i0 < items; i0 += RPF) {
#pragma unroll
    for (int r = 0; r < RPF; ++r) {
      const int row = i0 + r;  // ring item
      const int nit = min(row + RPF, last);  // refill target item
      const size_t nn = (size_t)min(gw + (DUAL ? nit >> 1 : nit) * NW, N - 1);
      // the refill target's matrix (i0 is a multiple of RPF)
      const bool up2 = DUAL && ((RPF % 2 == 0) ? (r & 1) != 0 : (nit & 1) != 0);
      // keep the rows in program order, so that each row waits only for its
      // own slots and the other RPF - 1 rows' loads stay in flight
      __builtin_amdgcn_sched_barrier(0);
      if (row >= 0) {  // uniform
        const bool vrow = row < items;
        float y = 0.f;
#pragma unroll
        for (int s = 0; s < SP; ++s) {
          const u32x4 w = wb[r][s];
          const float d = (vrow && gval[s]) ? db[r][s] : 0.f;
          const float zs = __builtin_fmaf((float)zb[r][s], cS[s], cC[s]);
          uint32_t e[8], o[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t x = w[t];
            const uint32_t x8 = x >> 8;
            e[2 * t] = and_or(x, ur.lo4, ur.magic);
            o[2 * t] = and_or(x, ur.hi4, ur.magic);
            e[2 * t + 1] = and_or(x8, ur.lo4, ur.magic);
            o[2 * t + 1] = and_or(x8, ur.hi4, ur.magic);
          }
          const int ps = seg * SP + s;
          floatx4 acc = mfma16(xs[ps][0][lane], u32x4{e[0], e[1], e[2], e[3]}, zero4);
          acc = mfma16(xs[ps][1][lane], u32x4{e[4], e[5], e[6], e[7]}, acc);
          acc = mfma16(xs[ps][2][lane], u32x4{o[0], o[1], o[2], o[3]}, acc);
          acc = mfma16(xs[ps][3][lane], u32x4{o[4], o[5], o[6], o[7]}, acc);
          float v = acc[0];
          v = rdiag == 1 ? acc[1] : v;
          v = rdiag == 2 ? acc[2] : v;
          v = rdiag == 3 ? acc[3] : v;
          y = __builtin_fmaf(d, v - zs, y);
        }
        // row done: the 16 diagonal lanes are quads 0 (lanes 0-3), 5, 10 and
        // 15 (lanes 60-63); add within quads with DPP, then the 4 quads
        float v = diag ? y : 0.f;
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0xB1, 0xF, 0xF, true));  // [1,0,3,2]
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0x4E, 0xF, 0xF, true));  // [2,3,0,1]
        const float sum =
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 20))) +
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 40)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 60)));
        if constexpr (DUAL) {
          const bool is_up = (RPF % 2 == 0) ? (r & 1) != 0 : (row & 1) != 0;
          const float val = silu_f(gsum) * sum;
          outv = (is_up && ((row >> 1) & 63) == lane) ? val : outv;
          gsum = sum;
        } else {
          outv = (row & 63) == lane ? sum : outv;
        }
      }
      // refill the slots with the same pieces of the row RPF ahead
      const uint32_t* qn = (up2 ? qlane2 : qlane) + nn * wpr;
      const void* sp = up2 ? S2 : S;
      const void* zp = up2 ? Z2 : Z;
      // rows past this wavefront's last need no loads (uniform branch)
      if (row + RPF < items) {
#pragma unroll
        for (int s = 0; s < SP; ++s) {
          wb[r][s] = ld_nt(reinterpret_cast<const u32x4*>(qn + 16 * (goff[s] - j)));
          db[r][s] = group_scale<CS>(sp, nn, ngr, goff[s] >> gshift);
          zb[r][s] = group_zero<CS>(zp, nn, ngr, goff[s] >> gshift);
        }
      }
      // A no-op (wavefront-scope) fence after the loads: a memory-writing
      // instruction between the loads and the loop back edge keeps the
      // compiler from merging them with the other loads that feed the ring.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    }
    // uniform: the first pass only fills the ring
    if constexpr (kLatePrep)
      if (i0 < 0) prep();
  }
  if constexpr (SEG > 1) {  // the row sums: segment 0 plus segment 1
    segp[wave][lane] = outv;
    __syncthreads();
    if (seg == 0) outv += segp[wave + 1][lane];
  }
  if (seg == 0 && lane < cnt) Y[gw + (size_t)lane * NW] = __half_as_ushort(__float2half_rn(outv));
}

// ---------------------------------------------------------------------------
// Decode, int4, 2 <= M <= 4 on rows of few pieces (M x pieces <= 8): the
// M = 1 streaming scheme with one set of diagonal MFMAs per token row. A
// wavefront reads a row as contiguous 1 KB pieces, unpacks each piece once
// and contracts it with the activation operands of every token row; those
// are prepared in LDS once per workgroup and then held in registers by every
// wavefront (16 VGPRs per token row and piece), so the loop reads no LDS.
// MT x 4 MFMAs per piece (MT = M): at M = 4, 16 per KB of weights, within
// the matrix cores' rate at full HBM bandwidth. SEG = 2: as in the M = 1
// kernel, wavefronts 2r and 2r + 1 read the first SP pieces of the same rows
// and the rest, and the first adds the second's sums (through LDS).
// Dynamic LDS: mt_lds_bytes(MT, SP * SEG, SEG).
// ---------------------------------------------------------------------------
constexpr size_t mt_lds_bytes(int mt, int np, int seg) {
  return (size_t)mt * np * (4 * 64 * 16 + 16 * 8) + (seg > 1 ? (size_t)4 * mt * 64 * 4 : 0);
}

template <int MT, int SP, bool FULL, bool CS, int SEG, bool DUAL = false>
__global__ __launch_bounds__(256) void gemv_w4_mt_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Q, const void* __restrict__ S,
    const void* __restrict__ Z, uint16_t* __restrict__ Y, int N, int K, int gshift,
    const uint32_t* __restrict__ Q2, const void* __restrict__ S2, const void* __restrict__ Z2) {
  static_assert(!DUAL || SEG == 1, "the gated form: one wavefront per row");
  static_assert(SEG == 1 || SEG == 2, "one or two wavefronts per row");
  constexpr int NP = SP * SEG;  // pieces of a row
  extern __shared__ __align__(16) uint8_t smem[];
  u32x4* xs = reinterpret_cast<u32x4*>(smem);                         // [MT][NP][4][64]
  float2* xcs = reinterpret_cast<float2*>(xs + MT * NP * 4 * 64);     // [MT][NP][16]: (C, S)
  float* segp = reinterpret_cast<float*>(xcs + MT * NP * 16);         // [4][MT][64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int seg = SEG > 1 ? wave % SEG : 0;  // pieces seg*SP .. seg*SP + SP - 1
  const RowMap rm = row_map(N, 4 / SEG, wave / SEG, false);
  const int gw = rm.first;  // rows gw, gw + NW, ... of this wavefront
  const int NW = rm.stride;
  const int j = lane & 15;
  const int jj = lane >> 4;
  const int nch = K >> 7;
  const int ngr = max(1, nch >> gshift);
  const int wpr = K >> 3;
  const int cnt = rm.count;  // rows of this wavefront (<= 64)
  const int rdiag = j & 3;
  const bool diag = jj == (j >> 2);

  int goff[SP];
  bool gval[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    const int g = 16 * (seg * SP + s) + j;
    gval[s] = FULL || g < nch;
    goff[s] = FULL ? g : min(g, nch - 1);
  }

  // operand prep: item t = (token row, piece, lane) as in the M = 1 kernel,
  // then every wavefront copies its pieces' operands and its groups' C, S to
  // registers
  constexpr int NI = MT * NP * 64;
  constexpr int XI = (NI + 255) / 256;
  constexpr bool kLatePrep = MT * SP >= 3;
  u32x4 av[MT][SP][4];
  float cC[MT][SP], cS[MT][SP];
  auto prep = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int t = (int)threadIdx.x + 256 * u;
      if (t < NI) {  // wave-uniform: NI is a multiple of 64
        const int tk = t / (NP * 64), ps = (t >> 6) % NP, pl = t & 63;
        const int g = min(16 * ps + (pl & 15), nch - 1);
        uint32_t d[16];
        load_x32(X + (size_t)tk * K + g * 128 + 32 * (pl >> 4), d);
#pragma unroll
        for (int i = 0; i < 16; ++i) {  // odd slots: x / 16 rounded to fp16
          const float od = h2f((uint16_t)(d[i] >> 16)) * 0.0625f;
          d[i] = (d[i] & 0xffffu) | ((uint32_t)__half_as_ushort(__float2half_rn(od)) << 16);
        }
        u32x4 o0, o1, o2, o3;
        permute_x32(d, o0, o1, o2, o3);
        float se = 0.f, so = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          se += h2f((uint16_t)(d[i] & 0xffffu));
          so += h2f((uint16_t)(d[i] >> 16));
        }
        se += __shfl_xor(se, 16);
        so += __shfl_xor(so, 16);
        se += __shfl_xor(se, 32);
        so += __shfl_xor(so, 32);
        u32x4* xo = xs + (size_t)(tk * NP + ps) * 4 * 64 + pl;
        xo[0] = o0;
        xo[64] = o1;
        xo[128] = o2;
        xo[192] = o3;
        if (pl < 16) xcs[(tk * NP + ps) * 16 + pl] = make_float2(1024.f * (se + so), se + 16.f * so);
      }
    }
    __syncthreads();
#pragma unroll
    for (int tk = 0; tk < MT; ++tk)
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        const int ps = tk * NP + seg * SP + s;
#pragma unroll
        for (int k = 0; k < 4; ++k) av[tk][s][k] = xs[(size_t)(ps * 4 + k) * 64 + lane];
        const float2 v = xcs[ps * 16 + j];
        cC[tk][s] = v.x;
        cS[tk][s] = v.y;
      }
  };
  if constexpr (!kLatePrep) prep();

  // a ring of one row; the loop starts one row early with an empty ring (no
  // prologue loads, as in the M = 1 kernel)
  u32x4 wb[SP];
  float db[SP];
  uint32_t zb[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    wb[s] = u32x4{0, 0, 0, 0};
    db[s] = 0.f;
    zb[s] = 0u;
  }
  const UnpackRegs ur = unpack_regs();
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t* qlane = Q + 16 * j + 4 * jj;
  const uint32_t* qlane2 = DUAL ? Q2 + (qlane - Q) : qlane;
  const int items = DUAL ? 2 * cnt : cnt;  // rows, or gate/up row pairs
  float gsum[MT];  // DUAL: the gate sums of the current row
#pragma unroll
  for (int tk = 0; tk < MT; ++tk) gsum[tk] = 0.f;
  float outv[MT];
#pragma unroll
  for (int tk = 0; tk < MT; ++tk) outv[tk] = 0.f;
  for (int row = -1; row < items; ++row) {  // row: item
    __builtin_amdgcn_sched_barrier(0);
    if (row >= 0) {  // uniform
      float y[MT];
#pragma unroll
      for (int tk = 0; tk < MT; ++tk) y[tk] = 0.f;
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        const u32x4 w = wb[s];
        const float d = gval[s] ? db[s] : 0.f;
        const float zf = (float)zb[s];
        uint32_t e[8], o[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t x = w[t];
          const uint32_t x8 = x >> 8;
          e[2 * t] = and_or(x, ur.lo4, ur.magic);
          o[2 * t] = and_or(x, ur.hi4, ur.magic);
          e[2 * t + 1] = and_or(x8, ur.lo4, ur.magic);
          o[2 * t + 1] = and_or(x8, ur.hi4, ur.magic);
        }
#pragma unroll
        for (int tk = 0; tk < MT; ++tk) {
          floatx4 acc = mfma16(av[tk][s][0], u32x4{e[0], e[1], e[2], e[3]}, zero4);
          acc = mfma16(av[tk][s][1], u32x4{e[4], e[5], e[6], e[7]}, acc);
          acc = mfma16(av[tk][s][2], u32x4{o[0], o[1], o[2], o[3]}, acc);
          acc = mfma16(av[tk][s][3], u32x4{o[4], o[5], o[6], o[7]}, acc);
          float v = acc[0];
          v = rdiag == 1 ? acc[1] : v;
          v = rdiag == 2 ? acc[2] : v;
          v = rdiag == 3 ? acc[3] : v;
          const float zs = __builtin_fmaf(zf, cS[tk][s], cC[tk][s]);
          y[tk] = __builtin_fmaf(d, v - zs, y[tk]);
        }
      }
      // row done: per token row, the 16 diagonal lanes (quads 0, 5, 10, 15)
      // added with DPP within quads, then the 4 quads
#pragma unroll
      for (int tk = 0; tk < MT; ++tk) {
        float v = diag ? y[tk] : 0.f;
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0xB1, 0xF, 0xF, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0x4E, 0xF, 0xF, true));
        const float sum =
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 20))) +
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 40)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 60)));
        if constexpr (DUAL) {
          if ((row & 1) == 0) {  // uniform: the gate item waits for its up item
            gsum[tk] = sum;
          } else {
            const float val = silu_f(gsum[tk]) * sum;
            outv[tk] = ((row >> 1) & 63) == lane ? val : outv[tk];
          }
        } else {
          outv[tk] = (row & 63) == lane ? sum : outv[tk];
        }
      }
    }
    if (row + 1 < items) {  // uniform: refill with the next item's pieces
      const int nit = row + 1;
      const bool up = DUAL && (nit & 1) != 0;
      const size_t nn = (size_t)gw + (size_t)(DUAL ? nit >> 1 : nit) * NW;
      const uint32_t* qn = (up ? qlane2 : qlane) + nn * wpr;
      const void* Sp = up ? S2 : S;
      const void* Zp = up ? Z2 : Z;
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        wb[s] = ld_nt(reinterpret_cast<const u32x4*>(qn + 16 * (goff[s] - j)));
        db[s] = group_scale<CS>(Sp, nn, ngr, goff[s] >> gshift);
        zb[s] = group_zero<CS>(Zp, nn, ngr, goff[s] >> gshift);
      }
    }
    // keeps the refill loads out of the loop head (see the M = 1 kernel)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if constexpr (kLatePrep)
      if (row < 0) prep();  // uniform: after the first row's loads are issued
  }
  if constexpr (SEG > 1) {  // the row sums: segment 0 plus segment 1
#pragma unroll
    for (int tk = 0; tk < MT; ++tk) segp[(wave * MT + tk) * 64 + lane] = outv[tk];
    __syncthreads();
    if (seg == 0) {
#pragma unroll
      for (int tk = 0; tk < MT; ++tk) outv[tk] += segp[((wave + 1) * MT + tk) * 64 + lane];
    }
  }
#pragma unroll
  for (int tk = 0; tk < MT; ++tk)
    if (seg == 0 && lane < cnt)
      Y[(size_t)tk * N + gw + (size_t)lane * NW] = __half_as_ushort(__float2half_rn(outv[tk]));
}

// ---------------------------------------------------------------------------
// Decode, int3, M = 1, group 128. The same streaming scheme as the int4
// kernel above: a wavefront reads one row at a time in pieces of 16 groups
// (16 x 13 words = 832 contiguous bytes) and contracts each piece with
// diagonal 16x16x32 MFMAs. Lane j + 16 jj loads the 4 words of group j that
// start at word {0, 4, 7, 9}[jj] (dword-aligned 16-byte loads) and uses all
// 4 (jj = 0), the first 3 (jj = 1, 2) or the last 3 (jj = 3), so the
// group's 13 words are used once and no load leaves the group.
//
// Unpacking. A word holds codes c0..c9 at bits 3i. Five AND-ORs with the
// fp16 magic number give five pairs (1024 + wl c_a, 1024 + wh c_b):
//   w & 0x001C0007 -> (c0, c6) weights (1, 4)
//   w & 0x00E00038 -> (c1, c7)         (8, 32)
//   (w >> 8) & 0x0007000E -> (c3, c8)  (2, 1)
//   (w >> 8) & 0x00380070 -> (c4, c9)  (16, 8)
//   (w << 1) & 0x00070380 -> (c2, c5)  (128, 1)
// The activation operand holds x / weight for each slot (exact: powers of
// two), so the MFMA gives 1024 * sum(A) + sum(c x); the first term C and
// the zero-point term z * S are removed per group as in the int4 kernel.
// Slots of unused words and of the two codes past the group's 128 (word 12,
// c8 and c9) have A = 0.
namespace {
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
constexpr int kW3Lo[5] = {0, 1, 3, 4, 2};
constexpr int kW3Hi[5] = {6, 7, 8, 9, 5};
constexpr float kW3InvLo[5] = {1.f, 0.125f, 0.5f, 0.0625f, 0.0078125f};
constexpr float kW3InvHi[5] = {0.25f, 0.03125f, 1.f, 0.125f, 1.f};
__device__ __forceinline__ int w3_first_word(int jj) { return jj == 0 ? 0 : (jj == 1 ? 4 : (jj == 2 ? 7 : 9)); }
}  // namespace

// DUAL: gate and up rows alternate in the ring as in the int4 kernel.
template <int SP, int RPF, bool FULL, bool DUAL, bool CS>
__global__ __launch_bounds__(256) void gemv_w3_m1_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Q, const void* __restrict__ S,
    const void* __restrict__ Z, const uint32_t* __restrict__ Q2, const void* __restrict__ S2,
    const void* __restrict__ Z2, uint16_t* __restrict__ Y, int N, int K, int wpr, int gshift) {
  __shared__ u32x4 xs[SP][5][64];  // [piece][operand][lane]
  __shared__ float2 xcs[SP][16];   // (C, S) of group 16*piece + j
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const RowMap rm = row_map(N, 4, wave);
  const int gw = rm.first;  // rows gw, gw + NW, ... of this wavefront
  const int NW = rm.stride;
  const int j = lane & 15;
  const int jj = lane >> 4;
  const int nch = K >> 7;  // 128-code blocks per row; SP = ceil(nch / 16)
  const int ngr = max(1, nch >> gshift);  // groups per row
  const int cnt = rm.count;  // rows of this wavefront (<= 64)
  const int rdiag = j & 3;
  const bool diag = jj == (j >> 2);
  const int woff = w3_first_word(jj);

  int goff[SP];
  bool gval[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    gval[s] = FULL || 16 * s + j < nch;
    goff[s] = FULL ? 16 * s + j : min(16 * s + j, nch - 1);
  }

  // operand prep: thread (piece s, lane l) builds lane l's 40 activation
  // slots of group 16 s + l%16. As in the int4 kernel the activations are
  // loaded first and, for long rows, prepared while the first ring loads are
  // in flight.
  constexpr bool kLatePrep = SP >= 3;
  constexpr int XI = (SP * 64 + 255) / 256;  // prep items per thread
  uint32_t xd[XI][20];
#pragma unroll
  for (int u = 0; u < XI; ++u) {
    const int t = min((int)threadIdx.x + 256 * u, SP * 64 - 1);
    const int pl = t & 63;
    const int g = min(16 * (t >> 6) + (pl & 15), nch - 1);
    const int pw = w3_first_word(pl >> 4);
    // dwords 5 pw .. 5 pw + 19 of the group's 64 (codes 10 pw .. 10 pw + 39)
    const uint32_t* xg = reinterpret_cast<const uint32_t*>(X + (size_t)g * 128);
#pragma unroll
    for (int i = 0; i < 20; ++i) xd[u][i] = xg[min(5 * pw + i, 63)];
  }
  float cC[SP], cS[SP];
  auto prep = [&]() {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int t = (int)threadIdx.x + 256 * u;
      const int ps = t >> 6, pl = t & 63;
      const int pq = pl >> 4;
      const int pw = w3_first_word(pq);
      const int wlo = pq == 3 ? 1 : 0, whi = pq == 1 || pq == 2 ? 3 : 4;  // used words [wlo, whi)
      uint32_t av[20];
      float cs = 0.f, ss = 0.f;
#pragma unroll
      for (int P = 0; P < 20; ++P) {
        const int w = P / 5, p = P % 5;
        const bool use = w >= wlo && w < whi;
        const int cl = 10 * w + kW3Lo[p], ch = 10 * w + kW3Hi[p];
        const float xl = h2f((uint16_t)(xd[u][cl >> 1] >> (16 * (cl & 1))));
        const float xh = h2f((uint16_t)(xd[u][ch >> 1] >> (16 * (ch & 1))));
        // a code past the group's 128 only occurs for word 12 (c8, c9)
        const bool lo_ok = use && 10 * (pw + w) + kW3Lo[p] < 128;
        const bool hi_ok = use && 10 * (pw + w) + kW3Hi[p] < 128;
        const __half al = __float2half_rn(lo_ok ? xl * kW3InvLo[p] : 0.f);
        const __half ah = __float2half_rn(hi_ok ? xh * kW3InvHi[p] : 0.f);
        av[P] = (uint32_t)__half_as_ushort(al) | ((uint32_t)__half_as_ushort(ah) << 16);
        const float fl = __half2float(al), fh = __half2float(ah);
        cs += fl + fh;
        ss += fl * (1.f / kW3InvLo[p]) + fh * (1.f / kW3InvHi[p]);
      }
      cs += __shfl_xor(cs, 16);
      ss += __shfl_xor(ss, 16);
      cs += __shfl_xor(cs, 32);
      ss += __shfl_xor(ss, 32);
      if (t < SP * 64) {  // wave-uniform: SP * 64 is a multiple of 64
#pragma unroll
        for (int o = 0; o < 5; ++o)
          xs[ps][o][pl] = u32x4{av[4 * o], av[4 * o + 1], av[4 * o + 2], av[4 * o + 3]};
        if (pl < 16) xcs[ps][pl] = make_float2(1024.f * cs, ss);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      const float2 v = xcs[s][j];
      cC[s] = v.x;
      cS[s] = v.y;
    }
  };
  if constexpr (!kLatePrep) prep();

  // ring of RPF rows x SP pieces, filled without prologue loads (see the
  // int4 kernel)
  u32x4 wb[RPF][SP];
  float db[RPF][SP];
  uint32_t zb[RPF][SP];
#pragma unroll
  for (int r = 0; r < RPF; ++r)
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      wb[r][s] = u32x4{0, 0, 0, 0};
      db[r][s] = 0.f;
      zb[r][s] = 0u;
    }
  const int items = DUAL ? 2 * cnt : cnt;  // ring items (rows, or gate/up row pairs)
  const int last = max(items - 1, 0);
  const UnpackRegs ur = unpack_regs();
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t* qlane = Q + woff;
  const uint32_t* qlane2 = DUAL ? Q2 + woff : qlane;
  float outv = 0.f;
  float gsum = 0.f;  // DUAL: the gate sum of the current row
  for (int i0 = -RPF; i0 < items; i0 += RPF) {
#pragma unroll
    for (int r = 0; r < RPF; ++r) {
      const int row = i0 + r;  // ring item
      const int nit = min(row + RPF, last);  // refill target item
      const size_t nn = (size_t)min(gw + (DUAL ? nit >> 1 : nit) * NW, N - 1);
      const bool up2 = DUAL && ((RPF % 2 == 0) ? (r & 1) != 0 : (nit & 1) != 0);
      __builtin_amdgcn_sched_barrier(0);
      if (row >= 0) {  // uniform
        const bool vrow = row < items;
        float y = 0.f;
#pragma unroll
        for (int s = 0; s < SP; ++s) {
          const u32x4 w = wb[r][s];
          const float dd = (vrow && gval[s]) ? db[r][s] : 0.f;
          const float zs = __builtin_fmaf((float)zb[r][s], cS[s], cC[s]);
          uint32_t pr[20];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x = w[q];
            const uint32_t t8 = x >> 8, u1 = x << 1;
            pr[5 * q + 0] = and_or(x, ur.m3[0], ur.magic);
            pr[5 * q + 1] = and_or(x, ur.m3[1], ur.magic);
            pr[5 * q + 2] = and_or(t8, ur.m3[2], ur.magic);
            pr[5 * q + 3] = and_or(t8, ur.m3[3], ur.magic);
            pr[5 * q + 4] = and_or(u1, ur.m3[4], ur.magic);
          }
          floatx4 acc = mfma16(xs[s][0][lane], u32x4{pr[0], pr[1], pr[2], pr[3]}, zero4);
          acc = mfma16(xs[s][1][lane], u32x4{pr[4], pr[5], pr[6], pr[7]}, acc);
          acc = mfma16(xs[s][2][lane], u32x4{pr[8], pr[9], pr[10], pr[11]}, acc);
          acc = mfma16(xs[s][3][lane], u32x4{pr[12], pr[13], pr[14], pr[15]}, acc);
          acc = mfma16(xs[s][4][lane], u32x4{pr[16], pr[17], pr[18], pr[19]}, acc);
          float v = acc[0];
          v = rdiag == 1 ? acc[1] : v;
          v = rdiag == 2 ? acc[2] : v;
          v = rdiag == 3 ? acc[3] : v;
          y = __builtin_fmaf(dd, v - zs, y);
        }
        float v = diag ? y : 0.f;
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0xB1, 0xF, 0xF, true));  // [1,0,3,2]
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0x4E, 0xF, 0xF, true));  // [2,3,0,1]
        const float sum =
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 20))) +
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 40)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 60)));
        if constexpr (DUAL) {
          const bool is_up = (RPF % 2 == 0) ? (r & 1) != 0 : (row & 1) != 0;
          const float val = silu_f(gsum) * sum;
          outv = (is_up && ((row >> 1) & 63) == lane) ? val : outv;
          gsum = sum;
        } else {
          outv = (row & 63) == lane ? sum : outv;
        }
      }
      const uint32_t* qn = (up2 ? qlane2 : qlane) + nn * wpr;
      const void* sp = up2 ? S2 : S;
      const void* zp = up2 ? Z2 : Z;
      // rows past this wavefront's last need no loads (uniform branch)
      if (row + RPF < items) {
#pragma unroll
        for (int s = 0; s < SP; ++s) {
          const u32x4a4 v = ld_nt(reinterpret_cast<const u32x4a4*>(qn + 13 * goff[s]));
          wb[r][s] = u32x4{v[0], v[1], v[2], v[3]};
          db[r][s] = group_scale<CS>(sp, nn, ngr, goff[s] >> gshift);
          zb[r][s] = group_zero<CS>(zp, nn, ngr, goff[s] >> gshift);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    }
    if constexpr (kLatePrep)
      if (i0 < 0) prep();
  }
  if (lane < cnt) Y[gw + (size_t)lane * NW] = __half_as_ushort(__float2half_rn(outv));
}

template <bool CS>
hipError_t launch_gemv_w3_m1_long(const __half* X, const uint32_t* q, const void* scales,
                                  const void* zeros, int N, int K, int group, __half* Y,
                                  hipStream_t st);

template <bool CS>
hipError_t launch_gemv_w3_m1_t(const __half* X, const uint32_t* q, const void* scales,
                               const void* zeros, int N, int K, int group, __half* Y,
                               hipStream_t st) {
  const int nch = K / 128;
  const int sp = (nch + 15) / 16;
  if (sp > 6) return launch_gemv_w3_m1_long<CS>(X, q, scales, zeros, N, K, group, Y, st);
  const int gshift = group_shift(group);
  const int wpr = words_per_row(K, 3, group);
  // wavefronts per compute unit: 3 per SIMD for rows of two pieces, else 2
  // (a kernel-trace sweep of 4-24 per CU and ring depths 1-3: 4096 x 11008
  // 8.8 -> 7.9 us, and a ring of two rows on 11008-long rows 10.0 -> 9.6 us)
  const int wpc = sp == 2 ? 12 : 8;
  const int nw = max(cu_count() * wpc, (N + 63) / 64);
  const dim3 g1((unsigned)((min(N, nw) + 3) / 4)), block(256);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  const bool full = nch % 16 == 0;
#define AWQ_W3(SM, RP)                                                                        \
  do {                                                                                        \
    if (full)                                                                                 \
      hipLaunchKernelGGL((gemv_w3_m1_kernel<SM, RP, true, false, CS>), g1, block, 0, st, x, q, \
                         scales, zeros, nullptr, nullptr, nullptr, y, N, K, wpr, gshift);     \
    else                                                                                      \
      hipLaunchKernelGGL((gemv_w3_m1_kernel<SM, RP, false, false, CS>), g1, block, 0, st, x,   \
                         q, scales, zeros, nullptr, nullptr, nullptr, y, N, K, wpr, gshift);  \
  } while (0)
  switch (sp) {
    case 1: AWQ_W3(1, 4); break;
    case 2: AWQ_W3(2, 2); break;
    case 3: AWQ_W3(3, 2); break;
    case 4: AWQ_W3(4, 1); break;
    case 5: AWQ_W3(5, 1); break;
    default: AWQ_W3(6, 2); break;
  }
#undef AWQ_W3
  return hipGetLastError();
}

hipError_t launch_gemv_w3_m1(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int N, int K, int group, __half* Y, hipStream_t st,
                             bool cs) {
  return cs ? launch_gemv_w3_m1_t<true>(X, q, scales, zeros, N, K, group, Y, st)
            : launch_gemv_w3_m1_t<false>(X, q, scales, zeros, N, K, group, Y, st);
}

// ---------------------------------------------------------------------------
// Decode, int3, 2 <= M <= 4 on rows of few pieces (M x pieces <= 8): the
// int3 M = 1 scheme (pieces of 16 groups x 13 words, five diagonal MFMAs
// per piece) with one set of MFMAs per token row, the activation operands
// of every token row held in registers (20 VGPRs per token row and piece)
// after a prep in LDS shared by the workgroup. SEG = 2: two wavefronts per
// row (first SP pieces and the rest), joined through LDS as in the int4
// kernels. Dynamic LDS: w3mt_lds_bytes(MT, SP * SEG, SEG).
// ---------------------------------------------------------------------------
constexpr size_t w3mt_lds_bytes(int mt, int np, int seg) {
  return (size_t)mt * np * (5 * 64 * 16 + 16 * 8) + (seg > 1 ? (size_t)4 * mt * 64 * 4 : 0);
}

template <int MT, int SP, bool FULL, bool CS, int SEG, bool DUAL = false>
__global__ __launch_bounds__(256) void gemv_w3_mt_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Q, const void* __restrict__ S,
    const void* __restrict__ Z, uint16_t* __restrict__ Y, int N, int K, int wpr, int gshift,
    const uint32_t* __restrict__ Q2, const void* __restrict__ S2, const void* __restrict__ Z2) {
  static_assert(!DUAL || SEG == 1, "the gated form: one wavefront per row");
  static_assert(SEG == 1 || SEG == 2, "one or two wavefronts per row");
  constexpr int NP = SP * SEG;  // pieces of a row
  extern __shared__ __align__(16) uint8_t smem[];
  u32x4* xs = reinterpret_cast<u32x4*>(smem);                      // [MT][NP][5][64]
  float2* xcs = reinterpret_cast<float2*>(xs + MT * NP * 5 * 64);  // [MT][NP][16]: (C, S)
  float* segp = reinterpret_cast<float*>(xcs + MT * NP * 16);      // [4][MT][64]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int seg = SEG > 1 ? wave % SEG : 0;
  const RowMap rm = row_map(N, 4 / SEG, wave / SEG);
  const int gw = rm.first;  // rows gw, gw + NW, ... of this wavefront
  const int NW = rm.stride;
  const int j = lane & 15;
  const int jj = lane >> 4;
  const int nch = K >> 7;
  const int ngr = max(1, nch >> gshift);
  const int cnt = rm.count;  // rows of this wavefront (<= 64)
  const int rdiag = j & 3;
  const bool diag = jj == (j >> 2);
  const int woff = w3_first_word(jj);

  int goff[SP];
  bool gval[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    const int g = 16 * (seg * SP + s) + j;
    gval[s] = FULL || g < nch;
    goff[s] = FULL ? g : min(g, nch - 1);
  }

  // operand prep: item t = (token row, piece, lane) builds that lane's 40
  // activation slots as in the int3 M = 1 kernel. It runs before the row
  // loop: run after the first ring loads (as in the other decode kernels),
  // the form with 2 token rows, 2 pieces per wavefront, two wavefronts per
  // row and whole pieces gave wrong, run-to-run varying sums for the first
  // token row; no cause was found in its LDS addressing, barriers or waits.
  constexpr int NI = MT * NP * 64;
  constexpr int XI = (NI + 255) / 256;
  u32x4 av[MT][SP][5];
  float cC[MT][SP], cS[MT][SP];
  auto prep = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < XI; ++u) {
      const int t = (int)threadIdx.x + 256 * u;
      if (t < NI) {  // wave-uniform: NI is a multiple of 64
        const int tk = t / (NP * 64), ps = (t >> 6) % NP, pl = t & 63;
        const int pq = pl >> 4;
        const int g = min(16 * ps + (pl & 15), nch - 1);
        const int pw = w3_first_word(pq);
        // dwords 5 pw .. 5 pw + 19 of the group's 64 (codes 10 pw .. 10 pw + 39)
        const uint32_t* xg = reinterpret_cast<const uint32_t*>(X + (size_t)tk * K + (size_t)g * 128);
        uint32_t xd[20];
#pragma unroll
        for (int i = 0; i < 20; ++i) xd[i] = xg[min(5 * pw + i, 63)];
        const int wlo = pq == 3 ? 1 : 0, whi = pq == 1 || pq == 2 ? 3 : 4;  // used words
        uint32_t ap[20];
        float cs = 0.f, ss = 0.f;
#pragma unroll
        for (int P = 0; P < 20; ++P) {
          const int w = P / 5, p = P % 5;
          const bool use = w >= wlo && w < whi;
          const int cl = 10 * w + kW3Lo[p], ch = 10 * w + kW3Hi[p];
          const float xl = h2f((uint16_t)(xd[cl >> 1] >> (16 * (cl & 1))));
          const float xh = h2f((uint16_t)(xd[ch >> 1] >> (16 * (ch & 1))));
          // a code past the group's 128 only occurs for word 12 (c8, c9)
          const bool lo_ok = use && 10 * (pw + w) + kW3Lo[p] < 128;
          const bool hi_ok = use && 10 * (pw + w) + kW3Hi[p] < 128;
          const __half al = __float2half_rn(lo_ok ? xl * kW3InvLo[p] : 0.f);
          const __half ah = __float2half_rn(hi_ok ? xh * kW3InvHi[p] : 0.f);
          ap[P] = (uint32_t)__half_as_ushort(al) | ((uint32_t)__half_as_ushort(ah) << 16);
          const float fl = __half2float(al), fh = __half2float(ah);
          cs += fl + fh;
          ss += fl * (1.f / kW3InvLo[p]) + fh * (1.f / kW3InvHi[p]);
        }
        cs += __shfl_xor(cs, 16);
        ss += __shfl_xor(ss, 16);
        cs += __shfl_xor(cs, 32);
        ss += __shfl_xor(ss, 32);
        u32x4* xo = xs + (size_t)(tk * NP + ps) * 5 * 64 + pl;
#pragma unroll
        for (int o = 0; o < 5; ++o)
          xo[64 * o] = u32x4{ap[4 * o], ap[4 * o + 1], ap[4 * o + 2], ap[4 * o + 3]};
        if (pl < 16) xcs[(tk * NP + ps) * 16 + pl] = make_float2(1024.f * cs, ss);
      }
    }
    __syncthreads();
#pragma unroll
    for (int tk = 0; tk < MT; ++tk)
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        const int ps = tk * NP + seg * SP + s;
#pragma unroll
        for (int o = 0; o < 5; ++o) av[tk][s][o] = xs[(size_t)(ps * 5 + o) * 64 + lane];
        const float2 v = xcs[ps * 16 + j];
        cC[tk][s] = v.x;
        cS[tk][s] = v.y;
      }
  };
  prep();

  // a ring of one row, no prologue loads (see the int4 M = 1 kernel)
  u32x4 wb[SP];
  float db[SP];
  uint32_t zb[SP];
#pragma unroll
  for (int s = 0; s < SP; ++s) {
    wb[s] = u32x4{0, 0, 0, 0};
    db[s] = 0.f;
    zb[s] = 0u;
  }
  const UnpackRegs ur = unpack_regs();
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t* qlane = Q + woff;
  const uint32_t* qlane2 = DUAL ? Q2 + (qlane - Q) : qlane;
  const int items = DUAL ? 2 * cnt : cnt;  // rows, or gate/up row pairs
  float gsum[MT];  // DUAL: the gate sums of the current row
#pragma unroll
  for (int tk = 0; tk < MT; ++tk) gsum[tk] = 0.f;
  float outv[MT];
#pragma unroll
  for (int tk = 0; tk < MT; ++tk) outv[tk] = 0.f;
  for (int row = -1; row < items; ++row) {  // row: item
    __builtin_amdgcn_sched_barrier(0);
    if (row >= 0) {  // uniform
      float y[MT];
#pragma unroll
      for (int tk = 0; tk < MT; ++tk) y[tk] = 0.f;
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        const u32x4 w = wb[s];
        const float dd = gval[s] ? db[s] : 0.f;
        const float zf = (float)zb[s];
        uint32_t pr[20];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = w[q];
          const uint32_t t8 = x >> 8, u1 = x << 1;
          pr[5 * q + 0] = and_or(x, ur.m3[0], ur.magic);
          pr[5 * q + 1] = and_or(x, ur.m3[1], ur.magic);
          pr[5 * q + 2] = and_or(t8, ur.m3[2], ur.magic);
          pr[5 * q + 3] = and_or(t8, ur.m3[3], ur.magic);
          pr[5 * q + 4] = and_or(u1, ur.m3[4], ur.magic);
        }
#pragma unroll
        for (int tk = 0; tk < MT; ++tk) {
          floatx4 acc = mfma16(av[tk][s][0], u32x4{pr[0], pr[1], pr[2], pr[3]}, zero4);
          acc = mfma16(av[tk][s][1], u32x4{pr[4], pr[5], pr[6], pr[7]}, acc);
          acc = mfma16(av[tk][s][2], u32x4{pr[8], pr[9], pr[10], pr[11]}, acc);
          acc = mfma16(av[tk][s][3], u32x4{pr[12], pr[13], pr[14], pr[15]}, acc);
          acc = mfma16(av[tk][s][4], u32x4{pr[16], pr[17], pr[18], pr[19]}, acc);
          float v = acc[0];
          v = rdiag == 1 ? acc[1] : v;
          v = rdiag == 2 ? acc[2] : v;
          v = rdiag == 3 ? acc[3] : v;
          const float zs = __builtin_fmaf(zf, cS[tk][s], cC[tk][s]);
          y[tk] = __builtin_fmaf(dd, v - zs, y[tk]);
        }
      }
#pragma unroll
      for (int tk = 0; tk < MT; ++tk) {
        float v = diag ? y[tk] : 0.f;
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0xB1, 0xF, 0xF, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                0x4E, 0xF, 0xF, true));
        const float sum =
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 20))) +
            (__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 40)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 60)));
        if constexpr (DUAL) {
          if ((row & 1) == 0) {  // uniform: the gate item waits for its up item
            gsum[tk] = sum;
          } else {
            const float val = silu_f(gsum[tk]) * sum;
            outv[tk] = ((row >> 1) & 63) == lane ? val : outv[tk];
          }
        } else {
          outv[tk] = (row & 63) == lane ? sum : outv[tk];
        }
      }
    }
    if (row + 1 < items) {  // uniform: refill with the next item's pieces
      const int nit = row + 1;
      const bool up = DUAL && (nit & 1) != 0;
      const size_t nn = (size_t)gw + (size_t)(DUAL ? nit >> 1 : nit) * NW;
      const uint32_t* qn = (up ? qlane2 : qlane) + nn * wpr;
      const void* Sp = up ? S2 : S;
      const void* Zp = up ? Z2 : Z;
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        const u32x4a4 v = ld_nt(reinterpret_cast<const u32x4a4*>(qn + 13 * goff[s]));
        wb[s] = u32x4{v[0], v[1], v[2], v[3]};
        db[s] = group_scale<CS>(Sp, nn, ngr, goff[s] >> gshift);
        zb[s] = group_zero<CS>(Zp, nn, ngr, goff[s] >> gshift);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
  if constexpr (SEG > 1) {  // the row sums: segment 0 plus segment 1
#pragma unroll
    for (int tk = 0; tk < MT; ++tk) segp[(wave * MT + tk) * 64 + lane] = outv[tk];
    __syncthreads();
    if (seg == 0) {
#pragma unroll
      for (int tk = 0; tk < MT; ++tk) outv[tk] += segp[((wave + 1) * MT + tk) * 64 + lane];
    }
  }
#pragma unroll
  for (int tk = 0; tk < MT; ++tk)
    if (seg == 0 && lane < cnt)
      Y[(size_t)tk * N + gw + (size_t)lane * NW] = __half_as_ushort(__float2half_rn(outv[tk]));
}

// 2 <= M <= 4, int3: all token rows in one launch when their operands fit
// the registers (M x pieces per wavefront <= kW3MtMaxItems, with two
// wavefronts per row past that; 8 would need 268-324 registers), else in
// launches of two token rows and a last single row, or of single token rows
// (each launch reading the weights once).
constexpr int kW3MtMaxItems = 6;

template <bool CS>
hipError_t launch_gemv_w3_mt_one(const uint16_t* x, const uint32_t* q, const void* scales,
                                 const void* zeros, int M, int N, int K, int wpr, int gshift,
                                 uint16_t* y, hipStream_t st, int sp, int seg) {
  const int nch = K / 128;
  // 2 wavefronts per SIMD; 1 past 6 token-row pieces (M = 1 on 13-14
  // pieces: 253-270 registers)
  const int wpc = M * sp > 6 ? 4 : 8;
  const int nrw = min(N, max(cu_count() * wpc / seg, (N + 63) / 64));  // row wavefronts
  const dim3 g1((unsigned)((nrw * seg + 3) / 4)), block(256);
  const bool full = nch == 16 * sp * seg;
  const size_t lds = w3mt_lds_bytes(M, sp * seg, seg);
#define AWQ_W3MTF(MV, SM, F, SG)                                                               \
  do {                                                                                         \
    const void* fn = (const void*)gemv_w3_mt_kernel<MV, SM, F, CS, SG>;                        \
    if (lds > 64 * 1024) {                                                                     \
      const hipError_t ea =                                                                    \
          hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);       \
      if (ea != hipSuccess) return ea;                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((gemv_w3_mt_kernel<MV, SM, F, CS, SG>), g1, block, lds, st, x, q,       \
                       scales, zeros, y, N, K, wpr, gshift, nullptr, nullptr, nullptr);        \
  } while (0)
#define AWQ_W3MT(MV, SM, SG)                \
  do {                                      \
    if (full) AWQ_W3MTF(MV, SM, true, SG);  \
    else AWQ_W3MTF(MV, SM, false, SG);      \
  } while (0)
  if (M == 1) {  // rows of 7-14 pieces, two wavefronts per row
    if (sp == 4) AWQ_W3MT(1, 4, 2);
    else if (sp == 5) AWQ_W3MT(1, 5, 2);
    else if (sp == 6) AWQ_W3MT(1, 6, 2);
    else AWQ_W3MT(1, 7, 2);
  } else if (seg == 1) {
    if (M == 2) {
      if (sp == 1) AWQ_W3MT(2, 1, 1);
      else if (sp == 2) AWQ_W3MT(2, 2, 1);
      else AWQ_W3MT(2, 3, 1);
    } else if (M == 3) {
      if (sp == 1) AWQ_W3MT(3, 1, 1);
      else AWQ_W3MT(3, 2, 1);
    } else {
      AWQ_W3MT(4, 1, 1);
    }
  } else {
    if (M == 2) {
      if (sp == 2) AWQ_W3MT(2, 2, 2);
      else AWQ_W3MT(2, 3, 2);
    } else if (M == 3) {
      AWQ_W3MT(3, 2, 2);
    } else {
      AWQ_W3MT(4, 1, 2);
    }
  }
#undef AWQ_W3MT
#undef AWQ_W3MTF
  return hipGetLastError();
}

template <bool CS>
hipError_t launch_gemv_w3_mt_t(const __half* X, const uint32_t* q, const void* scales,
                               const void* zeros, int M, int N, int K, int group, __half* Y,
                               hipStream_t st) {
  if (M < 2 || M > 4) return hipErrorNotSupported;
  const int nch = K / 128;
  const int np = (nch + 15) / 16;  // pieces of a row
  // wavefronts per row and pieces per wavefront for m token rows, or false
  auto shape = [&](int m, int& sp, int& seg) {
    seg = m * np <= kW3MtMaxItems ? 1 : 2;
    sp = (np + seg - 1) / seg;
    return m * sp <= kW3MtMaxItems;
  };
  const int gshift = group_shift(group);
  const int wpr = words_per_row(K, 3, group);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  int sp = 0, seg = 1;
  if (shape(M, sp, seg))
    return launch_gemv_w3_mt_one<CS>(x, q, scales, zeros, M, N, K, wpr, gshift, y, st, sp, seg);
  // pairs of token rows and an M = 1 launch for an odd last row, or one M = 1
  // launch per token row on longer rows (decided before anything is launched;
  // the M = 1 launches cover rows of up to 14 pieces)
  const bool single = np <= 14;
  const bool pairs = shape(2, sp, seg) && ((M & 1) == 0 || single);
  if (!pairs && !single) return hipErrorNotSupported;
  int m0 = 0;
  if (pairs) {
    for (; m0 + 1 < M; m0 += 2) {
      const hipError_t e = launch_gemv_w3_mt_one<CS>(x + (size_t)m0 * K, q, scales, zeros, 2, N,
                                                     K, wpr, gshift, y + (size_t)m0 * N, st, sp,
                                                     seg);
      if (e != hipSuccess) return e;
    }
  }
  for (; m0 < M; ++m0) {
    const hipError_t e = launch_gemv_w3_m1_t<CS>(X + (size_t)m0 * K, q, scales, zeros, N, K,
                                                 group, Y + (size_t)m0 * N, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// M = 1 on rows of 7-14 pieces (K up to 28672): the few-token kernel with
// one token row and two wavefronts per row (the M = 1 kernel holds 6 pieces)
template <bool CS>
hipError_t launch_gemv_w3_m1_long(const __half* X, const uint32_t* q, const void* scales,
                                  const void* zeros, int N, int K, int group, __half* Y,
                                  hipStream_t st) {
  const int np = (K / 128 + 15) / 16;
  if (np < 7 || np > 14) return hipErrorNotSupported;
  return launch_gemv_w3_mt_one<CS>(reinterpret_cast<const uint16_t*>(X), q, scales, zeros, 1, N,
                                   K, words_per_row(K, 3, group), group_shift(group),
                                   reinterpret_cast<uint16_t*>(Y), st, (np + 1) / 2, 2);
}

hipError_t launch_gemv_w3_mt(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int M, int N, int K, int group, __half* Y,
                             hipStream_t st, bool cs) {
  return cs ? launch_gemv_w3_mt_t<true>(X, q, scales, zeros, M, N, K, group, Y, st)
            : launch_gemv_w3_mt_t<false>(X, q, scales, zeros, M, N, K, group, Y, st);
}

// ---------------------------------------------------------------------------
// Decode, int4, 2 <= M <= 16 (gemv_w4_mx_kernel). K is covered in NP passes
// of PC 128-code chunks (one pass unless K > 8192). In a pass a workgroup of
// WV <= 8 wavefronts splits the pass's chunks into WV slices of CPW chunks;
// wavefront s keeps the activation operands of its slice (all token rows,
// MFMA A layout, prepared at the start of the pass) in registers and streams
// row block after row block (16 weight rows) against them, so the MFMA work
// does not grow with M and the activations are read once per workgroup.
// Lane (n, q) = (l % 16, l / 16) loads codes 32q .. 32q + 31 of a chunk of
// row n (16 bytes); the four 16x16x32 MFMAs of a chunk take word t of every
// lane, so one chunk gives the 16 rows x 16 token rows of one quantization
// group. Offset form as in gemv_w4_kernel: even slots (1024 + c) and odd
// slots (1024 + 16 c) are contracted separately, and C = 1024 sum(x even) +
// 64 sum(x odd) and z * S, S = sum(x), are removed per chunk and token.
// Weights stream through a 4-chunk register ring that runs across row blocks
// and passes; the scales and zero points of the next item are staged in LDS
// meanwhile, and the slices' partial sums of a row block are added in LDS in
// a fixed order (then, over the passes, in pass order).
// DUAL (gate and up of a gated MLP, one pass): the workgroup walks items 2j
// (gate row block j, from Q/S/Z) and 2j + 1 (up row block j, from
// Q2/S2/Z2); the gate sums wait in LDS and the up item stores
// fp16(silu(g) * u). MP: more than one pass (the single-pass form keeps the
// pass logic out of the loop).
template <int CPW, bool DUAL, bool CS, bool MP>
__global__ __launch_bounds__(512) void gemv_w4_mx_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Q, const void* __restrict__ S,
    const void* __restrict__ Z, const uint32_t* __restrict__ Q2, const void* __restrict__ S2,
    const void* __restrict__ Z2, uint16_t* __restrict__ Y, int M, int N, int K, int gshift,
    int rbw, int pc) {
  static_assert(CPW % 4 == 0, "the ring of 4 chunks must tile a slice");
  static_assert(!(MP && DUAL), "the gated form runs in one pass");
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WV = blockDim.x >> 6;
  const int nl = lane & 15, q = lane >> 4;
  const int nch = K >> 7;
  const int np = MP ? (nch + pc - 1) / pc : 1;  // passes over K
  const int ngr = max(1, nch >> gshift);
  // groups one pass touches at most (its first one is gbase(pass))
  const int gpp = MP ? min(ngr, ((pc + (1 << gshift) - 1) >> gshift) + 1) : ngr;
  const int wpr = K >> 3;
  const int nrb = (N + 15) >> 4;
  const int rb0 = blockIdx.x * rbw;
  const int nj = min(rbw, nrb - rb0);
  const int nb = DUAL ? 2 * nj : nj;  // items of a pass: row blocks, or gate/up pairs
  const int nit = np * nb;

  float2* csx = reinterpret_cast<float2*>(smem);                  // [nch][16] (C, S)
  float* szf = reinterpret_cast<float*>(csx + (size_t)nch * 16);  // [2][16][gpp] scales
  float* part = szf + 2 * 16 * gpp;                               // [2][WV][4][64] partials
  float* gsum = part + 2 * WV * 256;                              // [256] DUAL gate sums
  float* pacc = gsum + (DUAL ? 256 : 0);                          // [nj][256] earlier passes
  uint8_t* szb = reinterpret_cast<uint8_t*>(pacc + (MP ? nj * 256 : 0));  // [2][16][gpp]

  // item it (clamped to the last): pass, first row of its row block, and
  // whether it reads the up matrix
  auto item_pass = [&](int it) { return MP ? min(it, nit - 1) / nb : 0; };
  auto item_row = [&](int it) {
    const int c = MP ? min(it, nit - 1) % nb : min(it, nit - 1);
    return (rb0 + (DUAL ? c >> 1 : c)) * 16;
  };
  auto item_up = [&](int it) { return DUAL && (min(it, nit - 1) & 1) != 0; };
  // chunks of pass p: [p pc, pend(p)); this wavefront's slice starts at cbeg(p)
  auto pend = [&](int p) { return MP ? min((p + 1) * pc, nch) : nch; };
  auto cbeg = [&](int p) { return (MP ? p * pc : 0) + wave * CPW; };

  // ---- weight ring: 4 chunks ahead, across items ----------------------------
  // chunk i of the slice of item it; slots past the pass re-read its last chunk
  const uint32_t* qlane = Q + 4 * q;
  const uint32_t* qlane2 = DUAL ? Q2 + 4 * q : qlane;
  auto wload = [&](int it, int i) {
    const int p = item_pass(it);
    const size_t n = (size_t)min(item_row(it) + nl, N - 1);
    const int c = min(cbeg(p) + i, pend(p) - 1);
    return ld_nt(reinterpret_cast<const u32x4*>((item_up(it) ? qlane2 : qlane) + n * wpr + c * 16));
  };
  u32x4 ring[4];

  // ---- scales and zero points of item it (the groups of its pass): loaded
  // into registers, then stored to LDS buffer it & 1 --------------------------
  const int szn = 16 * gpp;  // values per item
  constexpr int SZI = 3;     // per thread (the launcher checks szn <= 3 * threads)
  float szv[SZI];
  uint8_t zzv[SZI];
  auto sz_load = [&](int it) {
    const void* Sp = item_up(it) ? S2 : S;
    const void* Zp = item_up(it) ? Z2 : Z;
    const int gb = MP ? (item_pass(it) * pc) >> gshift : 0;
#pragma unroll
    for (int u = 0; u < SZI; ++u) {
      const int idx = min((int)threadIdx.x + (int)blockDim.x * u, szn - 1);
      const int r = idx / gpp;
      const int g = min(gb + idx - r * gpp, ngr - 1);
      const size_t n = (size_t)min(item_row(it) + r, N - 1);
      szv[u] = group_scale<CS>(Sp, n, ngr, g);
      zzv[u] = (uint8_t)group_zero<CS>(Zp, n, ngr, g);
    }
  };
  auto sz_store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < SZI; ++u) {
      const int idx = (int)threadIdx.x + (int)blockDim.x * u;
      if (idx < szn) {
        szf[buf * szn + idx] = szv[u];
        szb[buf * szn + idx] = zzv[u];
      }
    }
  };
  // ---- activation operands of this slice of pass p (token row nl) and C, S:
  // prep loads and permutes chunk by chunk (LD), or permutes in place the raw
  // activations that xload put in av
  u32x4 av[CPW][4];
  auto xload = [&](int p) {
    const int ce = pend(p);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = cbeg(p) + i;
      const u32x4* src = reinterpret_cast<const u32x4*>(X + (size_t)min(nl, M - 1) * K +
                                                        min(c, ce - 1) * 128 + 32 * q);
#pragma unroll
      for (int t = 0; t < 4; ++t) av[i][t] = src[t];
    }
  };
  auto prep = [&](int p, auto LD) {
    const int ce = pend(p);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = cbeg(p) + i;
      const bool ok = c < ce && nl < M;
      uint32_t d[16];
      if constexpr (LD.value) {
        load_x32(X + (size_t)min(nl, M - 1) * K + min(c, ce - 1) * 128 + 32 * q, d);
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) d[t] = av[i][t >> 2][t & 3];
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) d[t] = ok ? d[t] : 0u;
      permute_x32(d, av[i][0], av[i][1], av[i][2], av[i][3]);
      float se = 0.f, so = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        se += h2f((uint16_t)(d[t] & 0xffffu));
        so += h2f((uint16_t)(d[t] >> 16));
      }
      se += __shfl_xor(se, 16);
      so += __shfl_xor(so, 16);
      se += __shfl_xor(se, 32);
      so += __shfl_xor(so, 32);
      if (q == 0 && c < ce) csx[c * 16 + nl] = make_float2(1024.f * se + 64.f * so, se + so);
    }
  };
  // one pass: the activations and the first item's scales first (the prep
  // and the barrier wait for them; the weight ring streams meanwhile).
  // Several passes: the ring first (that order needs fewer registers there)
  if constexpr (!MP) {
    xload(0);
    sz_load(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) ring[i] = wload(0, i);
  if constexpr (MP) sz_load(0);
  // keep the prep's arithmetic below every load (hoisted, it waits for the
  // first chunk before the other loads are issued)
  if constexpr (!MP) __builtin_amdgcn_sched_barrier(0);
  prep(0, std::integral_constant<bool, MP>{});
  sz_store(0);
  __syncthreads();

  const UnpackRegs ur = unpack_regs();
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nit; ++j) {  // j: item
    const int buf = j & 1;
    const int p = MP ? j / nb : 0, jj = j - p * nb;
    if (MP && jj == 0 && p > 0) {  // uniform: a new pass (csx of its chunks
      prep(p, std::true_type{});   // is written and read by the same wavefront)
    }
    if (j + 1 < nit) sz_load(j + 1);  // uniform
    const int cb = cbeg(p), ce = pend(p), gb = MP ? (p * pc) >> gshift : 0;
    floatx4 y = zero4;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const u32x4 w = ring[i & 3];
      // refill: chunk i + 4 of this item or the next one's
      ring[i & 3] = i + 4 < CPW ? wload(j, i + 4) : wload(j + 1, i + 4 - CPW);
      const int c = cb + i;
      if (c < ce) {  // uniform
        uint32_t e[8], o[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t x = w[t];
          const uint32_t x8 = x >> 8;
          e[2 * t] = and_or(x, ur.lo4, ur.magic);
          o[2 * t] = and_or(x, ur.hi4, ur.magic);
          e[2 * t + 1] = and_or(x8, ur.lo4, ur.magic);
          o[2 * t + 1] = and_or(x8, ur.hi4, ur.magic);
        }
        const floatx4 de = mfma16(av[i][1], u32x4{e[4], e[5], e[6], e[7]},
                                  mfma16(av[i][0], u32x4{e[0], e[1], e[2], e[3]}, zero4));
        const floatx4 dd = mfma16(av[i][3], u32x4{o[4], o[5], o[6], o[7]},
                                  mfma16(av[i][2], u32x4{o[0], o[1], o[2], o[3]}, zero4));
        const int gi = nl * gpp + (c >> gshift) - gb;
        const float dl = szf[buf * szn + gi];
        const float zf = (float)szb[buf * szn + gi];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float2 cv = csx[c * 16 + 4 * q + r];  // token 4q + r
          const float t = __builtin_fmaf(dd[r], 0.0625f, de[r]) - __builtin_fmaf(zf, cv.y, cv.x);
          y[r] = __builtin_fmaf(dl, t, y[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) part[((buf * WV + wave) * 4 + r) * 64 + lane] = y[r];
    if (j + 1 < nit) sz_store(buf ^ 1);
    __syncthreads();
    // slices' partials of item j, added in slice order, then over the passes
    // in pass order (thread t always handles the same entries, so gate sums
    // and earlier passes' sums are read back by their writer)
    for (int t = threadIdx.x; t < 256; t += blockDim.x) {
      const int l = t & 63, r = t >> 6;
      float v = 0.f;
      for (int w = 0; w < WV; ++w) v += part[((buf * WV + w) * 4 + r) * 64 + l];
      if constexpr (MP) {
        float* pa = pacc + jj * 256 + t;
        if (p > 0) v = *pa + v;
        if (p < np - 1) {
          *pa = v;
          continue;
        }
      }
      const int m = 4 * (l >> 4) + r;
      const int n = item_row(j) + (l & 15);
      if constexpr (DUAL) {
        if ((j & 1) == 0) {
          gsum[t] = v;
          continue;
        }
        v = silu_f(gsum[t]) * v;
      }
      if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(v));
    }
  }
}

constexpr int kGemvPF = 8;
// M = 1 kernel: rows of up to 14 pieces of 16 groups (K <= 28672; the
// activation operands of a whole row sit in 64 KB of LDS); rows of
// kM1SegMin or more pieces are read by two wavefronts each (timed on rows
// of 7-14 pieces: one wavefront per row is as fast up to 10 pieces; at 14,
// 28672 x 8192, one wavefront per row needs more than 256 registers and ran
// at 36 us, two per row at 25 us)
constexpr int kM1MaxPieces = 14;
// 2 <= M <= 4 on short rows: token rows x pieces held in registers
constexpr int kMtMaxItems = 8;
constexpr int kM1SegMin = 11;
static_assert(kM1SegMin == 11 && kM1MaxPieces == 14,
              "the launcher instantiates 1..10 pieces per row and 6..7 per half row");
constexpr size_t kLdsMax = 160 * 1024;  // LDS of one gfx950 compute unit
constexpr int kGemvMaxRbw = 8;

// raise a decode kernel's dynamic LDS limit once to the largest size used
template <int MODE, int MP, bool CS>
hipError_t allow_lds(size_t lds) {
  static size_t allowed = 0;
  if (lds <= allowed) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)gemv_w4_kernel<MODE, MP, kGemvPF, CS>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) allowed = lds;
  return e;
}

// 2 <= M <= 16: passes of at most 64 chunks (K 8192), each in slices of
// CPW in {4, 8} chunks over at most 8 wavefronts
template <bool CS>
hipError_t launch_gemv_w4_mx_t(const __half* X, const uint32_t* q, const void* scales,
                               const void* zeros, int M, int N, int K, int group, __half* Y,
                               hipStream_t st, const uint32_t* q2, const void* scales2,
                               const void* zeros2) {
  const bool dual = q2 != nullptr;
  const int gshift = log2i(group / 128);
  const int nch = K / 128;
  const int np = (nch + 63) / 64;
  if (dual && np > 1) return hipErrorNotSupported;
  const int pc = (nch + np - 1) / np;
  const int cpw = pc <= 32 ? 4 : 8;
  const int wv = (pc + cpw - 1) / cpw;
  const int ngr = max(1, nch >> gshift);
  const int gpp = np > 1 ? min(ngr, ((pc + (1 << gshift) - 1) >> gshift) + 1) : ngr;
  if (16 * gpp > 3 * 64 * wv) return hipErrorNotSupported;  // scale staging per thread
  const int nrb = (N + 15) / 16;
  // one workgroup of 8 wavefronts fills a compute unit at this register use
  const int resident = cu_count() * (wv <= 4 ? 8 / wv : 1);
  const int rbw = (nrb + resident - 1) / resident;
  const dim3 grid((unsigned)((nrb + rbw - 1) / rbw)), block((unsigned)(64 * wv));
  const size_t lds = (size_t)nch * 16 * 8 + (size_t)2 * 16 * gpp * 4 + (size_t)2 * wv * 256 * 4 +
                     (dual ? 256 * 4 : 0) + (np > 1 ? (size_t)rbw * 256 * 4 : 0) +
                     (size_t)2 * 16 * gpp;
  if (lds > 64 * 1024) return hipErrorNotSupported;  // the kernels' default LDS limit
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
#define AWQ_MX(CP, DU, MPV)                                                                      \
  hipLaunchKernelGGL((gemv_w4_mx_kernel<CP, DU, CS, MPV>), grid, block, lds, st, x, q, scales,    \
                     zeros, q2, scales2, zeros2, y, M, N, K, gshift, rbw, pc)
  if (np > 1) {
    if (cpw == 4) AWQ_MX(4, false, true);
    else AWQ_MX(8, false, true);
  } else if (cpw == 4) {
    if (dual) AWQ_MX(4, true, false);
    else AWQ_MX(4, false, false);
  } else {
    if (dual) AWQ_MX(8, true, false);
    else AWQ_MX(8, false, false);
  }
#undef AWQ_MX
  return hipGetLastError();
}

hipError_t launch_gemv_w4_mx(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int M, int N, int K, int group, __half* Y,
                             hipStream_t st, const uint32_t* q2, const void* scales2,
                             const void* zeros2, bool cs) {
  return cs ? launch_gemv_w4_mx_t<true>(X, q, scales, zeros, M, N, K, group, Y, st, q2, scales2,
                                        zeros2)
            : launch_gemv_w4_mx_t<false>(X, q, scales, zeros, M, N, K, group, Y, st, q2, scales2,
                                         zeros2);
}

// 2 <= M <= 4 on short rows: the M = 1 scheme per token row
// (gemv_w4_mt_kernel); the pieces of a row, wavefronts per row, pieces per
// wavefront and row wavefronts, and whether the automatic choice takes it
struct MtChoice {
  int np, seg, sp, rw;
  bool use;
};
MtChoice mt_choice(int M, int N, int nch) {
  MtChoice c;
  c.np = (nch + 15) / 16;
  c.seg = M * c.np <= kMtMaxItems ? 1 : 2;
  c.sp = (c.np + c.seg - 1) / c.seg;
  c.rw = cu_count() * (M * c.sp <= 4 ? 12 : 8) / c.seg;
  // Two wavefronts per row only at M = 2 on 5-6 pieces (11008x4096 18.9 ->
  // 12.2 us): at 7-8 pieces they would need more than 256 registers, and at
  // M = 3, 4 (16 and 12 MFMAs plus about 40 VALU instructions per KB) they
  // were slower than the 16-row-block kernel (8192x28672 M = 4 37.8 -> 50 us).
  c.use = M >= 2 && M <= 4 && M * c.sp <= kMtMaxItems && (c.seg == 1 || (M == 2 && c.sp <= 3)) &&
          (M == 2 || N >= 3 * c.rw);
  return c;
}

template <bool CS>
hipError_t launch_gemv_w4_t(const __half* X, const uint32_t* q, const void* scales,
                            const void* zeros, int M, int N, int K, int group, __half* Y,
                            hipStream_t st, int variant, void* ws, size_t ws_bytes) {
  const int gshift = log2i(group / 128);
  const int nrb = (N + 15) / 16;
  const int nch = K / 128;
  // all workgroups resident at once: ~3 per CU at this register budget
  const int cap = 3 * cu_count();
  int rbw = (nrb + cap - 1) / cap;
  if (rbw > kGemvMaxRbw) rbw = kGemvMaxRbw;
  const dim3 grid((nrb + rbw - 1) / rbw), block(256);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  // 2 <= M <= 4 on short rows: the M = 1 scheme per token row (gemv_w4_mt_kernel).
  // Timed with kernel traces against gemv_w4_mx_kernel over rotated weights:
  // M = 2 faster on every shape (4096x4096 7.7 -> 6.6 us, 4096x11008 12.8 ->
  // 9.4, 6144x6144 13.6 -> 9.4, 8192x28672 35.2 -> 27.4); M = 3 and 4 only
  // once every wavefront gets three or more rows (4096x11008 M = 4 13.2 ->
  // 12.6 us, while 4096 rows at M = 4 went from 7.9 to 8.1). 3 wavefronts
  // per SIMD at up to 4 token-row pieces (128-136 registers; 4096x11008
  // M = 2 10.2 -> 9.4 us), else 2.
  const MtChoice mt = mt_choice(M, N, nch);
  if (variant == 0 && mt.use) {
    const int sp = mt.sp, seg = mt.seg;
    const int nrw = min(N, max(mt.rw, (N + 63) / 64));
    const dim3 g1((unsigned)((nrw * seg + 3) / 4));
    const bool full = nch == 16 * sp * seg;
    const size_t lds = mt_lds_bytes(M, sp * seg, seg);
#define AWQ_MTF(MV, SM, F, SG)                                                                 \
  do {                                                                                         \
    const void* fn = (const void*)gemv_w4_mt_kernel<MV, SM, F, CS, SG>;                        \
    if (lds > 64 * 1024) {                                                                     \
      const hipError_t ea =                                                                    \
          hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);       \
      if (ea != hipSuccess) return ea;                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((gemv_w4_mt_kernel<MV, SM, F, CS, SG>), g1, block, lds, st, x, q,       \
                       scales, zeros, y, N, K, gshift, nullptr, nullptr, nullptr);             \
  } while (0)
#define AWQ_MT(MV, SM, SG)                \
  do {                                    \
    if (full) AWQ_MTF(MV, SM, true, SG);  \
    else AWQ_MTF(MV, SM, false, SG);      \
  } while (0)
    if (seg == 1) {
      if (M == 2) {
        if (sp == 1) AWQ_MT(2, 1, 1);
        else if (sp == 2) AWQ_MT(2, 2, 1);
        else if (sp == 3) AWQ_MT(2, 3, 1);
        else AWQ_MT(2, 4, 1);
      } else if (M == 3) {
        if (sp == 1) AWQ_MT(3, 1, 1);
        else AWQ_MT(3, 2, 1);
      } else {
        if (sp == 1) AWQ_MT(4, 1, 1);
        else AWQ_MT(4, 2, 1);
      }
    } else {  // two wavefronts per row: M = 2, 5 or 6 pieces
      AWQ_MT(2, 3, 2);
    }
#undef AWQ_MT
#undef AWQ_MTF
    return hipGetLastError();
  }
  if (variant == 0 && M >= 2) {
    if (mb_preferred(M, N, K)) {
      const hipError_t e =
          launch_gemv_w4_mb(X, q, scales, zeros, M, N, K, group, Y, st, CS, ws, ws_bytes);
      if (e != hipErrorNotSupported) return e;
    }
    const hipError_t e = launch_gemv_w4_mx_t<CS>(X, q, scales, zeros, M, N, K, group, Y, st,
                                                 nullptr, nullptr, nullptr);
    if (e != hipErrorNotSupported) return e;
  }
  if (variant == 0 && M == 1 && nch <= 16 * kM1MaxPieces) {
    const int np = (nch + 15) / 16;           // pieces of a row
    const int seg = np >= kM1SegMin ? 2 : 1;  // wavefronts per row
    const int sp = (np + seg - 1) / seg;      // pieces per wavefront
    // wavefronts: all resident, at most 64 rows each; 2 per SIMD, or 3 when
    // the registers allow it (up to 4 pieces) and every wavefront still gets
    // 5 or more rows (measured: 3 per SIMD is 2-4% faster there and slower
    // for fewer rows or longer rows); rows of 2 pieces: 4 per SIMD with a
    // ring of one row (measured 10-12% faster than 2-3 per SIMD with two)
    const int wpc = sp == 2 && seg == 1 ? 16 : (sp <= 4 && N >= 5 * 8 * cu_count() ? 12 : 8);
    const int nrw = min(N, max(cu_count() * wpc / seg, (N + 63) / 64));  // row wavefronts
    const dim3 g1((unsigned)((nrw * seg + 3) / 4));
    const bool full = nch == 16 * sp * seg;
#define AWQ_M1S(SM, RP, SG)                                                                    \
  do {                                                                                          \
    if (full)                                                                                   \
      hipLaunchKernelGGL((gemv_w4_m1_kernel<SM, RP, true, false, CS, SG>), g1, block, 0, st, x, \
                         q, scales, zeros, nullptr, nullptr, nullptr, y, N, K, gshift);         \
    else                                                                                        \
      hipLaunchKernelGGL((gemv_w4_m1_kernel<SM, RP, false, false, CS, SG>), g1, block, 0, st,  \
                         x, q, scales, zeros, nullptr, nullptr, nullptr, y, N, K, gshift);      \
  } while (0)
#define AWQ_M1(SM, RP) AWQ_M1S(SM, RP, 1)
    if (seg == 1) {
      switch (sp) {
        case 1: AWQ_M1(1, 4); break;
        case 2: AWQ_M1(2, 1); break;
        case 3: AWQ_M1(3, 2); break;
        case 4: AWQ_M1(4, 1); break;
        case 5: AWQ_M1(5, 1); break;
        case 6: AWQ_M1(6, 1); break;
        case 7: AWQ_M1(7, 1); break;
        case 8: AWQ_M1(8, 1); break;
        case 9: AWQ_M1(9, 1); break;
        default: AWQ_M1(10, 1); break;
      }
    } else {
      if (sp <= 6) AWQ_M1S(6, 1, 2);  // 11 or 12 pieces
      else AWQ_M1S(7, 1, 2);          // 13 or 14
    }
#undef AWQ_M1
#undef AWQ_M1S
    return hipGetLastError();
  }
  // LDS: activations in MFMA order and their C, S (offset form), the row
  // blocks' partial sums, and the staged scales and zero points
  const size_t sz = (size_t)rbw * 16 * max(1, nch >> gshift) * 5;
  if (variant == 0 && M <= 16) {
    const int mp = M == 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : (M <= 8 ? 8 : 16)));
    const int r = mp < 4 ? mp : 4;
    const size_t lds =
        (size_t)nch * 256 * mp + (size_t)nch * mp * 8 + (size_t)rbw * 4 * 64 * r * 4 + sz;
    if (lds <= kLdsMax) {
#define AWQ_GV(MPV)                                                                              \
  do {                                                                                            \
    const hipError_t ea = allow_lds<kOffset, MPV, CS>(lds);                                      \
    if (ea != hipSuccess) return ea;                                                              \
    hipLaunchKernelGGL((gemv_w4_kernel<kOffset, MPV, kGemvPF, CS>), grid, block, lds, st, x, q,   \
                       scales, zeros, y, M, N, K, gshift, rbw);                                   \
  } while (0)
      if (mp == 1) AWQ_GV(1);
      else if (mp == 2) AWQ_GV(2);
      else if (mp == 4) AWQ_GV(4);
      else if (mp == 8) AWQ_GV(8);
      else AWQ_GV(16);
#undef AWQ_GV
      return hipGetLastError();
    }
  }
  const size_t lds = (size_t)rbw * 4 * 64 * 4 * 4 + sz;
  if (lds > kLdsMax) return hipErrorNotSupported;
  const hipError_t ea = allow_lds<kExact, 16, CS>(lds);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((gemv_w4_kernel<kExact, 16, kGemvPF, CS>), grid, block, lds, st, x, q,
                     scales, zeros, y, M, N, K, gshift, rbw);
  return hipGetLastError();
}

size_t gemv_workspace_bytes(int M, int N, int K) {
  if (M < 2 || M > 16 || mt_choice(M, N, K / 128).use || !mb_preferred(M, N, K)) return 0;
  return mb_plan(M, N, K, true).ws_bytes;
}

hipError_t launch_gemv_w4(const __half* X, const uint32_t* q, const void* scales,
                          const void* zeros, int M, int N, int K, int group, __half* Y,
                          hipStream_t st, int variant, bool cs, void* ws, size_t ws_bytes) {
  return cs ? launch_gemv_w4_t<true>(X, q, scales, zeros, M, N, K, group, Y, st, variant, ws,
                                     ws_bytes)
            : launch_gemv_w4_t<false>(X, q, scales, zeros, M, N, K, group, Y, st, variant, ws,
                                      ws_bytes);
}

// Fused gate/up decode at M = 1, int4: Y = fp16(silu(X Wg^T) * (X Wu^T)).
hipError_t launch_gate_up_w4_m1(const __half* X, const uint32_t* qg, const float* sg,
                                const uint8_t* zg, const uint32_t* qu, const float* su,
                                const uint8_t* zu, int N, int K, int group, __half* Y,
                                hipStream_t st) {
  const int gshift = log2i(group / 128);
  const int nch = K / 128;
  const int sp = (nch + 15) / 16;
  if (sp > 6) return hipErrorNotSupported;
  // 2 wavefronts per SIMD, 4 for rows of two pieces (a kernel-trace sweep
  // of 8-16 per CU and ring depths 1-4: 2 x 4096 x 11008 12.9 -> 11.1 us)
  const int nw = max(cu_count() * (sp == 2 ? 16 : 8), (N + 63) / 64);
  const dim3 g1((unsigned)((min(N, nw) + 3) / 4)), block(256);
  const bool full = nch % 16 == 0;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
#define AWQ_GU(SM, RP)                                                                        \
  do {                                                                                        \
    if (full)                                                                                 \
      hipLaunchKernelGGL((gemv_w4_m1_kernel<SM, RP, true, true, false>), g1, block, 0, st, x,  \
                         qg, sg, zg, qu, su, zu, y, N, K, gshift);                            \
    else                                                                                      \
      hipLaunchKernelGGL((gemv_w4_m1_kernel<SM, RP, false, true, false>), g1, block, 0, st, x, \
                         qg, sg, zg, qu, su, zu, y, N, K, gshift);                            \
  } while (0)
  switch (sp) {
    case 1: AWQ_GU(1, 4); break;
    case 2: AWQ_GU(2, 2); break;
    case 3: AWQ_GU(3, 2); break;
    case 4: AWQ_GU(4, 2); break;
    case 5: AWQ_GU(5, 2); break;
    default: AWQ_GU(6, 2); break;
  }
#undef AWQ_GU
  return hipGetLastError();
}

// Fused gate/up decode at 2 <= M <= 4 on rows of few pieces: the few-token
// kernels in their gated form (one wavefront per row; items alternate gate
// and up rows). int4 at M = 2 only (event timing over rotated weights:
// 2 x 4096 x 11008 18.9 -> 17.8 us, 2 x 8192 x 28672 66 -> 58 us at M = 2,
// while M = 3, 4 got slower than the 16-row-block kernel: 18.9 -> 20.6,
// 20.0 -> 22.5 us); int3 whenever the operands fit (2 x 4096 x 11008 M = 2
// 56.8 -> 18.8 us, M = 3 54.8 -> 20.6 us against the prefill kernel), else
// in pairs of token rows and an M = 1 launch.
hipError_t launch_gate_up_w3_m1(const __half* X, const uint32_t* qg, const float* sg,
                                const uint8_t* zg, const uint32_t* qu, const float* su,
                                const uint8_t* zu, int N, int K, int group, __half* Y,
                                hipStream_t st);

hipError_t launch_gate_up_mt(const __half* X, const uint32_t* qg, const float* sg,
                             const uint8_t* zg, const uint32_t* qu, const float* su,
                             const uint8_t* zu, int M, int N, int K, int bits, int group,
                             __half* Y, hipStream_t st) {
  if (M < 2 || M > 4 || (bits == 4 && M != 2)) return hipErrorNotSupported;
  const int nch = K / 128;
  const int np = (nch + 15) / 16;
  const int cap = bits == 4 ? kMtMaxItems : kW3MtMaxItems;
  if (M * np > cap) {
    // int3: pairs of token rows and an M = 1 launch (decided before anything
    // is launched; the M = 1 gated kernel holds 6 pieces)
    if (bits != 3 || 2 * np > cap || ((M & 1) != 0 && np > 6)) return hipErrorNotSupported;
    for (int m0 = 0; m0 + 1 < M; m0 += 2) {
      const hipError_t e = launch_gate_up_mt(X + (size_t)m0 * K, qg, sg, zg, qu, su, zu, 2, N, K,
                                             bits, group, Y + (size_t)m0 * N, st);
      if (e != hipSuccess) return e;
    }
    if ((M & 1) != 0)
      return launch_gate_up_w3_m1(X + (size_t)(M - 1) * K, qg, sg, zg, qu, su, zu, N, K, group,
                                  Y + (size_t)(M - 1) * N, st);
    return hipSuccess;
  }
  const int wpc = bits == 4 && M * np <= 4 ? 12 : 8;
  const int nw = max(cu_count() * wpc, (N + 63) / 64);
  const dim3 g1((unsigned)((min(N, nw) + 3) / 4)), block(256);
  const bool full = nch == 16 * np;
  const int gshift = group_shift(group);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  if (bits == 4) {
    const size_t lds = mt_lds_bytes(M, np, 1);
#define AWQ_GUMT(MV, SM)                                                                         \
  do {                                                                                           \
    if (full)                                                                                    \
      hipLaunchKernelGGL((gemv_w4_mt_kernel<MV, SM, true, false, 1, true>), g1, block, lds, st, \
                         x, qg, sg, zg, y, N, K, gshift, qu, su, zu);                            \
    else                                                                                         \
      hipLaunchKernelGGL((gemv_w4_mt_kernel<MV, SM, false, false, 1, true>), g1, block, lds,    \
                         st, x, qg, sg, zg, y, N, K, gshift, qu, su, zu);                        \
  } while (0)
    if (M == 2) {
      if (np == 1) AWQ_GUMT(2, 1);
      else if (np == 2) AWQ_GUMT(2, 2);
      else if (np == 3) AWQ_GUMT(2, 3);
      else AWQ_GUMT(2, 4);
    } else if (M == 3) {
      if (np == 1) AWQ_GUMT(3, 1);
      else AWQ_GUMT(3, 2);
    } else {
      if (np == 1) AWQ_GUMT(4, 1);
      else AWQ_GUMT(4, 2);
    }
#undef AWQ_GUMT
  } else {
    const int wpr = words_per_row(K, 3, group);
    const size_t lds = w3mt_lds_bytes(M, np, 1);
#define AWQ_GUMT3(MV, SM)                                                                        \
  do {                                                                                           \
    if (full)                                                                                    \
      hipLaunchKernelGGL((gemv_w3_mt_kernel<MV, SM, true, false, 1, true>), g1, block, lds, st, \
                         x, qg, sg, zg, y, N, K, wpr, gshift, qu, su, zu);                       \
    else                                                                                         \
      hipLaunchKernelGGL((gemv_w3_mt_kernel<MV, SM, false, false, 1, true>), g1, block, lds,    \
                         st, x, qg, sg, zg, y, N, K, wpr, gshift, qu, su, zu);                   \
  } while (0)
    if (M == 2) {
      if (np == 1) AWQ_GUMT3(2, 1);
      else if (np == 2) AWQ_GUMT3(2, 2);
      else AWQ_GUMT3(2, 3);
    } else if (M == 3) {
      if (np == 1) AWQ_GUMT3(3, 1);
      else AWQ_GUMT3(3, 2);
    } else {
      AWQ_GUMT3(4, 1);
    }
#undef AWQ_GUMT3
  }
  return hipGetLastError();
}

// Fused gate/up decode at M = 1, int3, group 128.
hipError_t launch_gate_up_w3_m1(const __half* X, const uint32_t* qg, const float* sg,
                                const uint8_t* zg, const uint32_t* qu, const float* su,
                                const uint8_t* zu, int N, int K, int group, __half* Y,
                                hipStream_t st) {
  const int nch = K / 128;
  const int sp = (nch + 15) / 16;
  if (sp > 6) return hipErrorNotSupported;
  const int gshift = group_shift(group);
  const int wpr = words_per_row(K, 3, group);
  const int nw = max(cu_count() * 8, (N + 63) / 64);
  const dim3 g1((unsigned)((min(N, nw) + 3) / 4)), block(256);
  const bool full = nch % 16 == 0;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
#define AWQ_GU3(SM, RP)                                                                       \
  do {                                                                                        \
    if (full)                                                                                 \
      hipLaunchKernelGGL((gemv_w3_m1_kernel<SM, RP, true, true, false>), g1, block, 0, st, x,  \
                         qg, sg, zg, qu, su, zu, y, N, K, wpr, gshift);                       \
    else                                                                                      \
      hipLaunchKernelGGL((gemv_w3_m1_kernel<SM, RP, false, true, false>), g1, block, 0, st, x, \
                         qg, sg, zg, qu, su, zu, y, N, K, wpr, gshift);                       \
  } while (0)
  switch (sp) {
    case 1: AWQ_GU3(1, 4); break;
    case 2: AWQ_GU3(2, 2); break;
    case 3: AWQ_GU3(3, 2); break;
    case 4: AWQ_GU3(4, 2); break;
    case 5: AWQ_GU3(5, 2); break;
    default: AWQ_GU3(6, 2); break;
  }
#undef AWQ_GU3
  return hipGetLastError();
}

}  // namespace awq
