// Decode, int4, 2 <= M <= 16, on 16-row blocks with the activations in LDS
// (gemv_w4_mb_kernel).
//
// MFMA layout: in each v_mfma_f32_16x16x32_f16 the 16 A rows are token rows
// and the 16 B columns are 16 weight rows, so one activation operand serves
// 16 weight rows and the matrix-core work does not grow with M. Lane
// l = n + 16 q owns weight row n of the block and loads the 16 bytes
// (4 words, 32 codes) 32 q .. 32 q + 31 of each 128-code chunk; MFMA j of
// the chunk takes word j of every lane. A rows m >= M hold copies of other
// rows: an A row only reaches the output row of the same index, and output
// rows m >= M are never stored.
//
// Exact dequantization: a word's magic-number pairs are made exact integers
// c - z in fp16 by one packed op each, (1024 + c) - (1024 + z) for codes
// 0, 2, 4, 6 and (1024 + 16 c) / 16 - (64 + z) for codes 1, 3, 5, 7 (every
// value involved is an fp16 integer, so nothing rounds), the MFMAs contract
// them with the fp16 activations in float32, and the chunk's sums are scaled
// by the group step in float32. The lane's pairs come out in the order
// (c0, c4) (c1, c5) (c2, c6) (c3, c7) of the word; the activation operands
// are stored in LDS in that same order of k, x0 x4 x1 x5 x2 x6 x3 x7 (a
// common permutation of k leaves the sum unchanged).
//
// Work split. A workgroup of 8 wavefronts takes the chunks [c0, c1) of K
// (one of S splits, blockIdx.y) and prepares their activation operands in
// LDS once, for all 8 wavefronts; wavefront gw then streams its row blocks
// gw, gw + GW, ... (GW wavefronts per split) over those chunks with a ring
// of kMbRing chunk loads per row block, and keeps the block's sums in
// registers. With S > 1 the splits' float32 sums go to their own [M, N]
// planes of the caller's workspace, and the split that finishes a row block
// last (a counter per row block at the workspace's head) adds the planes
// in split order, so the result does not depend on which split is last;
// with S = 1 the wavefront stores fp16 directly.
//
// Full-line weight loads (FL). The MFMA layout puts 16 rows in every 16
// lanes, so a load in that layout fetches 16 rows x 64 B. With FL a
// wavefront instead loads a chunk pair of its 16 rows as two 8 rows x
// 128 B loads (lane i: bytes 16 (i % 8) of the 128-byte span of row i / 8),
// writes them to its own 2 KB of LDS, at 16-byte slot 8 n + (u ^ (n % 8))
// for row n and part u (both the write and the read below meet no bank
// conflict), and reads each chunk back in the MFMA layout (row nl, part
// 4 c + q). The plan takes FL when the staging buffers leave the split
// count unchanged.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}
__device__ __forceinline__ h2 hv(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t hbits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
// (a & m) | o as one v_and_or_b32 (m in an SGPR, o in a VGPR: unpack_regs);
// the compiler's own instruction, so it keeps the wait states an MFMA
// reading the result needs
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  return (a & m) | o;
}
// (lo half of a, lo half of b) and (hi half of a, hi half of b)
__device__ __forceinline__ uint32_t plo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t phi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

constexpr int kMbWaves = 8;  // wavefronts per workgroup
constexpr int kMbRing = 4;   // weight chunks in flight per wavefront

// chunks of a split, at most
constexpr int kMbMaxSpl = 40;

// LDS of a workgroup: the activation operands of spl chunks and one chunk
// of zeros (16 MP operands of 16 bytes per chunk), then per wavefront its
// row block's group parameters per chunk: float32 steps [16][pst] and uint8
// zero points [16][pst], pst = spl rounded up to odd (the 16 rows of a
// chunk fall in distinct banks), and with full-line loads (fl) a 2 KB
// staging buffer for a chunk pair of its 16 rows
struct MbLds {
  uint32_t a_bytes, pst, par_bytes, wave_bytes, total;
};
constexpr uint32_t kMbStage = 2048;
__host__ __device__ constexpr MbLds mb_lds(int spl, int mp, bool fl) {
  const uint32_t a = (uint32_t)(spl + 1) * 16u * (uint32_t)mp * 16u;
  const uint32_t pst = (uint32_t)spl | 1u;
  const uint32_t pb = (16u * pst * 5u + 15u) & ~15u;
  const uint32_t wb = pb + (fl ? kMbStage : 0u);
  return MbLds{a, pst, pb, wb, a + (uint32_t)kMbWaves * wb};
}

}  // namespace

// Plain group parameters (float32 steps, uint8 zero points, [N][ng] each).
// MP: token rows stored in LDS (8 or 16). PL: write float32 planes (S > 1)
// instead of fp16 Y. FL: full-line weight loads. LDS layout: mb_lds; the
// operands are
// [chunk][mfma j][q][m < MP].
// (4 wavefronts per SIMD: two workgroups per compute unit, 128 registers)
template <int MP, bool PL, bool FL>
__global__ __launch_bounds__(64 * kMbWaves) __attribute__((amdgpu_waves_per_eu(4, 8))) void
gemv_w4_mb_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Q, const void* __restrict__ S,
    const void* __restrict__ Z, uint16_t* __restrict__ Y, float* __restrict__ planes,
    uint32_t* __restrict__ counters, int M, int N, int K, int gshift, int spl) {
  extern __shared__ __align__(16) u32x4 a_lds[];
  constexpr int kChunkOps = 16 * MP;  // 16-byte operands of one chunk
  constexpr int kThreads = 64 * kMbWaves;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, q = lane >> 4;
  const int nch = K >> 7;
  const int ngr = max(1, nch >> gshift);
  const uint32_t rowq = (uint32_t)K >> 1;  // bytes of a packed row
  const int nrb = (N + 15) >> 4;
  const int c0 = blockIdx.y * spl;
  const int c1 = min(c0 + spl, nch);
  const int ncw = c1 - c0;                      // chunks of this split (>= 1)
  const int gw = blockIdx.x * kMbWaves + wave;  // wavefront among the split's
  const int GW = gridDim.x * kMbWaves;
  const int nrw = gw < nrb ? (nrb - 1 - gw) / GW + 1 : 0;  // row blocks of this wavefront
  const MbLds lay = mb_lds(spl, MP, FL);
  char* const lds = reinterpret_cast<char*>(a_lds);
  float* const p_step = reinterpret_cast<float*>(lds + lay.a_bytes + wave * lay.wave_bytes);
  uint8_t* const p_zero = reinterpret_cast<uint8_t*>(p_step + 16 * lay.pst);
  // FL staging (16-byte aligned: the operand and parameter blocks are)
  u32x4* const p_stage =
      reinterpret_cast<u32x4*>(lds + lay.a_bytes + wave * lay.wave_bytes + lay.par_bytes);

  const int nop = ncw * kChunkOps;

  // ---- one row block: its group parameters into this wavefront's LDS,
  // and a ring of kMbRing weight chunk loads (a load past the block's last
  // chunk repeats the last chunk, its result unused)
  u32x4 wr[kMbRing];
  const char* qrow = nullptr;  // uniform bases of the row block
  const char* srow = nullptr;
  const char* zrow = nullptr;
  uint32_t qoff = 0;  // this lane's offset from qrow
  // FL: this lane's row (i / 8 and 8 + i / 8) and 16-byte part of a
  // 128-byte span, and the two rows' offsets from qrow
  const int fr = lane >> 3, fu = lane & 7;
  uint32_t foff[2] = {0u, 0u};
  uint32_t prow = 0;  // this lane's row within the block (rows past N repeat row N - 1)
  // parameter loads: lane (nl, q) takes row nl, chunks q, q + 4, ... (a
  // load past the split's last chunk reads a later chunk of the row, or
  // the row's last one, and is not stored)
  constexpr int kPar = (kMbMaxSpl + 3) / 4;  // chunks per lane, at most
  float pstep[kPar];
  uint32_t pzero[kPar];
  auto row_setup = [&](int ri) {
    const int rb = min(gw + ri * GW, nrb - 1);
    prow = (uint32_t)min(nl, N - 1 - rb * 16);
    qrow = reinterpret_cast<const char*>(Q) + (size_t)rb * 16 * rowq;
    srow = static_cast<const char*>(S) + (size_t)rb * 16 * ngr * 4;
    zrow = static_cast<const char*>(Z) + (size_t)rb * 16 * ngr;
    qoff = prow * rowq + 16u * q;
    if constexpr (FL) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        foff[h] = (uint32_t)min(8 * h + fr, N - 1 - rb * 16) * rowq + 16u * (uint32_t)(fu & 3);
    }
#pragma unroll
    for (int i = 0; i < kPar; ++i) {
      if (4 * i < ncw) {  // uniform
        const uint32_t g = (uint32_t)min(c0 + 4 * i + q, nch - 1) >> gshift;
        pstep[i] = reinterpret_cast<const float*>(srow)[prow * (uint32_t)ngr + g];
        pzero[i] = reinterpret_cast<const uint8_t*>(zrow)[prow * (uint32_t)ngr + g];
      }
    }
  };
  auto row_store = [&]() {
#pragma unroll
    for (int i = 0; i < kPar; ++i) {
      if (4 * i + q < ncw) {
        p_step[nl * lay.pst + 4 * i + q] = pstep[i];
        p_zero[nl * lay.pst + 4 * i + q] = (uint8_t)pzero[i];
      }
    }
  };
  // slot r <- chunk t; FL: slots r, r + 1 (r even) <- the chunk pair
  // (t, t + 1) of rows 0-7 and 8-15 (a second chunk past the split's last
  // reads the last one again)
  auto load_w = [&](int r, int t) {
    if constexpr (FL) {
      if ((r & 1) == 0) {
        const int c = c0 + min(t + (fu >> 2), ncw - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wr[r + h] = ld_nt(reinterpret_cast<const u32x4*>(qrow + (size_t)c * 64 + foff[h]));
      }
    } else {
      const int c = c0 + min(t, ncw - 1);
      wr[r] = ld_nt(reinterpret_cast<const u32x4*>(qrow + (size_t)c * 64 + qoff));
    }
  };
  auto prologue = [&]() {
#pragma unroll
    for (int r = 0; r < kMbRing; ++r) load_w(r, r);
  };
  row_setup(0);
  prologue();

  // ---- activation operands of chunks [c0, c1) into LDS in MFMA order:
  // wavefront w stages token rows w and w + 8; lane l loads 16-byte pieces
  // l, l + 64, ... of the row's K range (a wavefront's load covers 1 KB of
  // the row), which go to operand (chunk piece / 16, j = l % 4,
  // q = l / 4 % 4, m). Then one chunk of zeros (the A operands of the
  // padding items). The first wait here also waits for the loads issued
  // above, which the first item would wait for anyway.
  {
    constexpr int kPI = (kMbMaxSpl + 3) / 4;  // pieces per lane and row, at most
    const uint32_t lane_op =
        ((uint32_t)((lane >> 4) * 4 + (lane & 3)) * 4u + (uint32_t)((lane >> 2) & 3)) * MP;
    const uint32_t kbytes = (uint32_t)(K - c0 * 128) * 2u;  // bytes from c0 to the row end
#pragma unroll
    for (int h = 0; h < MP / kMbWaves; ++h) {
      const int m = wave + kMbWaves * h;
      const char* xrow = reinterpret_cast<const char*>(X) +
                         ((size_t)min(m, M - 1) * K + (size_t)c0 * 128) * 2;
      u32x4 pv[kPI];
#pragma unroll
      for (int i = 0; i < kPI; ++i) {
        if (4 * i < ncw)  // uniform
          pv[i] = *reinterpret_cast<const u32x4*>(
              xrow + min((uint32_t)(lane + 64 * i) * 16u, kbytes - 16u));
      }
#pragma unroll
      for (int i = 0; i < kPI; ++i) {
        if (4 * i + (lane >> 4) < ncw) {
          const u32x4 d = pv[i];
          a_lds[lane_op + (uint32_t)(i * 64 * MP) + (uint32_t)m] =
              u32x4{plo(d[0], d[2]), phi(d[0], d[2]), plo(d[1], d[3]), phi(d[1], d[3])};
        }
      }
    }
    for (int t = threadIdx.x; t < kChunkOps; t += kThreads) a_lds[nop + t] = u32x4{0u, 0u, 0u, 0u};
  }
  row_store();
  __syncthreads();

  // this lane's A operand of MFMA 0 in chunk 0 (byte offset); MFMA j adds
  // j * 4 MP operands, chunk cc adds cc * kChunkOps
  const uint32_t abase = (uint32_t)(q * MP + (nl & (MP - 1))) * 16u;
  const float* const my_step = p_step + nl * lay.pst;
  const uint8_t* const my_zero = p_zero + nl * lay.pst;

  const UnpackRegs ur = unpack_regs();
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int ri = 0; ri < nrw; ++ri) {
    if (ri > 0) {
      row_setup(ri);
      prologue();
      row_store();
    }
    floatx4 acc = zero4;
    // the previous item's sums and step, added to acc one item late so that
    // the wavefront does not wait for the MFMAs it has just issued
    floatx4 sp = zero4;
    float dp = 0.f;
    // whole rounds of kMbRing items, so that the loop body has no branch;
    // the items past the last chunk (padding) take their A operands from the
    // zero chunk, which makes their sums exactly 0
    const int rounds = (ncw + kMbRing - 1) / kMbRing;
    uint32_t zn = my_zero[0];  // zero point of the next item
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int r = 0; r < kMbRing; ++r) {
        const int t = it * kMbRing + r;
        const uint32_t z = zn;
        zn = my_zero[min(t + 1, ncw - 1)];
        const float d = my_step[min(t, ncw - 1)];
        const h2 ze = hv((0xE400u + z) * 0x00010001u);       // -(1024 + z)
        const h2 zo = hv((0xD400u + 16u * z) * 0x00010001u);  // -(64 + z)
        const u32x4* ap = reinterpret_cast<const u32x4*>(lds + abase + (uint32_t)min(t, ncw) *
                                                                           (kChunkOps * 16u));
        u32x4 wv;
        if constexpr (FL) {
          // the pair through LDS: stored, its slots refilled, and this
          // item's 16 bytes read back in the MFMA layout
          if ((r & 1) == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) p_stage[8 * (8 * h + fr) + (fu ^ fr)] = wr[r + h];
            load_w(r, t + kMbRing);
          }
          wv = p_stage[8 * nl + ((4 * (r & 1) + q) ^ (nl & 7))];
        } else {
          wv = wr[r];
        }
        u32x4 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = wv[j], x8 = x >> 8;
          b[j] = u32x4{
              hbits(hv(and_or(x, ur.lo4, ur.magic)) + ze),
              hbits(__builtin_elementwise_fma(hv(and_or(x, ur.hi4, ur.magic)), sixteenth, zo)),
              hbits(hv(and_or(x8, ur.lo4, ur.magic)) + ze),
              hbits(__builtin_elementwise_fma(hv(and_or(x8, ur.hi4, ur.magic)), sixteenth, zo))};
        }
        // the slot's weights are unpacked: refill it with item t + kMbRing
        // (issued here, item by item: the scheduler would otherwise gather
        // the round's loads at its end, where the next round's first item
        // waits for them at once)
        if constexpr (!FL) load_w(r, t + kMbRing);
        floatx4 s = zero4;
#pragma unroll
        for (int j = 0; j < 4; ++j) s = mfma16(ap[j * 4 * MP], b[j], s);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(dp, sp[e], acc[e]);
        sp = s;
        dp = d;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(dp, sp[e], acc[e]);
    const int rb = gw + ri * GW;
    const int n = rb * 16 + nl;
    if constexpr (!PL) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * q + e;
        if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(acc[e]));
      }
    } else {
      // this split's sums to its plane; the split that finishes the row
      // block last adds the planes in split order and stores Y. The planes
      // are written through to the device-coherent level (agent-scope
      // stores) and the count is raised only once they have landed; the
      // last split reads them at that level (agent-scope loads). No fence:
      // a device-scope fence would write back and invalidate the whole L2.
      const size_t MN = (size_t)M * N;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * q + e;
        if (m < M && n < N)
          __hip_atomic_store(planes + blockIdx.y * MN + (size_t)m * N + n, acc[e],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0);  // the plane stores are complete
      uint32_t old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(counters + rb, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      old = __builtin_amdgcn_readfirstlane(old);
      if (old == gridDim.y - 1) {  // uniform: the last split of this row block
        const uint32_t S = gridDim.y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * q + e;
          const size_t at = (size_t)min(m, M - 1) * N + min(n, N - 1);
          // the planes 8 at a time (loads in flight together), added in
          // split order
          float sum = 0.f;
          for (uint32_t s0 = 0; s0 < S; s0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const uint32_t sp2 = min(s0 + u, S - 1);
              v[u] = __hip_atomic_load(planes + sp2 * MN + at, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const uint32_t sp2 = s0 + u;
              if (sp2 < S) {
                const float x = sp2 == blockIdx.y ? acc[e] : v[u];
                sum = sp2 == 0 ? x : sum + x;
              }
            }
          }
          if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(sum));
        }
        if (lane == 0)  // ready for the next call
          __hip_atomic_store(counters + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

namespace {
int mb_cu_count() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}

// LDS of a workgroup: at most 80 KB, so that two workgroups share a
// compute unit (kMbLdsWide: one workgroup per unit)
constexpr uint32_t kMbLdsMax = 80 * 1024;
constexpr uint32_t kMbLdsWide = 156 * 1024;
// wavefronts the plan aims for per compute unit when it sets the K splits
constexpr int kMbWavesPerCu = 8;
// ... and when it spreads the row blocks over the wavefronts: two
// workgroups per unit once the splits are set (kernel traces, same sums:
// 28672-code rows on 8192 rows at M = 2, 4, 8 40.8 -> 39.7, 41.6 -> 40.3,
// 41.6 -> 40.2 us; 8704-code rows on 28672 rows at M = 8 47.8 -> 45.7 us;
// other long-row shapes unchanged; raising the splits for it instead was
// slower on 11008-code rows, 13.6 -> 16.8 us at M = 4 and 8)
constexpr int kMbRowWavesPerCu = 16;

template <int MP, bool PL, bool FL>
hipError_t mb_allow_lds(size_t lds) {
  static size_t allowed = 64 * 1024;
  if (lds <= allowed) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)gemv_w4_mb_kernel<MP, PL, FL>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) allowed = lds;
  return e;
}
}  // namespace

// The K splits: as few as the LDS allows, raised (with a workspace) until
// the row blocks times the splits give about kMbWavesPerCu wavefronts per
// compute unit, keeping at least two chunks per split; then as many row
// blocks per wavefront as keep kMbRowWavesPerCu wavefronts per unit.
MbPlan mb_plan(int M, int N, int K, bool can_split) {
  MbPlan p{};
  const int mp = M <= 8 ? 8 : 16;
  const int nch = K / 128;
  const int nrb = (N + 15) / 16;
  const int cus = mb_cu_count();
  const int waves = kMbWavesPerCu * cus;
  // chunks per split: what the LDS and the staging registers hold
  auto spl_max_of = [&](bool fl, uint32_t cap) {
    int spl_max = kMbMaxSpl;
    while (spl_max > 1 && mb_lds(spl_max, mp, fl).total > cap) --spl_max;
    return spl_max;
  };
  auto splits_of = [&](bool fl) {
    const int spl_max = spl_max_of(fl, kMbLdsMax);
    int s = (nch + spl_max - 1) / spl_max;
    if (can_split) s = max(s, min((waves + nrb - 1) / nrb, max(1, nch / 2)));
    const int spl = (nch + s - 1) / s;
    return (nch + spl - 1) / spl;
  };
  int s = splits_of(false);
  const int spl = (nch + s - 1) / s;
  s = (nch + spl - 1) / spl;
  // full-line loads when their staging leaves the splits as they are
  const bool fl = splits_of(true) == s && mb_lds(spl, mp, true).total <= kMbLdsMax;
  if (s > 1 && (!can_split || nrb > kSplitMaxRowBlocks)) return p;  // splits == 0: not supported
  const int rbw = max(1, (nrb * s) / (kMbRowWavesPerCu * cus));
  p.mp = mp;
  p.splits = s;
  p.spl = spl;
  p.gx = (nrb + kMbWaves * rbw - 1) / (kMbWaves * rbw);
  p.fl = fl;
  p.lds = mb_lds(spl, mp, fl).total;
  // 16 stored token rows: their activation operands take twice the LDS, so
  // under the two-per-unit limit the splits get shorter and more numerous.
  // When that plan also has more workgroups than units, take one workgroup
  // per unit with up to kMbLdsWide of LDS if it needs at most 3/4 of the
  // splits and still gives 7/8 of the units a workgroup: the split count and
  // row blocks per wavefront with the most workgroups, the fewest splits
  // among equals (rows of 28672 codes on 8192 rows: 8 splits in 256
  // workgroups instead of 14 in 308)
  if (mp == 16 && can_split && s > 1 && p.gx * s > cus) {
    const int wmax = spl_max_of(false, kMbLdsWide);
    int best_w = 0, bs = 0, bspl = 0, bgx = 0;
    for (int s2 = max(2, (nch + wmax - 1) / wmax); 4 * s2 <= 3 * s; ++s2) {
      const int sp2 = (nch + s2 - 1) / s2;
      if ((nch + sp2 - 1) / sp2 != s2) continue;
      for (int r = 1; r <= 16; ++r) {
        const int gx = (nrb + kMbWaves * r - 1) / (kMbWaves * r);
        if (gx * s2 <= cus && gx * s2 > best_w) {
          best_w = gx * s2;
          bs = s2;
          bspl = sp2;
          bgx = gx;
        }
      }
    }
    if (bs > 1 && 8 * best_w >= 7 * cus) {
      p.splits = bs;
      p.spl = bspl;
      p.gx = bgx;
      p.fl = false;
      p.lds = mb_lds(bspl, mp, false).total;
    }
  }
  p.ws_bytes = p.splits > 1 ? kSplitCtrBytes + (size_t)p.splits * M * N * 4 : 0;
  return p;
}

// Timed with kernel traces against gemv_w4_mx_kernel (8 and 16 token rows,
// weights in HBM): on rows of 11008 codes (86 chunks, two passes of that
// kernel) this one takes 14.5 us against 19.5 (4096 rows, M = 4 and 8); on
// rows of up to 8192 codes that kernel stays ahead (4096 x 4096 M = 8:
// 10.7 against 8.1 us; 28672 x 8192 M = 8: 57 against 36 us), as this one's
// 16-row loads fetch 64 bytes per row per instruction and its K splits pay
// for the planes.
bool mb_preferred(int M, int N, int K) {
  (void)N;
  return M >= 2 && M <= 16 && K > 64 * 128;
}

hipError_t launch_gemv_w4_mb(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int M, int N, int K, int group, __half* Y,
                             hipStream_t st, bool cs, void* ws, size_t ws_bytes) {
  // 16 rows of K / 2 bytes each must have 32-bit offsets
  if (cs || M < 2 || M > 16 || K > (1 << 27)) return hipErrorNotSupported;
  const MbPlan p = mb_plan(M, N, K, ws != nullptr);
  if (p.splits == 0) return hipErrorNotSupported;
  if (p.splits > 1 && ws_bytes < p.ws_bytes) return hipErrorInvalidValue;
  const int gshift = group_shift(group);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  uint32_t* ctr = p.splits > 1 ? static_cast<uint32_t*>(ws) : nullptr;
  float* pl = p.splits > 1
                  ? reinterpret_cast<float*>(static_cast<char*>(ws) + kSplitCtrBytes)
                  : nullptr;
  const dim3 grid((unsigned)p.gx, (unsigned)p.splits), block(64 * kMbWaves);
#define AWQ_MB(MPV, PLV, FLV)                                                                  \
  do {                                                                                          \
    const hipError_t ea = mb_allow_lds<MPV, PLV, FLV>(p.lds);                                   \
    if (ea != hipSuccess) return ea;                                                            \
    hipLaunchKernelGGL((gemv_w4_mb_kernel<MPV, PLV, FLV>), grid, block, p.lds, st, x, q, scales, \
                       zeros, y, pl, ctr, M, N, K, gshift, p.spl);                              \
  } while (0)
#define AWQ_MB2(MPV, PLV)                   \
  do {                                      \
    if (p.fl) AWQ_MB(MPV, PLV, true);       \
    else AWQ_MB(MPV, PLV, false);           \
  } while (0)
  if (p.mp == 8) {
    if (pl) AWQ_MB2(8, true);
    else AWQ_MB2(8, false);
  } else {
    if (pl) AWQ_MB2(16, true);
    else AWQ_MB2(16, false);
  }
#undef AWQ_MB2
#undef AWQ_MB
  return hipGetLastError();
}

}  // namespace awq
