// Prefill / batched W4A16 (and W3A16) product on the fp16 matrix cores, and
// the fp16 "A * B^T" contraction the scale search uses.
//
// A workgroup of WGM x WGN wavefronts computes a BM x BN tile of Y = A B^T,
// A = X' [M, K] fp16, B = dequant(Q) [N, K]; each wavefront computes a
// (BM/WGM) x (BN/WGN) sub-tile with v_mfma_f32_32x32x16_f16. The K loop is
// software pipelined over two LDS buffers with one barrier per step: while
// the matrix cores work on step k from one buffer, two register stages hold
// steps k+1 and k+2 (loads in flight); after the MFMAs, step k+1 is
// dequantized into the other buffer and the loads for step k+3 are issued.
//
// K steps: 64 codes (half a group) for int4 and fp16 B, one whole 128-code
// group for int3 (an int3 group is 13 words; 64 codes would split a word).
// B tiles are dequantized to fp16 (q - z) * fp16(delta * 2^e_n). For int4 a
// group spans two steps: the scale and zero point are loaded with the even
// step only and reused for the odd one.
//
// Row exponent e_n. Before its K loop a workgroup finds, for each weight row
// n of its tile, the largest step of the row and picks the power of two that
// puts it in [2^10, 2^11); the epilogue multiplies the row's float32 sums by
// 2^-e_n. Multiplying by a power of two is exact in fp16 and float32 while
// the values stay in the normal range, so a row whose steps are ordinary
// gives the same bits as without it. A row whose steps lie below fp16's
// normal range (delta < 2^-14: small weights, or channels with a small
// activation statistic at large alpha) would otherwise be rounded to fp16
// subnormals (several percent off, or zero); with the exponent every group
// within 2^-24 of the row's largest step keeps fp16's full precision, and
// dequantized values stay below 15 * 2^11 < 65504.
//
// Code order in LDS. The packed words are unpacked with the fp16 magic-number
// trick, which yields codes in pairs that are not adjacent in k. For int4 the
// activation tile is stored with the same permutation of k (the contraction
// is a sum over k, so any common order is exact):
//   int4, per 8-code word:  c0 c4 c2 c6 c1 c5 c3 c7
// For int3 the five pairs of a word are put back in natural order with
// v_perm_b32, so the activation tile is a plain copy; an int3 group is 13
// words = 130 slots, of which the last 2 hold no code (their activation slots
// are zero), and slots 130..143 pad the step to 9 x 16. fp16 B tiles (the
// search's error terms) keep natural order.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));  // dword-aligned 16 B

__device__ __forceinline__ floatx16 mfma32(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// low halves of a and b -> (a.lo, b.lo); high halves -> (a.hi, b.hi)
__device__ __forceinline__ uint32_t plo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t phi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
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
__device__ __forceinline__ uint32_t hbits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 hv(uint32_t v) { return __builtin_bit_cast(h2, v); }

template <int BMODE, int BM, int BN, int NT>
struct Cfg {
  static constexpr int BK = BMODE == 3 ? 128 : 64;     // codes per step
  static constexpr int SLOTS = BMODE == 3 ? 144 : 64;  // LDS k slots per step
  static constexpr int STR = SLOTS + 8;                // LDS row stride (halves)
  static constexpr int ACH = BM * BK / 8 / NT;         // 16-byte A chunks per thread
  static constexpr int BCH = BN * BK / 8 / NT;         // 16-byte fp16 B chunks per thread
  static constexpr int BW = BN * 8 / NT;               // int4 B words per thread
  static constexpr int BIT = BN * 4 / NT;              // int3 B (row, quarter) items per thread
  // every thread loads whole items of both operands
  static_assert(BM * BK % (8 * NT) == 0 && ACH >= 1, "A chunks per thread");
  static_assert(BMODE != 0 || (BN * BK % (8 * NT) == 0 && BCH >= 1), "fp16 B chunks per thread");
  static_assert(BMODE != 4 || (BN * 8 % NT == 0 && BW >= 1), "int4 B words per thread");
  static_assert(BMODE != 3 || (BN * 4 % NT == 0 && BIT >= 1), "int3 B items per thread");
};

// register staging of one K step
template <int BMODE, int BM, int BN, int NT>
struct Stage;
template <int BM, int BN, int NT>
struct Stage<0, BM, BN, NT> {
  u32x4 a[Cfg<0, BM, BN, NT>::ACH], b[Cfg<0, BM, BN, NT>::BCH];
};
template <int BM, int BN, int NT>
struct Stage<4, BM, BN, NT> {
  u32x4 a[Cfg<4, BM, BN, NT>::ACH];
  uint32_t b[Cfg<4, BM, BN, NT>::BW];
  float d;           // scale of the step's group (even steps only)
  uint32_t zw, zsh;  // zero point = (zw >> zsh) & 0xff (even steps only)
};
template <int BM, int BN, int NT>
struct Stage<3, BM, BN, NT> {
  u32x4 a[Cfg<3, BM, BN, NT>::ACH];
  u32x4 b[Cfg<3, BM, BN, NT>::BIT];  // 4 words of a group from word {0,4,7,9}[quarter]
  float d[Cfg<3, BM, BN, NT>::BIT];
  uint32_t zw[Cfg<3, BM, BN, NT>::BIT], zsh[Cfg<3, BM, BN, NT>::BIT];
};

// first word loaded by quarter qt of an int3 group: 0, 4, 7, 9 (a shift and a
// mask; the nested ternary became branches)
__device__ __forceinline__ int int3_quarter_word(int qt) { return (0x09070400 >> (8 * qt)) & 0xff; }

// f(integral_constant<int, i>) for i = I .. N-1, in order
template <int I, int N, typename F>
__device__ __forceinline__ void unroll_c(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    unroll_c<I + 1, N>(f);
  }
}

// int4 dequantization constants of one (row, group): fp16 delta and the
// offsets -(1024 + z), -(64 + z) that turn magic-number halves into c - z
struct Dq {
  h2 dh, ze, zo;
};

}  // namespace

// EPI: 0 stores Y = fp16(A B^T); 1 writes the float64 square sum of the
// tile (the search); 2 is the gated-MLP form: B holds two weight matrices
// (gate from Bsrc/S/Z, up from B2/S2/Z2) and the tile's B rows alternate
// between them in blocks of 32 (tile row r reads row
// n0 + 32 (r / 64) + r % 32 of matrix (r / 32) % 2), so every wavefront holds
// the gate and up sums of the same outputs in neighbouring accumulators and
// stores fp16(silu(g) u), silu(g) = g / (1 + e^-g), in fp32. A tile then
// covers BN / 2 outputs.
//
// CS: compact group parameters (fp16 steps, 4-bit zero points 8 per word).
// ZW (plain storage): zero points are read as the aligned 32-bit word
// holding them (the zero-point array is a whole number of words); otherwise
// byte by byte.
// Word loads keep the loop-carried value 32 bits wide, so no byte
// extension is scheduled ahead of the MFMAs (it would wait on the newest
// loads).
template <int BMODE, int EPI, int BM, int BN, int WGM, int WGN, bool ZW, int NST, bool CS = false,
          bool SK = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(
    const uint16_t* __restrict__ A, const void* __restrict__ Bsrc, const void* __restrict__ S,
    const void* __restrict__ Z, int M, int N, int K, int wpr, int gshift,
    uint16_t* __restrict__ Y, double* __restrict__ partial, int hilo,
    const void* __restrict__ B2, const void* __restrict__ S2, const void* __restrict__ Z2,
    int nbase, int nend, float* __restrict__ ws, int spl) {
  constexpr int NT = 64 * WGM * WGN;
  static_assert(NST == 2 || NST == 4 || NST == 8, "register stages");
  using C = Cfg<BMODE, BM, BN, NT>;
  using St = Stage<BMODE, BM, BN, NT>;
  constexpr int STR = C::STR;
  constexpr int BK = C::BK;
  constexpr int TM = BM / WGM / 32, TN = BN / WGN / 32;  // 32x32 tiles per wavefront
  static_assert(TM >= 1 && TN >= 1 && BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "tile");
  static_assert(EPI != 2 || (TN % 2 == 0 && BMODE != 0), "gate/up pairs need an even TN");
  constexpr int BNO = EPI == 2 ? BN / 2 : BN;  // outputs per tile along N
  __shared__ __align__(16) uint16_t lds_a[2][BM * STR];
  __shared__ __align__(16) uint16_t lds_b[2][BN * STR];
  // per tile row of B: 2^-e_n (epilogue)
  __shared__ float row_post[BMODE != 0 ? BN : 1];
  // e_n of this thread's B row
  int rexp[1];
  // fp16 step delta * 2^e of a row: exact (a power-of-two product) unless it
  // leaves fp16's range; compact storage holds delta in fp16 already, and
  // v_ldexp_f16 scales it without a round trip through float32
  auto row_step = [](float d, int e) -> _Float16 {
    if constexpr (CS)
      return __builtin_amdgcn_ldexph((_Float16)d, e);
    else
      return (_Float16)__builtin_ldexpf(d, e);
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const UnpackRegs ur = unpack_regs();  // masks and magic number, loop-invariant
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // tile order: when the tile count splits evenly over the 8 XCDs, give each
  // XCD a contiguous run of tiles that walk M for a fixed N tile, so the
  // weight tile is reused from that XCD's L2
  const int mt = (M + BM - 1) / BM;
  // this launch covers outputs [nbase, nend) of the N (Y's row stride)
  const int ntl = (nend - nbase + BNO - 1) / BNO;
  const int total = mt * ntl;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
  const int m0 = (t % mt) * BM;
  const int n0 = nbase + (t / mt) * BNO;
  // fp16 B with hilo set holds each term as a hi and a lo fp16 part,
  // [N][2K]: 256-wide block c = (hi of k 128c..128c+127 | lo of the same k),
  // so a 64-wide step s reads activations 128*(s/4) + 64*(s%2)
  // split K (EPI 0, gridDim.y > 1): this workgroup takes steps
  // [kofs, kofs + nsteps) of its tile; partial tiles meet in the workspace
  const int nsteps_all = BMODE == 0 && hilo ? 2 * (K / BK) : K / BK;
  static_assert(!SK || EPI == 0, "split K stores plain products");
  const int nsplit = SK ? (int)gridDim.y : 1;
  const int kofs = nsplit > 1 ? (int)blockIdx.y * spl : 0;
  const int nsteps = nsplit > 1 ? min(spl, nsteps_all - kofs) : nsteps_all;
  const int ng = max(1, K >> (7 + gshift));  // quantization groups per row

  if (BMODE == 3) {
    // zero the slots 128..143 of every row of both buffers once: activation
    // slots 128..143 and weight slots 130..143 are never written again
    // (weight slots 128, 129 take the finite phantom codes of word 12)
    for (int i = tid; i < 2 * (BM + BN) * 16; i += NT) {
      const int buf = i / ((BM + BN) * 16);
      const int rr = (i / 16) % (BM + BN), c = i % 16;
      if (rr < BM)
        lds_a[buf][rr * STR + 128 + c] = 0;
      else
        lds_b[buf][(rr - BM) * STR + 128 + c] = 0;
    }
  }

  // output row of tile B row r, and whether it belongs to the second matrix
  auto brow_n = [&](int r) {
    return EPI == 2 ? min(n0 + 32 * (r >> 6) + (r & 31), N - 1) : min(n0 + r, N - 1);
  };
  auto bsel = [&](int r) { return EPI == 2 && ((r >> 5) & 1) != 0; };
  // zero point of row n, group g = (zw >> zsh) & ZMASK
  constexpr uint32_t ZMASK = CS ? 15u : 255u;
  auto load_zero = [&](const void* Zp, size_t n, int g, uint32_t& zw, uint32_t& zsh) {
    if constexpr (CS) {
      zw = static_cast<const uint32_t*>(Zp)[n * ((ng + 7) >> 3) + (g >> 3)];
      zsh = 4u * (uint32_t)(g & 7);
    } else if constexpr (ZW) {
      const size_t idx = n * ng + g;
      zw = static_cast<const uint32_t*>(Zp)[idx >> 2];
      zsh = 8u * (uint32_t)(idx & 3);
    } else {
      zw = static_cast<const uint8_t*>(Zp)[n * ng + g];
      zsh = 0u;
    }
  };
  // load step ks into st; for int4, SZ says whether this (even) step also
  // loads its group's scale and zero point
  auto load_step = [&](St& st, int ks, auto SZ) {
    ks += kofs;
    {
      const int ka = BMODE == 0 && hilo ? 128 * (ks >> 2) + 64 * (ks & 1) : BK * ks;
#pragma unroll
      for (int i = 0; i < C::ACH; ++i) {
        const int id = tid + NT * i;
        const int r = id / (BK / 8), c8 = id % (BK / 8);
        // rows past M read row M - 1: they only feed outputs never stored
        const int m = min(m0 + r, M - 1);
        st.a[i] = *reinterpret_cast<const u32x4*>(A + (size_t)m * K + ka + 8 * c8);
      }
    }
    if constexpr (BMODE == 0) {
      const uint16_t* B = static_cast<const uint16_t*>(Bsrc);
#pragma unroll
      for (int i = 0; i < C::BCH; ++i) {
        const int id = tid + NT * i;
        const int r = id / (BK / 8), c8 = id % (BK / 8);
        const int n = min(n0 + r, N - 1);
        st.b[i] = *reinterpret_cast<const u32x4*>(B + (size_t)n * (hilo ? 2 * K : K) + BK * ks +
                                                  8 * c8);
      }
    } else if constexpr (BMODE == 4) {
      // BW consecutive words of one row (8 words = 64 codes per row and step)
      const int r = (tid * C::BW) / 8, w0 = (tid * C::BW) % 8;
      const bool sel = bsel(r);
      const uint32_t* Q = static_cast<const uint32_t*>(sel ? B2 : Bsrc);
      const int n = brow_n(r);
      const uint32_t* p = Q + (size_t)n * wpr + 8 * ks + w0;
      if constexpr (SZ.value) {
        const int g = (ks * BK) >> (7 + gshift);
        st.d = group_scale<CS>(sel ? S2 : S, (size_t)n, ng, g);
        load_zero(sel ? Z2 : Z, (size_t)n, g, st.zw, st.zsh);
      }
      if constexpr (C::BW == 4) {
        const u32x4 v = ld_nt(reinterpret_cast<const u32x4*>(p));
        st.b[0] = v[0];
        st.b[1] = v[1];
        st.b[2] = v[2];
        st.b[3] = v[3];
      } else if constexpr (C::BW == 2) {
        const uint64_t v = ld_nt(reinterpret_cast<const uint64_t*>(p));
        st.b[0] = (uint32_t)v;
        st.b[1] = (uint32_t)(v >> 32);
      } else {
#pragma unroll
        for (int q = 0; q < C::BW; ++q) st.b[q] = ld_nt(p + q);
      }
    } else {  // int3: item = (row, quarter); quarters cover words 0-3, 4-6, 7-9, 10-12
#pragma unroll
      for (int i = 0; i < C::BIT; ++i) {
        const int id = tid + NT * i;
        const int r = id >> 2, qt = id & 3;
        const bool sel = bsel(r);
        const uint32_t* Q = static_cast<const uint32_t*>(sel ? B2 : Bsrc);
        const int n = brow_n(r);
        // dword-aligned 16-byte load that stays inside the group: quarter 3
        // reads words 9..12 and uses the last three
        const int w0 = int3_quarter_word(qt);
        const u32x4a4 v =
            ld_nt(reinterpret_cast<const u32x4a4*>(Q + (size_t)n * wpr + ks * 13 + w0));
        st.b[i] = u32x4{v[0], v[1], v[2], v[3]};
        st.d[i] = group_scale<CS>(sel ? S2 : S, (size_t)n, ng, ks >> gshift);
        load_zero(sel ? Z2 : Z, (size_t)n, ks >> gshift, st.zw[i], st.zsh[i]);
      }
    }
  };

  // dequantize / permute one register stage into LDS buffer buf, item by
  // item, so the work can be spread between the MFMAs of the current step
  constexpr int NA = C::ACH;                                               // A items
  constexpr int NB = BMODE == 3 ? C::BIT : (BMODE == 4 ? C::BW : C::BCH);  // B items
  Dq dq;  // int4: constants of the group of the last even step stored
  auto set_dq = [&](const St& st) {
    if constexpr (BMODE == 4) {
      const uint32_t z = (st.zw >> st.zsh) & ZMASK;
      const _Float16 dh = row_step(st.d, rexp[0]);
      dq.dh = h2{dh, dh};
      dq.ze = hv((0xE400u + z) * 0x00010001u);       // -(1024 + z)
      dq.zo = hv((0xD400u + 16u * z) * 0x00010001u);  // -(64 + z)
    }
  };
  auto store_a = [&](const St& st, int buf, int i) {
    uint16_t* la = lds_a[buf];
    if constexpr (BMODE == 0) {
      const int id = tid + NT * i;
      const int r = id / (BK / 8), c8 = id % (BK / 8);
      *reinterpret_cast<u32x4*>(&la[r * STR + 8 * c8]) = st.a[i];
    } else if constexpr (BMODE == 4) {
      const int id = tid + NT * i;
      const int r = id / (BK / 8), c8 = id % (BK / 8);
      const u32x4 d = st.a[i];
      const u32x4 p = {plo(d[0], d[2]), plo(d[1], d[3]), phi(d[0], d[2]), phi(d[1], d[3])};
      *reinterpret_cast<u32x4*>(&la[r * STR + 8 * c8]) = p;
    } else {  // int3: natural order, a plain copy
      const int id = tid + NT * i;
      const int r = id / (BK / 8), c8 = id % (BK / 8);
      *reinterpret_cast<u32x4*>(&la[r * STR + 8 * c8]) = st.a[i];
    }
  };
  auto store_b = [&](const St& st, int buf, int i) {
    uint16_t* lb = lds_b[buf];
    if constexpr (BMODE == 0) {
      const int id = tid + NT * i;
      const int r = id / (BK / 8), c8 = id % (BK / 8);
      *reinterpret_cast<u32x4*>(&lb[r * STR + 8 * c8]) = st.b[i];
    } else if constexpr (BMODE == 4) {
      const int r = (tid * C::BW) / 8, w0 = (tid * C::BW) % 8;
      const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
      const uint32_t w = st.b[i];
      const uint32_t w8 = w >> 8;
      const h2 e0 = (hv(and_or(w, ur.lo4, ur.magic)) + dq.ze) * dq.dh;
      const h2 e1 = (hv(and_or(w8, ur.lo4, ur.magic)) + dq.ze) * dq.dh;
      const h2 o0 =
          __builtin_elementwise_fma(hv(and_or(w, ur.hi4, ur.magic)), sixteenth, dq.zo) * dq.dh;
      const h2 o1 =
          __builtin_elementwise_fma(hv(and_or(w8, ur.hi4, ur.magic)), sixteenth, dq.zo) * dq.dh;
      *reinterpret_cast<u32x4*>(&lb[r * STR + 8 * (w0 + i)]) =
          u32x4{hbits(e0), hbits(e1), hbits(o0), hbits(o1)};
    } else {
      // codes: magic pairs with per-half power-of-two weights, made exact
      // integers c - z by one packed fma each, then scaled by delta
      const h2 mul[5] = {{(_Float16)1.f, (_Float16)0.25f},
                         {(_Float16)0.125f, (_Float16)0.03125f},
                         {(_Float16)0.5f, (_Float16)1.f},
                         {(_Float16)0.0625f, (_Float16)0.125f},
                         {(_Float16)0.0078125f, (_Float16)1.f}};
      // magic offsets of the five pairs, as 1024 - offset (fp16, exact)
      const float offl[5] = {1024.f, 128.f, 512.f, 64.f, 8.f};
      const float offh[5] = {256.f, 32.f, 1024.f, 128.f, 1024.f};
      const int id = tid + NT * i;
      const int r = id >> 2, qt = id & 3;
      const int w0 = int3_quarter_word(qt);
      const uint32_t z = (st.zw[i] >> st.zsh[i]) & ZMASK;
      const _Float16 d16 = row_step(st.d[i], rexp[0]);
      const h2 dh = {d16, d16};
      // -(offset + z) per half: -(1024 + z) from the fp16 bit pattern, plus
      // 1024 - offset, in packed fp16 (every value an integer below 2048,
      // so exact: the same bits as the float32 sums rounded to fp16)
      const h2 mz = hv((0xE400u + z) * 0x00010001u);
      h2 add[5];
#pragma unroll
      for (int p = 0; p < 5; ++p)
        add[p] = mz + h2{(_Float16)(1024.f - offl[p]), (_Float16)(1024.f - offh[p])};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // quarters load words 0-3, 4-7, 7-10 and 9-12 and store all four:
        // words 7, 9 and 10 are stored by two lanes of the same row with the
        // same values (same word, same step and zero point), so no lane
        // needs a branch around its stores (one kept the MFMAs of the step
        // from interleaving with this work)
        const uint32_t w = st.b[i][u];
        const uint32_t t8 = w >> 8, u1 = w << 1;
        const uint32_t raw[5] = {and_or(w, ur.m3[0], ur.magic), and_or(w, ur.m3[1], ur.magic),
                                 and_or(t8, ur.m3[2], ur.magic), and_or(t8, ur.m3[3], ur.magic),
                                 and_or(u1, ur.m3[4], ur.magic)};
        uint32_t pr[5];  // (c0,c6) (c1,c7) (c3,c8) (c4,c9) (c2,c5) as c - z times delta
#pragma unroll
        for (int p = 0; p < 5; ++p)
          pr[p] = hbits(__builtin_elementwise_fma(hv(raw[p]), mul[p], add[p]) * dh);
        uint32_t* pb = reinterpret_cast<uint32_t*>(&lb[r * STR + 10 * (w0 + u)]);
        pb[0] = plo(pr[0], pr[1]);                             // (c0, c1)
        pb[1] = plo(pr[4], pr[2]);                             // (c2, c3)
        pb[2] = __builtin_amdgcn_perm(pr[4], pr[3], 0x07060100u);  // (c4, c5)
        pb[3] = phi(pr[0], pr[1]);                             // (c6, c7)
        pb[4] = phi(pr[2], pr[3]);                             // (c8, c9)
      }
    }
  };
  auto store_all = [&](const St& st, int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) store_a(st, buf, i);
#pragma unroll
    for (int i = 0; i < NB; ++i) store_b(st, buf, i);
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int lr = lane & 31;
  const int lk = (lane >> 5) * 8;
  const int arow = (BM / WGM) * wm + lr;
  const int brow = (BN / WGN) * wn + lr;

  // operand fragments of sub-step kk, and the MFMAs of one sub-step
  auto frags = [&](const uint16_t* la, const uint16_t* lb, int kk, u32x4* fa, u32x4* fb) {
    const int ko = kk * 16 + lk;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[i] = *reinterpret_cast<const u32x4*>(&la[(arow + 32 * i) * STR + ko]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = *reinterpret_cast<const u32x4*>(&lb[(brow + 32 * j) * STR + ko]);
  };
  auto mfmas = [&](const u32x4* fa, const u32x4* fb) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
  };
  constexpr int NKS = C::SLOTS / 16;
  // one pipeline step: MFMAs on buffer cur, with the stores of stage sst
  // into the other buffer spread over the sub-steps, then the loads of
  // stage lst. The fragments of sub-step kk + 1 are read from LDS before
  // the MFMAs of sub-step kk, so their latency overlaps those MFMAs (two
  // sub-steps ahead measured the same).
  constexpr int PFD = 1;
  auto step = [&](int cur, const St& sst, St& lst, int lks, auto SZ) {
    if constexpr (SZ.value) set_dq(sst);
    const uint16_t* la = lds_a[cur];
    const uint16_t* lb = lds_b[cur];
    u32x4 fa[PFD + 1][TM], fb[PFD + 1][TN];
    unroll_c<0, (PFD < NKS ? PFD : NKS)>([&](auto I) {
      constexpr int i = decltype(I)::value;
      frags(la, lb, i, fa[i], fb[i]);
    });
    unroll_c<0, NKS>([&](auto KK) {
      constexpr int kk = decltype(KK)::value;
      constexpr int nb = (kk + PFD) % (PFD + 1);
      if constexpr (kk + PFD < NKS) frags(la, lb, kk + PFD, fa[nb], fb[nb]);
      mfmas(fa[kk % (PFD + 1)], fb[kk % (PFD + 1)]);
      if constexpr (kk < NKS - 1) {
        if constexpr (kk < NA) store_a(sst, cur ^ 1, kk);
        if constexpr (kk < NB) store_b(sst, cur ^ 1, kk);
      } else {
        unroll_c<kk, NA>([&](auto I) { store_a(sst, cur ^ 1, decltype(I)::value); });
        unroll_c<kk, NB>([&](auto I) { store_b(sst, cur ^ 1, decltype(I)::value); });
      }
    });
    load_step(lst, lks, SZ);
    __syncthreads();
    // keep the next step's dequantization below the barrier: hoisted above
    // it, it would wait for loads issued just before
    __builtin_amdgcn_sched_barrier(0);
  };

  // NST register stages in flight: stage i carries the steps i (mod NST).
  // While step t is computed from LDS, the stages hold steps t+1 .. t+NST;
  // during the MFMAs step t+1 is stored to the other LDS buffer and its
  // stage reloaded with step t+1+NST. With NST even, a stage's steps are all
  // even or all odd (int4: even stages carry the group's scale and zero
  // point). Loads past the last step re-read the last step (branch-free; the
  // extra stores land in the buffer no later step reads).
  St stg[NST];
  const int last = nsteps - 1;
  auto prime = [&](auto I) {
    constexpr int i = decltype(I)::value;
    load_step(stg[i], min(i, last), std::integral_constant<bool, BMODE == 4 && i % 2 == 0>{});
  };
  if constexpr (BMODE == 0) {
    unroll_c<0, NST>(prime);
  } else {
    // Row exponents. The TPR threads of tile row r (adjacent lanes) take the
    // largest step of the groups this workgroup's K range touches (a split's
    // own range: its partial sums are stored unscaled, so splits need not
    // agree on e). They are also the threads that dequantize row r, so each
    // keeps e in a register; only the epilogue's 2^-e goes through LDS (read
    // after the K loop's barriers). The first eight 16-byte scale loads go
    // out before the stages' loads, so waiting for them does not wait for
    // the stages (loads return in order).
    constexpr int TPR = NT / BN;
    static_assert(NT % BN == 0 && (TPR & (TPR - 1)) == 0 && TPR <= 64, "threads per tile row");
    static_assert(BMODE != 3 || C::BIT == 1, "int3: one B item (row) per thread");
    static_assert(BMODE != 4 || TPR <= 8, "int4: a thread's B words lie in row tid / TPR");
    const int r = tid / TPR, sub = tid % TPR;
    const size_t n = (size_t)brow_n(r);
    const void* Sp = bsel(r) ? S2 : S;
    const int glo = (kofs * BK) >> (7 + gshift);
    const int ghi = min(ng, ((((kofs + nsteps) * BK) - 1) >> (7 + gshift)) + 1);
    const int len = ghi - glo;
    float dmax = 0.f;
    if constexpr (!CS) {
      // float32 steps, four per 16-byte load; chunks past the range re-read
      // its last four steps (harmless for a max)
      const float* srow = static_cast<const float*>(Sp) + n * ng;
      const int nchunk = (len + 3) >> 2;
      auto chunk = [&](int c) {
        return *reinterpret_cast<const u32x4a4*>(srow + min(glo + 4 * c, ghi - 4));
      };
      u32x4a4 v[8];
      if (len >= 4) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = chunk(sub + TPR * u);
      }
      unroll_c<0, NST>(prime);
      if (len >= 4) {
        for (int c0 = 0;;) {
          // (through a float vector: __builtin_bit_cast of one element of an
          // integer vector reads element 0 in this compiler)
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const floatx4 f = __builtin_bit_cast(floatx4, v[u]);
            dmax = fmaxf(dmax, fmaxf(fmaxf(f[0], f[1]), fmaxf(f[2], f[3])));
          }
          c0 += 8 * TPR;
          if (c0 >= nchunk) break;
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = chunk(c0 + sub + TPR * u);
        }
      } else {
        for (int g = glo + sub; g < ghi; g += TPR) dmax = fmaxf(dmax, srow[g]);
      }
    } else {  // fp16 steps: 16 scalar loads in flight
      unroll_c<0, NST>(prime);
      for (int g0 = glo + 16 * sub; g0 < ghi; g0 += 16 * TPR) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = group_scale<CS>(Sp, n, ng, min(g0 + u, ghi - 1));
#pragma unroll
        for (int u = 0; u < 16; ++u) dmax = fmaxf(dmax, v[u]);
      }
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) dmax = fmaxf(dmax, __shfl_xor(dmax, off));
    // dmax = f 2^x with f in [1/2, 1): e = 11 - x; a zero or non-finite
    // maximum (nothing to scale) keeps e = 0
    int e = 0;
    if (dmax > 0.f && dmax <= 3.4e38f) e = 11 - __builtin_amdgcn_frexp_expf(dmax);
    e = max(-126, min(126, e));
    if (sub == 0) row_post[r] = __builtin_ldexpf(1.0f, -e);
    rexp[0] = e;  // int4: this thread's B row is (tid BW) / 8 = r; int3: (tid >> 2) = r
  }
  set_dq(stg[0]);
  store_all(stg[0], 0);
  load_step(stg[0], min(NST, last), std::integral_constant<bool, BMODE == 4>{});
  __syncthreads();
  // sub-step u of a group of NST steps starting at ks (a multiple of NST)
  auto sub = [&](int ks, auto U) {
    constexpr int u = decltype(U)::value;
    constexpr int si = (u + 1) % NST;
    step(u & 1, stg[si], stg[si], min(ks + u + 1 + NST, last),
         std::integral_constant<bool, BMODE == 4 && si % 2 == 0>{});
  };
  // full groups: no branch inside the loop body, so the compiler keeps the
  // in-flight loads counted exactly across the back edge
  int ks = 0;
  for (; ks + NST <= nsteps; ks += NST) unroll_c<0, NST>([&](auto U) { sub(ks, U); });
  // the last nsteps % NST steps (uniform branches)
  unroll_c<0, NST - 1>([&](auto U) {
    if (ks + decltype(U)::value < nsteps) sub(ks, U);
  });

  // D layout of the 32x32 MFMA: lane l holds column l % 32, rows
  // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15
  if constexpr (EPI == 0) {
    if (SK && nsplit > 1) {
      // Split K: this split's float32 products go to plane blockIdx.y of the
      // workspace ([split][M][N]), and the split that finishes the tile last
      // (the tile's counter at the workspace's head says which) adds the
      // planes in split order and stores Y. The planes are written through
      // to the device-coherent level (agent-scope stores), the count is
      // raised once every wavefront's stores have landed, and the last split
      // reads them at that level. No fence: a device-scope fence writes back
      // and invalidates the whole L2.
      const size_t MN = (size_t)M * N;
      float* plane = ws + (size_t)blockIdx.y * MN;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + (BN / WGN) * wn + 32 * j + lr;
          const float post = BMODE != 0 ? row_post[(BN / WGN) * wn + 32 * j + lr] : 1.0f;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int m =
                m0 + (BM / WGM) * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (m < M && n < nend) {
              __hip_atomic_store(plane + (size_t)m * N + n, acc[i][j][v] * post,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      {
        __builtin_amdgcn_s_waitcnt(0);  // this wavefront's plane stores are complete
        __syncthreads();                // and every wavefront's
        __shared__ uint32_t last_split;
        if (tid == 0) {
          uint32_t* ctr =
              reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) - kSplitCtrBytes) + t;
          const uint32_t old =
              __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last_split = old == (uint32_t)(nsplit - 1) ? 1u : 0u;
          // every split has counted: ready for the next call
          if (last_split) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (last_split == 0u) return;
        // the tile's outputs in a coalesced layout (thread -> column
        // tid % BN, rows RS apart; the row offset is the same for a whole
        // wavefront, so the addresses are a scalar base plus the column),
        // CH rows at a time, each split's loads in flight together, added
        // in split order; this split's own plane is read back like the others
        constexpr int NT = 64 * WGM * WGN;
        static_assert(BN % 64 == 0 && NT % BN == 0, "whole wavefronts per row");
        constexpr int RS = NT / BN;
        constexpr int RPT = BM / RS;
        constexpr int CH = RPT < 32 ? RPT : 32;
        const int rw = __builtin_amdgcn_readfirstlane(tid / BN);
        const int c = tid % BN;
        const unsigned cc = (unsigned)min(c, nend - 1 - n0);  // in the row
        for (int k0 = 0; k0 < RPT; k0 += CH) {
          float sum[CH];
          for (int sp = 0; sp < nsplit; ++sp) {
            float x[CH];
#pragma unroll
            for (int k = 0; k < CH; ++k) {
              const int m = min(m0 + rw + RS * (k0 + k), M - 1);
              const float* base = ws + (size_t)sp * MN + (size_t)m * N + n0;
              x[k] = __hip_atomic_load(base + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int k = 0; k < CH; ++k) sum[k] = sp == 0 ? x[k] : sum[k] + x[k];
          }
          if (n0 + c < nend) {
#pragma unroll
            for (int k = 0; k < CH; ++k) {
              const int m = m0 + rw + RS * (k0 + k);
              if (m < M) Y[(size_t)m * N + n0 + c] = __half_as_ushort(__float2half_rn(sum[k]));
            }
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + (BN / WGN) * wn + 32 * j + lr;
        const float post = BMODE != 0 ? row_post[(BN / WGN) * wn + 32 * j + lr] : 1.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m =
              m0 + (BM / WGM) * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (m < M && n < nend)
            Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(acc[i][j][v] * post));
        }
      }
  } else if constexpr (EPI == 2) {
    // accumulator pair (j, j + 1) = (gate, up) of outputs n
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const int n = n0 + (BNO / WGN) * wn + 32 * (j >> 1) + lr;
        const float pg = row_post[(BN / WGN) * wn + 32 * j + lr];
        const float pu = row_post[(BN / WGN) * wn + 32 * (j + 1) + lr];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m =
              m0 + (BM / WGM) * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const float g = acc[i][j][v] * pg;
          const float val = g / (1.0f + __expf(-g)) * (acc[i][j + 1][v] * pu);
          if (m < M && n < nend) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(val));
        }
      }
  } else {
    __shared__ double wsum[WGM * WGN];
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + (BN / WGN) * wn + 32 * j + lr;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m =
              m0 + (BM / WGM) * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const float e = acc[i][j][v];
          if (m < M && n < nend) sq = __builtin_fmaf(e, e, sq);
        }
      }
    double ds = (double)sq;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ds += __shfl_xor(ds, off);
    if (lane == 0) wsum[wave] = ds;
    __syncthreads();
    if (tid == 0) {
      double s = 0.0;
      for (int w = 0; w < WGM * WGN; ++w) s += wsum[w];
      partial[blockIdx.x] = s;
    }
  }
}

namespace {
int cu_n() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}
unsigned tiles_of(int M, int N, int bm, int bn) {
  return (unsigned)(((M + bm - 1) / bm) * ((N + bn - 1) / bn));
}
}  // namespace

namespace {
// The launch plan of the W4A16 / W3A16 product. Without a workspace: the
// largest tile that still gives every compute unit work (int4 256 x 256 with
// a 128 x 256 tail, or 128 x 128, or 64 x 64; int3 128 x 128 or 64 x 64).
// When the tiles leave compute units idle (small M x N; see gemm_plan) and a
// workspace is given, the K range splits over `splits` workgroups per tile
// (`spl` steps each, at least 8) so that about one workgroup per compute unit
// runs, on tiles as tall as M needs (32 (int4) or 64 rows, else 128) and 128
// wide: a tile re-reads its activation rows for every 128 outputs instead of
// every 64, and no rows past M are loaded and multiplied for nothing. Each
// split writes its float32 products to its own [M, N] plane of the
// workspace, and the split that finishes a tile last (a counter per tile at
// the workspace's head) adds the tile's planes in split order. Against a
// separate adding kernel (rocprofv3, weights in HBM): 4096x4096 M = 17 13.5
// -> 9.5 us, M = 64 17.8 -> 11.8, 4096x11008 M = 17 22.5 -> 18.0, M = 128
// 31.8 -> 29.3, int3 4096x4096 M = 32 21.3 -> 16.6.
struct GemmPlan {
  int bm, bn;    // tile
  int splits;    // K splits (1: none)
  int spl;       // steps per split
  unsigned tiles;
};

GemmPlan gemm_plan(int M, int N, int K, int bits, bool can_split) {
  const unsigned cus = (unsigned)cu_n();
  GemmPlan p{64, 64, 1, 0, 0};
  if (bits == 4) {
    // Rounds of tiles, one per compute unit at a time: a 256 x 256 tile
    // takes about 3 times as long as a 128 x 128 one, which takes about 2.5
    // times a 64 x 64 one (kernel traces, M x N at K = 4096: 256 x 11008
    // 57.6 us on 64 x 64 tiles -> 51.6 on 128 x 128, 1024 x 4096 92.8 ->
    // 55.3, 768 x 11008 149.1 -> 121.5 on 256 x 256, and at K = 8192
    // 512 x 28672 352.7 -> 276.6; the rule keeps 64 x 64 for 256 x 8192,
    // 41.1 against 47.1, and 128 x 128 for 256 x 28672, 189.1 against 208.6)
    const unsigned big = tiles_of(M, N, 256, 256), mid = tiles_of(M, N, 128, 128);
    const unsigned small = tiles_of(M, N, 64, 64);
    auto rounds = [&](unsigned t) { return (t + cus - 1) / cus; };
    if (big >= cus || 3 * rounds(big) <= rounds(mid)) p.bm = p.bn = 256;
    else if (5 * rounds(mid) <= 2 * rounds(small)) p.bm = p.bn = 128;
  } else if (tiles_of(M, N, 128, 128) * 2 >= cus) {
    p.bm = p.bn = 128;
  }
  const int nsteps = K / (bits == 3 ? 128 : 64);
  // split when 64 x 64 tiles fill at most half the compute units, or for a
  // long K (8192 or more) when 128 x 128 tiles do (measured with weights in
  // HBM: 4096 x 4096 at M = 17-64 23 -> 15 us, 11008 x 4096 at M = 17-256
  // 55-66 -> 23-45 us; 4096 x 11008 at M = 17-64, with 172 tiles of 64 x 64,
  // got no faster)
  if (can_split && (tiles_of(M, N, 64, 64) * 2 <= cus ||
                    (K >= 8192 && tiles_of(M, N, 128, 128) * 2 <= cus))) {
    const int bm = M <= 32 && bits == 4 ? 32 : (M <= 64 ? 64 : 128);
    const unsigned tiles = tiles_of(M, N, bm, 128);
    const int s = min((int)(cus / tiles), max(1, nsteps / 8));
    if (s > 1) {
      int spl = (nsteps + s - 1) / s;
      if (bits == 4) spl = (spl + 1) & ~1;  // int4 splits start on a group
      p = GemmPlan{bm, 128, (nsteps + spl - 1) / spl, spl, tiles};
    }
  }
  if (p.splits == 1) p.tiles = tiles_of(M, N, p.bm, p.bn);
  return p;
}

// planes after the counter region
size_t plan_workspace_bytes(const GemmPlan& p, int M, int N) {
  return p.splits <= 1 ? 0 : kSplitCtrBytes + (size_t)p.splits * M * N * 4;
}


}  // namespace

size_t gemm_workspace_bytes(int M, int N, int K, int bits) {
  return plan_workspace_bytes(gemm_plan(M, N, K, bits, true), M, N);
}

namespace {
template <bool CS>
hipError_t launch_gemm_t(const __half* X, const uint32_t* q, const void* scales, const void* zeros,
                         int M, int N, int K, int bits, int group, __half* Y, hipStream_t st,
                         void* ws, size_t ws_bytes) {
  const int gshift = group_shift(group);
  const int wpr = words_per_row(K, bits, group);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  const unsigned cus = (unsigned)cu_n();
  const bool zw = !CS && ((size_t)N * (size_t)(K / group)) % 4 == 0;
  const GemmPlan plan = gemm_plan(M, N, K, bits, ws != nullptr);
  if (plan.splits > 1 && ws_bytes < plan_workspace_bytes(plan, M, N)) return hipErrorInvalidValue;
  float* wsf = plan.splits > 1
                   ? reinterpret_cast<float*>(static_cast<char*>(ws) + kSplitCtrBytes)
                   : nullptr;
  const unsigned nsp = (unsigned)plan.splits;
#define AWQ_GEMM_K(BMODE, BM, BN, WGM, WGN, NST, NB, NE, SKV)                                  \
  do {                                                                                          \
    const dim3 grid(tiles_of(M, (NE) - (NB), BM, BN), nsp);                                     \
    if (zw)                                                                                     \
      hipLaunchKernelGGL((gemm_kernel<BMODE, 0, BM, BN, WGM, WGN, true, NST, CS, SKV>),         \
                         grid, dim3(64 * WGM * WGN), 0, st, x, q, scales, zeros, M, N, K, wpr,  \
                         gshift, y, nullptr, 0, nullptr, nullptr, nullptr, NB, NE, wsf,         \
                         plan.spl);                                                             \
    else                                                                                        \
      hipLaunchKernelGGL((gemm_kernel<BMODE, 0, BM, BN, WGM, WGN, false, NST, CS, SKV>),        \
                         grid, dim3(64 * WGM * WGN), 0, st, x, q, scales, zeros, M, N, K, wpr,  \
                         gshift, y, nullptr, 0, nullptr, nullptr, nullptr, NB, NE, wsf,         \
                         plan.spl);                                                             \
  } while (0)
#define AWQ_GEMM(BMODE, BM, BN, WGM, WGN, NST, NB, NE) \
  AWQ_GEMM_K(BMODE, BM, BN, WGM, WGN, NST, NB, NE, false)
#define AWQ_GEMM_S(BMODE, BM, BN, WGM, WGN, NST) \
  AWQ_GEMM_K(BMODE, BM, BN, WGM, WGN, NST, 0, N, true)
  if (plan.splits > 1) {
    // split K: int4 32 x 128 (4 wavefronts of 32 x 32), 64 x 128 (2 x 2 of
    // 32 x 64) or 128 x 128 tiles
    if (bits == 4) {
      if (plan.bm == 32) AWQ_GEMM_S(4, 32, 128, 1, 4, 4);
      else if (plan.bm == 64) AWQ_GEMM_S(4, 64, 128, 2, 2, 4);
      else AWQ_GEMM_S(4, 128, 128, 2, 2, 4);
    } else {
      // int3 on 8 wavefronts, one B item per thread (two put the register
      // stages in scratch memory): 64 x 128 also serves M <= 32
      if (plan.bm == 128) AWQ_GEMM_S(3, 128, 128, 4, 2, 4);
      else AWQ_GEMM_S(3, 64, 128, 2, 4, 4);
    }
  } else if (bits == 4) {
    if (plan.bm == 256) {
      // Whole rounds of 256 x 256 tiles (one per compute unit each), and the
      // columns past them on 128 x 256 tiles when those fit in one round:
      // a partial last round of big tiles would leave compute units idle for
      // a whole tile time, the small tiles take about half of it.
      const unsigned big = plan.tiles;
      const int mt = (M + 255) / 256;
      const int nsplit = (int)((big / cus) * cus / (unsigned)mt) * 256;
      const bool split = big % cus != 0 && nsplit > 0 && nsplit < N &&
                         tiles_of(M, N - nsplit, 128, 256) <= cus;
      if (split) {
        AWQ_GEMM(4, 256, 256, 2, 4, 2, 0, nsplit);
        AWQ_GEMM(4, 128, 256, 2, 4, 4, nsplit, N);
      } else {
        AWQ_GEMM(4, 256, 256, 2, 4, 2, 0, N);
      }
    } else if (plan.bm == 128) {
      AWQ_GEMM(4, 128, 128, 2, 2, 4, 0, N);
    } else {
      AWQ_GEMM(4, 64, 64, 2, 2, 4, 0, N);
    }
  } else if (plan.bm == 128) {
    // 8 wavefronts of 32 x 64 (one B item per thread) once the 128 x 128
    // tiles fill half the compute units (measured: 256 x 4096 x 11008 in
    // 62 us against 77 us on 64 x 64 tiles; 2048 x 4096 x 11008 382 / 548 us)
    AWQ_GEMM(3, 128, 128, 4, 2, 4, 0, N);
  } else {
    AWQ_GEMM(3, 64, 64, 2, 2, 4, 0, N);
  }
#undef AWQ_GEMM_S
#undef AWQ_GEMM
#undef AWQ_GEMM_K
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm(const __half* X, const uint32_t* q, const void* scales, const void* zeros,
                       int M, int N, int K, int bits, int group, __half* Y, hipStream_t st,
                       bool cs, void* ws, size_t ws_bytes) {
  return cs ? launch_gemm_t<true>(X, q, scales, zeros, M, N, K, bits, group, Y, st, ws, ws_bytes)
            : launch_gemm_t<false>(X, q, scales, zeros, M, N, K, bits, group, Y, st, ws, ws_bytes);
}

// gated MLP: Y = fp16(silu(X Wg^T) * (X Wu^T)), both products on one A tile
hipError_t launch_gemm_gate_up(const __half* X, const uint32_t* qg, const float* sg,
                               const uint8_t* zg, const uint32_t* qu, const float* su,
                               const uint8_t* zu, int M, int N, int K, int bits, int group,
                               __half* Y, hipStream_t st) {
  const int gshift = group_shift(group);
  const int wpr = words_per_row(K, bits, group);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(X);
  uint16_t* y = reinterpret_cast<uint16_t*>(Y);
  const unsigned cus = (unsigned)cu_n();
  const bool zw = ((size_t)N * (size_t)(K / group)) % 4 == 0;
#define AWQ_GU(BMODE, BM, BN, WGM, WGN, NST)                                                     \
  do {                                                                                            \
    if (zw)                                                                                       \
      hipLaunchKernelGGL((gemm_kernel<BMODE, 2, BM, BN, WGM, WGN, true, NST>),                    \
                         dim3(tiles_of(M, N, BM, BN / 2)), dim3(64 * WGM * WGN), 0, st, x, qg, sg, \
                         zg, M, N, K, wpr, gshift, y, nullptr, 0, qu, su, zu, 0, N, nullptr, 0);  \
    else                                                                                          \
      hipLaunchKernelGGL((gemm_kernel<BMODE, 2, BM, BN, WGM, WGN, false, NST>),                   \
                         dim3(tiles_of(M, N, BM, BN / 2)), dim3(64 * WGM * WGN), 0, st, x, qg, sg, \
                         zg, M, N, K, wpr, gshift, y, nullptr, 0, qu, su, zu, 0, N, nullptr, 0);  \
  } while (0)
  if (bits == 4) {
    // the bigger tile once its tiles fill 5/8 of the compute units (kernel
    // traces, same outputs: 2 x 28672 x 8192 at M = 256 402.6 -> 275.9 us,
    // 2 x 11008 x 4096 at M = 512 152.3 -> 131.5 us and at M = 128
    // 70.3 -> 49.3 us; at 86 big tiles, 2 x 11008 x 4096 at M = 192 and
    // 256, the 128 x 128 tile stays faster: 85.9 against 107.1 us)
    if (tiles_of(M, N, 256, 128) * 8 >= cus * 5)
      AWQ_GU(4, 256, 256, 2, 4, 2);
    else if (tiles_of(M, N, 128, 64) * 8 >= cus * 5)
      AWQ_GU(4, 128, 128, 2, 2, 4);
    else
      AWQ_GU(4, 64, 128, 2, 2, 4);
  } else {
    // 8 wavefronts, so each thread loads one (row, quarter) item per step
    // (two items per thread put the register stages in scratch memory)
    AWQ_GU(3, 128, 128, 4, 2, 4);
  }
#undef AWQ_GU
  return hipGetLastError();
}

// ||A B^T||_F^2 as one float64 partial per workgroup tile; A is [M, K] fp16,
// B is [N, K] fp16, or with hilo [N, 2K] holding hi and lo parts per
// 128-wide k chunk (then the product is A (Bhi + Blo)^T)
namespace {
// 256 x 256 tiles when one round of them is shorter than the rounds of
// 128 x 128 tiles it replaces (a big tile does 4 small tiles' work at about
// 4/3 of their speed: half the operand traffic per flop)
bool sqnorm_big(int M, int N) {
  const unsigned cus = (unsigned)cu_n();
  const unsigned big = tiles_of(M, N, 256, 256), small = tiles_of(M, N, 128, 128);
  const double t_big = 3.0 * (double)((big + cus - 1) / cus);
  const double t_small = 1.0 * (double)((small + cus - 1) / cus);
  return t_big < t_small;
}
}  // namespace

hipError_t launch_sqnorm_abt(const uint16_t* A, const uint16_t* B, int M, int N, int K, bool hilo,
                             double* partial, hipStream_t st) {
  if (sqnorm_big(M, N))
    hipLaunchKernelGGL((gemm_kernel<0, 1, 256, 256, 2, 4, false, 2>),
                       dim3(tiles_of(M, N, 256, 256)), dim3(512), 0, st, A, B, nullptr, nullptr,
                       M, N, K, 0, 0, nullptr, partial, hilo ? 1 : 0, nullptr, nullptr, nullptr, 0,
                       N, nullptr, 0);
  else
    hipLaunchKernelGGL((gemm_kernel<0, 1, 128, 128, 2, 2, false, 2>),
                       dim3(tiles_of(M, N, 128, 128)), dim3(256), 0, st, A, B, nullptr, nullptr,
                       M, N, K, 0, 0, nullptr, partial, hilo ? 1 : 0, nullptr, nullptr, nullptr, 0,
                       N, nullptr, 0);
  return hipGetLastError();
}

unsigned sqnorm_abt_tiles(int M, int N) {
  return sqnorm_big(M, N) ? tiles_of(M, N, 256, 256) : tiles_of(M, N, 128, 128);
}

}  // namespace awq
