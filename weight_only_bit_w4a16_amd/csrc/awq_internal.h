// Internal launch interface between the C-ABI layer (awq_api.hip) and the
// kernel translation units. Every launcher enqueues on `st` and returns the
// launch status; shapes have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

// words of one packed group: int4 -> group/8; int3 -> 13 per 128-code block
// (every block starts on a word boundary, whatever the group)
inline int words_per_group(int bits, int group) { return bits == 4 ? group / 8 : 13 * (group / 128); }

// Kernels index a group's scale by (128-code block) >> gshift, with
// gshift = ceil(log2(group / 128)), and take max(1, blocks >> gshift) groups
// per row: exact for groups of 128, 256 and 512, and for a group of the
// whole row (then every block maps to group 0).
// per-output-channel groups (the whole row) are quantized with the row in
// registers: K <= 4096 kRowMaxChunks
constexpr int kRowMaxChunks = 8;

// a group the per-group kernels do not tile (128, 256 or 512 codes): one
// group of the whole row, quantized by the per-row kernels
inline bool row_group(int group) { return group != 128 && group != 256 && group != 512; }

inline int group_shift(int group) {
  int s = 0;
  while ((128 << s) < group) ++s;
  return s;
}
inline int words_per_row(int K, int bits, int group) {
  int w = (K / group) * words_per_group(bits, group);
  return (w + 3) & ~3;
}

hipError_t launch_act_stats(const __half* X, int T, int K, double* m, hipStream_t st);
hipError_t launch_scale_candidates(const double* m, int K, const float* alpha, int n_alpha,
                                   float* s, hipStream_t st);
// zero_point false: the symmetric grid
hipError_t launch_quant_pack(const __half* W, const float* s, int N, int K, int bits, int group,
                             bool zero_point, uint32_t* q, float* scales, uint8_t* zeros,
                             hipStream_t st);
hipError_t launch_fold(const __half* X, const float* s, int M, int K, __half* Y, hipStream_t st);

// The product kernels read the group parameters in plain storage (float32
// steps, uint8 zero points; cs = false) or compact storage (fp16 steps,
// 4-bit zero points 8 per uint32 word, rows of ceil(groups / 8) words;
// cs = true).
//
// decode, int4, M <= 16. variant 0 picks the fastest kernel for the shape;
// variant 1 forces the exact-dequant kernel (kept selectable for tests).
// ws / ws_bytes: a workspace of at least gemv_workspace_bytes(M, N, K)
// bytes lets 2 <= M <= 16 split K over workgroups (nullptr: no split).
hipError_t launch_gemv_w4(const __half* X, const uint32_t* q, const void* scales,
                          const void* zeros, int M, int N, int K, int group, __half* Y,
                          hipStream_t st, int variant, bool cs, void* ws = nullptr,
                          size_t ws_bytes = 0);
// bytes of workspace the automatic int4 decode choice splits K with (0:
// none for this shape)
size_t gemv_workspace_bytes(int M, int N, int K);
// decode, int4, 2 <= M <= 16 on 16-row blocks with the activations in LDS
// (gemv_w4_mb_kernel): token rows stored (8 or 16), K splits, chunks of 128
// codes per split, workgroups per split, full-line weight loads, LDS bytes,
// workspace bytes. splits is 0 when the shape needs a split and can_split is
// false.
struct MbPlan {
  int mp, splits, spl, gx;
  bool fl;
  size_t lds, ws_bytes;
};
MbPlan mb_plan(int M, int N, int K, bool can_split);
// whether the automatic int4 decode choice for 2 <= M <= 16 takes this
// kernel (rows longer than one pass of gemv_w4_mx_kernel)
bool mb_preferred(int M, int N, int K);
// hipErrorNotSupported (nothing launched) when the plan has no splits
hipError_t launch_gemv_w4_mb(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int M, int N, int K, int group, __half* Y,
                             hipStream_t st, bool cs, void* ws, size_t ws_bytes);
// decode, int3, M <= 4
hipError_t launch_gemv_w3(const __half* X, const uint32_t* q, const void* scales,
                          const void* zeros, int M, int N, int K, int group, __half* Y,
                          hipStream_t st, bool cs);
constexpr int kGemvW3MaxM = 4;
// decode, int3, 2 <= M <= 4 on rows of up to 8 pieces of 16 blocks
// (hipErrorNotSupported, with nothing launched, otherwise)
hipError_t launch_gemv_w3_mt(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int M, int N, int K, int group, __half* Y,
                             hipStream_t st, bool cs);
// decode, int3, M = 1 (K up to 96 blocks of 128 codes)
hipError_t launch_gemv_w3_m1(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int N, int K, int group, __half* Y, hipStream_t st,
                             bool cs);
// The workspace of a product that splits K: a counter region first (one
// uint32 per 16-row block of outputs; zero before the first call, and every
// call leaves it zero), then the splits' float32 [M, N] planes.
constexpr size_t kSplitCtrBytes = 64 * 1024;
constexpr int kSplitMaxRowBlocks = (int)(kSplitCtrBytes / 4);
// prefill (any M)
hipError_t launch_gemm(const __half* X, const uint32_t* q, const void* scales, const void* zeros,
                       int M, int N, int K, int bits, int group, __half* Y, hipStream_t st,
                       bool cs,
                       void* ws = nullptr, size_t ws_bytes = 0);
// bytes of workspace the prefill product uses to split K for this shape (0:
// it does not split)
size_t gemm_workspace_bytes(int M, int N, int K, int bits);
// decode, int4, 2 <= M <= 16, K <= 8192 (NotSupported otherwise); with q2
// set, the gated-MLP form silu(X Wq^T) * (X Wq2^T)
hipError_t launch_gemv_w4_mx(const __half* X, const uint32_t* q, const void* scales,
                             const void* zeros, int M, int N, int K, int group, __half* Y,
                             hipStream_t st, const uint32_t* q2, const void* scales2,
                             const void* zeros2, bool cs);
// gated MLP: Y = fp16(silu(X Wg^T) * (X Wu^T)), plain storage; M = 1 int4 /
// int3 decode (K up to 96 blocks), and the prefill kernel for any M
// fused gate/up, 2 <= M <= 4 on rows of few pieces (hipErrorNotSupported,
// with nothing launched, otherwise)
hipError_t launch_gate_up_mt(const __half* X, const uint32_t* qg, const float* sg,
                             const uint8_t* zg, const uint32_t* qu, const float* su,
                             const uint8_t* zu, int M, int N, int K, int bits, int group,
                             __half* Y, hipStream_t st);
hipError_t launch_gate_up_w4_m1(const __half* X, const uint32_t* qg, const float* sg,
                                const uint8_t* zg, const uint32_t* qu, const float* su,
                                const uint8_t* zu, int N, int K, int group, __half* Y,
                                hipStream_t st);
hipError_t launch_gate_up_w3_m1(const __half* X, const uint32_t* qg, const float* sg,
                                const uint8_t* zg, const uint32_t* qu, const float* su,
                                const uint8_t* zu, int N, int K, int group, __half* Y,
                                hipStream_t st);
hipError_t launch_gemm_gate_up(const __half* X, const uint32_t* qg, const float* sg,
                               const uint8_t* zg, const uint32_t* qu, const float* su,
                               const uint8_t* zu, int M, int N, int K, int bits, int group,
                               __half* Y, hipStream_t st);
// plain -> compact group parameters
hipError_t launch_compact_params(const float* scales, const uint8_t* zeros, int N, int ng,
                                 uint16_t* scales16, uint32_t* zeros4, hipStream_t st);

// scale search pieces
size_t search_workspace_bytes(int N, int K, int T, int n_alpha, int bits, int group);
hipError_t launch_search(const __half* W, const __half* Xc, int N, int K, int T,
                         const float* alpha_dev, int n_alpha, int bits, int group,
                         bool zero_point, void* ws, double* loss_dev, int* best_dev, float* s_out,
                         hipStream_t st);

// layers sharing one input: losses added per candidate in layer order
size_t search_workspace_bytes_joint(const int* N, int n_layers, int K, int T, int n_alpha);
hipError_t launch_search_joint(const __half* const* W, const int* N, int n_layers, const __half* Xc,
                               int K, int T, const float* alpha_dev, int n_alpha, int bits,
                               int group, bool zero_point, void* ws, double* loss_dev,
                               int* best_dev, float* s_out, hipStream_t st);

// RMSNorm with the scale folded into its weight
hipError_t launch_fold_norm_weight(const __half* gamma, const float* s, int K, __half* out,
                                   hipStream_t st);
constexpr int kRmsNormMaxK = 16384;
hipError_t launch_rmsnorm(const __half* X, const __half* gamma, int M, int K, float eps, __half* Y,
                          hipStream_t st);

}  // namespace awq
