/*
 * awq.h -- C ABI of libawq: the data-parallel hot path of AWQ
 * (activation-aware weight quantization) with 4-bit or 3-bit group-wise
 * weights and fp16 activations (W4A16 / W3A16), for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (as stated on the pages this library follows):
 *   - a linear layer Y = W X is rewritten as (W diag(s)) (diag(s)^-1 X),
 *     which is exact before quantization (hungho77 blog "AWQ explained" --
 *     "Scaling instead of mixed precision"; AWQ Explained: Protecting the
 *     Weights That Matter Most -- "Scaling instead of mixed precision");
 *   - s_j = mean_t |x_tj| ** alpha with alpha grid-searched in [0, 1] to
 *     minimise the layer-output error on a calibration batch (AWQ Explained
 *     -- "How the scale is chosen");
 *   - W diag(s) is quantized with plain round-to-nearest, group-wise along
 *     the input dimension, 3 or 4 bits, groups of 128, asymmetric grid with
 *     an integer zero point (ai360xpert "AWQ" -- "How It Works"; Real Python
 *     glossary "activation-aware weight quantization (AWQ)"; AWQ Explained --
 *     "How the scale is chosen");
 *   - at run time the packed weights are loaded, unpacked, dequantized and
 *     multiplied with fp16 activations (hungho77 blog -- "Why the engine is
 *     part of the method").
 *
 * Conventions for every call:
 *   - All arrays are dense, row-major and contiguous. fp16 values are passed
 *     as uint16_t bit patterns.
 *   - W is [N, K]: row n = output channel, column k = input channel.
 *     Activations are [tokens, K]; Y = X' dequant(Q)^T is [M, N].
 *   - "dev" pointers are HIP device memory; "host" pointers are host memory.
 *     Device pointers must be 16-byte aligned.
 *   - The caller owns every buffer. The library never allocates or frees
 *     device memory; its only scratch is the caller's `workspace`.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls enqueue
 *     their kernels on it and return without waiting, except
 *     awq_scale_search, which synchronizes `stream` (it returns host values).
 *   - Arguments are validated before any HIP call; a bad argument returns
 *     AWQ_ERR_INVALID_ARG or AWQ_ERR_UNSUPPORTED and enqueues nothing. With
 *     no usable GPU the calls return AWQ_ERR_NO_DEVICE. A failed launch
 *     returns AWQ_ERR_HIP.
 *   - Inputs must be finite; the result is unspecified otherwise.
 *   - The library keeps no state between calls; calls on different streams
 *     may run concurrently as long as their output buffers do not overlap.
 *
 * Supported shapes: bits in {3, 4}; group in {128, 256, 512} with K a
 * multiple of group, or group = -1 (or K): one group per output channel
 * (the whole row, AwqConfig group_size = -1), for K a multiple of 128 up to
 * 32768.
 *
 * Packed weight layout (Qpacked, uint32 [N, awq_packed_words_per_row]):
 *   codes along K, lowest slot in the lowest bits. int4: the code at
 *   position k of a row sits in word k / 8, bits [4 (k % 8), 4 (k % 8) + 4).
 *   int3: the row is cut into blocks of 128 codes, each starting on a word
 *   boundary and taking 13 words of 10 codes (bits 30-31 zero; the 13th word
 *   holds 8 codes); code j = k % 128 of block k / 128 sits in word
 *   13 (k / 128) + j / 10, bits [3 (j % 10), 3 (j % 10) + 3). The layout does
 *   not depend on the group (groups are whole blocks). Unused slots are
 *   zero; each row is padded with zero words to a multiple of 4 words
 *   (16 bytes).
 *   scales: float32 [N, K/group], the grid step delta of each group.
 *   zeros:  uint8   [N, K/group], the integer zero point z of each group.
 *   A weight dequantizes to (q - z) * delta.
 */
#ifndef AWQ_H
#define AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misaligned pointer */
  AWQ_ERR_UNSUPPORTED = 2, /* valid request outside the supported shapes */
  AWQ_ERR_NO_DEVICE = 3,   /* no HIP device visible */
  AWQ_ERR_HIP = 4,         /* a HIP runtime call or a launch failed */
  AWQ_ERR_WORKSPACE = 5    /* workspace NULL or smaller than required */
} awq_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* awq_status_string(int status);

/* ABI version of this library (major * 100 + minor). */
int awq_version(void);

/* uint32 words per packed row for (K, bits, group); 0 if the combination is
 * invalid. int4: K/8. int3: 13 words per 128 codes, rounded up to a
 * multiple of 4. */
size_t awq_packed_words_per_row(int K, int bits, int group);

/* Activation statistic (AWQ Explained -- "How the scale is chosen": the
 * scale is driven by mean(|x_j|) per input channel):
 *   m[k] = (sum_t |Xcal[t, k]|) / T, in float64.
 * Xcal: dev fp16 [T, K]; m: dev float64 [K]. 1 <= T < 8192 (the fp16 sum is
 * then exact in float64, so the result does not depend on summation order). */
awq_status awq_act_stats(const uint16_t* Xcal, int T, int K, double* m, void* stream);

/* Scale candidates s = s_X ** alpha for every alpha of the grid (AWQ
 * Explained -- "How the scale is chosen"):
 *   s[a, k] = float32(pow(m[k], alpha[a])) (pow in float64), or 1 if
 *   m[k] == 0.
 * m: dev float64 [K]; alpha: dev float32 [n_alpha]; s: dev float32
 * [n_alpha, K]. */
awq_status awq_scale_candidates(const double* m, int K, const float* alpha, int n_alpha,
                                float* s, void* stream);

/* Round-to-nearest quantize-and-pack of W diag(s) (ai360xpert "AWQ" --
 * "How It Works", step 4; AWQ Explained -- "Scaling instead of mixed
 * precision" and "How the scale is chosen"). Per row n and group g, in
 * float32 with single roundings and round-half-to-even:
 *   W' = float32(W) * s[k]          (s == NULL means s = 1, plain RTN)
 *   lo = min(0, min W'), hi = max(0, max W'), r = hi - lo
 *   r == 0:  delta = 1, z = 0
 *   else:    delta = r / (2^bits - 1), z = rint(-lo / delta)
 *   q = clamp(rint(W' / delta) + z, 0, 2^bits - 1)
 * W: dev fp16 [N, K]; s: dev float32 [K] or NULL; outputs as in the layout
 * above (qpacked dev uint32 [N, words_per_row], scales dev float32
 * [N, K/group], zeros dev uint8 [N, K/group]). Padding words are written as
 * zero. Asynchronous on `stream`. */
awq_status awq_quantize_pack(const uint16_t* W, const float* s, int N, int K, int bits, int group,
                             uint32_t* qpacked, float* scales, uint8_t* zeros, void* stream);

/* awq_quantize_pack with the grid chosen by `zero_point` (the AwqConfig
 * option of AWQ Explained -- "How the scale is chosen", last paragraph):
 * 1 = the asymmetric grid above (awq_quantize_pack is this call with 1);
 * 0 = the symmetric grid, per row n and group g:
 *   a = max |W'|
 *   a == 0:  delta = 1
 *   else:    delta = a / (2^(bits-1) - 1)
 *   z = 2^(bits-1),  q = rint(W' / delta) + z   (in [1, 2^bits - 1])
 * so the codes are signed integers stored with a fixed offset and the packed
 * layout, the zeros array and awq_w4a16_matmul are unchanged. Any other
 * value of zero_point returns AWQ_ERR_INVALID_ARG. */
awq_status awq_quantize_pack_ex(const uint16_t* W, const float* s, int N, int K, int bits,
                                int group, int zero_point, uint32_t* qpacked, float* scales,
                                uint8_t* zeros, void* stream);

/* Fold diag(s)^-1 into the activation (AWQ Explained -- "Scaling instead of
 * mixed precision": the matching activation channel is divided by s):
 *   Xout[m, k] = fp16(float32(X[m, k]) / s[k])   (round-to-nearest-even)
 * X, Xout: dev fp16 [M, K] (may be the same buffer); s: dev float32 [K]. */
awq_status awq_fold_inv_scale(const uint16_t* X, const float* s, int M, int K, uint16_t* Xout,
                              void* stream);

/* The W4A16 (or W3A16) product (hungho77 blog -- "Why weight-only
 * quantization fits decoding" and "Why the engine is part of the method"):
 *   Y[m, n] = sum_k X'[m, k] * (q[n, k] - z[n, g(k)]) * delta[n, g(k)]
 * accumulated in float32 and rounded once to fp16.
 * X': dev fp16 [M, K] (already divided by s); qpacked/scales/zeros as
 * produced by awq_quantize_pack; Y: dev fp16 [M, N].
 * M <= 16 runs the decode kernels (memory-bound weight streaming), larger M
 * the prefill kernels (fp16 matrix cores). Asynchronous on `stream`. */
awq_status awq_w4a16_matmul(const uint16_t* X, const uint32_t* qpacked, const float* scales,
                            const uint8_t* zeros, int M, int N, int K, int bits, int group,
                            uint16_t* Y, void* stream);

/* awq_w4a16_matmul with an explicit kernel choice, so that every kernel can
 * be checked and timed on every shape: kernel 0 = automatic (as
 * awq_w4a16_matmul), 1 = decode kernel (M <= 16 for int4, M <= 4 for int3),
 * 2 = int4 decode kernel in exact-dequant form (M <= 16), 3 = prefill
 * kernel (any M). Returns AWQ_ERR_UNSUPPORTED for a kernel that does not
 * cover the request. */
awq_status awq_w4a16_matmul_kernel(const uint16_t* X, const uint32_t* qpacked, const float* scales,
                                   const uint8_t* zeros, int M, int N, int K, int bits, int group,
                                   uint16_t* Y, int kernel, void* stream);

/* Bytes of device workspace with which awq_w4a16_matmul_ws splits the K
 * range of this product over several workgroups per output tile (0: the
 * shape runs without splitting, or the arguments are invalid). Splitting is
 * used when even the smallest prefill tiles leave compute units idle (M
 * beyond the decode range with few output tiles, for example M = 17..256 on
 * a 4096-wide layer), and by the int4 decode kernel for 2 <= M <= 16 on
 * rows of more than 8192 codes. The bytes are a 64 KiB counter region
 * followed by one float32 [M, N] plane per split. */
size_t awq_w4a16_matmul_workspace_bytes(int M, int N, int K, int bits, int group);

/* awq_w4a16_matmul with a workspace (same arithmetic contract). With a
 * split, every split writes its float32 sums over its part of K to its own
 * [M, N] plane of the workspace, and the split that finishes an output
 * tile last (prefill: a tile of up to 128 x 128 outputs; int4 decode: a
 * 16-row block), which it learns from that tile's counter in the
 * workspace's first 64 KiB, adds the tile's planes in split order, so the
 * result does not depend on timing. workspace: dev, 16-byte aligned, at least
 * awq_w4a16_matmul_workspace_bytes(M, N, K, bits, group) bytes, owned by
 * the caller; its first 64 KiB zero-filled before the first call that uses
 * it (every call leaves them zero; the rest may hold anything); calls that
 * share a workspace must be ordered on one stream. NULL runs without
 * splitting; a non-NULL workspace that is too small returns
 * AWQ_ERR_WORKSPACE. Asynchronous on `stream`. */
awq_status awq_w4a16_matmul_ws(const uint16_t* X, const uint32_t* qpacked, const float* scales,
                               const uint8_t* zeros, int M, int N, int K, int bits, int group,
                               uint16_t* Y, void* workspace, size_t workspace_bytes,
                               void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * product of awq_w4a16_matmul_ws, same arguments, kernels and results,
 * with the workspace (counter region and split-K planes) in a scratch
 * array the library holds in device memory (16 MiB + 64 KiB on each GPU it
 * runs on, zero when loaded, from first load to the end of the process)
 * instead of a caller workspace. The call allocates nothing; the caller
 * still owns X, qpacked, scales, zeros and Y. A shape whose split plan
 * needs more than that returns AWQ_ERR_WORKSPACE (on a 256-unit GPU every
 * prefill plan fits, and every decode plan with N * K up to about 1.9e9 at
 * M <= 8, 5.4e8 at M <= 16). Every call on one GPU shares that
 * GPU's scratch and leaves its planes behind and its counters zero, so calls
 * that overlap on one GPU race: order them on one stream. The first call on
 * a device looks up the scratch's address there (no allocation).
 * Asynchronous on `stream`. */
awq_status awq_w4a16_matmul_noalloc(const uint16_t* X, const uint32_t* qpacked,
                                    const float* scales, const uint8_t* zeros, int M, int N, int K,
                                    int bits, int group, uint16_t* Y, void* stream);

/* The gate and up projections of a gated MLP fused into one call (hungho77
 * blog -- "Why the engine is part of the method": the speed-up comes from
 * kernels that fuse operators). Both projections read the same activation
 * X' once and the elementwise epilogue runs on their float32 sums:
 *   G[m, n] = sum_k X'[m, k] * (qg[n, k] - zg[n, g(k)]) * dg[n, g(k)]
 *   U[m, n] = the same with (qu, su, zu)
 *   Y[m, n] = fp16(silu(G) * U),  silu(v) = v / (1 + e^-v), in float32.
 * X': dev fp16 [M, K], already divided by the scale s both matrices were
 * quantized with (one s per activation: gate and up share their input);
 * (qg, sg, zg) and (qu, su, zu): two [N, K] matrices packed as by
 * awq_quantize_pack(_ex); Y: dev fp16 [M, N]. Kernel choice, every one
 * reading X' once for the two matrices: M = 1 (int4 and int3) the M = 1
 * decode kernels; 2 <= M <= 4 the few-token decode kernels where their
 * operands fit (int4 at M = 2, int3 at M = 2-4); int4 up to M = 16 the
 * 16-row-block decode kernel; anything else the prefill kernel.
 * Asynchronous on `stream`. */
awq_status awq_w4a16_gate_up_silu(const uint16_t* X, const uint32_t* qg, const float* sg,
                                  const uint8_t* zg, const uint32_t* qu, const float* su,
                                  const uint8_t* zu, int M, int N, int K, int bits, int group,
                                  uint16_t* Y, void* stream);

/* Compact storage of the group parameters (the fp16-scale, packed-zero
 * format of common AWQ checkpoints; AWQ Explained -- "How the scale is
 * chosen" names the group size and zero-point options it stores):
 *   scales16[n, g] = fp16(scales[n, g])             (round-to-nearest-even)
 *   zeros4[n, g / 8] bits [4 (g % 8), 4 (g % 8) + 4) = zeros[n, g]
 * scales, zeros: dev, as written by awq_quantize_pack(_ex) for this
 * (N, K, group) (every zero point fits 4 bits); scales16: dev fp16
 * [N, K/group]; zeros4: dev uint32 [N, ceil(K/group / 8)], unused fields
 * zero. A step of 65520 or more becomes infinite in fp16 (the weights' scale
 * must keep the steps below that). Asynchronous on `stream`. */
awq_status awq_compact_group_params(const float* scales, const uint8_t* zeros, int N, int K,
                                    int group, uint16_t* scales16, uint32_t* zeros4,
                                    void* stream);

/* The product over compactly stored group parameters:
 *   Y[m, n] = sum_k X'[m, k] * (q[n, k] - z[n, g(k)]) * float(fp16 step)
 * with the same kernels, accumulation and rounding as
 * awq_w4a16_matmul_kernel (kernel 0 = automatic, 1 = decode, 2 = int4 exact
 * decode, 3 = prefill). The parameters take 2.5 of the plain 5 bytes per
 * group. Asynchronous on `stream`. */
awq_status awq_w4a16_matmul_compact(const uint16_t* X, const uint32_t* qpacked,
                                    const uint16_t* scales16, const uint32_t* zeros4, int M, int N,
                                    int K, int bits, int group, uint16_t* Y, int kernel,
                                    void* stream);

/* Bytes of device workspace awq_scale_search needs for these sizes
 * (0 if the sizes are invalid). */
size_t awq_scale_search_workspace_bytes(int N, int K, int T, int n_alpha, int bits, int group);

/* Per-layer grid search over alpha (AWQ Explained -- "How the scale is
 * chosen"; hungho77 blog -- "Scaling instead of mixed precision"):
 *   m = awq_act_stats(Xcalib); for each alpha_i: s_i = m ** alpha_i,
 *   D_i = W - Q(W diag(s_i)) diag(s_i)^-1  (Q as in awq_quantize_pack),
 *   loss[i] = || Xcalib D_i^T ||_F^2  (sum over tokens and output channels),
 *   best = first index of the minimum loss; s_out = s_best.
 * W: dev fp16 [N, K]; Xcalib: dev fp16 [T, K]; alpha_grid: host float32
 * [n_alpha] (values in [0, 1]); s_out: dev float32 [K]; loss_out: host
 * float64 [n_alpha] (may be NULL); best_index: host int (may be NULL);
 * workspace: dev, at least awq_scale_search_workspace_bytes(...) bytes.
 * The contraction runs on the fp16 matrix cores (float32 accumulation, tile
 * sums in float64). For T*N >= 2^18 it is evaluated in the scaled domain,
 * x_k D_nk = (x_k / s_k) * (w_nk s_k - Q(W s)_nk), both factors rounded to
 * fp16 (loss error below about 1.2e-5 relative, shrinking as 1/sqrt(T N));
 * smaller problems contract Xcalib against D split into fp16 hi and lo parts
 * (about 1e-6). Either way well inside 1e-4.
 * Synchronizes `stream` before returning. */
awq_status awq_scale_search(const uint16_t* W, const uint16_t* Xcalib, int N, int K, int T,
                            const float* alpha_grid, int n_alpha, int bits, int group, float* s_out,
                            double* loss_out, int* best_index, void* workspace,
                            size_t workspace_bytes, void* stream);

/* awq_scale_search with Q the grid chosen by `zero_point` (1 = asymmetric,
 * as awq_scale_search; 0 = symmetric, as awq_quantize_pack_ex). Same
 * arguments, workspace, accuracy and synchronization otherwise; any other
 * value of zero_point returns AWQ_ERR_INVALID_ARG. */
awq_status awq_scale_search_ex(const uint16_t* W, const uint16_t* Xcalib, int N, int K, int T,
                               const float* alpha_grid, int n_alpha, int bits, int group,
                               int zero_point, float* s_out, double* loss_out, int* best_index,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Layers that read the same normalized input (q/k/v projections; gate and
 * up) can carry only one s, since it is folded into the one norm in front of
 * them (AWQ Explained -- "Scaling instead of mixed precision"). Their search
 * adds the layers' losses per candidate, in layer order, and picks the first
 * minimum of the sum:
 *   loss[i] = sum_l || Xcalib D_l,i^T ||_F^2,  D_l,i as in awq_scale_search.
 * W: host array of n_layers (1..16) dev pointers to fp16 [N[l], K] matrices;
 * N: host int [n_layers]; the other arguments, the accuracy and the
 * synchronization are those of awq_scale_search_ex (one layer gives exactly
 * awq_scale_search_ex). workspace: dev, at least
 * awq_scale_search_joint_workspace_bytes(...) bytes (0 if the sizes are
 * invalid). */
size_t awq_scale_search_joint_workspace_bytes(const int* N, int n_layers, int K, int T,
                                              int n_alpha, int bits, int group);
awq_status awq_scale_search_joint(const uint16_t* const* W, const int* N, int n_layers,
                                  const uint16_t* Xcalib, int K, int T, const float* alpha_grid,
                                  int n_alpha, int bits, int group, int zero_point, float* s_out,
                                  double* loss_out, int* best_index, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* The fold of diag(s)^-1 into the RMSNorm in front of the layer (AWQ
 * Explained -- "Scaling instead of mixed precision": done offline; what
 * ships is a slightly modified norm):
 *   gamma_out[k] = fp16(float32(gamma[k]) / s[k])   (round-to-nearest-even)
 * gamma, gamma_out: dev fp16 [K] (may be the same buffer); s: dev float32
 * [K]. Asynchronous on `stream`. */
awq_status awq_fold_norm_weight(const uint16_t* gamma, const float* s, int K, uint16_t* gamma_out,
                                void* stream);

/* RMSNorm, which with the folded weight yields X' = norm(X) diag(s)^-1 for
 * the W4A16 product directly:
 *   r = 1 / sqrt(sum_k X[m, k]^2 / K + eps),  Y[m, k] = fp16(X[m, k] r gamma[k])
 * in float32 (r from a fixed-order tree sum), one rounding to fp16; within
 * one fp16 ulp of the exact value. X, Y: dev fp16 [M, K] (may be the same
 * buffer); gamma: dev fp16 [K]; eps >= 0. K must be a multiple of 8 and at
 * most 16384 (else AWQ_ERR_UNSUPPORTED). Asynchronous on `stream`. */
awq_status awq_rmsnorm(const uint16_t* X, const uint16_t* gamma, int M, int K, float eps,
                       uint16_t* Y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_H */
