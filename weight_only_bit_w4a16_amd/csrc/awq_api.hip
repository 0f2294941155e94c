// C-ABI layer of libawq: argument validation (before any HIP call), device
// check, dispatch to the kernel launchers, error mapping. Stateless apart
// from the per-device address of the allocation-free product's scratch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/awq.h"
#include "awq_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// layers of one joint search (q, k, v or gate, up, and room to spare)
constexpr int kMaxLayers = 16;

// normalise the group argument (-1 means the whole row); 0 if unsupported.
// Groups of 128, 256 or 512 codes, or of the whole row (per output channel)
// when K is a multiple of 128 and the row fits the per-row kernels.
int resolve_group(int K, int group) {
  if (group == -1) group = K;
  if (K <= 0 || K % group != 0) return 0;
  if (group == 128 || group == 256 || group == 512) return group;
  if (group == K && K % 128 == 0 && K <= 4096 * awq::kRowMaxChunks) return group;
  return 0;
}

awq_status device_ready() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return AWQ_ERR_NO_DEVICE;
  }
  return AWQ_OK;
}

awq_status from_hip(hipError_t e) {
  if (e == hipSuccess) return AWQ_OK;
  if (e == hipErrorNotSupported) return AWQ_ERR_UNSUPPORTED;
  return AWQ_ERR_HIP;
}

awq_status check_group(int K, int bits, int group, int* g_out) {
  if (bits != 3 && bits != 4) return AWQ_ERR_UNSUPPORTED;
  if (K <= 0) return AWQ_ERR_INVALID_ARG;
  if (group == 0 || group < -1) return AWQ_ERR_INVALID_ARG;
  if (group > 0 && K % group != 0) return AWQ_ERR_INVALID_ARG;
  const int g = resolve_group(K, group);
  if (g == 0) return AWQ_ERR_UNSUPPORTED;
  *g_out = g;
  return AWQ_OK;
}

// whether the automatic choice runs this shape on a decode kernel
bool auto_decode(int M, int bits) { return bits == 4 ? M <= 16 : M <= awq::kGemvW3MaxM; }

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of awq_w4a16_matmul_noalloc: the workspace of a split product
// (its counter region, then the split-K planes) in a file-scope device array
// instead of a caller workspace. A prefill split plan runs at most one
// workgroup per compute unit on tiles of at most 128 x 128 outputs, one
// float32 per output and split, so 256 units x 128 x 128 x 4 B = 16 MiB of
// planes hold every prefill plan on a 256-unit GPU; the array adds the
// counter region. It is zero when the code object is loaded (a zero-filled
// section), and every call leaves its counters zero. Each GPU the library
// runs on holds its own copy of the array until the process ends; host code
// reaches it only through the device address looked up below, never by its
// name (which on the host is a stand-in, not a device address).
constexpr size_t kNoAllocScratchBytes = ((size_t)16 << 20) + awq::kSplitCtrBytes;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// the current device's address of `scratch`, looked up once per device with
// that device current
awq_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return AWQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return AWQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return AWQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AWQ_OK;
}

// ws / ws_bytes: a caller workspace (nullptr: none); noalloc: use the
// file-scope scratch as the workspace
awq_status matmul_impl(const uint16_t* X, const uint32_t* qpacked, const void* scales,
                       const void* zeros, int M, int N, int K, int bits, int group, uint16_t* Y,
                       void* stream, int kernel, bool cs, void* ws = nullptr,
                       size_t ws_bytes = 0, bool noalloc = false) {
  if (!X || !qpacked || !scales || !zeros || !Y) return AWQ_ERR_INVALID_ARG;
  if (M <= 0 || N <= 0 || K <= 0) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(qpacked) || !aligned16(scales) || !aligned16(zeros) ||
      !aligned16(Y))
    return AWQ_ERR_INVALID_ARG;
  if (kernel < 0 || kernel > 3) return AWQ_ERR_INVALID_ARG;
  int g = 0;
  awq_status st = check_group(K, bits, group, &g);
  if (st != AWQ_OK) return st;
  if ((long long)M * K > (1LL << 31) || (long long)N * K > (1LL << 34)) return AWQ_ERR_UNSUPPORTED;
  if ((kernel == 1 || kernel == 2) && (M > 16 || (bits == 3 && M > awq::kGemvW3MaxM)))
    return AWQ_ERR_UNSUPPORTED;
  if (kernel == 2 && bits == 3) return AWQ_ERR_UNSUPPORTED;
  if (ws != nullptr && !aligned16(ws)) return AWQ_ERR_INVALID_ARG;
  const bool decode = kernel == 1 || kernel == 2 || (kernel == 0 && auto_decode(M, bits));
  // the workspace the automatic choice splits K with (the forced decode
  // kernels take none)
  const size_t need = kernel != 0 ? 0
                      : decode    ? (bits == 4 ? awq::gemv_workspace_bytes(M, N, K) : 0)
                                  : awq::gemm_workspace_bytes(M, N, K, bits);
  if (ws != nullptr && ws_bytes < need) return AWQ_ERR_WORKSPACE;
  if (noalloc && need > kNoAllocScratchBytes) return AWQ_ERR_WORKSPACE;
  st = device_ready();
  if (st != AWQ_OK) return st;
  if (noalloc && need > 0) {
    st = noalloc_scratch(&ws);
    if (st != AWQ_OK) return st;
    ws_bytes = kNoAllocScratchBytes;
  }
  if (kernel != 0) ws = nullptr;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const __half* x = reinterpret_cast<const __half*>(X);
  __half* y = reinterpret_cast<__half*>(Y);
  hipError_t e;
  if (decode) {
    if (bits == 4)
      e = awq::launch_gemv_w4(x, qpacked, scales, zeros, M, N, K, g, y, s, kernel == 2 ? 1 : 0,
                              cs, ws, ws_bytes);
    else if (M == 1 && kernel == 0)
      e = awq::launch_gemv_w3_m1(x, qpacked, scales, zeros, N, K, g, y, s, cs);
    else if (kernel == 0)
      e = awq::launch_gemv_w3_mt(x, qpacked, scales, zeros, M, N, K, g, y, s, cs);
    else
      e = hipErrorNotSupported;
    if (bits == 3 && e == hipErrorNotSupported) {
      (void)hipGetLastError();
      e = awq::launch_gemv_w3(x, qpacked, scales, zeros, M, N, K, g, y, s, cs);
    }
    // a shape the decode kernel does not cover (its LDS budget) runs on the
    // prefill kernel when the caller let the library choose
    if (e == hipErrorNotSupported && kernel == 0) {
      (void)hipGetLastError();
      e = awq::launch_gemm(x, qpacked, scales, zeros, M, N, K, bits, g, y, s, cs);
    }
  } else {
    e = awq::launch_gemm(x, qpacked, scales, zeros, M, N, K, bits, g, y, s, cs, ws, ws_bytes);
  }
  return from_hip(e);
}

}  // namespace

extern "C" {

const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_ERR_INVALID_ARG: return "AWQ_ERR_INVALID_ARG";
    case AWQ_ERR_UNSUPPORTED: return "AWQ_ERR_UNSUPPORTED";
    case AWQ_ERR_NO_DEVICE: return "AWQ_ERR_NO_DEVICE";
    case AWQ_ERR_HIP: return "AWQ_ERR_HIP";
    case AWQ_ERR_WORKSPACE: return "AWQ_ERR_WORKSPACE";
    default: return "AWQ_ERR_UNKNOWN";
  }
}

int awq_version(void) { return 101; }

size_t awq_packed_words_per_row(int K, int bits, int group) {
  int g = 0;
  if (check_group(K, bits, group, &g) != AWQ_OK) return 0;
  return (size_t)awq::words_per_row(K, bits, g);
}

awq_status awq_act_stats(const uint16_t* Xcal, int T, int K, double* m, void* stream) {
  if (!Xcal || !m) return AWQ_ERR_INVALID_ARG;
  if (T <= 0 || K <= 0) return AWQ_ERR_INVALID_ARG;
  if (T >= 8192) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(Xcal) || !aligned16(m)) return AWQ_ERR_INVALID_ARG;
  awq_status st = device_ready();
  if (st != AWQ_OK) return st;
  return from_hip(awq::launch_act_stats(reinterpret_cast<const __half*>(Xcal), T, K, m,
                                        reinterpret_cast<hipStream_t>(stream)));
}

awq_status awq_scale_candidates(const double* m, int K, const float* alpha, int n_alpha, float* s,
                                void* stream) {
  if (!m || !alpha || !s) return AWQ_ERR_INVALID_ARG;
  if (K <= 0 || n_alpha <= 0) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(m) || !aligned16(alpha) || !aligned16(s)) return AWQ_ERR_INVALID_ARG;
  awq_status st = device_ready();
  if (st != AWQ_OK) return st;
  return from_hip(awq::launch_scale_candidates(m, K, alpha, n_alpha, s,
                                               reinterpret_cast<hipStream_t>(stream)));
}

awq_status awq_quantize_pack_ex(const uint16_t* W, const float* s, int N, int K, int bits,
                                int group, int zero_point, uint32_t* qpacked, float* scales,
                                uint8_t* zeros, void* stream) {
  if (!W || !qpacked || !scales || !zeros) return AWQ_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0) return AWQ_ERR_INVALID_ARG;
  if (zero_point != 0 && zero_point != 1) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(qpacked) || !aligned16(scales) || !aligned16(zeros) ||
      (s && !aligned16(s)))
    return AWQ_ERR_INVALID_ARG;
  int g = 0;
  awq_status st = check_group(K, bits, group, &g);
  if (st != AWQ_OK) return st;
  if ((long long)N * K > (1LL << 34)) return AWQ_ERR_UNSUPPORTED;
  st = device_ready();
  if (st != AWQ_OK) return st;
  return from_hip(awq::launch_quant_pack(reinterpret_cast<const __half*>(W), s, N, K, bits, g,
                                         zero_point != 0, qpacked, scales, zeros,
                                         reinterpret_cast<hipStream_t>(stream)));
}

awq_status awq_quantize_pack(const uint16_t* W, const float* s, int N, int K, int bits, int group,
                             uint32_t* qpacked, float* scales, uint8_t* zeros, void* stream) {
  return awq_quantize_pack_ex(W, s, N, K, bits, group, 1, qpacked, scales, zeros, stream);
}

awq_status awq_fold_inv_scale(const uint16_t* X, const float* s, int M, int K, uint16_t* Xout,
                              void* stream) {
  if (!X || !s || !Xout) return AWQ_ERR_INVALID_ARG;
  if (M <= 0 || K <= 0) return AWQ_ERR_INVALID_ARG;
  if (K % 8 != 0) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(s) || !aligned16(Xout)) return AWQ_ERR_INVALID_ARG;
  awq_status st = device_ready();
  if (st != AWQ_OK) return st;
  return from_hip(awq::launch_fold(reinterpret_cast<const __half*>(X), s, M, K,
                                   reinterpret_cast<__half*>(Xout),
                                   reinterpret_cast<hipStream_t>(stream)));
}

awq_status awq_w4a16_matmul(const uint16_t* X, const uint32_t* qpacked, const float* scales,
                            const uint8_t* zeros, int M, int N, int K, int bits, int group,
                            uint16_t* Y, void* stream) {
  return matmul_impl(X, qpacked, scales, zeros, M, N, K, bits, group, Y, stream, 0, false);
}

awq_status awq_w4a16_matmul_kernel(const uint16_t* X, const uint32_t* qpacked, const float* scales,
                                   const uint8_t* zeros, int M, int N, int K, int bits, int group,
                                   uint16_t* Y, int kernel, void* stream) {
  return matmul_impl(X, qpacked, scales, zeros, M, N, K, bits, group, Y, stream, kernel, false);
}

size_t awq_w4a16_matmul_workspace_bytes(int M, int N, int K, int bits, int group) {
  int g = 0;
  if (M <= 0 || N <= 0 || check_group(K, bits, group, &g) != AWQ_OK) return 0;
  if (auto_decode(M, bits)) return bits == 4 ? awq::gemv_workspace_bytes(M, N, K) : 0;
  return awq::gemm_workspace_bytes(M, N, K, bits);
}

awq_status awq_w4a16_matmul_ws(const uint16_t* X, const uint32_t* qpacked, const float* scales,
                               const uint8_t* zeros, int M, int N, int K, int bits, int group,
                               uint16_t* Y, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return matmul_impl(X, qpacked, scales, zeros, M, N, K, bits, group, Y, stream, 0, false,
                     workspace, workspace_bytes);
}

awq_status awq_w4a16_matmul_noalloc(const uint16_t* X, const uint32_t* qpacked,
                                    const float* scales, const uint8_t* zeros, int M, int N, int K,
                                    int bits, int group, uint16_t* Y, void* stream) {
  return matmul_impl(X, qpacked, scales, zeros, M, N, K, bits, group, Y, stream, 0, false,
                     nullptr, 0, true);
}

awq_status awq_compact_group_params(const float* scales, const uint8_t* zeros, int N, int K,
                                    int group, uint16_t* scales16, uint32_t* zeros4,
                                    void* stream) {
  if (!scales || !zeros || !scales16 || !zeros4) return AWQ_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(scales) || !aligned16(zeros) || !aligned16(scales16) || !aligned16(zeros4))
    return AWQ_ERR_INVALID_ARG;
  int g = 0;
  awq_status st = check_group(K, 4, group, &g);
  if (st != AWQ_OK) return st;
  st = device_ready();
  if (st != AWQ_OK) return st;
  return from_hip(awq::launch_compact_params(scales, zeros, N, K / g, scales16, zeros4,
                                             reinterpret_cast<hipStream_t>(stream)));
}

awq_status awq_w4a16_matmul_compact(const uint16_t* X, const uint32_t* qpacked,
                                    const uint16_t* scales16, const uint32_t* zeros4, int M, int N,
                                    int K, int bits, int group, uint16_t* Y, int kernel,
                                    void* stream) {
  return matmul_impl(X, qpacked, scales16, zeros4, M, N, K, bits, group, Y, stream, kernel, true);
}

awq_status awq_w4a16_gate_up_silu(const uint16_t* X, const uint32_t* qg, const float* sg,
                                  const uint8_t* zg, const uint32_t* qu, const float* su,
                                  const uint8_t* zu, int M, int N, int K, int bits, int group,
                                  uint16_t* Y, void* stream) {
  if (!X || !qg || !sg || !zg || !qu || !su || !zu || !Y) return AWQ_ERR_INVALID_ARG;
  if (M <= 0 || N <= 0 || K <= 0) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(qg) || !aligned16(sg) || !aligned16(zg) || !aligned16(qu) ||
      !aligned16(su) || !aligned16(zu) || !aligned16(Y))
    return AWQ_ERR_INVALID_ARG;
  int g = 0;
  awq_status st = check_group(K, bits, group, &g);
  if (st != AWQ_OK) return st;
  if ((long long)M * K > (1LL << 31) || (long long)N * K > (1LL << 34)) return AWQ_ERR_UNSUPPORTED;
  st = device_ready();
  if (st != AWQ_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const __half* x = reinterpret_cast<const __half*>(X);
  __half* y = reinterpret_cast<__half*>(Y);
  hipError_t e = hipErrorNotSupported;
  if (M == 1)
    e = bits == 4 ? awq::launch_gate_up_w4_m1(x, qg, sg, zg, qu, su, zu, N, K, g, y, s)
                  : awq::launch_gate_up_w3_m1(x, qg, sg, zg, qu, su, zu, N, K, g, y, s);
  else if (M <= 4)
    e = awq::launch_gate_up_mt(x, qg, sg, zg, qu, su, zu, M, N, K, bits, g, y, s);
  if (e == hipErrorNotSupported && bits == 4 && M >= 2 && M <= 16) {
    (void)hipGetLastError();
    e = awq::launch_gemv_w4_mx(x, qg, sg, zg, M, N, K, g, y, s, qu, su, zu, false);
  }
  if (e == hipErrorNotSupported) {
    (void)hipGetLastError();
    e = awq::launch_gemm_gate_up(x, qg, sg, zg, qu, su, zu, M, N, K, bits, g, y, s);
  }
  return from_hip(e);
}

size_t awq_scale_search_workspace_bytes(int N, int K, int T, int n_alpha, int bits, int group) {
  int g = 0;
  if (N <= 0 || T <= 0 || T >= 8192 || n_alpha <= 0) return 0;
  if (check_group(K, bits, group, &g) != AWQ_OK) return 0;
  return awq::search_workspace_bytes(N, K, T, n_alpha, bits, g);
}

static awq_status awq_scale_search_joint_workspace_bytes_impl(const int* N, int n_layers, int K,
                                                             int T, int n_alpha, int bits,
                                                             int group, size_t* out) {
  *out = 0;
  if (!N || n_layers <= 0 || n_layers > kMaxLayers) return AWQ_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l)
    if (N[l] <= 0) return AWQ_ERR_INVALID_ARG;
  if (T <= 0 || n_alpha <= 0) return AWQ_ERR_INVALID_ARG;
  if (T >= 8192) return AWQ_ERR_UNSUPPORTED;
  int g = 0;
  const awq_status st = check_group(K, bits, group, &g);
  if (st != AWQ_OK) return st;
  *out = awq::search_workspace_bytes_joint(N, n_layers, K, T, n_alpha);
  return AWQ_OK;
}

awq_status awq_scale_search_joint(const uint16_t* const* W, const int* N, int n_layers,
                                  const uint16_t* Xcalib, int K, int T, const float* alpha_grid,
                                  int n_alpha, int bits, int group, int zero_point, float* s_out,
                                  double* loss_out, int* best_index, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!W || !N || !Xcalib || !alpha_grid || !s_out) return AWQ_ERR_INVALID_ARG;
  if (n_layers <= 0 || n_layers > kMaxLayers || K <= 0 || T <= 0 || n_alpha <= 0)
    return AWQ_ERR_INVALID_ARG;
  if (zero_point != 0 && zero_point != 1) return AWQ_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l)
    if (!W[l] || N[l] <= 0 || !aligned16(W[l])) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(Xcalib) || !aligned16(s_out)) return AWQ_ERR_INVALID_ARG;
  for (int i = 0; i < n_alpha; ++i)
    if (!(alpha_grid[i] >= 0.0f && alpha_grid[i] <= 1.0f)) return AWQ_ERR_INVALID_ARG;
  size_t need = 0;
  awq_status st =
      awq_scale_search_joint_workspace_bytes_impl(N, n_layers, K, T, n_alpha, bits, group, &need);
  if (st != AWQ_OK) return st;
  int g = 0;
  (void)check_group(K, bits, group, &g);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return AWQ_ERR_WORKSPACE;
  st = device_ready();
  if (st != AWQ_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // workspace head: alpha grid (float32), losses (float64), best index (int)
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* alpha_dev = reinterpret_cast<float*>(ws);
  const size_t a_bytes = ((size_t)n_alpha * 4 + 255) & ~(size_t)255;
  double* loss_dev = reinterpret_cast<double*>(ws + a_bytes);
  const size_t l_bytes = ((size_t)n_alpha * 8 + 255) & ~(size_t)255;
  int* best_dev = reinterpret_cast<int*>(ws + a_bytes + l_bytes);
  void* rest = ws + a_bytes + l_bytes + 256;

  hipError_t e = hipMemcpyAsync(alpha_dev, alpha_grid, (size_t)n_alpha * 4, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return AWQ_ERR_HIP;
  const __half* wl[kMaxLayers];
  for (int l = 0; l < n_layers; ++l) wl[l] = reinterpret_cast<const __half*>(W[l]);
  e = awq::launch_search_joint(wl, N, n_layers, reinterpret_cast<const __half*>(Xcalib), K, T,
                               alpha_dev, n_alpha, bits, g, zero_point != 0, rest, loss_dev,
                               best_dev, s_out, s);
  if (e != hipSuccess) return from_hip(e);
  int host_best = 0;
  if (loss_out) {
    e = hipMemcpyAsync(loss_out, loss_dev, (size_t)n_alpha * 8, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return AWQ_ERR_HIP;
  }
  e = hipMemcpyAsync(&host_best, best_dev, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return AWQ_ERR_HIP;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return AWQ_ERR_HIP;
  if (best_index) *best_index = host_best;
  return AWQ_OK;
}

size_t awq_scale_search_joint_workspace_bytes(const int* N, int n_layers, int K, int T,
                                              int n_alpha, int bits, int group) {
  size_t need = 0;
  (void)awq_scale_search_joint_workspace_bytes_impl(N, n_layers, K, T, n_alpha, bits, group,
                                                    &need);
  return need;
}

awq_status awq_scale_search_ex(const uint16_t* W, const uint16_t* Xcalib, int N, int K, int T,
                               const float* alpha_grid, int n_alpha, int bits, int group,
                               int zero_point, float* s_out, double* loss_out, int* best_index,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!W) return AWQ_ERR_INVALID_ARG;
  const uint16_t* wl[1] = {W};
  return awq_scale_search_joint(wl, &N, 1, Xcalib, K, T, alpha_grid, n_alpha, bits, group,
                                zero_point, s_out, loss_out, best_index, workspace,
                                workspace_bytes, stream);
}

awq_status awq_fold_norm_weight(const uint16_t* gamma, const float* s, int K, uint16_t* gamma_out,
                                void* stream) {
  if (!gamma || !s || !gamma_out) return AWQ_ERR_INVALID_ARG;
  if (K <= 0) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(gamma) || !aligned16(s) || !aligned16(gamma_out)) return AWQ_ERR_INVALID_ARG;
  const awq_status st = device_ready();
  if (st != AWQ_OK) return st;
  return from_hip(awq::launch_fold_norm_weight(reinterpret_cast<const __half*>(gamma), s, K,
                                               reinterpret_cast<__half*>(gamma_out),
                                               reinterpret_cast<hipStream_t>(stream)));
}

awq_status awq_rmsnorm(const uint16_t* X, const uint16_t* gamma, int M, int K, float eps,
                       uint16_t* Y, void* stream) {
  if (!X || !gamma || !Y) return AWQ_ERR_INVALID_ARG;
  if (M <= 0 || K <= 0 || !(eps >= 0.0f)) return AWQ_ERR_INVALID_ARG;
  if (K % 8 != 0 || K > awq::kRmsNormMaxK) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(gamma) || !aligned16(Y)) return AWQ_ERR_INVALID_ARG;
  const awq_status st = device_ready();
  if (st != AWQ_OK) return st;
  return from_hip(awq::launch_rmsnorm(reinterpret_cast<const __half*>(X),
                                      reinterpret_cast<const __half*>(gamma), M, K, eps,
                                      reinterpret_cast<__half*>(Y),
                                      reinterpret_cast<hipStream_t>(stream)));
}

awq_status awq_scale_search(const uint16_t* W, const uint16_t* Xcalib, int N, int K, int T,
                            const float* alpha_grid, int n_alpha, int bits, int group, float* s_out,
                            double* loss_out, int* best_index, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return awq_scale_search_ex(W, Xcalib, N, K, T, alpha_grid, n_alpha, bits, group, 1, s_out,
                             loss_out, best_index, workspace, workspace_bytes, stream);
}

}  // extern "C"
