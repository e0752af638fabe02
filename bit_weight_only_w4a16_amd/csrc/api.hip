// C ABI entry points: argument checks (all before any launch), then the launchers.
#include "../../include/awq.h"
#include "awq_internal.hpp"

#include <math.h>

namespace {

using awq::kGroup;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

// Shape checks shared by every weight entry point.
int check_shape(int64_t N, int64_t K, int32_t group, int32_t fmt) {
  if (N <= 0 || K <= 0 || group <= 0) return AWQ_ERR_INVALID_ARG;
  if (fmt != AWQ_FMT_ASYM && fmt != AWQ_FMT_SYM8) return AWQ_ERR_INVALID_ARG;
  if (N % 8 != 0 || K % 8 != 0 || K % group != 0) return AWQ_ERR_INVALID_ARG;
  // groups of 32 or 64 channels, or any multiple of 128 that divides K (per-channel
  // included: group == K); K itself a multiple of 128 (the unit width)
  if (K % kGroup != 0) return AWQ_ERR_UNSUPPORTED;
  if (group != 32 && group != 64 && group % kGroup != 0) return AWQ_ERR_UNSUPPORTED;
  if (N * K >= (int64_t{1} << 31) || N >= (int64_t{1} << 30) || K > (int64_t{1} << 22))
    return AWQ_ERR_UNSUPPORTED;
  return AWQ_OK;
}

}  // namespace

namespace awq {

// Argument checks of the product entry points (also used by awq_gemm_noalloc).
int check_product(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
                  int64_t N, int64_t K, int32_t group, int32_t fmt, const uint16_t* y,
                  const void* ws, size_t ws_bytes) {
  int rc = check_shape(N, K, group, fmt);
  if (rc != AWQ_OK) return rc;
  if (M < 0 || M >= (int64_t{1} << 30)) return AWQ_ERR_INVALID_ARG;
  if (M > 0 && (x == nullptr || packed == nullptr || y == nullptr)) return AWQ_ERR_INVALID_ARG;
  if (ws == nullptr && ws_bytes != 0) return AWQ_ERR_INVALID_ARG;
  if (M * K >= (int64_t{1} << 32) || M * N >= (int64_t{1} << 32)) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(inv_s_c) || !aligned16(packed) || !aligned16(y) ||
      !aligned16(ws))
    return AWQ_ERR_MISALIGNED;
  if (ws != nullptr && ws_bytes < awq_workspace_bytes(M, N, K, group)) return AWQ_ERR_WORKSPACE;
  return AWQ_OK;
}

}  // namespace awq

namespace {
using awq::check_product;
}  // namespace

extern "C" {

const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_OK: return "ok";
    case AWQ_ERR_INVALID_ARG: return "invalid argument (NULL buffer, bad size or enum value)";
    case AWQ_ERR_UNSUPPORTED: return "unsupported request (group size, M range or size limit)";
    case AWQ_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case AWQ_ERR_WORKSPACE: return "packed or workspace buffer too small";
    case AWQ_ERR_HIP: return "HIP runtime rejected a kernel launch";
    default: return "unknown status";
  }
}

int awq_layout_version(void) { return awq::kLayoutVersion; }

int awq_channel_scale(const uint16_t* x_cal, int64_t rows, int64_t K, double alpha,
                      uint16_t* s_c, uint16_t* inv_s_c, hipStream_t stream) {
  if (x_cal == nullptr || s_c == nullptr) return AWQ_ERR_INVALID_ARG;
  if (rows < 1 || rows > 8192 || K < 1 || K >= (int64_t{1} << 30)) return AWQ_ERR_INVALID_ARG;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return AWQ_ERR_INVALID_ARG;
  if (rows * K >= (int64_t{1} << 40)) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(x_cal) || !aligned16(s_c) || !aligned16(inv_s_c)) return AWQ_ERR_MISALIGNED;
  return hip_status(awq::launch_channel_scale(x_cal, rows, K, alpha, s_c, inv_s_c, stream));
}

int awq_pack(const uint16_t* w, const uint16_t* s_c, int64_t N, int64_t K, int32_t group,
             int32_t fmt, int32_t* qweight, uint16_t* scales, int32_t* qzeros,
             hipStream_t stream) {
  int rc = check_shape(N, K, group, fmt);
  if (rc != AWQ_OK) return rc;
  if (w == nullptr || qweight == nullptr || scales == nullptr) return AWQ_ERR_INVALID_ARG;
  if ((fmt == AWQ_FMT_ASYM) != (qzeros != nullptr)) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(s_c) || !aligned16(qweight) || !aligned16(scales) ||
      !aligned16(qzeros))
    return AWQ_ERR_MISALIGNED;
  return hip_status(
      awq::launch_pack(w, s_c, N, K, group, fmt, qweight, scales, qzeros, stream));
}

size_t awq_repacked_bytes(int64_t N, int64_t K, int32_t group, int32_t fmt) {
  if (check_shape(N, K, group, fmt) != AWQ_OK) return 0;
  return static_cast<size_t>(awq::make_layout(N, K, group, fmt).total_bytes);
}

int awq_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
               int64_t N, int64_t K, int32_t group, int32_t fmt, void* packed,
               size_t packed_bytes, hipStream_t stream) {
  int rc = check_shape(N, K, group, fmt);
  if (rc != AWQ_OK) return rc;
  if (qweight == nullptr || scales == nullptr || packed == nullptr) return AWQ_ERR_INVALID_ARG;
  if ((fmt == AWQ_FMT_ASYM) != (qzeros != nullptr)) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(qweight) || !aligned16(scales) || !aligned16(qzeros) || !aligned16(packed))
    return AWQ_ERR_MISALIGNED;
  if (packed_bytes < awq_repacked_bytes(N, K, group, fmt)) return AWQ_ERR_WORKSPACE;
  return hip_status(
      awq::launch_repack(qweight, scales, qzeros, N, K, group, fmt, packed, stream));
}

int awq_dequant(const void* w, const uint16_t* scales, const int32_t* qzeros, int32_t layout,
                int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* w_out,
                hipStream_t stream) {
  int rc = check_shape(N, K, group, fmt);
  if (rc != AWQ_OK) return rc;
  if (w == nullptr || w_out == nullptr) return AWQ_ERR_INVALID_ARG;
  if (layout == AWQ_LAYOUT_CANONICAL) {
    if (scales == nullptr) return AWQ_ERR_INVALID_ARG;
    if ((fmt == AWQ_FMT_ASYM) != (qzeros != nullptr)) return AWQ_ERR_INVALID_ARG;
  } else if (layout == AWQ_LAYOUT_GFX950) {
    if (scales != nullptr || qzeros != nullptr) return AWQ_ERR_INVALID_ARG;
  } else {
    return AWQ_ERR_INVALID_ARG;
  }
  if (!aligned16(w) || !aligned16(scales) || !aligned16(qzeros) || !aligned16(w_out))
    return AWQ_ERR_MISALIGNED;
  if (layout == AWQ_LAYOUT_CANONICAL) {
    return hip_status(awq::launch_dequant_canonical(static_cast<const int32_t*>(w), scales,
                                                    qzeros, N, K, group, fmt, w_out, stream));
  }
  return hip_status(awq::launch_dequant_packed(w, N, K, group, fmt, w_out, stream));
}

size_t awq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (M <= 0 || check_shape(N, K, group, AWQ_FMT_ASYM) != AWQ_OK) return 0;
  const size_t a = M <= 16 ? awq::gemv_workspace_bytes(M, N, K) : 0;
  const size_t b = awq::gemm_workspace_bytes(M, N, K);
  return a > b ? a : b;
}

int awq_gemv(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
             int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y, void* ws,
             size_t ws_bytes, hipStream_t stream) {
  int rc = check_product(x, inv_s_c, packed, M, N, K, group, fmt, y, ws, ws_bytes);
  if (rc != AWQ_OK) return rc;
  if (M > 16) return AWQ_ERR_UNSUPPORTED;
  if (M == 0) return AWQ_OK;
  return hip_status(awq::launch_gemv(x, inv_s_c, packed, M, N, K, group, fmt, y, ws, ws_bytes, stream));
}

int awq_gemm(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
             int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y, void* ws,
             size_t ws_bytes, hipStream_t stream) {
  int rc = check_product(x, inv_s_c, packed, M, N, K, group, fmt, y, ws, ws_bytes);
  if (rc != AWQ_OK) return rc;
  if (M == 0) return AWQ_OK;
  return hip_status(awq::launch_gemm(x, inv_s_c, packed, M, N, K, group, fmt, y, ws, ws_bytes, stream));
}

size_t awq_chain_state_bytes(void) { return awq::chain_state_bytes(); }

int awq_gemv_chain(const awq_chain_layer* layers, int32_t n_layers, void* state,
                   hipStream_t stream) {
  if (n_layers < 0) return AWQ_ERR_INVALID_ARG;
  if (n_layers == 0) return AWQ_OK;
  if (layers == nullptr || state == nullptr) return AWQ_ERR_INVALID_ARG;
  if (n_layers > awq::chain_max_layers()) return AWQ_ERR_UNSUPPORTED;
  for (int i = 0; i < n_layers; ++i) {
    const awq_chain_layer& l = layers[i];
    int rc = check_shape(l.N, l.K, l.group, l.fmt);
    if (rc != AWQ_OK) return rc;
    if (l.packed == nullptr || l.y == nullptr) return AWQ_ERR_INVALID_ARG;
    if (l.src < -1 || l.src >= i) return AWQ_ERR_INVALID_ARG;
    if (l.src == -1 && l.x == nullptr) return AWQ_ERR_INVALID_ARG;
    if (l.src >= 0 && layers[l.src].N != l.K) return AWQ_ERR_INVALID_ARG;
    // every wavefront of a workgroup takes at least one 128-channel unit of a tile, and
    // the staged inputs fit in LDS
    if (l.group < kGroup || l.K < awq::chain_min_k() || l.K > awq::chain_max_k()) return AWQ_ERR_UNSUPPORTED;
    if ((l.src == -1 && !aligned16(l.x)) || !aligned16(l.inv_s_c) || !aligned16(l.packed) ||
        !aligned16(l.y))
      return AWQ_ERR_MISALIGNED;
  }
  if (!aligned16(state)) return AWQ_ERR_MISALIGNED;
  return hip_status(awq::launch_chain(layers, n_layers, static_cast<uint32_t*>(state), stream));
}

size_t awq_scale_search_workspace_bytes(int64_t rows, int64_t N, int64_t K, int32_t group,
                                        int32_t fmt) {
  if (rows < 1 || rows > 256 || check_shape(N, K, group, fmt) != AWQ_OK) return 0;
  return awq::scale_search_workspace_bytes(rows, N, K, group, fmt);
}

int awq_scale_search(const uint16_t* w, const uint16_t* x_cal, int64_t rows, int64_t N,
                     int64_t K, int32_t group, int32_t fmt, int32_t grid, double* losses,
                     double* best_alpha, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(N, K, group, fmt);
  if (rc != AWQ_OK) return rc;
  if (w == nullptr || x_cal == nullptr || losses == nullptr || best_alpha == nullptr ||
      ws == nullptr)
    return AWQ_ERR_INVALID_ARG;
  if (rows < 1 || rows > 256 || grid < 1 || grid > 1000) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(x_cal) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(losses) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(best_alpha) & 7u) != 0)
    return AWQ_ERR_MISALIGNED;
  if (ws_bytes < awq::scale_search_workspace_bytes(rows, N, K, group, fmt)) return AWQ_ERR_WORKSPACE;
  return hip_status(awq::launch_scale_search(w, x_cal, rows, N, K, group, fmt, grid, losses,
                                             best_alpha, ws, stream));
}

}  // extern "C"
