// AWQ scale search: the exponent alpha of s = (mean |X_cal|)^alpha that minimises the
// output error of the quantized layer on the calibration rows ("Quantization Paradigms
// for Edge Inference: AWQ, GPTQ, and FP8 Matrix Cores", section 3, second equation:
// s* = argmin_s || W X - Q(W diag(s)) diag(s)^-1 X ||). The pages leave the search space
// open; it is the grid alpha = i / grid, i = 0 .. grid, ties to the smallest alpha.
//
// Every candidate goes through the library's own kernels, exactly as it would be
// deployed: channel scale -> fold + RTN + pack -> gfx950 repack -> matrix-core product
// of the calibration rows (X' = binary16(X * inv_s_c), binary16 output). The reference
// X_cal . W^T is formed once, in float32 on the matrix cores from the unquantized
// binary16 weights. The squared error is summed in float64 with a fixed reduction
// order, so the losses (and the choice) are the same bits on every call.
#include "awq_internal.hpp"

namespace awq {
namespace {

constexpr int kLossBlocks = 256;  // partial sums per loss (fixed: the reduction order)

// y[r][n] = sum_k x[r][k] * w[n][k] in float32; blockIdx.y takes rows 32 y .. 32 y + 31
// as two 16-row matrix tiles. One wavefront per 16 output columns; the plain row-major
// operands are the matrix-core fragments directly (lane l: row / column l % 16, channels
// 8 (l / 16)..+7 of each 32-channel step). Rows past `rows` and columns past N read as 0
// and are not stored.
__global__ void __launch_bounds__(256) dense_ref_kernel(const uint16_t* x, const uint16_t* w,
                                                        int rows, int N, int K, float* y) {
  const int row0 = 32 * blockIdx.y;
  x += static_cast<int64_t>(row0) * K;
  y += static_cast<int64_t>(row0) * N;
  rows = min(rows - row0, 32);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, p = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  if (n0 >= N) return;  // whole wavefront
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, static_cast<uint32_t>(N) * K * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(rows) * K * 2);
  const int n = n0 + r;
  const uint32_t woff = n < N ? static_cast<uint32_t>(n * K + 8 * p) * 2 : kNoLoad;
  const uint32_t xoff0 = r < rows ? static_cast<uint32_t>(r * K + 8 * p) * 2 : kNoLoad;
  const uint32_t xoff1 = r + 16 < rows ? static_cast<uint32_t>((r + 16) * K + 8 * p) * 2 : kNoLoad;
  float4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < K; k0 += 32) {
    const uint32_t so = static_cast<uint32_t>(k0) * 2;
    const uint4 b = buf_load16(rw, woff, so);
    const uint4 a0 = buf_load16(rx, xoff0, so);
    const uint4 a1 = buf_load16(rx, xoff1, so);
    const half8_t bf = __builtin_bit_cast(half8_t, b);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a0), bf, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a1), bf, acc1, 0, 0, 0);
  }
  // element q of acc is row 4 p + q (tile 0) or 16 + 4 p + q (tile 1), column r
  if (n < N) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m0 = 4 * p + q, m1 = 16 + 4 * p + q;
      if (m0 < rows) y[static_cast<int64_t>(m0) * N + n] = acc0[q];
      if (m1 < rows) y[static_cast<int64_t>(m1) * N + n] = acc1[q];
    }
  }
}

// partial[b] = sum over elements i = b, b + kLossBlocks * 256, ... of (ref - y)^2 in
// float64: thread t of block b takes i = b * 256 + t + j * kLossBlocks * 256, then the
// block adds its 256 values in a fixed tree order.
__global__ void __launch_bounds__(256) loss_partial_kernel(const float* ref, const uint16_t* y,
                                                           int64_t total, double* partial) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(kLossBlocks) * 256) {
    const double d = static_cast<double>(ref[i]) - f16_bits_to_f64(y[i]);
    acc += d * d;
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// loss = sqrt(sum of the partials, in block order)
__global__ void loss_final_kernel(const double* partial, double* loss) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double s = 0.0;
  for (int b = 0; b < kLossBlocks; ++b) s += partial[b];
  *loss = sqrt(s);
}

// best = i / grid for the first i with the smallest loss
__global__ void argmin_kernel(const double* losses, int grid, double* best) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int bi = 0;
  for (int i = 1; i <= grid; ++i)
    if (losses[i] < losses[bi]) bi = i;
  *best = static_cast<double>(bi) / grid;
}

inline int64_t align256(int64_t b) { return (b + 255) & ~int64_t{255}; }

struct SearchLayout {
  int64_t s_c, inv, qweight, scales, qzeros, packed, ref, yq, gemm_ws, partial, total;
  int64_t packed_bytes, gemm_ws_bytes;
};

SearchLayout search_layout(int64_t rows, int64_t N, int64_t K, int32_t group, int32_t fmt) {
  SearchLayout L;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.s_c = take(2 * K);
  L.inv = take(2 * K);
  L.qweight = take(N * K / 2);
  L.scales = take(2 * (K / group) * N);
  L.qzeros = take(fmt == 0 ? (K / group) * N / 2 : 0);
  L.packed_bytes = make_layout(N, K, group, fmt).total_bytes;
  L.packed = take(L.packed_bytes);
  L.ref = take(4 * rows * N);
  L.yq = take(2 * rows * N);
  L.gemm_ws_bytes = static_cast<int64_t>(gemm_workspace_bytes(rows, N, K));
  L.gemm_ws = take(L.gemm_ws_bytes);
  L.partial = take(8 * kLossBlocks);
  L.total = o;
  return L;
}

}  // namespace

size_t scale_search_workspace_bytes(int64_t rows, int64_t N, int64_t K, int32_t group,
                                    int32_t fmt) {
  return static_cast<size_t>(search_layout(rows, N, K, group, fmt).total);
}

hipError_t launch_scale_search(const uint16_t* w, const uint16_t* x_cal, int64_t rows,
                               int64_t N, int64_t K, int32_t group, int32_t fmt, int32_t grid,
                               double* losses, double* best_alpha, void* ws, hipStream_t st) {
  const SearchLayout L = search_layout(rows, N, K, group, fmt);
  unsigned char* base = static_cast<unsigned char*>(ws);
  uint16_t* s_c = reinterpret_cast<uint16_t*>(base + L.s_c);
  uint16_t* inv = reinterpret_cast<uint16_t*>(base + L.inv);
  int32_t* qweight = reinterpret_cast<int32_t*>(base + L.qweight);
  uint16_t* scales = reinterpret_cast<uint16_t*>(base + L.scales);
  int32_t* qzeros = fmt == 0 ? reinterpret_cast<int32_t*>(base + L.qzeros) : nullptr;
  void* packed = base + L.packed;
  float* ref = reinterpret_cast<float*>(base + L.ref);
  uint16_t* yq = reinterpret_cast<uint16_t*>(base + L.yq);
  void* gws = L.gemm_ws_bytes > 0 ? base + L.gemm_ws : nullptr;
  double* partial = reinterpret_cast<double*>(base + L.partial);

  hipLaunchKernelGGL(dense_ref_kernel,
                     dim3(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>((rows + 31) / 32)),
                     dim3(256), 0,
                     st, x_cal, w, static_cast<int>(rows), static_cast<int>(N),
                     static_cast<int>(K), ref);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i <= grid; ++i) {
    const double alpha = static_cast<double>(i) / grid;
    if ((e = launch_channel_scale(x_cal, rows, K, alpha, s_c, inv, st)) != hipSuccess) return e;
    if ((e = launch_pack(w, s_c, N, K, group, fmt, qweight, scales, qzeros, st)) != hipSuccess) return e;
    if ((e = launch_repack(qweight, scales, qzeros, N, K, group, fmt, packed, st)) != hipSuccess) return e;
    if ((e = launch_gemm(x_cal, inv, packed, rows, N, K, group, fmt, yq, gws,
                         static_cast<size_t>(L.gemm_ws_bytes), st)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(loss_partial_kernel, dim3(kLossBlocks), dim3(256), 0, st, ref, yq,
                       rows * N, partial);
    hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(64), 0, st, partial, losses + i);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(argmin_kernel, dim3(1), dim3(64), 0, st, losses, grid, best_alpha);
  return hipGetLastError();
}

}  // namespace awq
