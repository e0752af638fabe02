// Offline steps on the device: the AWQ channel scale from calibration activations and
// the fold + round-to-nearest group quantization + 4-bit packing of a weight matrix.
//
// Rules: "Quantization Paradigms for Edge Inference", section 3 (channel scale from
// calibration activation magnitudes; W' = W diag(s)); edgesiliconlab ?p=2015, section
// "What Is the Core Difference Between AWQ and GPTQ Quantization?" (plain
// round-to-nearest on the scaled matrix); "The Ultimate Guide to Quantized LLMs:
// GPTQ", section "Understanding Quantized Model Compression" (a scale and a zero point
// per block). Every floating-point decision that picks an integer code is taken in
// float64 so that it is exact for binary16 inputs (see the notes at each step).
#include "awq_internal.hpp"

namespace awq {
namespace {

// binary16 RNE of sqrt(m), exact even where the float64 square root is off by an ulp:
// the candidate is checked against the squares of its two neighbouring midpoints,
// which have at most 12 significant bits, so their squares are exact in float64.
__device__ uint16_t sqrt_to_f16_rn(double m) {
  uint16_t h = f64_to_f16_rn(__builtin_sqrt(m));
  if (h >= 0x7C00u || h == 0) return h;
  const double a = f16_bits_to_f64(h);
  const double lo = f16_bits_to_f64(static_cast<uint16_t>(h - 1));
  const double hi = f16_bits_to_f64(static_cast<uint16_t>(h + 1));
  const double mlo = 0.5 * (lo + a), mhi = 0.5 * (a + hi);
  const double mlo2 = mlo * mlo, mhi2 = mhi * mhi;
  if (m < mlo2 || (m == mlo2 && (h & 1))) return static_cast<uint16_t>(h - 1);
  if (m > mhi2 || (m == mhi2 && (h & 1))) return static_cast<uint16_t>(h + 1);
  return h;
}

__global__ void channel_scale_kernel(const uint16_t* __restrict__ x_cal, int rows, int K,
                                     double alpha, uint16_t* __restrict__ s_c,
                                     uint16_t* __restrict__ inv_s_c) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  // Sum of binary16 magnitudes: every term is a multiple of 2^-24 below 2^16, so up to
  // 8192 terms sum exactly in float64 in any order.
  double sum = 0.0;
  for (int r = 0; r < rows; ++r) {
    sum += __builtin_fabs(f16_bits_to_f64(x_cal[static_cast<int64_t>(r) * K + k]));
  }
  const double m = sum / rows;
  uint16_t s;
  if (m == 0.0) {
    s = 0x3C00;  // 1.0
  } else if (alpha == 0.5) {
    s = sqrt_to_f16_rn(m);
  } else if (alpha == 0.0) {
    s = 0x3C00;
  } else if (alpha == 1.0) {
    s = f64_to_f16_rn(m);
  } else {
    s = f64_to_f16_rn(pow(m, alpha));
  }
  s_c[k] = s;
  if (inv_s_c) inv_s_c[k] = f64_to_f16_rn(1.0 / f16_bits_to_f64(s));
}

// One workgroup quantizes 8 consecutive rows of one group: TPR = min(group / 8, 16)
// threads per row, each owning every TPR-th 8-channel vector (one output word each).
// Rows sit in contiguous lanes so that the group min/max reduce within a wavefront.
template <int TPR>
__global__ void __launch_bounds__(8 * TPR)
pack_kernel(const uint16_t* __restrict__ w, const uint16_t* __restrict__ s_c, int K, int group,
            int fmt, int32_t* __restrict__ qweight, uint16_t* __restrict__ scales,
            int32_t* __restrict__ qzeros, int N) {
  // a block quantizes one group of 8 rows; TPR threads per row, each taking the
  // 8-channel vectors t, t + TPR, ... of the group (group / (8 TPR) of them)
  const int row_in_blk = threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int n = blockIdx.x * 8 + row_in_blk;
  const int g = blockIdx.y;
  const int nvec = group / (8 * TPR);
  const int64_t row_base = static_cast<int64_t>(n) * K + static_cast<int64_t>(g) * group;

  // Fold: binary16 x binary16 is exact in float64; one rounding to binary16.
  auto fold8 = [&](int j, double v[8]) {
    const int k = g * group + (t + j * TPR) * 8;
    const uint4 wraw = *reinterpret_cast<const uint4*>(w + row_base + (t + j * TPR) * 8);
    uint4 sraw = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
    if (s_c) sraw = *reinterpret_cast<const uint4*>(s_c + k);
    const uint32_t wv[4] = {wraw.x, wraw.y, wraw.z, wraw.w};
    const uint32_t sv[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t wb = static_cast<uint16_t>(wv[i >> 1] >> (16 * (i & 1)));
      const uint16_t sb = static_cast<uint16_t>(sv[i >> 1] >> (16 * (i & 1)));
      v[i] = f16_bits_to_f64(f64_to_f16_rn(f16_bits_to_f64(wb) * f16_bits_to_f64(sb)));
    }
  };

  double vmin = 0.0, vmax = 0.0;
  for (int j = 0; j < nvec; ++j) {
    double v[8];
    fold8(j, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vmin = (j == 0 && i == 0) ? v[i] : __builtin_fmin(vmin, v[i]);
      vmax = (j == 0 && i == 0) ? v[i] : __builtin_fmax(vmax, v[i]);
    }
  }
  // group extrema across the TPR lanes of this row (binary16 values: exact in float32)
  float fmin = static_cast<float>(vmin), fmax = static_cast<float>(vmax);
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) {
    fmin = __builtin_fminf(fmin, __shfl_xor(fmin, off, TPR));
    fmax = __builtin_fmaxf(fmax, __shfl_xor(fmax, off, TPR));
  }
  vmin = fmin;
  vmax = fmax;

  // Scale and zero. The range (hi - lo) of two binary16 values is exact in float64.
  // A binary16 midpoint is a multiple of 2^-25, the range a multiple of 2^-24, so the
  // quotient range/15 is either exactly a midpoint or at least 2^-45 (relative) away
  // from one: a float64 quotient then rounds to binary16 exactly as the real quotient.
  double s;
  int z;
  if (fmt == 0) {
    const double lo = __builtin_fmin(vmin, 0.0), hi = __builtin_fmax(vmax, 0.0);
    s = f16_bits_to_f64(f64_to_f16_rn((hi - lo) / 15.0));
    s = __builtin_fmax(s, 5.9604644775390625e-08);  // 2^-24
    z = static_cast<int>(__builtin_rint(-lo / s));
    z = z < 0 ? 0 : (z > 15 ? 15 : z);
  } else {
    const double a = __builtin_fmax(__builtin_fabs(vmin), __builtin_fabs(vmax));
    s = f16_bits_to_f64(f64_to_f16_rn(a / 7.0));
    s = __builtin_fmax(s, 5.9604644775390625e-08);
    z = 8;
  }
  // Codes (the fold recomputed: cheaper than holding a whole group per thread). v/s is
  // either an exact tie (k + 1/2) or at least 2^-41 away from one, so the float64
  // quotient rounds half-to-even exactly like the real quotient.
  for (int j = 0; j < nvec; ++j) {
    double v[8];
    fold8(j, v);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int q = static_cast<int>(__builtin_rint(v[i] / s)) + z;
      q = q < 0 ? 0 : (q > 15 ? 15 : q);
      word |= static_cast<uint32_t>(q) << (4 * i);
    }
    if (n < N)
      qweight[static_cast<int64_t>(n) * (K / 8) + (static_cast<int64_t>(g) * group + (t + j * TPR) * 8) / 8] =
          static_cast<int32_t>(word);
  }
  if (n < N && t == 0) scales[static_cast<int64_t>(g) * N + n] = f64_to_f16_rn(s);
  if (fmt == 0) {
    __shared__ uint32_t zsh[8];
    if (t == 0) zsh[row_in_blk] = static_cast<uint32_t>(z);
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t zw = 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) zw |= zsh[r] << (4 * r);
      qzeros[static_cast<int64_t>(g) * (N / 8) + blockIdx.x] = static_cast<int32_t>(zw);
    }
  }
}

}  // namespace

hipError_t launch_channel_scale(const uint16_t* x_cal, int64_t rows, int64_t K, double alpha,
                                uint16_t* s_c, uint16_t* inv_s_c, hipStream_t st) {
  const int threads = 256;
  const unsigned blocks = static_cast<unsigned>((K + threads - 1) / threads);
  hipLaunchKernelGGL(channel_scale_kernel, dim3(blocks), dim3(threads), 0, st, x_cal,
                     static_cast<int>(rows), static_cast<int>(K), alpha, s_c, inv_s_c);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w, const uint16_t* s_c, int64_t N, int64_t K,
                       int32_t group, int32_t fmt, int32_t* qweight, uint16_t* scales,
                       int32_t* qzeros, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(N / 8), static_cast<unsigned>(K / group));
  const int k = static_cast<int>(K), n = static_cast<int>(N), g = static_cast<int>(group);
  if (group == 32) {
    hipLaunchKernelGGL(pack_kernel<4>, grid, dim3(32), 0, st, w, s_c, k, g, fmt, qweight,
                       scales, qzeros, n);
  } else if (group == 64) {
    hipLaunchKernelGGL(pack_kernel<8>, grid, dim3(64), 0, st, w, s_c, k, g, fmt, qweight,
                       scales, qzeros, n);
  } else if (group % kGroup == 0) {
    hipLaunchKernelGGL(pack_kernel<16>, grid, dim3(128), 0, st, w, s_c, k, g, fmt, qweight,
                       scales, qzeros, n);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace awq
