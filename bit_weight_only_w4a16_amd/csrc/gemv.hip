// Decode product y[M, N] = X' . deq(Wq)^T for 1 <= M <= 8 on gfx950.
//
// At batch 1 the product reads every weight once and does two flops per weight, so it
// is bound by memory bandwidth (edgesiliconlab ?p=2015, section "The Mathematics of
// Memory Bandwidth Saturation"; section "GEMM vs. GEMV Kernels and Batch Size
// Dynamics"). The kernel is built around streaming the 4-bit codes at full HBM rate:
//
//  * a workgroup owns one 16-row tile and the whole of K, so no partial sums leave
//    the workgroup (no split-K workspace, no atomics, no cross-XCD cache traffic);
//  * its wavefronts take interleaved 128-channel groups; for each group one wavefront
//    load moves a whole 1 KiB unit (one 128-bit load per lane, fully coalesced), and the
//    loads of the next batch of groups are issued before the current batch is consumed;
//  * dequantization is folded into the dot products: a nibble OR-ed into binary16 1024
//    (or 64) is (off + q) exactly, v_dot2_f32_f16 accumulates X' * (off + q) in float32,
//    and per group y += s * (acc - O - z * S), where O = sum X' * off and S = sum X' over
//    the lane's 32 channels are computed once per workgroup into LDS. That is 5 VALU ops
//    per 8 weights to unpack plus 4 per 8 weights and row for the products;
//  * X' = binary16(X * inv_s_c) is staged in LDS once per workgroup; the 16 lanes that
//    share a channel slice read it with the same address (LDS broadcast);
//  * the four 32-channel slices of a row are summed with two cross-lane shuffles, the
//    wavefronts through LDS, and one thread per (row, output) writes y.
#include "awq_internal.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace awq {
namespace {

constexpr int kLdsBudget = 61440;  // bytes of LDS a workgroup may use for X', O and S

struct GemvArgs {
  const uint16_t* x;
  const uint16_t* inv;
  const uint8_t* packed;
  uint16_t* y;
  int64_t scales_off;
  int64_t zeros_off;  // < 0: symmetric format (zero 8)
  int N, K, n_groups, phase_groups;
};

// X' for channels [k0, k0 + nk) of every row into xs[m][nk], and O, S for every
// 32-channel slice into osum/ssum[m][nk / 32]. A thread converts 8 channels; the 4
// threads of a slice are consecutive lanes and add their partial sums with shuffles.
// Channel k of a word has offset 1024 if k % 8 is in {0, 1, 4, 5}, else 64.
template <int M, int NT>
__device__ __forceinline__ void stage_phase(const GemvArgs& a, int k0, int nk, _Float16* xs,
                                            float* osum, float* ssum) {
  const int vec_per_row = nk / 8;  // a multiple of 16
  const half2_t one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  const half2_t o1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  const half2_t o64 = {static_cast<_Float16>(64.0f), static_cast<_Float16>(64.0f)};
  for (int i = threadIdx.x; i < M * vec_per_row; i += NT) {
    const int m = i / vec_per_row, v = i - m * vec_per_row;
    uint4 val = *reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(m) * a.K + k0 + 8 * v);
    if (a.inv) {
      const uint4 iv = *reinterpret_cast<const uint4*>(a.inv + k0 + 8 * v);
      const uint32_t xw[4] = {val.x, val.y, val.z, val.w};
      const uint32_t iw[4] = {iv.x, iv.y, iv.z, iv.w};
      uint32_t ow[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half2_t xh = as_h2(xw[j]), ih = as_h2(iw[j]);
        half2_t rr;
        rr.x = static_cast<_Float16>(static_cast<float>(xh.x) * static_cast<float>(ih.x));
        rr.y = static_cast<_Float16>(static_cast<float>(xh.y) * static_cast<float>(ih.y));
        ow[j] = as_u32(rr);
      }
      val = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
    *reinterpret_cast<uint4*>(xs + m * nk + 8 * v) = val;
    float sv = __builtin_amdgcn_fdot2(as_h2(val.x), one2, 0.0f, false);
    sv = __builtin_amdgcn_fdot2(as_h2(val.y), one2, sv, false);
    sv = __builtin_amdgcn_fdot2(as_h2(val.z), one2, sv, false);
    sv = __builtin_amdgcn_fdot2(as_h2(val.w), one2, sv, false);
    float ov = __builtin_amdgcn_fdot2(as_h2(val.x), o1024, 0.0f, false);
    ov = __builtin_amdgcn_fdot2(as_h2(val.y), o64, ov, false);
    ov = __builtin_amdgcn_fdot2(as_h2(val.z), o1024, ov, false);
    ov = __builtin_amdgcn_fdot2(as_h2(val.w), o64, ov, false);
    sv += __shfl_xor(sv, 1, 4);
    ov += __shfl_xor(ov, 1, 4);
    sv += __shfl_xor(sv, 2, 4);
    ov += __shfl_xor(ov, 2, 4);
    if ((v & 3) == 0) {
      const int e = m * (nk / 32) + (v >> 2);
      ssum[e] = sv;
      osum[e] = ov;
    }
  }
  __syncthreads();
}

template <int M, int WAVES, int BATCH>
__global__ void __launch_bounds__(WAVES * 64) gemv_kernel(GemvArgs a) {
  constexpr int NT = WAVES * 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int t = blockIdx.x;
  // the wavefront index is uniform: keep it (and every group index) in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, p = lane >> 4;
  const int ng = a.n_groups;

  _Float16* xs = reinterpret_cast<_Float16*>(smem);
  float* osum = reinterpret_cast<float*>(smem + 2 * M * a.phase_groups * kGroup);
  float* ssum = osum + M * a.phase_groups * 4;
  float* red = ssum + M * a.phase_groups * 4;  // [WAVES][M][16]

  // buffer resources over this tile's codes, scales and zeros: the per-group offset is
  // wavefront-uniform (SGPR), the per-lane offset constant (VGPR)
  const __amdgpu_buffer_rsrc_t rcodes =
      make_rsrc(a.packed + static_cast<int64_t>(t) * ng * kUnitBytes, ng * kUnitBytes);
  const __amdgpu_buffer_rsrc_t rscales =
      make_rsrc(a.packed + a.scales_off + static_cast<int64_t>(t) * ng * (2 * kTileN), ng * 2 * kTileN);
  const bool asym = a.zeros_off >= 0;
  const __amdgpu_buffer_rsrc_t rzeros =
      make_rsrc(a.packed + (asym ? a.zeros_off : 0) + static_cast<int64_t>(t) * ng * 8, ng * 8);
  const uint32_t lane_code = 16u * lane, lane_scale = 2u * r, lane_zero = 4u * (r >> 3);
  const int zshift = 4 * (r & 7);

  float yacc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) yacc[m] = 0.0f;

  struct Batch {
    uint4 c[BATCH];
    uint32_t s[BATCH], z[BATCH];
  };
  auto load = [&](Batch& b, int ph0, int jb, int nj) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (jb + u < nj) {
        const uint32_t g = static_cast<uint32_t>(ph0 + wave + WAVES * (jb + u));
        b.c[u] = buf_load16(rcodes, lane_code, g * kUnitBytes);
        b.s[u] = buf_load2(rscales, lane_scale, g * (2 * kTileN));
        b.z[u] = asym ? buf_load4(rzeros, lane_zero, g * 8) : 0u;
      }
    }
  };
  auto compute = [&](const Batch& b, int jb, int nj, int ngp, int nk) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (jb + u < nj) {
        const int gl = wave + WAVES * (jb + u);
        const _Float16* xg = xs + gl * kGroup + 32 * p;
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
        const uint32_t words[4] = {b.c[u].x, b.c[u].y, b.c[u].z, b.c[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const Pairs4 pr = unpack_word(words[i]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xg + m * nk + 8 * i);
            acc[m] = __builtin_amdgcn_fdot2(as_h2(pr.p[0]), as_h2(xv.x), acc[m], false);
            acc[m] = __builtin_amdgcn_fdot2(as_h2(pr.p[1]), as_h2(xv.y), acc[m], false);
            acc[m] = __builtin_amdgcn_fdot2(as_h2(pr.p[2]), as_h2(xv.z), acc[m], false);
            acc[m] = __builtin_amdgcn_fdot2(as_h2(pr.p[3]), as_h2(xv.w), acc[m], false);
          }
        }
        const float s = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b.s[u])));
        const float z = asym ? static_cast<float>((b.z[u] >> zshift) & 0xFu) : 8.0f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int e = (m * ngp + gl) * 4 + p;
          yacc[m] += s * (acc[m] - osum[e] - z * ssum[e]);
        }
      }
    }
  };

  for (int ph0 = 0; ph0 < ng; ph0 += a.phase_groups) {
    const int ngp = min(a.phase_groups, ng - ph0);
    const int nk = ngp * kGroup;
    // this wavefront's groups in the phase: gl = wave + WAVES * j, j < nj
    const int nj = wave < ngp ? (ngp - wave + WAVES - 1) / WAVES : 0;
    Batch b0, b1;
    load(b0, ph0, 0, nj);
    if (ph0 != 0) __syncthreads();  // the previous phase is done with LDS
    stage_phase<M, NT>(a, ph0 * kGroup, nk, xs, osum, ssum);
    for (int jb = 0; jb < nj; jb += 2 * BATCH) {
      load(b1, ph0, jb + BATCH, nj);
      compute(b0, jb, nj, ngp, nk);
      load(b0, ph0, jb + 2 * BATCH, nj);
      compute(b1, jb + BATCH, nj, ngp, nk);
    }
  }

  // sum the four channel slices of each row (lanes r, r+16, r+32, r+48), then the waves
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = yacc[m];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (p == 0) red[(wave * M + m) * kTileN + r] = v;
  }
  __syncthreads();
  if (threadIdx.x < M * kTileN) {
    const int m = threadIdx.x / kTileN, rr = threadIdx.x % kTileN;
    float v = red[m * kTileN + rr];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v += red[(w * M + m) * kTileN + rr];
    const int n = t * kTileN + rr;
    if (n < a.N) {
      a.y[static_cast<int64_t>(m) * a.N + n] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
  }
}

// Two groups in flight per wavefront per batch (double-buffered), and 16 wavefronts per
// workgroup when there are few tiles (N <= 8192: one workgroup per CU, more loads in
// flight per CU), 8 otherwise (several workgroups per CU).
constexpr int kBatchDefault = 2;
inline bool many_waves(int64_t n_tiles) { return n_tiles <= 512; }

int phase_groups_for(int M, int n_groups) {
  int pg = kLdsBudget / (M * (2 * kGroup + 32));
  if (pg > n_groups) pg = n_groups;
  return pg < 1 ? 1 : pg;
}

size_t smem_bytes(int M, int phase_groups, int waves) {
  return static_cast<size_t>(2) * M * phase_groups * kGroup + 32ull * M * phase_groups +
         4ull * waves * M * kTileN;
}

template <int M, int WAVES, int BATCH>
hipError_t launch_cfg(const GemvArgs& a, int64_t n_tiles, hipStream_t st) {
  const size_t lds = smem_bytes(M, a.phase_groups, WAVES);
  hipLaunchKernelGGL((gemv_kernel<M, WAVES, BATCH>), dim3(static_cast<unsigned>(n_tiles)),
                     dim3(WAVES * 64), lds, st, a);
  return hipGetLastError();
}

template <int M>
hipError_t launch_m(const GemvArgs& a, int64_t n_tiles, hipStream_t st) {
  if (many_waves(n_tiles)) return launch_cfg<M, 16, kBatchDefault>(a, n_tiles, st);
  return launch_cfg<M, 8, kBatchDefault>(a, n_tiles, st);
}

// Tuning override for sweeps (M = 1 only): AWQ_GEMV_CFG = "waves,batch".
hipError_t launch_m1(const GemvArgs& a, int64_t n_tiles, hipStream_t st) {
  const char* env = getenv("AWQ_GEMV_CFG");
  if (env) {
    int w = 0, b = 0;
    if (sscanf(env, "%d,%d", &w, &b) == 2) {
      if (w == 4 && b == 4) return launch_cfg<1, 4, 4>(a, n_tiles, st);
      if (w == 8 && b == 1) return launch_cfg<1, 8, 1>(a, n_tiles, st);
      if (w == 8 && b == 2) return launch_cfg<1, 8, 2>(a, n_tiles, st);
      if (w == 8 && b == 4) return launch_cfg<1, 8, 4>(a, n_tiles, st);
      if (w == 16 && b == 1) return launch_cfg<1, 16, 1>(a, n_tiles, st);
      if (w == 16 && b == 2) return launch_cfg<1, 16, 2>(a, n_tiles, st);
      if (w == 16 && b == 4) return launch_cfg<1, 16, 4>(a, n_tiles, st);
    }
  }
  return launch_m<1>(a, n_tiles, st);
}

}  // namespace

size_t gemv_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemv(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                       int64_t M, int64_t N, int64_t K, int32_t fmt, uint16_t* y, void*, size_t,
                       hipStream_t st) {
  const PackedLayout L = make_layout(N, K, kGroup, fmt);
  GemvArgs a;
  a.x = x;
  a.inv = inv_s_c;
  a.packed = static_cast<const uint8_t*>(packed);
  a.y = y;
  a.scales_off = L.scales_off;
  a.zeros_off = L.zeros_off;
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.n_groups = static_cast<int>(L.n_groups);
  a.phase_groups = phase_groups_for(static_cast<int>(M), a.n_groups);
  switch (M) {
    case 1: return launch_m1(a, L.n_tiles, st);
    case 2: return launch_m<2>(a, L.n_tiles, st);
    case 3: return launch_m<3>(a, L.n_tiles, st);
    case 4: return launch_m<4>(a, L.n_tiles, st);
    case 5: return launch_m<5>(a, L.n_tiles, st);
    case 6: return launch_m<6>(a, L.n_tiles, st);
    case 7: return launch_m<7>(a, L.n_tiles, st);
    case 8: return launch_m<8>(a, L.n_tiles, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
