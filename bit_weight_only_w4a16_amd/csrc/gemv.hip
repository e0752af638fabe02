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
//  * every load is issued unconditionally: a load with nothing to fetch gets a per-lane
//    offset past the end of its buffer resource, which returns zeros without a memory
//    access. With no branch around a load the compiler's wait counts are exact, so a
//    wavefront waits for the batch it is about to use and never for the one behind it;
//  * the activations are requested before the weights, so staging them waits only for
//    the activation loads;
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
  int64_t zeros_off;
  int N, K, n_groups, phase_groups;
};

// Staging of X' for channels [k0, k0 + nk) of every row: thread `tid` handles the 8-channel
// vectors i = tid + NT * j (row i / (nk / 8)). Loads come from buffer resources, so a
// vector past the end reads zeros and no load needs a branch.
struct XStage {
  __amdgpu_buffer_rsrc_t rx, rinv;
  int vpr;    // vectors per row in this phase (a multiple of 16)
  int total;  // M * vpr
  int k0;
};

__device__ __forceinline__ uint32_t x_voff(const GemvArgs& a, const XStage& s, int i) {
  const int m = i / s.vpr, v = i - m * s.vpr;
  const uint32_t off = 2u * static_cast<uint32_t>(m * a.K + s.k0 + 8 * v);
  return i < s.total ? off : kNoLoad;
}
__device__ __forceinline__ uint32_t inv_voff(const XStage& s, int i) {
  const int v = i % s.vpr;
  return i < s.total ? 2u * static_cast<uint32_t>(s.k0 + 8 * v) : kNoLoad;
}

// X' = binary16(x * inv) for one vector; writes it and, from the first lane of each
// group of 4 (one 32-channel slice), O and S for the slice. Channel k of a word has
// offset 1024 if k % 8 is in {0, 1, 4, 5}, else 64. All four lanes of a slice are
// active together: `total` is a multiple of 16 and NT of 64.
__device__ __forceinline__ void stage_store(const XStage& s, int i, uint4 val, uint4 iv,
                                            bool has_inv, int nk, _Float16* xs, float* osum,
                                            float* ssum) {
  const half2_t one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  const half2_t o1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  const half2_t o64 = {static_cast<_Float16>(64.0f), static_cast<_Float16>(64.0f)};
  // with no inv_s_c the factor is 1 (exact); a select rather than a branch keeps the
  // inv_s_c load unconditional
  if (!has_inv) iv = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  {
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
  if (i < s.total) {
    const int m = i / s.vpr, v = i - m * s.vpr;
    *reinterpret_cast<uint4*>(xs + m * nk + 8 * v) = val;
    if ((v & 3) == 0) {
      const int e = m * (nk / 32) + (v >> 2);
      ssum[e] = sv;
      osum[e] = ov;
    }
  }
}

template <int M, int WAVES, int BATCH, bool ASYM>
__global__ void __launch_bounds__(WAVES * 64) gemv_kernel(GemvArgs a) {
  constexpr int NT = WAVES * 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int t = blockIdx.x;
  // the wavefront index is uniform: keep it (and every group index) in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, p = lane >> 4;
  const int ng = a.n_groups;
  const bool has_inv = a.inv != nullptr;

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
  const __amdgpu_buffer_rsrc_t rzeros =
      make_rsrc(a.packed + (ASYM ? a.zeros_off : 0) + static_cast<int64_t>(t) * ng * 8, ng * 8);
  const uint32_t lane_code = 16u * lane, lane_scale = 2u * r, lane_zero = 4u * (r >> 3);
  const int zshift = 4 * (r & 7);

  XStage xst;
  xst.rx = make_rsrc(a.x, static_cast<uint32_t>(M * a.K * 2));
  xst.rinv = make_rsrc(has_inv ? a.inv : a.x, has_inv ? static_cast<uint32_t>(a.K * 2) : 0u);

  float yacc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) yacc[m] = 0.0f;

  struct Batch {
    uint4 c[BATCH];
    uint32_t s[BATCH], z[BATCH];
  };
  // groups gl = wave + WAVES * j of the phase, j < nj; a slot past nj loads nothing
  auto load = [&](Batch& b, int ph0, int jb, int nj) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const bool live = jb + u < nj;
      const uint32_t g = live ? static_cast<uint32_t>(ph0 + wave + WAVES * (jb + u)) : 0u;
      const uint32_t skip = live ? 0u : kNoLoad;
      b.c[u] = buf_load16(rcodes, lane_code + skip, g * kUnitBytes);
      b.s[u] = buf_load2(rscales, lane_scale + skip, g * (2 * kTileN));
      if (ASYM) b.z[u] = buf_load4(rzeros, lane_zero + skip, g * 8);
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
        const float z = ASYM ? static_cast<float>((b.z[u] >> zshift) & 0xFu) : 8.0f;
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
    xst.vpr = nk / 8;
    xst.total = M * xst.vpr;
    xst.k0 = ph0 * kGroup;
    // activations first (two vectors per thread), then this wavefront's first batch
    const int i0 = threadIdx.x, i1 = threadIdx.x + NT;
    const uint4 x0 = buf_load16(xst.rx, x_voff(a, xst, i0), 0);
    const uint4 v0 = buf_load16(xst.rinv, inv_voff(xst, i0), 0);
    const uint4 x1 = buf_load16(xst.rx, x_voff(a, xst, i1), 0);
    const uint4 v1 = buf_load16(xst.rinv, inv_voff(xst, i1), 0);
    const int nj = wave < ngp ? (ngp - wave + WAVES - 1) / WAVES : 0;
    Batch b0, b1;
    load(b0, ph0, 0, nj);
    if (ph0 != 0) __syncthreads();  // the previous phase is done with LDS
    stage_store(xst, i0, x0, v0, has_inv, nk, xs, osum, ssum);
    stage_store(xst, i1, x1, v1, has_inv, nk, xs, osum, ssum);
    for (int i = threadIdx.x + 2 * NT; i < ((xst.total + NT - 1) / NT) * NT; i += NT) {
      const uint4 xv = buf_load16(xst.rx, x_voff(a, xst, i), 0);
      const uint4 iv = buf_load16(xst.rinv, inv_voff(xst, i), 0);
      stage_store(xst, i, xv, iv, has_inv, nk, xs, osum, ssum);
    }
    __syncthreads();
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
  if (a.zeros_off >= 0) {
    hipLaunchKernelGGL((gemv_kernel<M, WAVES, BATCH, true>), dim3(static_cast<unsigned>(n_tiles)),
                       dim3(WAVES * 64), lds, st, a);
  } else {
    hipLaunchKernelGGL((gemv_kernel<M, WAVES, BATCH, false>), dim3(static_cast<unsigned>(n_tiles)),
                       dim3(WAVES * 64), lds, st, a);
  }
  return hipGetLastError();
}

// Eight wavefronts with two groups in flight each; for long rows (K >= 16384) sixteen
// wavefronts with one group each, which keeps more loads in flight per CU when there are
// few tiles per CU. (Sweeps on MI355X over 4096 <= K, N <= 28672.)
template <int M>
hipError_t launch_m(const GemvArgs& a, int64_t n_tiles, hipStream_t st) {
  if (a.n_groups >= 128) return launch_cfg<M, 16, 1>(a, n_tiles, st);
  return launch_cfg<M, 8, 2>(a, n_tiles, st);
}

// Tuning override for sweeps (M = 1 only): AWQ_GEMV_CFG = "waves,batch".
hipError_t launch_m1(const GemvArgs& a, int64_t n_tiles, hipStream_t st) {
  const char* env = getenv("AWQ_GEMV_CFG");
  if (env) {
    int w = 0, b = 0;
    if (sscanf(env, "%d,%d", &w, &b) == 2) {
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
