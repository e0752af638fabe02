// Batched-decode / prefill product y[M, N] = X' . deq(Wq)^T on the gfx950 matrix cores.
//
// Larger batches turn the product into a matrix-matrix multiply that is bound by
// arithmetic rather than bandwidth (edgesiliconlab ?p=2015, section "GEMM vs. GEMV
// Kernels and Batch Size Dynamics"). The weights are turned into binary16 in registers
// right before the matrix instruction (same page, section "Kernel Execution: Marlin vs.
// ExLlamaV2 INT4 GEMM Micro-Architecture", item 3), with exactly the dequantized values
// W_d = binary16((q - z) * s):
//
//  * v_mfma_f32_16x16x32_f16: lane l feeds row/column l % 16 and k slots 8 (l / 16)..+7.
//    In the gfx950 layout a lane's 16 bytes of a unit are row l % 16, channels
//    32 (l / 16) + 8 i + 0..7 for word i, so word i is exactly the B operand of k-step i
//    of the group (the slots of step i stand for channels 32 j + 8 i + e, j = l / 16): one
//    128-bit global load per lane gives the B operands of a 16-row tile for a whole
//    group, with no LDS round trip. The X' operand uses the same slot-to-channel map.
//  * X' tiles (binary16(X * inv_s_c)) are staged in LDS one group (128 channels) at a
//    time, rows padded by 16 bytes; the next group's X' and weights are loaded into
//    registers while the current group is multiplied.
//  * Four wavefronts per workgroup in a 2 x 2 arrangement; each computes WM x WN
//    matrix-core tiles of 16 x 16.
#include "awq_internal.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace awq {
namespace {

constexpr int kLdsStride = kGroup + 8;  // halfs per LDS row (16-byte pad)
constexpr int kGThreads = 256;

struct GemmArgs {
  const uint16_t* x;
  const uint16_t* inv;
  const uint8_t* packed;
  uint16_t* y;
  int64_t scales_off;
  int64_t zeros_off;
  int M, N, K, n_groups, n_tiles, n_blocks_n, n_blocks_m;
};

__device__ __forceinline__ uint4 scale_x(uint4 val, uint4 iv) {
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
  return make_uint4(ow[0], ow[1], ow[2], ow[3]);
}

template <int WM, int WN>
__global__ void __launch_bounds__(kGThreads) gemm_kernel(GemmArgs a) {
  constexpr int BM = 2 * WM * 16, BN = 2 * WN * 16;
  constexpr int A_VEC = BM * (kGroup / 8) / kGThreads;  // 16-byte X' vectors per thread
  __shared__ __attribute__((aligned(16))) _Float16 xs[BM * kLdsStride];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, p = lane >> 4;

  // workgroup -> output block; consecutive workgroups walk down M first so that the
  // ones running together share their weight tiles in L2
  const int bid = blockIdx.x;
  const int bm = bid % a.n_blocks_m, bn = bid / a.n_blocks_m;
  const int m_blk = bm * BM, n_blk = bn * BN;
  const int ng = a.n_groups;

  // this wavefront's weight tiles (clamped: tiles past the last one are read but their
  // rows are >= N and never stored), as buffer resources: the per-group offset is
  // uniform (SGPR), the per-lane offset constant
  __amdgpu_buffer_rsrc_t rb[WN], rs[WN], rz[WN];
  const bool asym = a.zeros_off >= 0;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int64_t tile = min(n_blk / kTileN + wn * WN + j, a.n_tiles - 1);
    rb[j] = make_rsrc(a.packed + tile * ng * kUnitBytes, ng * kUnitBytes);
    rs[j] = make_rsrc(a.packed + a.scales_off + tile * ng * (2 * kTileN), ng * 2 * kTileN);
    rz[j] = make_rsrc(a.packed + (asym ? a.zeros_off : 0) + tile * ng * 8, ng * 8);
  }
  const uint32_t lane_code = 16u * lane, lane_scale = 2u * r, lane_zero = 4u * (r >> 3);

  // X' staging: thread -> (row, 8-channel vector) pairs of the BM x 128 tile
  int a_row[A_VEC], a_col[A_VEC];
  bool a_ok[A_VEC];
#pragma unroll
  for (int it = 0; it < A_VEC; ++it) {
    const int v = threadIdx.x + it * kGThreads;
    a_row[it] = v >> 4;
    a_col[it] = (v & 15) * 8;
    a_ok[it] = m_blk + a_row[it] < a.M;
  }
  const uint16_t* xrow[A_VEC];
#pragma unroll
  for (int it = 0; it < A_VEC; ++it)
    xrow[it] = a.x + static_cast<int64_t>(a_ok[it] ? m_blk + a_row[it] : 0) * a.K + a_col[it];

  uint4 areg[A_VEC];
  uint4 breg[WN];
  uint32_t sreg[WN], zreg[WN];

  auto load_group = [&](int g) {
#pragma unroll
    for (int it = 0; it < A_VEC; ++it) {
      areg[it] = a_ok[it] ? *reinterpret_cast<const uint4*>(xrow[it] + g * kGroup)
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      breg[j] = buf_load16(rb[j], lane_code, g * kUnitBytes);
      sreg[j] = buf_load2(rs[j], lane_scale, g * (2 * kTileN));
      zreg[j] = asym ? buf_load4(rz[j], lane_zero, g * 8) : 0u;
    }
  };

  float4_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  load_group(0);
  const int zshift = 4 * (r & 7);
  for (int g = 0; g < ng; ++g) {
    // X' of group g into LDS (scaled by inv_s_c), weights of group g into the B registers
    uint4 iv[A_VEC];
    if (a.inv) {
#pragma unroll
      for (int it = 0; it < A_VEC; ++it)
        iv[it] = *reinterpret_cast<const uint4*>(a.inv + g * kGroup + a_col[it]);
    }
    __syncthreads();  // everyone is done reading the previous group's tile
#pragma unroll
    for (int it = 0; it < A_VEC; ++it) {
      const uint4 val = a.inv ? scale_x(areg[it], iv[it]) : areg[it];
      *reinterpret_cast<uint4*>(&xs[a_row[it] * kLdsStride + a_col[it]]) = val;
    }
    uint4 bcur[WN];
    half2_t s2[WN];
    uint32_t nz1024[WN], nz64[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      bcur[j] = breg[j];
      const uint32_t z = asym ? (zreg[j] >> zshift) & 0xFu : 8u;
      s2[j] = as_h2(sreg[j] | (sreg[j] << 16));
      nz1024[j] = neg_off1024(z);
      nz64[j] = neg_off64(z);
    }
    __syncthreads();
    if (g + 1 < ng) load_group(g + 1);

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half8_t bf[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint32_t w = i == 0 ? bcur[j].x : i == 1 ? bcur[j].y : i == 2 ? bcur[j].z : bcur[j].w;
        half2_t d[4];
        dequant_word(w, nz1024[j], nz64[j], s2[j], d);
        bf[j] = half8_t{d[0].x, d[0].y, d[1].x, d[1].y, d[2].x, d[2].y, d[3].x, d[3].y};
      }
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int row = wm * WM * 16 + ms * 16 + r;
        const half8_t af =
            *reinterpret_cast<const half8_t*>(&xs[row * kLdsStride + 32 * p + 8 * i]);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[ms][j], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: element q of acc[ms][j] is row 4 (l / 16) + q, column l % 16 of its tile
#pragma unroll
  for (int ms = 0; ms < WM; ++ms) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n_blk + (wn * WN + j) * 16 + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m_blk + wm * WM * 16 + ms * 16 + 4 * p + q;
        if (m < a.M && n < a.N) {
          a.y[static_cast<int64_t>(m) * a.N + n] =
              __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[ms][j][q]));
        }
      }
    }
  }
}

template <int WM, int WN>
hipError_t launch_tiles(GemmArgs a, hipStream_t st) {
  constexpr int BM = 2 * WM * 16, BN = 2 * WN * 16;
  a.n_blocks_m = (a.M + BM - 1) / BM;
  a.n_blocks_n = (a.N + BN - 1) / BN;
  const unsigned blocks = static_cast<unsigned>(a.n_blocks_m) * static_cast<unsigned>(a.n_blocks_n);
  hipLaunchKernelGGL((gemm_kernel<WM, WN>), dim3(blocks), dim3(kGThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                       int64_t M, int64_t N, int64_t K, int32_t fmt, uint16_t* y, void*, size_t,
                       hipStream_t st) {
  const PackedLayout L = make_layout(N, K, kGroup, fmt);
  GemmArgs a;
  a.x = x;
  a.inv = inv_s_c;
  a.packed = static_cast<const uint8_t*>(packed);
  a.y = y;
  a.scales_off = L.scales_off;
  a.zeros_off = L.zeros_off;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.n_groups = static_cast<int>(L.n_groups);
  a.n_tiles = static_cast<int>(L.n_tiles);
  const char* env = getenv("AWQ_GEMM_TILE");
  int wm = 0, wn = 0;
  if (env && sscanf(env, "%d,%d", &wm, &wn) == 2) {
    if (wm == 2 && wn == 2) return launch_tiles<2, 2>(a, st);
    if (wm == 4 && wn == 2) return launch_tiles<4, 2>(a, st);
    if (wm == 4 && wn == 4) return launch_tiles<4, 4>(a, st);
  }
  if (M <= 32) return launch_tiles<1, 4>(a, st);
  if (M <= 64) return launch_tiles<2, 4>(a, st);
  return launch_tiles<4, 4>(a, st);
}

}  // namespace awq
