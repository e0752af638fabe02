// Prefill product y[M, N] = X' . deq(Wq)^T with the weights dequantized once per
// workgroup into LDS.
//
// In the register-fed kernel (gemm.hip) every wavefront turns its own weight words into
// binary16, so one dequantized fragment feeds only the wavefront's own rows; at large M
// that VALU work rivals the matrix-core time. Here the workgroup dequantizes each
// weight tile once (exactly W_d = binary16((q - z) * s), the same unpack as everywhere
// else) into LDS, next to the X' tile, and the four wavefronts run a plain
// LDS -> v_mfma_f32_16x16x32_f16 loop over both (edgesiliconlab ?p=2015, section
// "Kernel Execution: Marlin vs. ExLlamaV2 INT4 GEMM Micro-Architecture": tiles staged in
// on-chip memory, double-buffered so that the next tile's transfer overlaps the current
// tile's matrix instructions, 4-bit values expanded to binary16 before the multiply).
//
//  * a stage is 64 input channels (half a group): X' [BM][64] and W_d [BN][64] binary16
//    tiles, rows padded by 16 bytes; two stages in LDS (double buffering), one barrier per
//    stage;
//  * while stage s is multiplied, the packed weights and X' of stage s + 1 (loaded into
//    registers during stage s - 1) are dequantized / scaled and written to the other
//    buffer, and the loads for stage s + 2 are issued;
//  * four wavefronts in a 2 x 2 arrangement, each WM x WN matrix-core tiles of 16 x 16.
#include "awq_internal.hpp"

#include <stdlib.h>

namespace awq {
namespace {

constexpr int kStageK = 64;                 // channels per stage
constexpr int kRow = kStageK + 8;           // halfs per LDS row (16-byte pad)
constexpr int kThreadsL = 256;
constexpr int kXcdsL = 8;

struct GemmLdsArgs {
  const uint16_t* x;
  const uint16_t* inv;
  const uint8_t* packed;
  uint16_t* y;
  int64_t scales_off;
  int64_t zeros_off;
  uint32_t packed_bytes;
  int M, N, K, n_groups, n_tiles, n_blocks_m, n_blocks_n;
};

template <int WM, int WN>
__global__ void __launch_bounds__(kThreadsL) gemm_lds_kernel(GemmLdsArgs a) {
  constexpr int BM = 2 * WM * 16, BN = 2 * WN * 16;
  constexpr int A_VEC = BM * (kStageK / 8) / kThreadsL;  // 16-byte X' vectors per thread
  constexpr int B_UNITS = BN * 2 / kThreadsL;            // half-unit lane slices per thread
  static_assert(A_VEC >= 1 && B_UNITS >= 1, "tile too small for 256 threads");
  constexpr int ABUF = BM * kRow, BBUF = BN * kRow;      // halfs per stage buffer
  extern __shared__ __attribute__((aligned(16))) _Float16 lds[];  // [2][ABUF + BBUF]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, p = lane >> 4;

  const int nb = a.n_blocks_m * a.n_blocks_n;
  int bid = blockIdx.x;
  if (nb % kXcdsL == 0) bid = (bid % kXcdsL) * (nb / kXcdsL) + bid / kXcdsL;
  const int bm = bid % a.n_blocks_m, bn = bid / a.n_blocks_m;
  const int m_blk = bm * BM, n_blk = bn * BN;
  const int ng = a.n_groups;
  const int n_stages = 2 * ng;
  const bool asym = a.zeros_off >= 0;

  // ---- X' staging: thread -> (row, 8-channel vector) of the BM x 64 stage tile
  const int rows_here = min(BM, a.M - m_blk);
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(a.x + static_cast<int64_t>(m_blk) * a.K, static_cast<uint32_t>(rows_here) * a.K * 2);
  uint32_t a_voff[A_VEC];
  int a_lds[A_VEC], a_col[A_VEC];
#pragma unroll
  for (int it = 0; it < A_VEC; ++it) {
    const int v = tid + it * kThreadsL;
    const int row = v >> 3, col = (v & 7) * 8;
    a_voff[it] = static_cast<uint32_t>(row * a.K + col) * 2;
    a_lds[it] = row * kRow + col;
    a_col[it] = col;
  }

  // ---- weight staging: thread -> (tile, lane slice with channel slice p in {2h, 2h+1})
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.packed, a.packed_bytes);
  uint32_t b_code_base[B_UNITS], b_scale_base[B_UNITS], b_zero_base[B_UNITS];
  uint32_t b_lane16[B_UNITS];
  int b_lds[B_UNITS], b_zshift[B_UNITS], b_psub[B_UNITS], b_r[B_UNITS];
#pragma unroll
  for (int u = 0; u < B_UNITS; ++u) {
    const int v = tid + u * kThreadsL;
    const int tl = v >> 5, sl = v & 31;  // tile in block, slice lane
    const int rr = sl & 15, ps = sl >> 4;  // row in tile, which of the two channel slices
    const uint32_t tile = static_cast<uint32_t>(min(n_blk / kTileN + tl, a.n_tiles - 1));
    b_code_base[u] = tile * ng * kUnitBytes;
    b_scale_base[u] = static_cast<uint32_t>(a.scales_off) + tile * ng * (2 * kTileN) + 2u * rr;
    b_zero_base[u] = asym ? static_cast<uint32_t>(a.zeros_off) + tile * ng * 8 + 4u * (rr >> 3) : 0u;
    b_lane16[u] = 16u * rr;  // lane (rr + 16 p) of the unit; p added per stage
    b_zshift[u] = 4 * (rr & 7);
    b_psub[u] = ps;
    b_r[u] = rr;
    b_lds[u] = (tl * kTileN + rr) * kRow + 32 * ps;
  }

  struct Stage {
    uint4 a[A_VEC];
    uint4 c[B_UNITS];
    uint32_t s[B_UNITS], z[B_UNITS];
  };
  auto load_stage = [&](Stage& st, int s) {
    const int g = s >> 1, h = s & 1;
#pragma unroll
    for (int it = 0; it < A_VEC; ++it) st.a[it] = buf_load16(rx, a_voff[it], s * kStageK * 2);
#pragma unroll
    for (int u = 0; u < B_UNITS; ++u) {
      // per-lane parts in the VGPR offset, the (uniform) group offset in the SGPR one
      const uint32_t lane_off = b_code_base[u] + b_lane16[u] + 256u * (2 * h + b_psub[u]);
      st.c[u] = buf_load16(rp, lane_off, g * kUnitBytes);
      st.s[u] = buf_load2(rp, b_scale_base[u], g * (2 * kTileN));
      st.z[u] = asym ? buf_load4(rp, b_zero_base[u], g * 8) : 0u;
    }
  };
  auto store_stage = [&](const Stage& st, int s, int buf) {
    _Float16* abuf = lds + buf * (ABUF + BBUF);
    _Float16* bbuf = abuf + ABUF;
    if (a.inv) {
#pragma unroll
      for (int it = 0; it < A_VEC; ++it) {
        const uint4 iv = *reinterpret_cast<const uint4*>(a.inv + s * kStageK + a_col[it]);
        const uint4 x = st.a[it];
        const half2_t h0 = as_h2(x.x) * as_h2(iv.x), h1 = as_h2(x.y) * as_h2(iv.y);
        const half2_t h2 = as_h2(x.z) * as_h2(iv.z), h3 = as_h2(x.w) * as_h2(iv.w);
        *reinterpret_cast<uint4*>(abuf + a_lds[it]) =
            make_uint4(as_u32(h0), as_u32(h1), as_u32(h2), as_u32(h3));
      }
    } else {
#pragma unroll
      for (int it = 0; it < A_VEC; ++it) *reinterpret_cast<uint4*>(abuf + a_lds[it]) = st.a[it];
    }
#pragma unroll
    for (int u = 0; u < B_UNITS; ++u) {
      const uint32_t z = asym ? (st.z[u] >> b_zshift[u]) & 0xFu : 8u;
      const half2_t s2 = as_h2(st.s[u] | (st.s[u] << 16));
      const uint32_t n1024 = neg_off1024(z), n64 = neg_off64(z);
      const uint32_t words[4] = {st.c[u].x, st.c[u].y, st.c[u].z, st.c[u].w};
      _Float16* dst = bbuf + b_lds[u];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half2_t d[4];
        dequant_word(words[i], n1024, n64, s2, d);
        *reinterpret_cast<uint4*>(dst + 8 * i) =
            make_uint4(as_u32(d[0]), as_u32(d[1]), as_u32(d[2]), as_u32(d[3]));
      }
    }
    (void)b_r;
  };

  float4_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int buf) {
    const _Float16* abuf = lds + buf * (ABUF + BBUF);
    const _Float16* bbuf = abuf + ABUF;
#pragma unroll
    for (int kk = 0; kk < kStageK / 32; ++kk) {
      half8_t bf[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int row = (wn * WN + j) * 16 + r;
        bf[j] = *reinterpret_cast<const half8_t*>(bbuf + row * kRow + 32 * kk + 8 * p);
      }
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int row = (wm * WM + ms) * 16 + r;
        const half8_t af = *reinterpret_cast<const half8_t*>(abuf + row * kRow + 32 * kk + 8 * p);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[ms][j], 0, 0, 0);
        }
      }
    }
  };

  // prologue: stage 0 in LDS buffer 0, stage 1 in registers. One register set: in
  // iteration s the registers holding stage s + 1 are written to LDS right after the
  // stage-s multiply, then refilled with stage s + 2, which has the whole of iteration
  // s + 1 to arrive.
  Stage st;
  load_stage(st, 0);
  store_stage(st, 0, 0);
  if (n_stages > 1) load_stage(st, 1);
  __syncthreads();
  for (int s = 0; s < n_stages; ++s) {
    const int buf = s & 1;
    compute(buf);
    if (s + 1 < n_stages) {
      store_stage(st, s + 1, buf ^ 1);
      if (s + 2 < n_stages) load_stage(st, s + 2);
    }
    __syncthreads();
  }

#pragma unroll
  for (int ms = 0; ms < WM; ++ms) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n_blk + (wn * WN + j) * 16 + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m_blk + (wm * WM + ms) * 16 + 4 * p + q;
        if (m < a.M && n < a.N) {
          a.y[static_cast<int64_t>(m) * a.N + n] =
              __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[ms][j][q]));
        }
      }
    }
  }
}

template <int WM, int WN>
hipError_t launch_lds_tiles(GemmLdsArgs a, hipStream_t st) {
  constexpr int BM = 2 * WM * 16, BN = 2 * WN * 16;
  const size_t lds = 2ull * (BM + BN) * kRow * sizeof(_Float16);
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_lds_kernel<WM, WN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  a.n_blocks_m = (a.M + BM - 1) / BM;
  a.n_blocks_n = (a.N + BN - 1) / BN;
  const unsigned blocks = static_cast<unsigned>(a.n_blocks_m) * static_cast<unsigned>(a.n_blocks_n);
  hipLaunchKernelGGL((gemm_lds_kernel<WM, WN>), dim3(blocks), dim3(kThreadsL), lds, st, a);
  return hipGetLastError();
}

}  // namespace

// cfg: 0 = default for the shape; otherwise WM * 10 + WN
hipError_t launch_gemm_lds(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                           int64_t M, int64_t N, int64_t K, int32_t fmt, uint16_t* y, int cfg,
                           hipStream_t st) {
  const PackedLayout L = make_layout(N, K, kGroup, fmt);
  GemmLdsArgs a;
  a.x = x;
  a.inv = inv_s_c;
  a.packed = static_cast<const uint8_t*>(packed);
  a.y = y;
  a.scales_off = L.scales_off;
  a.zeros_off = L.zeros_off;
  a.packed_bytes = static_cast<uint32_t>(L.total_bytes);
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.n_groups = static_cast<int>(L.n_groups);
  a.n_tiles = static_cast<int>(L.n_tiles);
  switch (cfg) {
    case 44: return launch_lds_tiles<4, 4>(a, st);
    case 48: return launch_lds_tiles<4, 8>(a, st);
    case 84: return launch_lds_tiles<8, 4>(a, st);
    default: return launch_lds_tiles<8, 4>(a, st);
  }
}

}  // namespace awq
