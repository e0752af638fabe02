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
//    of the group (the slots of step i stand for channels 32 j + 8 i + e, j = l / 16):
//    one 128-bit buffer load per lane gives the B operands of a 16-row weight tile for
//    a whole group, with no LDS round trip. The X' operand uses the same slot map.
//  * X' (binary16(X * inv_s_c)) goes through LDS, one 128-channel group per stage,
//    double-buffered: while group g is multiplied from one buffer, group g + 1 is
//    written to the other from registers loaded a stage earlier, and group g + 2 is
//    being fetched from memory; one barrier per group. Rows are padded by 16 bytes so
//    the 16 rows read by one instruction fall in distinct LDS banks.
//  * The weights of group g + 1 are in registers while group g is multiplied. Every
//    load is issued unconditionally (a group past the end reads zeros through an
//    out-of-range lane offset), so the compiler's wait counts cover exactly the loads
//    each step needs and never drain the prefetches behind them.
//  * Four wavefronts per workgroup, side by side along N (or 2 x 2); each computes
//    WM x WN matrix-core tiles of 16 x 16 (up to 128 x 64 outputs, accumulators in
//    VGPRs), so one dequantized weight fragment feeds WM instructions.
//  * At small M the weights are the whole cost and the output blocks are few, so K is
//    split: over KS slices of four wavefronts inside the workgroup (each slice with its
//    own X' buffers and share of the groups, sums added through LDS in slice order),
//    and, when even that leaves too few workgroups, across workgroups (float32 partial
//    sums in the caller's workspace, added in split order by a second launch).
//  * Workgroups are numbered so that the ones a given XCD (L2 slice) runs are
//    neighbours along M: they share the same weight columns in that L2.
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
  uint32_t packed_bytes;
  float* part;  // split-K partial sums [splits][M][N], or NULL (one split)
  int M, N, K, n_groups, n_tiles, n_blocks_n, n_blocks_m, splits, sets;
};

// SCHED > 0: ask the scheduler to issue each matrix instruction followed by SCHED VALU
// instructions (and an LDS read every WN of them), so that the dequantization of the
// next weight fragments runs while the matrix core is busy.
// The arguments are thirteen scalar dwords (the rest of the layout is derived from
// them), which the compiler preloads into SGPRs at wavefront launch: no wait for the
// argument block before the first load. `out` is y (binary16) or, with K split, the
// float32 partial sums.
template <int WAVES_M, int WM, int WN, int SCHED, bool ASYM, int KS>
__global__ void __launch_bounds__(kGThreads * KS)
    gemm_kernel(const uint16_t* x, const uint16_t* inv, const uint8_t* packed, void* out, int M,
                int N, int K, int splits, int sets) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int BM = WAVES_M * WM * 16, BN = WAVES_N * WN * 16;
  const PackedLayout L = make_layout_sets(N, K, sets, ASYM);
  GemmArgs a;
  a.x = x;
  a.inv = inv;
  a.packed = packed;
  a.y = splits > 1 ? nullptr : static_cast<uint16_t*>(out);
  a.part = splits > 1 ? static_cast<float*>(out) : nullptr;
  a.scales_off = L.scales_off;
  a.zeros_off = L.zeros_off;
  a.packed_bytes = static_cast<uint32_t>(L.total_bytes);
  a.M = M;
  a.N = N;
  a.K = K;
  a.n_groups = static_cast<int>(L.n_groups);
  a.n_tiles = static_cast<int>(L.n_tiles);
  a.n_blocks_m = (M + BM - 1) / BM;
  a.n_blocks_n = (N + BN - 1) / BN;
  a.splits = splits;
  a.sets = sets;
  constexpr int A_VEC = BM * (kGroup / 8) / kGThreads;  // 16-byte X' vectors per thread
  constexpr int BUF = BM * kLdsStride;                  // halfs per LDS buffer
  extern __shared__ __attribute__((aligned(16))) _Float16 xs_all[];  // [KS][2][BM][kLdsStride]

  // KS > 1: the workgroup's wavefronts form KS slices of four, each with its own pair of
  // LDS buffers and its own consecutive share of the workgroup's groups
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int ks = wave_all >> 2, wave = wave_all & 3;
  const int tid = threadIdx.x & (kGThreads - 1);  // thread index inside the slice
  _Float16* xs = xs_all + ks * 2 * BUF;
  const int lane = threadIdx.x & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int r = lane & 15, p = lane >> 4;

  // workgroup -> output block. Blocks are dealt to the XCDs round-robin; renumber so
  // that each XCD gets a contiguous run, walked down M first (shared weight columns).
  const int nb = a.n_blocks_m * a.n_blocks_n;
  const int bid = xcd_block(blockIdx.x, nb);
  const int bm = bid % a.n_blocks_m, bn = bid / a.n_blocks_m;
  const int m_blk = bm * BM, n_blk = bn * BN;
  const int ng = a.n_groups;
  const bool has_inv = a.inv != nullptr;
  // this workgroup's share of K: groups [ga, gb); this slice's: [g0, g1), `per` of them
  // at most (every slice makes the same number of trips, so the barriers match)
  const int split = blockIdx.y;
  const int ga = split * ng / a.splits, gb = (split + 1) * ng / a.splits;
  const int per = (gb - ga + KS - 1) / KS;
  const int g0 = min(gb, ga + ks * per), g1 = min(gb, g0 + per);

  // one buffer resource over the whole packed layer; this wavefront's weight tiles are
  // addressed by wavefront-uniform (SGPR) offsets (tiles past the last one are clamped:
  // their rows are >= N and never stored). Few SGPRs: no resource ends up in VGPRs.
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.packed, a.packed_bytes);
  const uint32_t sbytes = 2 * kTileN * a.sets, zbytes = 8 * a.sets;  // per unit
  uint32_t code_off[WN], scale_off[WN], zero_off[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const uint32_t tile = static_cast<uint32_t>(min(n_blk / kTileN + wn * WN + j, a.n_tiles - 1));
    code_off[j] = tile * ng * kUnitBytes;
    scale_off[j] = static_cast<uint32_t>(a.scales_off) + tile * ng * sbytes;
    zero_off[j] = ASYM ? static_cast<uint32_t>(a.zeros_off) + tile * ng * zbytes : 0u;
  }
  const int lset = lane_set(p, a.sets);
  const uint32_t lane_code = 16u * lane, lane_scale = 2u * (kTileN * lset + r),
                 lane_zero = 4u * (2 * lset + (r >> 3));
  const int zshift = 4 * (r & 7);

  // X' rows of this block as one buffer resource (rows past M read as 0), and inv_s_c
  // (an empty resource when the activations come pre-scaled)
  const int rows_here = min(BM, a.M - m_blk);
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(a.x + static_cast<int64_t>(m_blk) * a.K, static_cast<uint32_t>(rows_here) * a.K * 2);
  const __amdgpu_buffer_rsrc_t rinv =
      make_rsrc(has_inv ? a.inv : a.x, has_inv ? static_cast<uint32_t>(a.K) * 2 : 0u);
  // thread -> X' vectors: rows tid / 16 + 16 it, channels 8 (tid % 16)..+7 of the group
  const int a_col = (tid & 15) * 8;
  uint32_t a_voff[A_VEC];
  int a_lds[A_VEC];
#pragma unroll
  for (int it = 0; it < A_VEC; ++it) {
    const int row = (tid + it * kGThreads) >> 4;
    a_voff[it] = static_cast<uint32_t>(row * a.K + a_col) * 2;
    a_lds[it] = row * kLdsStride + a_col;
  }

  // Every load below is issued unconditionally; a group past the last one gets a lane
  // offset past the end of its resource and reads zeros without touching memory. With
  // no branches around loads, each wait covers exactly the loads it needs.
  uint4 areg[A_VEC];
  uint4 ireg;
  auto load_a = [&](int g) {
    const bool live = g < g1;
    const uint32_t skip = live ? 0u : kNoLoad;
    const uint32_t soff = live ? static_cast<uint32_t>(g) * kGroup * 2 : 0u;
#pragma unroll
    for (int it = 0; it < A_VEC; ++it) areg[it] = buf_load16(rx, a_voff[it] + skip, soff);
    ireg = buf_load16(rinv, 2u * a_col + skip, soff);
  };
  // X' = binary16(x * inv); with no inv_s_c the factor is 1 (exact). A select rather
  // than a branch keeps the inv_s_c load unconditional.
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  auto store_a = [&](int buf) {
    _Float16* dst = xs + buf * BUF;
    const uint4 iv = has_inv ? ireg : ones;
#pragma unroll
    for (int it = 0; it < A_VEC; ++it) *reinterpret_cast<uint4*>(dst + a_lds[it]) = scale_x8(areg[it], iv);
  };
  struct BRegs {
    uint4 c[WN];
    uint32_t s[WN], z[WN];
  };
  auto load_b = [&](BRegs& b, int g) {
    const bool live = g < g1;
    const uint32_t skip = live ? 0u : kNoLoad;
    const uint32_t gg = live ? static_cast<uint32_t>(g) : 0u;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      b.c[j] = buf_load16(rp, lane_code + skip, code_off[j] + gg * kUnitBytes);
      b.s[j] = buf_load2(rp, lane_scale + skip, scale_off[j] + gg * sbytes);
      if (ASYM) b.z[j] = buf_load4(rp, lane_zero + skip, zero_off[j] + gg * zbytes);
    }
  };

  float4_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const BRegs& b, int buf) {
    const _Float16* src = xs + buf * BUF;
    half2_t s2[WN];
    uint32_t nz1024[WN], nz64[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const uint32_t z = ASYM ? (b.z[j] >> zshift) & 0xFu : 8u;
      s2[j] = as_h2(b.s[j] | (b.s[j] << 16));
      nz1024[j] = neg_off1024(z);
      nz64[j] = neg_off64(z);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half8_t bf[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint32_t w = i == 0 ? b.c[j].x : i == 1 ? b.c[j].y : i == 2 ? b.c[j].z : b.c[j].w;
        half2_t d[4];
        dequant_word(w, nz1024[j], nz64[j], s2[j], d);
        bf[j] = half8_t{d[0].x, d[0].y, d[1].x, d[1].y, d[2].x, d[2].y, d[3].x, d[3].y};
      }
#pragma unroll
      for (int ms = 0; ms < WM; ++ms) {
        const int row = wm * WM * 16 + ms * 16 + r;
        const half8_t af = *reinterpret_cast<const half8_t*>(src + row * kLdsStride + 32 * p + 8 * i);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[ms][j], 0, 0, 0);
        }
      }
    }
    if constexpr (SCHED > 0) {
#pragma unroll
      for (int q = 0; q < 4 * WM * WN; ++q) {
        if (q % WN == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, SCHED, 0);               // VALU
      }
    }
  };

  // prologue: X'(0) in LDS buffer 0, X'(1) and B(0) in registers
  BRegs b0, b1;
  load_a(g0);
  load_b(b0, g0);
  store_a(0);
  load_a(g0 + 1);
  __syncthreads();

  // two groups per trip: g from buffer 0 / b0, g + 1 from buffer 1 / b1. While one group
  // is multiplied, the weights of the next are in flight and its X' goes into the other
  // LDS buffer; one barrier per group.
  // (sched_barrier keeps the scheduler from sinking the prefetches below the math)
  for (int t = 0; t < per; t += 2) {
    const int g = g0 + t;
    load_b(b1, g + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (g < g1) compute(b0, 0);
    store_a(1);
    load_a(g + 2);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    load_b(b0, g + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (g + 1 < g1) compute(b1, 1);
    store_a(0);
    load_a(g + 3);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  if constexpr (KS > 1) {
    // the slices' sums meet in LDS (the X' buffers are free after the last barrier):
    // slices 1 .. KS-1 write, slice 0 adds them in slice order (the same bits every call)
    float4_t* red = reinterpret_cast<float4_t*>(xs_all);
    if (ks > 0) {
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          red[((((ks - 1) * 4 + wave) * WM + ms) * WN + j) * 64 + lane] = acc[ms][j];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[ms][j] += red[((((k2 - 1) * 4 + wave) * WM + ms) * WN + j) * 64 + lane];
  }

  // epilogue: element q of acc[ms][j] is row 4 (l / 16) + q, column l % 16 of its tile;
  // binary16 y, or with split K this split's float32 partial sums
  float* part = a.part ? a.part + static_cast<int64_t>(split) * a.M * a.N : nullptr;
#pragma unroll
  for (int ms = 0; ms < WM; ++ms) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n_blk + (wn * WN + j) * 16 + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m_blk + wm * WM * 16 + ms * 16 + 4 * p + q;
        if (m < a.M && n < a.N) {
          const int64_t o = static_cast<int64_t>(m) * a.N + n;
          if (part) {
            part[o] = acc[ms][j][q];
          } else {
            a.y[o] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[ms][j][q]));
          }
        }
      }
    }
  }
}

// y = binary16(sum over the splits of the partial sums, in split order): deterministic.
// Four outputs per thread; M * N is a multiple of 8. The split count is a template
// argument so that all S loads are in flight before the first add (with a run-time
// count the loop waited one memory round trip per split).
template <int S>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* part, int64_t mn,
                                                            uint16_t* y) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  float4_t p[S];
#pragma unroll
  for (int s = 0; s < S; ++s) p[s] = *reinterpret_cast<const float4_t*>(part + s * mn + i);
  float4_t v = p[0];
#pragma unroll
  for (int s = 1; s < S; ++s) v += p[s];
  const half2_t lo = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1])};
  const half2_t hi = {static_cast<_Float16>(v[2]), static_cast<_Float16>(v[3])};
  *reinterpret_cast<uint2*>(y + i) = make_uint2(as_u32(lo), as_u32(hi));
}

// Splits of K for a launch of `blocks` output blocks (from sweeps on MI355X): about 640
// workgroups (2.5 per CU) when the output alone gives fewer than 512, each split at least
// 8 units, at most 8 splits, and the partial sums' traffic (written once, read once) no
// more than the weights' bytes.
int pick_splits(int64_t blocks, int64_t M, int64_t N, int64_t K, int n_groups) {
  if (blocks >= 512) return 1;
  int64_t s = (640 + blocks - 1) / blocks;
  s = s < n_groups / 8 ? s : n_groups / 8;
  const int64_t traffic_cap = K / (16 * M);  // 8 S M N <= N K / 2
  s = s < traffic_cap ? s : traffic_cap;
  s = s < 8 ? s : 8;
  return s < 1 ? 1 : static_cast<int>(s);
}

template <int WAVES_M, int WM, int WN, int SCHED, bool ASYM, int KS>
hipError_t launch_tiles_fmt(GemmArgs a, hipStream_t st) {
  constexpr int BM = WAVES_M * WM * 16, BN = (4 / WAVES_M) * WN * 16;
  constexpr size_t lds_x = 2ull * KS * BM * kLdsStride * sizeof(_Float16);
  constexpr size_t lds_red = (KS - 1) * 4ull * WM * WN * 64 * 16;
  const size_t lds = lds_x > lds_red ? lds_x : lds_red;
  static std::atomic<uint64_t> lds_done{0};
  const hipError_t ea = ensure_lds_limit(
      reinterpret_cast<const void*>(&gemm_kernel<WAVES_M, WM, WN, SCHED, ASYM, KS>), static_cast<int>(lds),
      lds_done);
  if (ea != hipSuccess) return ea;
  a.n_blocks_m = (a.M + BM - 1) / BM;
  a.n_blocks_n = (a.N + BN - 1) / BN;
  const unsigned blocks = static_cast<unsigned>(a.n_blocks_m) * static_cast<unsigned>(a.n_blocks_n);
  void* out = a.splits > 1 ? static_cast<void*>(a.part) : static_cast<void*>(a.y);
  hipLaunchKernelGGL((gemm_kernel<WAVES_M, WM, WN, SCHED, ASYM, KS>), dim3(blocks, a.splits),
                     dim3(kGThreads * KS), lds, st, a.x, a.inv, a.packed, out, a.M, a.N, a.K, a.splits,
                     a.sets);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_splitk_reduce(a.part, a.splits, static_cast<int64_t>(a.M) * a.N, a.y, st);
}

// How the narrow tiles split K (from sweeps on MI355X at M = 8 .. 64 on the 7B and 70B
// layers): S = pick_splits splits in all; with at least 80 output blocks they are taken
// inside the workgroup (two or four slices of four wavefronts, partial sums added
// through LDS, one launch: 8-15 % faster on 4096 -> 11008 and 8192 -> 28672), with fewer
// blocks two slices and up to four workgroups per block (the partial sums of the
// workgroups go through the workspace and a second launch; 0-10 % faster than eight
// workgroups). Four slices only for wavefront tiles of at most four matrix-core tiles.
struct NarrowSplit {
  int ks, splits;
};
NarrowSplit pick_narrow(int64_t blocks, int64_t M, int64_t N, int64_t K, int n_groups, int tiles) {
  const int s = pick_splits(blocks, M, N, K, n_groups);
  if (s <= 1) return {1, 1};
  if (blocks >= 80) return {s >= 3 && tiles <= 4 ? 4 : 2, 1};
  return {2, s < 4 ? s : 4};
}

// Output blocks of the default tiling for an M x N product (see launch_gemm).
template <int WAVES_M, int WM, int WN>
int64_t blocks_of(int64_t M, int64_t N) {
  constexpr int BM = WAVES_M * WM * 16, BN = (4 / WAVES_M) * WN * 16;
  return ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
}
// matrix-core tiles per wavefront of the default small-M tiling (M <= 64)
int default_wave_tiles(int64_t M, int64_t N, int64_t K) {
  if (M <= 16) return N * K <= (int64_t{1} << 26) ? 1 : 2;
  if (M <= 32) return N * K <= (int64_t{1} << 26) ? 2 : 4;
  return N * K <= (int64_t{1} << 26) ? 4 : 8;
}

int64_t default_blocks(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 && N * K <= (int64_t{1} << 26)) return blocks_of<1, 1, 1>(M, N);
  if (M <= 16) return blocks_of<1, 1, 2>(M, N);
  if (M <= 32 && N * K <= (int64_t{1} << 26)) return blocks_of<1, 2, 1>(M, N);
  if (M <= 32) return blocks_of<1, 2, 2>(M, N);
  if (M <= 64 && N * K <= (int64_t{1} << 26)) return blocks_of<1, 2, 2>(M, N);
  if (M <= 64) return blocks_of<1, 4, 2>(M, N);
  if (K >= 8192 || N >= 16384) return blocks_of<1, 8, 2>(M, N);
  return blocks_of<1, 4, 4>(M, N);
}

template <int WAVES_M, int WM, int WN, int SCHED = 0, int KS = 1>
hipError_t launch_tiles(GemmArgs a, hipStream_t st) {
  if (a.zeros_off >= 0) return launch_tiles_fmt<WAVES_M, WM, WN, SCHED, true, KS>(a, st);
  return launch_tiles_fmt<WAVES_M, WM, WN, SCHED, false, KS>(a, st);
}

// the small-M tilings with K also split inside the workgroup (KS slices of four wavefronts)
template <int WAVES_M, int WM, int WN>
hipError_t launch_tiles_ks(GemmArgs a, int ks, hipStream_t st) {
  // four slices (1024 threads, 128 VGPRs per lane) only for wavefront tiles of at most
  // four matrix-core tiles: larger ones would spill
  if constexpr (WM * WN <= 4) {
    if (ks == 4) return launch_tiles<WAVES_M, WM, WN, 0, 4>(a, st);
  }
  if (ks >= 2) return launch_tiles<WAVES_M, WM, WN, 0, 2>(a, st);
  return launch_tiles<WAVES_M, WM, WN, 0, 1>(a, st);
}

template <int S>
hipError_t launch_reduce_s(const float* part, int64_t mn, uint16_t* y, hipStream_t st) {
  hipLaunchKernelGGL(splitk_reduce_kernel<S>, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)),
                     dim3(256), 0, st, part, mn, y);
  return hipGetLastError();
}

}  // namespace

// splits in [2, 16] (every K split the launchers pick or accept)
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t mn, uint16_t* y,
                                hipStream_t st) {
  switch (splits) {
    case 2: return launch_reduce_s<2>(part, mn, y, st);
    case 3: return launch_reduce_s<3>(part, mn, y, st);
    case 4: return launch_reduce_s<4>(part, mn, y, st);
    case 5: return launch_reduce_s<5>(part, mn, y, st);
    case 6: return launch_reduce_s<6>(part, mn, y, st);
    case 7: return launch_reduce_s<7>(part, mn, y, st);
    case 8: return launch_reduce_s<8>(part, mn, y, st);
    case 9: return launch_reduce_s<9>(part, mn, y, st);
    case 10: return launch_reduce_s<10>(part, mn, y, st);
    case 11: return launch_reduce_s<11>(part, mn, y, st);
    case 12: return launch_reduce_s<12>(part, mn, y, st);
    case 13: return launch_reduce_s<13>(part, mn, y, st);
    case 14: return launch_reduce_s<14>(part, mn, y, st);
    case 15: return launch_reduce_s<15>(part, mn, y, st);
    case 16: return launch_reduce_s<16>(part, mn, y, st);
    default: return hipErrorInvalidValue;
  }
}

// Where the decode kernel (whole 16-row tiles and all of K per workgroup: no split, no
// second launch, no workspace) is faster than the split-K tiles (measured on MI355X, 4096
// <= K, N <= 28672): always at M <= 2 (4096 -> 11008: 6.5 / 7.0 instead of 10.2 / 10.4
// us; the 70B layers: 21.6 / 23.5 instead of 28.0 / 27.8 us); at M <= 4 on layers of at
// most 2^15 16 x 128 units (4096 -> 11008 at M = 4: 7.5 instead of 10.6 us) or of more than
// 512 row tiles (two tiles per workgroup there: 4096 -> 22016 / 8192 -> 28672 at M = 3,
// 11.7 / 25.3 instead of 14.5 / 27.4 us; with 512 tiles or fewer and long rows it runs
// sixteen wavefronts per tile, and 28672 -> 8192 at M = 3 / 4 takes 31 / 35 us there
// against 29 / 29 us for the split-K tiles); up to 16 rows
// on layers of at most 256 row tiles while the staged activations of its groups fit in
// LDS in about one pass (4096 -> 4096 at M = 8, 5.3 instead of 8.2 us; 11008 -> 4096 at
// M = 8, 11.4 instead of 12.7 us); and up to 16 rows on 257 .. 768 row tiles, where it
// runs one workgroup of two or three tiles per CU, when the activations fit in one pass
// (two for two tiles and K <= 8192): 4096 -> 6144 / 8192 / 11008 / 12288 at M = 8 6.5 /
// 6.7 / 8.6 / 8.7 instead of 9.3 / 9.4 / 9.5 / 9.6 us, 8192 -> 8192 at M = 16 14.2
// instead of 15.2 us; with more phases (5120 -> 12288 at M = 16, 28672 -> 8192 at M >= 5)
// the split-K tiles stay faster.
static bool small_m_takes_decode_kernel(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = (N + kTileN - 1) / kTileN, groups = K / kGroup;
  if (M <= 2) return true;
  if (M <= 4 && (tiles * groups <= (int64_t{1} << 15) || tiles > 512)) return true;
  if (M > 16) return false;
  if (tiles <= 256) return M * groups <= 704;
  if (tiles > 768) return false;
  const int phases = gemv_phases(M, N, K);
  return phases == 1 || (gemv_tiles_per_wg(M, N) == 2 && phases == 2 && groups <= 64);
}

// Large M runs the wide-tile kernel, which needs X' in the workspace when inv_s_c is
// given.
constexpr int64_t kWideMinM = 256;

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M >= kWideMinM) return gemm_wide_workspace_bytes(M, N, K);
  if (small_m_takes_decode_kernel(M, N, K)) return 0;
  const int64_t blocks = default_blocks(M, N, K);
  const int n_groups = static_cast<int>(K / kGroup);
  const int s = M <= 64 ? pick_narrow(blocks, M, N, K, n_groups, default_wave_tiles(M, N, K)).splits
                        : pick_splits(blocks, M, N, K, n_groups);
  return s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                       int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y,
                       void* ws, size_t ws_bytes, hipStream_t st) {
  // large M: wide wavefront tiles, X' from the workspace (or pre-scaled by the caller).
  // Tuning overrides for sweeps (libraries built for tuning): AWQ_GEMM_WIDE = "0" keeps the
  // narrow kernel, "[splits]<column tiles><K split>" (41, 42, 31, 32, 21, 22, 442, ...)
  // forces a wide configuration.
  const char* wide_str = tuning_env("AWQ_GEMM_WIDE");
  const int wide_env = wide_str == nullptr ? -1 : (wide_str[0] == '0' ? 0 : atoi(wide_str));
  const bool wide_ok =
      inv_s_c == nullptr || (ws != nullptr && ws_bytes >= static_cast<size_t>(M) * K * 2);
  if (M >= kWideMinM && wide_ok && wide_env != 0) {
    const int cfg = wide_env > 0 ? wide_env : 0;
    return launch_gemm_wide(x, inv_s_c, packed, M, N, K, group, fmt, y, ws, ws_bytes, cfg, st);
  }
  const PackedLayout L = make_layout(N, K, group, fmt);
  if (small_m_takes_decode_kernel(M, N, K)) {
    return launch_gemv(x, inv_s_c, packed, M, N, K, group, fmt, y, nullptr, 0, st);
  }
  GemmArgs a;
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
  a.sets = static_cast<int>(L.sets);
  // split K when the output blocks alone leave CUs idle and the caller gave a workspace
  // for the partial sums (without one the product runs unsplit)
  a.splits = 1;
  a.part = nullptr;
  const int64_t blocks = default_blocks(M, N, K);
  int want = pick_splits(blocks, M, N, K, a.n_groups);
  int ks = 1;
  if (M <= 64) {
    const NarrowSplit ns = pick_narrow(blocks, M, N, K, a.n_groups, default_wave_tiles(M, N, K));
    ks = ns.ks;
    want = ns.splits;
  }
  // AWQ_GEMM_SPLITS = "<splits>" forces the K split (tuning sweeps; needs a
  // workspace of splits * M * N * 4 bytes, else the product runs unsplit)
  const char* splits_str = tuning_env("AWQ_GEMM_SPLITS");
  const int splits_env = splits_str == nullptr ? 0 : atoi(splits_str);
  if (splits_env >= 1 && splits_env <= 16 && splits_env <= a.n_groups) want = splits_env;
  // AWQ_GEMM_KS = "<slices>,<splits>" (tuning sweeps): K split inside the workgroup over
  // 1, 2 or 4 slices of four wavefronts, and across <splits> workgroups
  if (const char* e = tuning_env("AWQ_GEMM_KS")) {
    int k1 = 1, s1 = 1;
    if (sscanf(e, "%d,%d", &k1, &s1) == 2 && (k1 == 1 || k1 == 2 || k1 == 4) && s1 >= 1 && s1 <= 16) {
      ks = k1;
      want = s1;
    }
  }
  if (want > 1 && ws != nullptr && ws_bytes >= static_cast<size_t>(want) * M * N * sizeof(float)) {
    a.splits = want;
    a.part = static_cast<float*>(ws);
  }
  // AWQ_GEMM_TILE = "waves_m,wm,wn,sched" selects another tiling (tuning sweeps)
  struct TileEnv {
    int wv = 0, wm = 0, wn = 0, sc = 0;
    bool set = false;
  };
  TileEnv tile_env;
  if (const char* env = tuning_env("AWQ_GEMM_TILE")) {
    tile_env.set = sscanf(env, "%d,%d,%d,%d", &tile_env.wv, &tile_env.wm, &tile_env.wn, &tile_env.sc) == 4;
  }
  if (tile_env.set) {
    const int wv = tile_env.wv, wm = tile_env.wm, wn = tile_env.wn, sc = tile_env.sc;
    if (wv == 1 && wm == 4 && wn == 4 && sc == 0) return launch_tiles<1, 4, 4, 0>(a, st);
    if (wv == 1 && wm == 4 && wn == 4 && sc == 2) return launch_tiles<1, 4, 4, 2>(a, st);
    if (wv == 1 && wm == 4 && wn == 4 && sc == 3) return launch_tiles<1, 4, 4, 3>(a, st);
    if (wv == 1 && wm == 4 && wn == 4 && sc == 4) return launch_tiles<1, 4, 4, 4>(a, st);
    if (wv == 1 && wm == 8 && wn == 4 && sc == 0) return launch_tiles<1, 8, 4, 0>(a, st);
    if (wv == 1 && wm == 8 && wn == 4 && sc == 2) return launch_tiles<1, 8, 4, 2>(a, st);
    if (wv == 1 && wm == 8 && wn == 2 && sc == 0) return launch_tiles<1, 8, 2, 0>(a, st);
    if (wv == 1 && wm == 8 && wn == 2 && sc == 3) return launch_tiles<1, 8, 2, 3>(a, st);
    if (wv == 1 && wm == 4 && wn == 2 && sc == 0) return launch_tiles<1, 4, 2, 0>(a, st);
    if (wv == 1 && wm == 4 && wn == 8 && sc == 0) return launch_tiles<1, 4, 8, 0>(a, st);
    if (wv == 2 && wm == 4 && wn == 4 && sc == 0) return launch_tiles<2, 4, 4, 0>(a, st);
    if (wv == 1 && wm == 2 && wn == 4 && sc == 0) return launch_tiles<1, 2, 4, 0>(a, st);
    if (wv == 1 && wm == 1 && wn == 4 && sc == 0) return launch_tiles<1, 1, 4, 0>(a, st);
    if (wv == 1 && wm == 1 && wn == 2 && sc == 0) return launch_tiles<1, 1, 2, 0>(a, st);
    if (wv == 1 && wm == 1 && wn == 1 && sc == 0) return launch_tiles<1, 1, 1, 0>(a, st);
    if (wv == 1 && wm == 2 && wn == 1 && sc == 0) return launch_tiles<1, 2, 1, 0>(a, st);
    if (wv == 1 && wm == 2 && wn == 2 && sc == 0) return launch_tiles<1, 2, 2, 0>(a, st);
  }
  // Defaults from sweeps on MI355X: at M <= 64 the product is bound by streaming the
  // weights, and narrow workgroup tiles give the most workgroups (16 x 64 up to M = 16 for
  // layers of at most 2^26 weights, else 16 x 128; 32 x 64 / 32 x 128 up to M = 32, where
  // each dequantized weight fragment serves both row tiles: 10-20 % faster than two
  // 16-row blocks; up to M = 64, 32 x 128 on layers of at most 2^26 weights (more
  // workgroups than 64 x 128: 5-22 % faster there), else 64 x 128), K split so that
  // the workgroups cover the CUs about 2.5 times; at larger M a 64 x 256 tile (each wavefront
  // 64 x 64) runs best, or for long K or wide N a 128 x 128 tile (each wavefront 128 x
  // 32), which dequantizes each weight fragment for 8 row tiles.
  if (M <= 16 && N * K <= (int64_t{1} << 26)) return launch_tiles_ks<1, 1, 1>(a, ks, st);
  if (M <= 16) return launch_tiles_ks<1, 1, 2>(a, ks, st);
  if (M <= 32 && N * K <= (int64_t{1} << 26)) return launch_tiles_ks<1, 2, 1>(a, ks, st);
  if (M <= 32) return launch_tiles_ks<1, 2, 2>(a, ks, st);
  if (M <= 64 && N * K <= (int64_t{1} << 26)) return launch_tiles_ks<1, 2, 2>(a, ks, st);
  if (M <= 64) return launch_tiles_ks<1, 4, 2>(a, ks, st);
  if (K >= 8192 || N >= 16384) return launch_tiles<1, 8, 2>(a, st);
  return launch_tiles<1, 4, 4>(a, st);
}

}  // namespace awq
