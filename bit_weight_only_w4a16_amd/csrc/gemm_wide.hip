// Prefill product y[M, N] = X' . deq(Wq)^T for large M on the gfx950 matrix cores, with
// wide wavefront tiles.
//
// Prefill is bound by matrix-core throughput (edgesiliconlab ?p=2015, section "GEMM vs.
// GEMV Kernels and Batch Size Dynamics"); the weights are turned into binary16 in
// registers right before the matrix instruction (same page, section "Kernel Execution:
// Marlin vs. ExLlamaV2 INT4 GEMM Micro-Architecture", item 3), exactly
// W_d = binary16((q - z) * s). Three resources compete per 128-channel group: the
// matrix core, the VALU work of that dequantization (13 instructions per 8 weights),
// and LDS bandwidth for the activation operand. A wavefront tile of 128 rows x 64
// columns (8 x 4 matrix-core tiles of 16 x 16) reuses each dequantized weight fragment
// for 8 row tiles and each activation fragment for 4 column tiles, which keeps the
// dequantization near 40 % and the LDS reads near 50 % of the matrix-core time.
//
//  * X' = binary16(X * inv_s_c) is formed once per call by `prescale_kernel` (into the
//    caller's workspace) or passed in pre-scaled, so the activation tile can go from
//    memory straight into LDS: `buffer_load_dwordx4 ... lds` writes each lane's 16 bytes
//    at LDS base + 16 * lane, no registers involved. Rows are 256 bytes with no padding;
//    16-byte chunk c of row r is stored at chunk position c ^ (r % 16) (the lanes pick
//    their global chunk accordingly), so the 16 rows read by one matrix-core fragment
//    load fall in 16 different bank groups.
//  * Activation tiles are double-buffered in LDS (2 x 32 KiB), one barrier per group; the
//    weights of the next group are in registers while a group is multiplied; every load
//    is issued unconditionally: a prefetch past the wavefront's last group re-reads that
//    group (an L2 hit, never multiplied), so no load needs a per-lane offset of its own.
//  * Four wavefronts side by side along N: a workgroup covers 128 x 256 outputs (or
//    128 x 192 / 128 x 128 with three / two column tiles per wavefront); accumulators in
//    VGPRs. With few output blocks, eight wavefronts split K in two (see KS below).
#include "awq_internal.hpp"

namespace awq {
namespace {

constexpr int kBM = 128;              // rows of X' per workgroup
constexpr int kRowBytes = kGroup * 2;  // one activation row of a group: 256 B
constexpr int kTileBytes = kBM * kRowBytes;

struct WideArgs {
  const uint16_t* xs;  // X' [M][K] binary16
  const uint8_t* packed;
  uint16_t* y;
  int64_t scales_off;
  int64_t zeros_off;
  uint32_t packed_bytes;
  int M, N, K, n_groups, n_tiles, n_blocks_m, n_blocks_n, sets;
  float* part;  // splits > 1: float32 partial sums [splits][M][N]
  int splits;
};

__global__ void __launch_bounds__(256) prescale_kernel(const uint16_t* x, const uint16_t* inv,
                                                       int64_t total, int K, uint16_t* xs) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= total) return;
  const uint4 xv = *reinterpret_cast<const uint4*>(x + i);
  const uint4 iv = *reinterpret_cast<const uint4*>(inv + i % K);
  *reinterpret_cast<uint4*>(xs + i) = scale_x8(xv, iv);
}

// KS = 2 splits K inside the workgroup: wavefronts 4..7 take the second half of the
// groups with their own pair of LDS buffers, and add their sums to those of wavefronts
// 0..3 through LDS at the end (in a fixed order), which gives two wavefronts per SIMD
// when there are too few output blocks to fill the CUs twice.
template <int WN, int KS, bool ASYM>
__global__ void __launch_bounds__(256 * KS) gemm_wide_kernel(WideArgs a) {
  constexpr int WM = 8;
  constexpr int BN = 4 * WN * 16;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_all[];  // [KS][2][kBM][256 B]

  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave_all >> 2;        // which part of K
  const int wave = wave_all & 3;          // column slot within the workgroup
  unsigned char* smem = smem_all + half * 2 * kTileBytes;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, p = lane >> 4;

  const int nb = a.n_blocks_m * a.n_blocks_n;
  const int bid = xcd_block(blockIdx.x, nb);
  // output blocks in bands of 8 row blocks, row block fastest within a band: the ~64
  // workgroups resident on one XCD at a time (consecutive block numbers) then cover about
  // 8 row blocks x 8 column blocks, so its L2 holds fewer distinct X' rows and weight
  // columns than with all row blocks x a few column blocks (measured: 1.5-3.5 % faster
  // on the Llama-3-8B prefill shapes)
  const int per_band = 8 * a.n_blocks_n;
  const int band = bid / per_band;
  const int rows_in = min(8, a.n_blocks_m - band * 8);
  const int lb = bid - band * per_band;
  const int bm = band * 8 + lb % rows_in, bn = lb / rows_in;
  const int m_blk = bm * kBM, n_blk = bn * BN;
  const int ng = a.n_groups;
  // this workgroup's units [ga, gb) (split blockIdx.y of K), then this wavefront's
  // [g0, g1); both halves run the same number of trips
  const int per = (ng + a.splits - 1) / a.splits;
  const int ga = min(ng, static_cast<int>(blockIdx.y) * per), gb = min(ng, ga + per);
  const int span = gb - ga, hspan = (span + 1) / 2;
  const int g0 = ga + half * hspan;
  const int g1 = KS == 1 ? gb : min(gb, g0 + hspan);
  const int trips = KS == 1 ? span : hspan;

  // weights: one resource over the packed layer, per-tile SGPR offsets (tiles past the
  // last are clamped: their outputs are never stored)
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.packed, a.packed_bytes);
  const uint32_t sbytes = 2 * kTileN * a.sets, zbytes = 8 * a.sets;  // per unit
  uint32_t code_off[WN], scale_off[WN], zero_off[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const uint32_t tile = static_cast<uint32_t>(min(n_blk / kTileN + wave * WN + j, a.n_tiles - 1));
    code_off[j] = tile * ng * kUnitBytes;
    scale_off[j] = static_cast<uint32_t>(a.scales_off) + tile * ng * sbytes;
    zero_off[j] = ASYM ? static_cast<uint32_t>(a.zeros_off) + tile * ng * zbytes : 0u;
  }
  const int lset = lane_set(p, a.sets);
  const uint32_t lane_code = 16u * lane, lane_scale = 2u * (kTileN * lset + r),
                 lane_zero = 4u * (2 * lset + (r >> 3));
  const int zshift = 4 * (r & 7);

  // activations: this block's rows (rows past M read as 0). Wavefront w fills LDS rows
  // 32 w .. 32 w + 31 of a buffer with 8 instructions of 4 rows each; lane l of
  // instruction j writes row 32 w + 4 j + l / 16, chunk position l % 16, which holds the
  // global chunk (l % 16) ^ (row % 16).
  const int rows_here = min(kBM, a.M - m_blk);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xs + static_cast<int64_t>(m_blk) * a.K,
                                              static_cast<uint32_t>(rows_here) * a.K * 2);
  uint32_t a_voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 32 * wave + 4 * j + (lane >> 4);
    const int chunk = (lane & 15) ^ (row & 15);
    a_voff[j] = static_cast<uint32_t>(row * a.K + 8 * chunk) * 2;
  }
  auto dma_a = [&](int g, int buf) {
    const int soff = max(min(g, g1 - 1), 0) * kRowBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      unsigned char* dst = smem + buf * kTileBytes + (32 * wave + 4 * j) * kRowBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(dst), 16,
          static_cast<int>(a_voff[j]), __builtin_amdgcn_readfirstlane(soff), 0, 0);
    }
  };

  struct BRegs {
    uint4 c[WN];
    uint32_t s[WN], z[WN];
  };
  auto load_b = [&](BRegs& b, int g) {
    const uint32_t gg = static_cast<uint32_t>(max(min(g, g1 - 1), 0));
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      b.c[j] = buf_load16(rp, lane_code, code_off[j] + gg * kUnitBytes);
      b.s[j] = buf_load2(rp, lane_scale, scale_off[j] + gg * sbytes);
      if (ASYM) b.z[j] = buf_load4(rp, lane_zero, zero_off[j] + gg * zbytes);
    }
  };

  float4_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // The unpack constants live in registers whose values the compiler does not see (mask
  // in an SGPR, magic in a VGPR), so (w & mask) | magic stays one ordinary v_and_or_b32:
  // an instruction the scheduler can place between matrix instructions and whose
  // read-after-write distance to them it tracks (gfx9 VOP3 takes no literal constants).
  uint32_t mask0, mask1, magic0, magic1;
  asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(mask0));
  asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(mask1));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic0));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(magic1));
  // exact dequantization of one word (eight weights of one column): (off + q) - (off + z)
  // is an exact small integer, times s rounded once to binary16
  auto deq = [&](uint32_t w, uint32_t nz1024, uint32_t nz64, half2_t s2) -> half8_t {
    const uint32_t w8 = w >> 8;
    const half2_t d0 = (as_h2((w & mask0) | magic0) + as_h2(nz1024)) * s2;
    const half2_t d1 = (as_h2((w & mask1) | magic1) + as_h2(nz64)) * s2;
    const half2_t d2 = (as_h2((w8 & mask0) | magic0) + as_h2(nz1024)) * s2;
    const half2_t d3 = (as_h2((w8 & mask1) | magic1) + as_h2(nz64)) * s2;
    return half8_t{d0.x, d0.y, d1.x, d1.y, d2.x, d2.y, d3.x, d3.y};
  };

  auto compute = [&](const BRegs& b, int buf) {
    const unsigned char* src = smem + buf * kTileBytes;
    half2_t s2[WN];
    uint32_t nz1024[WN], nz64[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const uint32_t z = ASYM ? (b.z[j] >> zshift) & 0xFu : 8u;
      s2[j] = as_h2(b.s[j] | (b.s[j] << 16));
      nz1024[j] = neg_off1024(z);
      nz64[j] = neg_off64(z);
    }
    auto word = [&](int i, int j) -> uint32_t {
      return i == 0 ? b.c[j].x : i == 1 ? b.c[j].y : i == 2 ? b.c[j].z : b.c[j].w;
    };
    // A fragment of row tile ms at k-step i: row 16 ms + r, chunk 4 p + i (swizzled)
    auto afrag = [&](int i, int ms) -> half8_t {
      const int chunk = (4 * p + i) ^ r;
      return *reinterpret_cast<const half8_t*>(src + (16 * ms + r) * kRowBytes + 16 * chunk);
    };
    // Software pipeline over the (k-step, column) blocks of the group: while column j of
    // k-step i is multiplied (eight matrix instructions, one per row tile), the next
    // column's weights (or column 0 of k-step i + 1) are dequantized, and during the last
    // column of a k-step the next k-step's X' fragments are read, each right after its
    // last use. Scheduling groups place one matrix instruction, then up to two ALU
    // instructions and one LDS read, so that a wavefront's ALU work issues while its own
    // matrix instructions run (about two ALU instructions fit under one): matrix-core
    // busy 0.59 -> 0.62 and co-issued cycles 0.22 -> 0.35 of it on 4096 -> 28672 at
    // M = 2048, with the same sums in the same order.
    half8_t af[WM];
#pragma unroll
    for (int ms = 0; ms < WM; ++ms) af[ms] = afrag(0, ms);
    half8_t bcur = deq(word(0, 0), nz1024[0], nz64[0], s2[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const bool last = j == WN - 1;
        const int ni = last ? i + 1 : i, nj = last ? 0 : j + 1;
        half8_t bnext = bcur;
        if (ni < 4) bnext = deq(word(ni, nj), nz1024[nj], nz64[nj], s2[nj]);
#pragma unroll
        for (int ms = 0; ms < WM; ++ms) {
          acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[ms], bcur, acc[ms][j], 0, 0, 0);
          if (last && i < 3) af[ms] = afrag(i + 1, ms);
        }
        // 13 ALU instructions of the next dequantization: 2, 2, 2, 2, 2, 1, 1, 1
#pragma unroll
        for (int ms = 0; ms < WM; ++ms) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
          if (ni < 4) {
            if (ms < 5) {
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // ALU
            } else {
              __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
            }
          }
          if (last && i < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
        bcur = bnext;
      }
    }
  };

  // prologue: A(0) in LDS buffer 0, B(0) in registers
  BRegs b0, b1;
  dma_a(g0, 0);
  load_b(b0, g0);
  __builtin_amdgcn_s_waitcnt(0);  // the A(g0) transfers have landed
  __syncthreads();

  // two groups per trip; while group g is multiplied from one buffer, A(g + 1) streams
  // into the other and B(g + 1) into registers; one barrier per group (every wavefront
  // of the workgroup takes the same number of trips, so the barriers match)
  // the multiply runs at raised wavefront priority: a wavefront that has its operands
  // keeps the matrix core while the other wavefronts of the SIMD wait at the barrier or
  // issue their loads, which keeps the wavefronts of a SIMD out of phase
  for (int t = 0; t < trips; t += 2) {
    const int g = g0 + t;
    dma_a(g + 1, 1);
    load_b(b1, g + 1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if (g < g1) compute(b0, 0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    dma_a(g + 2, 0);
    load_b(b0, g + 2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if (g + 1 < g1) compute(b1, 1);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if constexpr (KS == 2) {
    // the second half's sums through LDS (its buffers are free now): float4 i of lane l
    // of column slot w at [i][w][l], so that consecutive lanes write consecutive 16 bytes
    float4_t* red = reinterpret_cast<float4_t*>(smem_all);
    if (half == 1) {
#pragma unroll
      for (int ms = 0; ms < WM; ++ms)
#pragma unroll
        for (int j = 0; j < WN; ++j) red[((ms * WN + j) * 4 + wave) * 64 + lane] = acc[ms][j];
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int ms = 0; ms < WM; ++ms) {
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[ms][j] += red[((ms * WN + j) * 4 + wave) * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);  // one row tile at a time: no reloads held live
    }
  }

  // binary16 results, or with K split across workgroups this split's float32 sums
  float* part = a.part + static_cast<int64_t>(blockIdx.y) * a.M * a.N;
#pragma unroll
  for (int ms = 0; ms < WM; ++ms) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n_blk + (wave * WN + j) * 16 + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m_blk + ms * 16 + 4 * p + q;
        if (m < a.M && n < a.N) {
          const int64_t o = static_cast<int64_t>(m) * a.N + n;
          if (a.splits > 1) {
            part[o] = acc[ms][j][q];
          } else {
            a.y[o] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[ms][j][q]));
          }
        }
      }
    }
  }
}

template <int WN, int KS, bool ASYM>
hipError_t launch_wide_fmt(WideArgs a, hipStream_t st) {
  constexpr int BN = 4 * WN * 16;
  const size_t lds = 2ull * KS * kTileBytes;
  static std::atomic<uint64_t> lds_done{0};
  const hipError_t ea = ensure_lds_limit(reinterpret_cast<const void*>(&gemm_wide_kernel<WN, KS, ASYM>),
                                         static_cast<int>(lds), lds_done);
  if (ea != hipSuccess) return ea;
  a.n_blocks_m = (a.M + kBM - 1) / kBM;
  a.n_blocks_n = (a.N + BN - 1) / BN;
  const unsigned blocks = static_cast<unsigned>(a.n_blocks_m) * static_cast<unsigned>(a.n_blocks_n);
  hipLaunchKernelGGL((gemm_wide_kernel<WN, KS, ASYM>), dim3(blocks, a.splits), dim3(256 * KS),
                     lds, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_splitk_reduce(a.part, a.splits, static_cast<int64_t>(a.M) * a.N, a.y, st);
}

template <int WN, int KS>
hipError_t launch_wide(const WideArgs& a, hipStream_t st) {
  return a.zeros_off >= 0 ? launch_wide_fmt<WN, KS, true>(a, st) : launch_wide_fmt<WN, KS, false>(a, st);
}

// Column tiles per wavefront and K split for an M x N product, aiming at two workgroups
// per CU (from sweeps on MI355X): 128 x 256 workgroup tiles when they give that many;
// else 128 x 192 tiles when N divides into them and they do; else, with at most one
// 128 x 256 block per CU, K split in two inside the workgroup, and when the blocks
// cover fewer than half of the CUs, K split across floor(256 / blocks) workgroups as
// well (float32 partial sums in the workspace; each split at least 4 units, at most
// 16). In that last case 128 x 192 tiles are taken instead when they fill more of the
// 256 CUs (ragged N: 4096 -> 11008 at M = 256 and 512).
struct WidePick {
  int wn, ks, splits;
};
WidePick pick_wide(int64_t M, int64_t N, int64_t K) {
  const int64_t mb = (M + kBM - 1) / kBM;
  const int64_t blocks4 = mb * ((N + 255) / 256), blocks3 = mb * ((N + 191) / 192);
  if (blocks4 >= 512) return {4, 1, 1};
  if (N % 192 == 0 && blocks3 >= 512) return {3, 1, 1};
  if (blocks4 > 256) return {4, 1, 1};
  auto splits_for = [&](int64_t blocks) {
    int64_t s = 256 / blocks;
    s = s < K / (4 * kGroup) ? s : K / (4 * kGroup);
    s = s < 16 ? s : 16;
    return s < 1 ? int64_t{1} : s;
  };
  const int64_t s4 = splits_for(blocks4);
  if (blocks3 <= 256) {
    const int64_t s3 = splits_for(blocks3);
    if (blocks3 * s3 > blocks4 * s4) return {3, 2, s3 < 2 ? 1 : static_cast<int>(s3)};
  }
  return {4, 2, s4 < 2 ? 1 : static_cast<int>(s4)};
}

inline int64_t align256(int64_t b) { return (b + 255) & ~int64_t{255}; }

}  // namespace

// X' first ([M][K] binary16, 256-byte aligned), then the partial sums of a K split.
size_t gemm_wide_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const WidePick w = pick_wide(M, N, K);
  const int64_t part = w.splits > 1 ? static_cast<int64_t>(w.splits) * M * N * 4 : 0;
  return static_cast<size_t>(align256(M * K * 2) + part);
}

// X' into the workspace when inv_s_c is given, then the product; the K split across
// workgroups only when the workspace (ws_bytes) holds its partial sums as well.
// cfg = 100 * splits + 10 * column tiles per wavefront + K split in the workgroup, or 0
// for the default choice.
hipError_t launch_gemm_wide(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                            int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                            uint16_t* y, void* ws, size_t ws_bytes, int cfg, hipStream_t st) {
  const PackedLayout L = make_layout(N, K, group, fmt);
  const uint16_t* xs = x;
  if (inv_s_c != nullptr) {
    uint16_t* dst = static_cast<uint16_t*>(ws);
    const int64_t total = M * K;
    hipLaunchKernelGGL(prescale_kernel, dim3(static_cast<unsigned>((total / 8 + 255) / 256)),
                       dim3(256), 0, st, x, inv_s_c, total, static_cast<int>(K), dst);
    xs = dst;
  }
  WideArgs a;
  a.xs = xs;
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
  WidePick w = pick_wide(M, N, K);
  if (cfg != 0) w = {(cfg / 10) % 10, cfg % 10, cfg >= 100 ? (cfg / 100 < 16 ? cfg / 100 : 16) : 1};
  const int64_t part_off = align256(M * K * 2);
  a.splits = 1;
  a.part = nullptr;
  if (w.splits > 1 && ws != nullptr &&
      ws_bytes >= static_cast<size_t>(part_off + static_cast<int64_t>(w.splits) * M * N * 4)) {
    a.splits = w.splits;
    a.part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + part_off);
  }
  const int wn = w.wn, ks = w.ks;
  if (wn == 4 && ks == 1) return launch_wide<4, 1>(a, st);
  if (wn == 4 && ks == 2) return launch_wide<4, 2>(a, st);
  if (wn == 3 && ks == 1) return launch_wide<3, 1>(a, st);
  if (wn == 3 && ks == 2) return launch_wide<3, 2>(a, st);
  if (wn == 2 && ks == 1) return launch_wide<2, 1>(a, st);
  if (wn == 2 && ks == 2) return launch_wide<2, 2>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace awq
