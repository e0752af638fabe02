// Decode product y[M, N] = X' . deq(Wq)^T for 1 <= M <= 16 on gfx950.
//
// At batch 1 the product reads every weight once and does two flops per weight, so it
// is bound by memory bandwidth (edgesiliconlab ?p=2015, section "The Mathematics of
// Memory Bandwidth Saturation"; section "GEMM vs. GEMV Kernels and Batch Size
// Dynamics"). The kernel is built around streaming the 4-bit codes:
//
//  * a workgroup owns one 16-row weight tile and the whole of K, so no partial sums
//    leave the workgroup (no split-K workspace, no atomics, no cross-XCD traffic);
//  * its wavefronts take interleaved 128-channel groups; for each group one wavefront
//    load moves a whole 1 KiB unit (one 128-bit load per lane, fully coalesced). Two
//    batches of groups are in flight per wavefront: both are requested before the
//    activations are staged, and each batch is refilled as soon as it is consumed;
//  * the code loads are marked non-temporal (each code byte is read once per call), which
//    leaves the caches to the activations and the scales: 1-8 % faster, most on the 70B
//    layers;
//  * every load is issued unconditionally: a load with nothing to fetch gets a per-lane
//    offset past the end of its buffer resource, which returns zeros without a memory
//    access. With no branch around a load the compiler's wait counts are exact, so a
//    wavefront waits for the batch it is about to use and never for the one behind it;
//  * each wavefront stages X' = binary16(X * inv_s_c) in LDS for its own groups only
//    (activations requested before the weights), so the wavefronts never wait for each
//    other before the final sum of their partial results.
//
// The arithmetic runs on the matrix cores. A nibble OR-ed into binary16 1024 (or 64) is
// (off + q) exactly; in the gfx950 layout the four words a lane loads are the B operands
// of the four k-steps of v_mfma_f32_16x16x32_f16 for the group, so after the 5-op unpack
// per word the matrix core forms D[m][n] = sum_k X'[m][k] (off_k + q[n][k]) over the
// group in four instructions (v_dot2 would take 16 per lane and row). Per group,
// y[m][n] += s[n] * (D[m][n] - O[m] - z[n] S[m]), where O[m] = sum_k X'[m][k] off_k and
// S[m] = sum_k X'[m][k] over the group are formed once when X' is staged. This is the
// decode-time dequantize-in-registers of edgesiliconlab ?p=2015 (section "Kernel
// Execution: Marlin vs. ExLlamaV2 INT4 GEMM Micro-Architecture"), with the zero point
// and scale applied once per group and output instead of once per weight.
//
// The A operand of lane l is X' row l % 16; lanes of rows >= M repeat row M - 1, whose
// results are dropped. Lane (r, p) holds D rows 4 p .. 4 p + 3 for weight row r.
#include "awq_internal.hpp"

#include <stdio.h>
#include <stdlib.h>

namespace awq {
namespace {

// LDS a workgroup may use for X', O and S: with several workgroups per CU 60 KiB (two
// fit beside each other), with at most one per CU 144 KiB
constexpr int kLdsShared = 61440, kLdsAlone = 147456;

struct MvArgs {
  const uint16_t* x;
  const uint16_t* inv;
  const uint8_t* packed;
  uint16_t* y;
  int64_t scales_off;
  int64_t zeros_off;
  int N, K, n_groups, phase_groups, sets;
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// v + (v from lane `ctrl` of the same 16-lane row), one data-parallel-primitive move
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}

// Sum over the 16 lanes of a row, left in every lane of it: swap neighbours, swap pairs
// (quad permutations [1,0,3,2] and [2,3,0,1]), then add the mirrored half-row and the
// mirrored row. Every lane adds the same two operands at each step, so all 16 hold the
// same bits. Four ALU operations with no LDS round trip.
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  return dpp_add<0x140>(v);
}

// Orders a wavefront's LDS accesses for the compiler: staging stores by some lanes are
// read back by other lanes of the same wavefront, which a per-lane view of memory does
// not see as a dependence. A wavefront-scope release/acquire fence pair is an IR-level
// memory operation (wave_barrier alone is not), so no load is hoisted above it and no
// store is sunk below it; the hardware executes one wavefront's LDS operations in order,
// so nothing more is needed.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int M>
struct XPass {
  uint4 x[M];
  uint4 inv;
};

// EXACT (groups of 32 or 64 channels, several scale sets per unit): the weights are
// dequantized exactly to W_d before the matrix core, which then sums across groups; the
// per-group correction needs one scale per matrix-core sum and does not apply.
// The arguments are scalars rather than one struct, fourteen dwords in all, so that the
// compiler marks them for kernarg preloading: the command processor writes them into
// SGPRs when it launches a wavefront, and the kernel starts without waiting for a load
// of its argument block (0.3-0.4 us of a 4-7 us decode launch on MI355X).
template <int M, int WAVES, int BATCH, bool ASYM, bool EXACT, int T>
__global__ void __launch_bounds__(WAVES * 64)
    gemv_kernel(const uint16_t* x, const uint16_t* inv, const uint8_t* packed, uint16_t* y,
                uint32_t scales_off, uint32_t zeros_off, int N, int K, int phase_groups, int n_sets) {
  MvArgs a;
  a.x = x;
  a.inv = inv;
  a.packed = packed;
  a.y = y;
  a.scales_off = scales_off;
  a.zeros_off = zeros_off;
  a.N = N;
  a.K = K;
  a.n_groups = K / kGroup;
  a.phase_groups = phase_groups;
  a.sets = n_sets;
  constexpr int JM = M < 4 ? M : 4;  // D rows per lane that can be real rows
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // T > 1: the workgroup takes T consecutive 16-row tiles (every wavefront's staged X'
  // then serves T weight tiles); a tile past the last one reads the last one again and
  // stores nothing (its rows are >= N)
  const int t0 = blockIdx.x * T;
  const int n_tiles = (a.N + kTileN - 1) / kTileN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, p = lane >> 4;
  const int ng = a.n_groups;
  const bool has_inv = a.inv != nullptr;
  // LDS slots use fixed strides (the largest phase), so a group's slots belong to the
  // wavefront that owns the group in every phase
  const int PG = a.phase_groups, PK = a.phase_groups * kGroup;
  _Float16* xs = reinterpret_cast<_Float16*>(smem);        // [M][PK]
  float* osum = reinterpret_cast<float*>(smem + 2 * M * PK);  // [M][PG]
  float* ssum = osum + M * PG;                               // [M][PG]
  float* red = ssum + M * PG;                                // [WAVES][M][T * 16]

  const int sets = a.sets;
  const uint32_t sbytes = 2 * kTileN * sets, zbytes = 8 * sets;  // per unit
  __amdgpu_buffer_rsrc_t rcodes[T], rscales[T], rzeros[T];
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const int64_t t = T == 1 ? t0 : min(t0 + j, n_tiles - 1);
    rcodes[j] = make_rsrc(a.packed + t * ng * kUnitBytes, ng * kUnitBytes);
    rscales[j] = make_rsrc(a.packed + a.scales_off + t * ng * sbytes, ng * sbytes);
    rzeros[j] = make_rsrc(a.packed + (ASYM ? a.zeros_off : 0) + t * ng * zbytes, ng * zbytes);
  }
  const int lset = lane_set(p, sets);
  const uint32_t lane_code = 16u * lane, lane_scale = 2u * (kTileN * lset + r),
                 lane_zero = 4u * (2 * lset + (r >> 3));
  const int zshift = 4 * (r & 7);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, static_cast<uint32_t>(M * a.K * 2));
  const __amdgpu_buffer_rsrc_t rinv =
      make_rsrc(has_inv ? a.inv : a.x, has_inv ? static_cast<uint32_t>(a.K * 2) : 0u);
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  const int arow = r < M ? r : M - 1;

  float yacc[T][JM];
#pragma unroll
  for (int tj = 0; tj < T; ++tj)
#pragma unroll
    for (int j = 0; j < JM; ++j) yacc[tj][j] = 0.0f;
  float4_t dacc[T];  // EXACT: sum over groups of X' W_d
#pragma unroll
  for (int tj = 0; tj < T; ++tj) dacc[tj] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  struct Batch {
    uint4 c[BATCH][T];
    uint32_t s[BATCH][T], z[BATCH][T];
  };
  // groups gl = wave + WAVES * j of the phase, j < nj; a slot past nj loads nothing
  auto load = [&](Batch& b, int ph0, int jb, int nj) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const bool live = jb + u < nj;
      const uint32_t g = live ? static_cast<uint32_t>(ph0 + wave + WAVES * (jb + u)) : 0u;
      const uint32_t skip = live ? 0u : kNoLoad;
#pragma unroll
      for (int tj = 0; tj < T; ++tj) {
        b.c[u][tj] = buf_load16_stream(rcodes[tj], lane_code + skip, g * kUnitBytes);
        b.s[u][tj] = buf_load2(rscales[tj], lane_scale + skip, g * sbytes);
        if (ASYM) b.z[u][tj] = buf_load4(rzeros[tj], lane_zero + skip, g * zbytes);
      }
    }
  };
  auto compute = [&](const Batch& b, int jb, int nj) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (jb + u < nj) {
        const int gl = wave + WAVES * (jb + u);
        const _Float16* xg = xs + arow * PK + gl * kGroup + 32 * p;
        if constexpr (EXACT) {
          half2_t s2[T];
          uint32_t nz1024[T], nz64[T];
#pragma unroll
          for (int tj = 0; tj < T; ++tj) {
            const uint32_t z = ASYM ? (b.z[u][tj] >> zshift) & 0xFu : 8u;
            s2[tj] = as_h2(b.s[u][tj] | (b.s[u][tj] << 16));
            nz1024[tj] = neg_off1024(z);
            nz64[tj] = neg_off64(z);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const half8_t af = *reinterpret_cast<const half8_t*>(xg + 8 * i);
#pragma unroll
            for (int tj = 0; tj < T; ++tj) {
              const uint32_t w = i == 0 ? b.c[u][tj].x : i == 1 ? b.c[u][tj].y : i == 2 ? b.c[u][tj].z : b.c[u][tj].w;
              half2_t dq[4];
              dequant_word(w, nz1024[tj], nz64[tj], s2[tj], dq);
              const half8_t bf = {dq[0].x, dq[0].y, dq[1].x, dq[1].y, dq[2].x, dq[2].y, dq[3].x, dq[3].y};
              dacc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, dacc[tj], 0, 0, 0);
            }
          }
          continue;
        }
#pragma unroll
        for (int tj = 0; tj < T; ++tj) {
          const uint32_t words[4] = {b.c[u][tj].x, b.c[u][tj].y, b.c[u][tj].z, b.c[u][tj].w};
          float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const Pairs4 pr = unpack_word_mfma(words[i]);
            const u32x4_t bw = {pr.p[0], pr.p[1], pr.p[2], pr.p[3]};
            const half8_t af = *reinterpret_cast<const half8_t*>(xg + 8 * i);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, __builtin_bit_cast(half8_t, bw), d, 0, 0, 0);
          }
          const float s = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b.s[u][tj])));
          const float z = ASYM ? static_cast<float>((b.z[u][tj] >> zshift) & 0xFu) : 8.0f;
#pragma unroll
          for (int j = 0; j < JM; ++j) {
            const int m = min(4 * p + j, M - 1);
            const int e = m * PG + gl;
            yacc[tj][j] += s * (d[j] - osum[e] - z * ssum[e]);
          }
        }
      }
    }
  };

  // Activation staging per wavefront, four groups per pass: lane (r, p) converts
  // channels 8 r .. 8 r + 7 of the pass's group p; the 16 lanes of a group then add up
  // O and S for it.
  auto xpass_load = [&](XPass<M>& P, int ph0, int c, int nj) {
    const int j = 4 * c + p;
    const bool live = j < nj;
    const uint32_t ch = static_cast<uint32_t>((ph0 + wave + WAVES * j) * kGroup + 8 * r);
#pragma unroll
    for (int m = 0; m < M; ++m) P.x[m] = buf_load16(rx, live ? 2u * (m * a.K + ch) : kNoLoad, 0);
    P.inv = buf_load16(rinv, live ? 2u * ch : kNoLoad, 0);
  };
  auto xpass_store = [&](const XPass<M>& P, int c, int nj) {
    const half2_t one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    const half2_t o1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
    const half2_t o64 = {static_cast<_Float16>(64.0f), static_cast<_Float16>(64.0f)};
    const int j = 4 * c + p;
    const int gl = wave + WAVES * j;
    const uint4 iv = has_inv ? P.inv : ones;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4 val = scale_x8(P.x[m], iv);
      // channel k of a word has offset 1024 if k % 8 is in {0, 1, 4, 5}, else 64
      float sv = __builtin_amdgcn_fdot2(as_h2(val.x), one2, 0.0f, false);
      sv = __builtin_amdgcn_fdot2(as_h2(val.y), one2, sv, false);
      sv = __builtin_amdgcn_fdot2(as_h2(val.z), one2, sv, false);
      sv = __builtin_amdgcn_fdot2(as_h2(val.w), one2, sv, false);
      float ov = __builtin_amdgcn_fdot2(as_h2(val.x), o1024, 0.0f, false);
      ov = __builtin_amdgcn_fdot2(as_h2(val.y), o64, ov, false);
      ov = __builtin_amdgcn_fdot2(as_h2(val.z), o1024, ov, false);
      ov = __builtin_amdgcn_fdot2(as_h2(val.w), o64, ov, false);
      sv = row_sum16(sv);
      ov = row_sum16(ov);
      if (j < nj) {
        *reinterpret_cast<uint4*>(xs + m * PK + gl * kGroup + 8 * r) = val;
        if (!EXACT && r == 0) {
          ssum[m * PG + gl] = sv;
          osum[m * PG + gl] = ov;
        }
      }
    }
  };
  constexpr int PRE = M <= 2 ? 2 : 1;  // passes whose loads go out before the weights

  for (int ph0 = 0; ph0 < ng; ph0 += PG) {
    const int ngp = min(PG, ng - ph0);
    const int nj = wave < ngp ? (ngp - wave + WAVES - 1) / WAVES : 0;
    const int npass = (nj + 3) / 4;
    XPass<M> P[PRE];
#pragma unroll
    for (int c = 0; c < PRE; ++c) xpass_load(P[c], ph0, c, nj);
    Batch b0, b1;
    load(b0, ph0, 0, nj);
    load(b1, ph0, BATCH, nj);
#pragma unroll
    for (int c = 0; c < PRE; ++c) xpass_store(P[c], c, nj);
    for (int c = PRE; c < npass; ++c) {
      XPass<M> Q;
      xpass_load(Q, ph0, c, nj);
      xpass_store(Q, c, nj);
    }
    wave_lds_sync();  // staged X', O, S visible to every lane before the products
    for (int jb = 0; jb < nj; jb += 2 * BATCH) {
      compute(b0, jb, nj);
      load(b0, ph0, jb + 2 * BATCH, nj);
      compute(b1, jb + BATCH, nj);
      load(b1, ph0, jb + 3 * BATCH, nj);
    }
    wave_lds_sync();  // this phase's reads done before the next phase restages the slots
  }

  if constexpr (EXACT) {
#pragma unroll
    for (int tj = 0; tj < T; ++tj)
#pragma unroll
      for (int j = 0; j < JM; ++j) yacc[tj][j] = dacc[tj][j];
  }
  // the wavefronts' partial sums through LDS; one thread per (row, output) writes y
  constexpr int TN = T * kTileN;
#pragma unroll
  for (int tj = 0; tj < T; ++tj)
#pragma unroll
    for (int j = 0; j < JM; ++j) {
      const int m = 4 * p + j;
      if (m < M) red[(wave * M + m) * TN + tj * kTileN + r] = yacc[tj][j];
    }
  __syncthreads();
  for (int i = threadIdx.x; i < M * TN; i += WAVES * 64) {
    const int m = i / TN, c = i % TN;
    float v = red[m * TN + c];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v += red[(w * M + m) * TN + c];
    const int n = t0 * kTileN + c;
    if (n < a.N) {
      a.y[static_cast<int64_t>(m) * a.N + n] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
  }
}

// X' phase length (groups staged at once). One workgroup per tile (T = 1): 144 KiB of LDS
// when at most one workgroup runs per CU (n_tiles <= 256), else 60 KiB (two fit beside
// each other). With T tiles per workgroup the same two cases, less the partial-sum area.
int phase_groups_for(int M, int n_groups, int64_t n_tiles, int T, int waves) {
  const int64_t wgs = (n_tiles + T - 1) / T;
  int budget;
  if (T == 1) {
    budget = n_tiles <= 256 ? kLdsAlone : kLdsShared;
  } else {
    budget = (wgs <= 256 ? 163840 : 81920) - 4 * waves * M * kTileN * T - 1024;
  }
  int pg = budget / (M * (2 * kGroup + 8));
  if (pg > n_groups) pg = n_groups;
  return pg < 1 ? 1 : pg;
}

size_t smem_bytes(int M, int phase_groups, int waves, int T) {
  return static_cast<size_t>(2) * M * phase_groups * kGroup + 8ull * M * phase_groups +
         4ull * waves * M * kTileN * T;
}

template <int M, int WAVES, int BATCH, bool ASYM, bool EXACT, int T>
hipError_t launch_fmt(const MvArgs& a, int64_t n_tiles, hipStream_t st) {
  const size_t lds = smem_bytes(M, a.phase_groups, WAVES, T);
  static std::atomic<uint64_t> lds_done{0};
  const hipError_t ea = ensure_lds_limit(
      reinterpret_cast<const void*>(&gemv_kernel<M, WAVES, BATCH, ASYM, EXACT, T>), 163840, lds_done);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((gemv_kernel<M, WAVES, BATCH, ASYM, EXACT, T>),
                     dim3(static_cast<unsigned>((n_tiles + T - 1) / T)), dim3(WAVES * 64), lds, st,
                     a.x, a.inv, a.packed, a.y, static_cast<uint32_t>(a.scales_off),
                     static_cast<uint32_t>(ASYM ? a.zeros_off : 0), a.N, a.K, a.phase_groups, a.sets);
  return hipGetLastError();
}

// The per-group correction needs the activation sums O and S of every row: from five
// rows on, staging them costs more than dequantizing each weight exactly, so M > 4 (and
// groups of 32 or 64) take the exact form.
template <int M, int WAVES, int BATCH, int T = 1>
hipError_t launch_cfg(const MvArgs& a, int64_t n_tiles, hipStream_t st) {
  const bool asym = a.zeros_off >= 0;
  if (M > 4 || a.sets > 1) {
    return asym ? launch_fmt<M, WAVES, BATCH, true, true, T>(a, n_tiles, st)
                : launch_fmt<M, WAVES, BATCH, false, true, T>(a, n_tiles, st);
  }
  if constexpr (M <= 4) {
    return asym ? launch_fmt<M, WAVES, BATCH, true, false, T>(a, n_tiles, st)
                : launch_fmt<M, WAVES, BATCH, false, false, T>(a, n_tiles, st);
  }
  return hipErrorInvalidValue;
}

// Tiles per workgroup at M >= 2. Each wavefront stages the activations of every row for
// its groups, and with T tiles per workgroup that staging serves T weight tiles; a
// workgroup's time also grows with its share of a CU. From sweeps of T = 1 .. 4 at
// M = 1 .. 16 on K = 4096 with 256 .. 1792 row tiles and on the 70B layers (MI355X): up
// to 768 tiles, T = ceil(tiles / 256), one workgroup per CU (4096 -> 11008 at M = 2 / 4 /
// 8 / 16: 7.0 / 7.5 / 8.6 / 9.4 us against 8.6 / 9.6 / 13.1 / 21.6 with one tile); beyond
// that two tiles, four from M = 12 (8192 -> 28672 at M = 2 / 16: 23.5 / 50 instead of
// 28.2 / 89 us). At M = 1 the differences stayed within the run-to-run spread (4096 ->
// 11008: 6.47 / 6.45 us with one / three tiles), and the tuned one-tile launch is kept.
// Tuning builds: AWQ_GEMV_T forces 1 .. 4.
int tiles_per_wg(int M, int64_t n_tiles) {
  if (const char* env = tuning_env("AWQ_GEMV_T")) {
    const int t = atoi(env);
    if (t >= 1 && t <= 4) return t;
  }
  if (M == 1 || n_tiles <= 256) return 1;
  if (n_tiles <= 768) return static_cast<int>((n_tiles + 255) / 256);
  return M >= 12 ? 4 : 2;
}

// From sweeps on MI355X (4096 <= K, N <= 28672): long rows on few tiles (K >= 8192,
// N <= 8192, so at most two workgroups per CU) take 16 wavefronts with one group in
// flight each; everything else eight wavefronts with one group each. Sixteen
// wavefronts leave 128 VGPRs per lane, which the staging of more than four activation
// rows overflows (spills to scratch), so M > 4 always takes eight.
int waves_for(int M, int n_groups, int64_t n_tiles) {
  return M <= 4 && n_groups >= 64 && n_tiles <= 512 ? 16 : 8;
}

template <int M>
hipError_t launch_m(const MvArgs& a, int64_t n_tiles, int T, hipStream_t st) {
  if constexpr (M <= 4) {
    if (waves_for(M, a.n_groups, n_tiles) == 16) return launch_cfg<M, 16, 1>(a, n_tiles, st);
  }
  if (T == 4) return launch_cfg<M, 8, 1, 4>(a, n_tiles, st);
  if (T == 3) return launch_cfg<M, 8, 1, 3>(a, n_tiles, st);
  if (T == 2) return launch_cfg<M, 8, 1, 2>(a, n_tiles, st);
  return launch_cfg<M, 8, 1>(a, n_tiles, st);
}

// Tuning override for sweeps (M = 1 only, libraries built for tuning): AWQ_GEMV_CFG =
// "waves,batch".
hipError_t launch_m1(const MvArgs& a, int64_t n_tiles, int T, hipStream_t st) {
  int cfg = 0;
  if (const char* env = tuning_env("AWQ_GEMV_CFG")) {
    int w = 0, b = 0;
    if (sscanf(env, "%d,%d", &w, &b) == 2) cfg = 10 * w + b;
  }
  switch (cfg) {
    case 42: return launch_cfg<1, 4, 2>(a, n_tiles, st);
    case 44: return launch_cfg<1, 4, 4>(a, n_tiles, st);
    case 84: return launch_cfg<1, 8, 4>(a, n_tiles, st);
    case 81: return launch_cfg<1, 8, 1>(a, n_tiles, st);
    case 82: return launch_cfg<1, 8, 2>(a, n_tiles, st);
    case 161: return launch_cfg<1, 16, 1>(a, n_tiles, st);
    case 162: return launch_cfg<1, 16, 2>(a, n_tiles, st);
    default: return launch_m<1>(a, n_tiles, T, st);
  }
}

}  // namespace

size_t gemv_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

int gemv_tiles_per_wg(int64_t M, int64_t N) {
  return tiles_per_wg(static_cast<int>(M), (N + kTileN - 1) / kTileN);
}

int gemv_phases(int64_t M, int64_t N, int64_t K) {
  const int64_t n_tiles = (N + kTileN - 1) / kTileN;
  const int ng = static_cast<int>(K / kGroup);
  const int T = tiles_per_wg(static_cast<int>(M), n_tiles);
  const int pg = phase_groups_for(static_cast<int>(M), ng, n_tiles, T,
                                  T == 1 ? waves_for(static_cast<int>(M), ng, n_tiles) : 8);
  return (ng + pg - 1) / pg;
}

hipError_t launch_gemv(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                       int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y,
                       void*, size_t, hipStream_t st) {
  const PackedLayout L = make_layout(N, K, group, fmt);
  MvArgs a;
  a.x = x;
  a.inv = inv_s_c;
  a.packed = static_cast<const uint8_t*>(packed);
  a.y = y;
  a.scales_off = L.scales_off;
  a.zeros_off = L.zeros_off;
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.n_groups = static_cast<int>(L.n_groups);
  a.sets = static_cast<int>(L.sets);
  const int T = tiles_per_wg(static_cast<int>(M), L.n_tiles);
  a.phase_groups = phase_groups_for(static_cast<int>(M), a.n_groups, L.n_tiles, T,
                                    T == 1 ? waves_for(static_cast<int>(M), a.n_groups, L.n_tiles) : 8);
  switch (M) {
    case 1: return launch_m1(a, L.n_tiles, T, st);
    case 2: return launch_m<2>(a, L.n_tiles, T, st);
    case 3: return launch_m<3>(a, L.n_tiles, T, st);
    case 4: return launch_m<4>(a, L.n_tiles, T, st);
    case 5: return launch_m<5>(a, L.n_tiles, T, st);
    case 6: return launch_m<6>(a, L.n_tiles, T, st);
    case 7: return launch_m<7>(a, L.n_tiles, T, st);
    case 8: return launch_m<8>(a, L.n_tiles, T, st);
    case 9: return launch_m<9>(a, L.n_tiles, T, st);
    case 10: return launch_m<10>(a, L.n_tiles, T, st);
    case 11: return launch_m<11>(a, L.n_tiles, T, st);
    case 12: return launch_m<12>(a, L.n_tiles, T, st);
    case 13: return launch_m<13>(a, L.n_tiles, T, st);
    case 14: return launch_m<14>(a, L.n_tiles, T, st);
    case 15: return launch_m<15>(a, L.n_tiles, T, st);
    case 16: return launch_m<16>(a, L.n_tiles, T, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
