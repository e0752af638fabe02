// Internal declarations and device helpers of the gfx950 W4A16 library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/awq.h"

#include <stdio.h>
#include <stdlib.h>

#include <atomic>

namespace awq {

// ---------------------------------------------------------------- layout constants
// gfx950 packed layout, version 3: a 1 KiB unit holds 16 output rows x 128 input
// channels. Lane l of a wavefront owns 16 bytes of a unit: row l % 16, channels
// 32 (l / 16) + 0..31 of the unit, as four 32-bit words of eight channels each. Each
// unit carries S = max(1, 128 / G) sets of 16 scales (and zeros) for group size G: with
// G = 32 or 64 one set per group inside the unit (lane l uses set (l / 16) * S / 4),
// with G a multiple of 128 (per-channel included) the set of the group the unit lies in.
constexpr int kTileN = 16;        // output rows per unit
constexpr int kGroup = 128;       // input channels per unit
constexpr int kUnitBytes = 1024;  // 16 rows x 128 channels x 4 bits
constexpr int kLayoutVersion = 3;

struct PackedLayout {
  int64_t n_tiles;       // ceil(N / 16)
  int64_t n_groups;      // units along K: K / 128
  int64_t sets;          // scale / zero sets per unit: max(1, 128 / group)
  int64_t codes_off;     // byte offsets inside the packed buffer
  int64_t scales_off;
  int64_t zeros_off;     // -1 for the symmetric format
  int64_t total_bytes;
};

// the layout of an N x K layer with `sets` scale / zero sets per unit; kernels whose
// arguments are kept few call it on the device
__host__ __device__ inline PackedLayout make_layout_sets(int64_t N, int64_t K, int64_t sets, bool asym) {
  PackedLayout L;
  L.n_tiles = (N + kTileN - 1) / kTileN;
  L.n_groups = K / kGroup;
  L.sets = sets;
  L.codes_off = 0;
  L.scales_off = L.n_tiles * L.n_groups * kUnitBytes;
  int64_t end = L.scales_off + L.n_tiles * L.n_groups * L.sets * kTileN * 2;
  if (asym) {
    L.zeros_off = (end + 255) / 256 * 256;
    end = L.zeros_off + L.n_tiles * L.n_groups * L.sets * (kTileN / 2);
  } else {
    L.zeros_off = -1;
  }
  L.total_bytes = (end + 255) / 256 * 256;
  return L;
}

inline PackedLayout make_layout(int64_t N, int64_t K, int32_t group, int32_t fmt) {
  return make_layout_sets(N, K, group < kGroup ? kGroup / group : 1, fmt == 0);
}

// the scale / zero set lane (r, p) of a unit uses: p * S / 4 for S sets per unit
__host__ __device__ inline int lane_set(int p, int sets) { return (p * sets) >> 2; }

// ------------------------------------------------------------ launch helpers
// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once per device
// (the attribute is held per device); `done` is that kernel's bit set of devices done.
// Safe to call from several host threads: at worst two of them set the same value.
inline hipError_t ensure_lds_limit(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Tuning overrides for configuration sweeps: read from the environment only in a library
// built with -DAWQ_TUNING (python -m bit_weight_only_w4a16_amd.build --tuning); the
// product library reads no environment variable and always takes its default choices.
inline const char* tuning_env(const char* name) {
#ifdef AWQ_TUNING
  return getenv(name);
#else
  (void)name;
  return nullptr;
#endif
}

// Argument checks shared by the product entry points: an AWQ_* status.
int check_product(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
                  int64_t N, int64_t K, int32_t group, int32_t fmt, const uint16_t* y,
                  const void* ws, size_t ws_bytes);

// ------------------------------------------------------------ launchers (per file)
hipError_t launch_channel_scale(const uint16_t* x_cal, int64_t rows, int64_t K, double alpha,
                                uint16_t* s_c, uint16_t* inv_s_c, hipStream_t st);
hipError_t launch_pack(const uint16_t* w, const uint16_t* s_c, int64_t N, int64_t K,
                       int32_t group, int32_t fmt, int32_t* qweight, uint16_t* scales,
                       int32_t* qzeros, hipStream_t st);
hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                         int64_t N, int64_t K, int32_t group, int32_t fmt, void* packed,
                         hipStream_t st);
hipError_t launch_dequant_canonical(const int32_t* qweight, const uint16_t* scales,
                                    const int32_t* qzeros, int64_t N, int64_t K, int32_t group,
                                    int32_t fmt, uint16_t* w_out, hipStream_t st);
hipError_t launch_dequant_packed(const void* packed, int64_t N, int64_t K, int32_t group,
                                 int32_t fmt, uint16_t* w_out, hipStream_t st);

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K);
// The decode kernel's row tiles per workgroup and its number of X' staging phases for an
// M x N x K product (1 <= M <= 16)
int gemv_tiles_per_wg(int64_t M, int64_t N);
int gemv_phases(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                       int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y,
                       void* ws, size_t ws_bytes, hipStream_t st);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
size_t gemm_wide_workspace_bytes(int64_t M, int64_t N, int64_t K);
// y = binary16(sum over s of part[s]), part [splits][mn] float32, in split order
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t mn, uint16_t* y,
                                hipStream_t st);
size_t scale_search_workspace_bytes(int64_t rows, int64_t N, int64_t K, int32_t group,
                                    int32_t fmt);
hipError_t launch_scale_search(const uint16_t* w, const uint16_t* x_cal, int64_t rows,
                               int64_t N, int64_t K, int32_t group, int32_t fmt, int32_t grid,
                               double* losses, double* best_alpha, void* ws, hipStream_t st);
hipError_t launch_gemm_wide(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                            int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt,
                            uint16_t* y, void* ws, size_t ws_bytes, int cfg, hipStream_t st);
hipError_t launch_gemm(const uint16_t* x, const uint16_t* inv_s_c, const void* packed,
                       int64_t M, int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y,
                       void* ws, size_t ws_bytes, hipStream_t st);

size_t chain_state_bytes();
int chain_max_layers();
int chain_max_k();
int chain_min_k();
hipError_t launch_chain(const awq_chain_layer* layers, int n, uint32_t* state, hipStream_t st);

// ------------------------------------------------------------------ device helpers
// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin by workgroup
// number: workgroup i runs on XCD i % 8. Output block numbers are handed out so that
// each XCD gets a contiguous run of them (XCD x the blocks [x q + min(x, r), ...) with
// q = nb / 8, r = nb % 8, one more for the first r XCDs): a kernel that walks blocks down
// M first then keeps the blocks that share weight columns in one L2. A bijection on
// [0, nb) for any nb.
__device__ __forceinline__ int xcd_block(int i, int nb) {
  constexpr int kXcd = 8;
  const int q = nb / kXcd, r = nb % kXcd;
  const int x = i % kXcd, slot = i / kXcd;
  return x * q + (x < r ? x : r) + slot;
}

// Buffer resource over [base, base + bytes): loads take a wavefront-uniform SGPR offset
// plus a per-lane VGPR offset, so streaming through the weights costs no 64-bit address
// arithmetic; an offset past `bytes` reads 0. Word 3 is the gfx9 raw-buffer format.
// The SGPR offset goes through readfirstlane: callers pass uniform values, and this
// keeps the compiler from treating them as divergent (which would wrap every load in
// a scalarisation loop).
// Per-lane offset that lies past the end of every buffer resource used here (each covers
// less than 2^31 bytes: the entry points reject larger layers), so a load given it
// returns zeros without a memory access. Loads use it instead of a branch.
constexpr uint32_t kNoLoad = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                              __builtin_amdgcn_readfirstlane(static_cast<int>(soff)), 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// The same 16-byte load marked non-temporal (the `nt` cache-policy bit): for data read
// exactly once per call, so the caches keep the lines that are reused instead.
__device__ __forceinline__ uint4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  constexpr int kNonTemporal = 2;
  const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                              __builtin_amdgcn_readfirstlane(static_cast<int>(soff)),
                                              kNonTemporal);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff),
                                              __builtin_amdgcn_readfirstlane(static_cast<int>(soff)), 0);
}
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff),
                                              __builtin_amdgcn_readfirstlane(static_cast<int>(soff)), 0);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__host__ __device__ inline double f16_bits_to_f64(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int f = h & 0x3FF;
  double mag;
  if (e == 0x1F) {
    mag = f ? __builtin_nan("") : __builtin_inf();
  } else if (e == 0) {
    mag = __builtin_ldexp(static_cast<double>(f), -24);
  } else {
    mag = __builtin_ldexp(static_cast<double>(f + 1024), e - 25);
  }
  return (h & 0x8000) ? -mag : mag;
}

// Nearest binary16 to a float64, ties to even, subnormals kept, overflow to infinity.
// The value is scaled by a power of two (exact) so that one rint() in float64 does the
// rounding: in the subnormal range the units are 2^-24, elsewhere 2^(e-10).
__host__ __device__ inline uint16_t f64_to_f16_rn(double d) {
  const uint16_t sign = __builtin_signbit(d) ? 0x8000 : 0;
  const double a = __builtin_fabs(d);
  if (a != a) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;  // 65520 ties to the even neighbour: infinity
  if (a < 6.103515625e-05) {               // below 2^-14: subnormal units of 2^-24
    const double m = __builtin_rint(__builtin_ldexp(a, 24));
    return sign | static_cast<uint16_t>(m);  // m == 1024 is the smallest normal
  }
  int e;
  (void)__builtin_frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)  ->  a in [2^(e-1), 2^e)
  const int ex = e - 1;          // -14 .. 15
  const double m = __builtin_rint(__builtin_ldexp(a, 10 - ex));  // 1024 .. 2048
  const int bits = ((ex + 15) << 10) + (static_cast<int>(m) - 1024);
  return sign | static_cast<uint16_t>(bits);
}

// Four pairs of binary16 from one packed word in the gfx950 nibble order: pair p holds
// channels (2p, 2p + 1) of the word as binary16 (off + q), off = 1024 for p = 0, 2 and
// 64 for p = 1, 3. OR-ing a nibble into the fraction of 1024 (0x6400, unit 1) or of 64
// (0x5400, unit 1/16, nibble at bits 4..7) yields the integer exactly.
struct Pairs4 {
  uint32_t p[4];
};

// (a & mask) | magic in one v_and_or_b32. gfx9 VOP3 encodings take no literal
// constants, so left to itself the compiler splits this into a v_and and a v_or with
// literals; here the mask sits in an SGPR and the magic in a VGPR (one SGPR operand:
// the constant-bus limit).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

// For pairs that go on through ordinary ALU instructions (dequant_word): the compiler
// orders those after the asm like any other dependence.
__device__ __forceinline__ Pairs4 unpack_word(uint32_t w) {
  Pairs4 r;
  const uint32_t w8 = w >> 8;
  r.p[0] = and_or(w, 0x000F000Fu, 0x64006400u);
  r.p[1] = and_or(w, 0x00F000F0u, 0x54005400u);
  r.p[2] = and_or(w8, 0x000F000Fu, 0x64006400u);
  r.p[3] = and_or(w8, 0x00F000F0u, 0x54005400u);
  return r;
}

// For pairs that a matrix instruction reads directly. On gfx950 an MFMA may read a VGPR
// only two wait states after an ALU instruction wrote it; the compiler inserts those
// waits for the instructions it generates, but it does not treat inline asm as an ALU
// write, so an MFMA scheduled right behind an asm v_and_or_b32 could read the old
// register contents (this returned wrong sums in a decode variant where it happened).
// Here the four v_and_or_b32 are one asm block that ends with s_nop 1: whatever the
// compiler places next is at least two wait states after the last write. The outputs
// are early-clobber because the block writes them while still reading its inputs.
__device__ __forceinline__ Pairs4 unpack_word_mfma(uint32_t w) {
  Pairs4 r;
  const uint32_t w8 = w >> 8;
  asm("v_and_or_b32 %0, %4, %6, %7\n\t"
      "v_and_or_b32 %1, %4, %8, %9\n\t"
      "v_and_or_b32 %2, %5, %6, %7\n\t"
      "v_and_or_b32 %3, %5, %8, %9\n\t"
      "s_nop 1"
      : "=&v"(r.p[0]), "=&v"(r.p[1]), "=&v"(r.p[2]), "=&v"(r.p[3])
      : "v"(w), "v"(w8), "s"(0x000F000Fu), "v"(0x64006400u), "s"(0x00F000F0u), "v"(0x54005400u));
  return r;
}

// binary16 bit patterns of -(1024 + z) and -(64 + z), duplicated in both halves.
__device__ __forceinline__ uint32_t neg_off1024(uint32_t z) {
  const uint32_t h = 0xE400u | z;
  return h | (h << 16);
}
__device__ __forceinline__ uint32_t neg_off64(uint32_t z) {
  const uint32_t h = 0xD400u | (z << 4);
  return h | (h << 16);
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) {
  return __builtin_bit_cast(half2_t, u);
}
__device__ __forceinline__ uint32_t as_u32(half2_t h) {
  return __builtin_bit_cast(uint32_t, h);
}

// Exact dequantization of one word: eight binary16 values (q - z) * s in channel order.
// (off + q) - (off + z) is an exact small integer; one binary16 multiply rounds once.
// binary16(x * inv) for 8 channels (v_pk_mul_f16): the product of two binary16 values
// is exact before its one rounding to nearest even, as in the definition X' = X * inv_s_c
// rounded to binary16.
__device__ __forceinline__ uint4 scale_x8(uint4 val, uint4 iv) {
  const half2_t a0 = as_h2(val.x) * as_h2(iv.x), a1 = as_h2(val.y) * as_h2(iv.y);
  const half2_t a2 = as_h2(val.z) * as_h2(iv.z), a3 = as_h2(val.w) * as_h2(iv.w);
  return make_uint4(as_u32(a0), as_u32(a1), as_u32(a2), as_u32(a3));
}

__device__ __forceinline__ void dequant_word(uint32_t w, uint32_t nz1024, uint32_t nz64,
                                             half2_t s2, half2_t out[4]) {
  const Pairs4 pr = unpack_word(w);
  out[0] = (as_h2(pr.p[0]) + as_h2(nz1024)) * s2;
  out[1] = (as_h2(pr.p[1]) + as_h2(nz64)) * s2;
  out[2] = (as_h2(pr.p[2]) + as_h2(nz1024)) * s2;
  out[3] = (as_h2(pr.p[3]) + as_h2(nz64)) * s2;
}

// Offset of channel pair p of a word: 1024 for p even, 64 for p odd.
__host__ __device__ constexpr float pair_offset(int p) { return (p & 1) ? 64.0f : 1024.0f; }

}  // namespace awq
