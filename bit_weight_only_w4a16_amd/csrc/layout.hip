// Repack of the canonical 4-bit layout into the gfx950 layout, and the two bit-exact
// dequantizers (one per layout) used as parity probes and as the unfused baseline.
//
// gfx950 layout (byte-level definition in awq.h): a 1 KiB unit holds 16 output rows x
// 128 input channels, with one scale (and zero) set per group inside it for groups of
// 32 or 64 channels, or the set of its group for groups of 128 or more. Lane l of a
// wavefront owns the 16 bytes at 16 l: row l % 16, channels 32 (l / 16) .. + 31 of the
// unit, as four words of eight channels.
// One wavefront load instruction therefore moves a whole unit, fully coalesced; for the
// matrix cores the same 16 bytes are the B operands of four v_mfma_f32_16x16x32_f16
// (word i feeds step i: lane l gives column l % 16 and k slots 8 (l / 16) .. + 7).
// Inside each word the nibbles are interleaved (channel e at position
// (e >> 1) + 4 (e & 1)) so that one mask pulls channels (2p, 2p + 1) into the two
// halves of a register, ready to become binary16 by OR-ing in an exponent
// (edgesiliconlab ?p=2015, section "Kernel Execution: Marlin vs. ExLlamaV2 INT4 GEMM
// Micro-Architecture", item 3: 4-bit values are separated by shifts and masks and
// turned into binary16 right before the multiply).
#include "awq_internal.hpp"

namespace awq {
namespace {

__device__ __forceinline__ uint32_t interleave_nibbles(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t q = (w >> (4 * e)) & 0xFu;
    r |= q << (4 * ((e >> 1) + 4 * (e & 1)));
  }
  return r;
}

// one thread per (tile t, unit g, lane l): 16 bytes of codes; lanes with p < S also
// write row r's scale of set p (and, for r = 0 and 8, the set's two zero words). Set p
// of unit g is canonical group g * 128 / G + p for G < 128, else g * 128 / G.
__global__ void repack_kernel(const int32_t* __restrict__ qweight,
                              const uint16_t* __restrict__ scales,
                              const int32_t* __restrict__ qzeros, int N, int K, int n_groups,
                              int group, int sets, uint4* __restrict__ codes,
                              uint16_t* __restrict__ pscales, uint32_t* __restrict__ pzeros,
                              int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int l = static_cast<int>(i & 63);
  const int64_t unit = i >> 6;
  const int g = static_cast<int>(unit % n_groups);
  const int64_t t = unit / n_groups;
  const int r = l & 15, p = l >> 4;
  const int64_t n = t * kTileN + r;
  uint4 out = make_uint4(0, 0, 0, 0);
  if (n < N) {
    // canonical words (g * 128 + 32 p) / 8 .. + 3 of row n: 16 contiguous bytes
    const uint4 in =
        *reinterpret_cast<const uint4*>(qweight + n * (K / 8) + (g * kGroup + 32 * p) / 8);
    out.x = interleave_nibbles(in.x);
    out.y = interleave_nibbles(in.y);
    out.z = interleave_nibbles(in.z);
    out.w = interleave_nibbles(in.w);
  }
  codes[i] = out;
  if (p < sets) {
    const int64_t cg = static_cast<int64_t>(g) * kGroup / group + (group < kGroup ? p : 0);
    const int64_t set = unit * sets + p;
    pscales[set * kTileN + r] = n < N ? scales[cg * N + n] : uint16_t{0};
    if (pzeros && (r & 7) == 0) {
      // zeros of rows 16 t + r .. + 7: the canonical word (16 t + r) / 8 of group cg
      pzeros[set * 2 + (r >> 3)] =
          n < N ? static_cast<uint32_t>(qzeros[cg * (N / 8) + n / 8]) : 0u;
    }
  }
}

// canonical layout -> W_d, one thread per 32-bit word (8 channels of one row)
__global__ void dequant_canonical_kernel(const int32_t* __restrict__ qweight,
                                         const uint16_t* __restrict__ scales,
                                         const int32_t* __restrict__ qzeros, int N, int K,
                                         int group, uint4* __restrict__ out, int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int wpr = K / 8;
  const int64_t n = i / wpr;
  const int wi = static_cast<int>(i % wpr);
  const int g = wi * 8 / group;
  const uint32_t word = static_cast<uint32_t>(qweight[i]);
  const double s = f16_bits_to_f64(scales[static_cast<int64_t>(g) * N + n]);
  int z = 8;
  if (qzeros) {
    const uint32_t zw = static_cast<uint32_t>(qzeros[static_cast<int64_t>(g) * (N / 8) + n / 8]);
    z = static_cast<int>((zw >> (4 * (n % 8))) & 0xFu);
  }
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int q0 = static_cast<int>((word >> (8 * p)) & 0xFu);
    const int q1 = static_cast<int>((word >> (8 * p + 4)) & 0xFu);
    const uint32_t h0 = f64_to_f16_rn(static_cast<double>(q0 - z) * s);
    const uint32_t h1 = f64_to_f16_rn(static_cast<double>(q1 - z) * s);
    o[p] = h0 | (h1 << 16);
  }
  out[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

// gfx950 layout -> W_d, one thread per (tile, group, lane): 32 channels of one row,
// through the same magic-number unpack the matrix-core kernel uses.
__global__ void dequant_packed_kernel(const uint8_t* __restrict__ packed, int N, int K,
                                      int n_groups, int sets, int64_t scales_off,
                                      int64_t zeros_off, uint16_t* __restrict__ out,
                                      int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int l = static_cast<int>(i & 63);
  const int64_t unit = i >> 6;
  const int g = static_cast<int>(unit % n_groups);
  const int64_t t = unit / n_groups;
  const int r = l & 15, p = l >> 4;
  const int64_t n = t * kTileN + r;
  if (n >= N) return;
  const int64_t set = unit * sets + lane_set(p, sets);
  const uint16_t sb = reinterpret_cast<const uint16_t*>(packed + scales_off)[set * kTileN + r];
  uint32_t z = 8;
  if (zeros_off >= 0) {
    const uint32_t zw = reinterpret_cast<const uint32_t*>(packed + zeros_off)[set * 2 + (r >> 3)];
    z = (zw >> (4 * (r & 7))) & 0xFu;
  }
  const half2_t s2 = as_h2(static_cast<uint32_t>(sb) | (static_cast<uint32_t>(sb) << 16));
  const uint32_t nz1024 = neg_off1024(z), nz64 = neg_off64(z);
  const uint4 cw = reinterpret_cast<const uint4*>(packed)[i];
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
  uint4* dst = reinterpret_cast<uint4*>(out + n * K + static_cast<int64_t>(g) * kGroup + 32 * p);
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    half2_t h[4];
    dequant_word(words[wi], nz1024, nz64, s2, h);
    dst[wi] = make_uint4(as_u32(h[0]), as_u32(h[1]), as_u32(h[2]), as_u32(h[3]));
  }
}

inline unsigned blocks_for(int64_t total, int threads) {
  return static_cast<unsigned>((total + threads - 1) / threads);
}

}  // namespace

hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                         int64_t N, int64_t K, int32_t group, int32_t fmt, void* packed,
                         hipStream_t st) {
  const PackedLayout L = make_layout(N, K, group, fmt);
  uint8_t* base = static_cast<uint8_t*>(packed);
  const int64_t total = L.n_tiles * L.n_groups * 64;
  hipLaunchKernelGGL(repack_kernel, dim3(blocks_for(total, 256)), dim3(256), 0, st, qweight,
                     scales, fmt == 0 ? qzeros : nullptr, static_cast<int>(N),
                     static_cast<int>(K), static_cast<int>(L.n_groups), static_cast<int>(group),
                     static_cast<int>(L.sets), reinterpret_cast<uint4*>(base + L.codes_off),
                     reinterpret_cast<uint16_t*>(base + L.scales_off),
                     fmt == 0 ? reinterpret_cast<uint32_t*>(base + L.zeros_off) : nullptr, total);
  return hipGetLastError();
}

hipError_t launch_dequant_canonical(const int32_t* qweight, const uint16_t* scales,
                                    const int32_t* qzeros, int64_t N, int64_t K, int32_t group,
                                    int32_t fmt, uint16_t* w_out, hipStream_t st) {
  const int64_t total = N * (K / 8);
  hipLaunchKernelGGL(dequant_canonical_kernel, dim3(blocks_for(total, 256)), dim3(256), 0, st,
                     qweight, scales, fmt == 0 ? qzeros : nullptr, static_cast<int>(N),
                     static_cast<int>(K), static_cast<int>(group),
                     reinterpret_cast<uint4*>(w_out), total);
  return hipGetLastError();
}

hipError_t launch_dequant_packed(const void* packed, int64_t N, int64_t K, int32_t group,
                                 int32_t fmt, uint16_t* w_out, hipStream_t st) {
  const PackedLayout L = make_layout(N, K, group, fmt);
  const int64_t total = L.n_tiles * L.n_groups * 64;
  hipLaunchKernelGGL(dequant_packed_kernel, dim3(blocks_for(total, 256)), dim3(256), 0, st,
                     static_cast<const uint8_t*>(packed), static_cast<int>(N),
                     static_cast<int>(K), static_cast<int>(L.n_groups), static_cast<int>(L.sets),
                     L.scales_off, L.zeros_off, w_out, total);
  return hipGetLastError();
}

}  // namespace awq
