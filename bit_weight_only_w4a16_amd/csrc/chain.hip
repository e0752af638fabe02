// Decode chain: the M = 1 products of a decoder block in one launch on gfx950.
//
// At batch 1 each product streams its weights once and is bound by memory bandwidth
// (edgesiliconlab ?p=2015, section "The Mathematics of Memory Bandwidth Saturation":
// tokens per second = bandwidth / bytes per token). A decoder block is a short sequence
// of such products, some of which take an earlier product's output as their input. Run
// as one launch per product, every product pays the launch (about 1.6 us between two
// dependent kernels on MI355X) and a full memory round trip before its first weight
// arrives, which at 4096 x 4096 is as long as the transfer itself. Here one launch runs
// the whole sequence on a grid of one workgroup per CU:
//
//  * the layers' 16-row tiles are numbered one after another and dealt to the
//    workgroups round-robin, so every workgroup walks its tiles in layer order;
//  * fifteen streaming wavefronts per workgroup take interleaved 128-channel units of
//    each tile, as the single-product decode kernel does, but their weight loads run a
//    fixed number of units ahead through a ring of registers that does not stop at a
//    layer boundary: while a layer waits for its input, the next layer's weights are
//    already on the way. Each wavefront converts its own units' slice of a layer's input
//    to X' = binary16(X * inv_s_c) and forms the per-group sums, as that kernel does;
//  * a control wavefront does all of the workgroup's global synchronisation, so the
//    streaming wavefronts never wait on a global memory operation other than their own
//    weight loads: it loads each layer's inv_s_c and, once it exists, its input into LDS
//    with direct-to-LDS loads (several layers' inputs are held at once), adds the
//    streaming wavefronts' partial sums of a tile in fixed order, writes y, and
//    publishes the layer's completion;
//  * a layer whose input is an earlier layer's output waits until every tile of that
//    layer is complete. Outputs are written with returning agent-scope atomics, which
//    are performed where all XCDs see them; once they have returned, a per-XCD counter
//    is incremented. Consumers poll the counters with agent-scope loads and load the
//    input with agent-scope loads, so no L2 write-back or invalidation is needed;
//  * every wait is bounded by the real-time counter: a wait that runs out is counted in
//    word 0 of the state buffer and the kernel goes on, so it always ends.
//
// Workgroups wait only for tiles of earlier layers and for their own wavefronts, and
// the grid is no larger than the number of workgroups the device holds at once, so
// every wait ends. The arithmetic per unit is the decode kernel's per-group correction
// (y += s (D - O - z S), D on the matrix cores), in the same order.
#include "../../include/awq.h"
#include "awq_internal.hpp"

namespace awq {
namespace {

constexpr int kMaxChain = AWQ_CHAIN_MAX_LAYERS;  // layers per launch
constexpr int kSub = 8;             // completion counters per layer (by workgroup % 8 = XCD)
constexpr int kSlots = 8;           // LDS slots for the partial sums of a tile
constexpr int kMaxBufs = 3;         // layer inputs held in LDS at once
constexpr int kMaxK = 16384;        // input channels per layer
constexpr int kMinK = 15 * 128;     // one unit per streaming wavefront and tile
constexpr int kLdsLimit = 160 * 1024;
constexpr int kCounterStride = 32;  // words between counters (128 bytes)
constexpr uint64_t kSpinTicks = uint64_t{1} << 24;  // about 0.17 s at 100 MHz

// state words: [0] count of waits that ran out, [32] workgroups done, counters from word 64
constexpr int kErrWord = 0, kDoneWord = 32, kCntWord = 64;
constexpr size_t kStateBytes = 4u * (kCntWord + kMaxChain * kSub * kCounterStride);

__host__ __device__ constexpr int cnt_word(int layer, int sub) {
  return kCntWord + (layer * kSub + sub) * kCounterStride;
}

struct ChainLayerDev {
  const uint16_t* x;  // input: the caller's x, or the y of layer `src`
  const uint16_t* inv;
  const uint8_t* packed;
  uint16_t* y;
  uint32_t packed_bytes;
  uint32_t scales_off;
  uint32_t zeros_off;
  int32_t N;
  int32_t K;
  int32_t ng;          // units along K
  int32_t n_tiles;
  int32_t tile_begin;  // first global tile number
  int32_t src;         // -1 or an earlier layer
  int32_t asym;
};

struct ChainArgs {
  ChainLayerDev L[kMaxChain];
  uint32_t* state;
  int32_t n_layers;
  int32_t nbuf;      // layer inputs held in LDS at once
  uint32_t consumed; // bit l: some layer reads layer l's output
  int32_t kpad;  // binary16 values per input buffer: the largest K rounded up to 512
};
// The kernel reads its arguments in place through the kernel-argument segment: scalar
// loads, also when indexed by layer (a by-value copy would go to scratch).
typedef __attribute__((address_space(4))) const ChainArgs KArgs;

// ---------------------------------------------------------------- uniform values
// Everything that steers the wavefronts (layer, tile and unit cursors, buffer bases,
// flags) is the same in every lane. Reading it through readfirstlane keeps it in scalar
// registers, so buffer resources and offsets never need a per-lane loop and the waits
// stay uniform branches.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// a flag or counter in LDS, read by every lane and taken from the first
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
  return uni(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
// the same value stored by every lane: no branch on the lane number
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup"); }
__device__ __forceinline__ void lds_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); }

// the 100 MHz real-time counter, uniform across the wavefront
__device__ __forceinline__ uint64_t now_ticks() {
  const uint64_t t = __builtin_amdgcn_s_memrealtime();
  const uint32_t lo = uni(static_cast<uint32_t>(t));
  const uint32_t hi = uni(static_cast<uint32_t>(t >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Buffer resource over the state words; an access given kNoLoad as its lane offset is
// not performed, so "lane 0 only" needs no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_rsrc(uint32_t* state) {
  return make_rsrc(state, static_cast<uint32_t>(kStateBytes));
}
__device__ __forceinline__ uint32_t lane0_off(uint32_t word) {
  return (threadIdx.x & 63) == 0 ? 4u * word : kNoLoad;
}
// count a wait that ran out (word 0 of the state), at agent scope or wider (sc1)
__device__ __forceinline__ void flag_error(uint32_t* state) {
  (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, state_rsrc(state), static_cast<int>(lane0_off(kErrWord)), 0, 16);
}

// v + (v from lane `ctrl` of the same 16-lane row)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
// sum over the 16 lanes of a row, the same bits in every lane of it
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  return dpp_add<0x140>(v);
}

struct Lds {
  KArgs* args;            // the kernel arguments
  _Float16* xs;           // [nbuf][kpad] a layer's input X, turned into X' in place
  _Float16* xinv;         // [nbuf][kpad] its inv_s_c
  float* os;              // [nbuf][kpad / 128]  sum of X' * offset per group
  float* ss;              // [nbuf][kpad / 128]  sum of X' per group
  float* part;            // [kSlots][WAVES][16] partial sums of a tile
  uint32_t* arrive;       // [kSlots][WAVES] generation of the partial a wavefront delivered
  uint32_t* gen;          // [kSlots] generations of the slot summed
  uint32_t* landed;       // [kMaxChain] the layer's input is in its buffer
  uint32_t* err;          // a streaming wavefront's wait ran out
  int kpad, gpad, nbuf;
};

// per-layer fields (scalar loads)
#define LF(s, li, field) ((s).args->L[uni(li)].field)
__device__ __forceinline__ int n_layers(const Lds& s) { return s.args->n_layers; }

// first global tile of layer li that workgroup b owns, or -1
__device__ __forceinline__ int first_tile(const Lds& s, int li, int b, int P) {
  const int tb = LF(s, li, tile_begin);
  const int g0 = tb + ((b - tb) % P + P) % P;
  return g0 < tb + LF(s, li, n_tiles) ? g0 : -1;
}

// A workgroup's position in the global tile order: tile g of layer li (tile t of it),
// unit u of the tile.
struct Cursor {
  int li, g, tend, t, u, ng;
};

__device__ __forceinline__ void cursor_seek(const Lds& s, Cursor& c) {
  const int n = n_layers(s);
  while (c.li < n && c.g >= LF(s, c.li, tile_begin) + LF(s, c.li, n_tiles)) c.li = uni(c.li + 1);
  if (c.li < n) {
    const int tb = LF(s, c.li, tile_begin);
    c.tend = uni(tb + LF(s, c.li, n_tiles));
    c.t = uni(c.g - tb);
    c.ng = LF(s, c.li, ng);
  }
}

template <int WAVES>
__device__ __forceinline__ void cursor_next(const Lds& s, Cursor& c, int wave, int P) {
  c.u = uni(c.u + WAVES);
  if (c.u >= c.ng) {
    c.u = wave;
    c.g = uni(c.g + P);
    c.t = uni(c.t + P);
    if (c.g >= c.tend) cursor_seek(s, c);
  }
}

// ----------------------------------------------------------------- streaming wavefronts
// Turn this wavefront's units of layer li's input (units wave, wave + WAVES, ...) into
// X' = binary16(X * inv_s_c) in place, and form per unit S = sum X' and O = sum X' *
// offset (offset 1024 or 64 by channel, as the unpacked codes carry it). Lane (r, p)
// takes channels 8 r .. 8 r + 7 of unit 4 c + p of pass c; the 16 lanes of a unit then
// add up its sums (all of them store the same bits).
template <int WAVES>
__device__ __forceinline__ void convert_input(const Lds& s, int li, int bf, int wave) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, p = lane >> 4;
  const int ng = LF(s, li, ng);
  const bool has_inv = LF(s, li, inv) != nullptr;
  const int nj = (ng - wave + WAVES - 1) / WAVES;
  const half2_t one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  const half2_t o1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  const half2_t o64 = {static_cast<_Float16>(64.0f), static_cast<_Float16>(64.0f)};
  _Float16* xb = s.xs + bf * s.kpad;
  const _Float16* ib = s.xinv + bf * s.kpad;
  for (int c = 0; c < nj; c += 4) {
    // a lane past this wavefront's units reads the last unit of the buffer and stores nothing
    const int u = wave + WAVES * (c + p);
    const bool live = c + p < nj;
    const int ch = (live ? u : s.gpad - 1) * kGroup + 8 * r;
    uint4 val = *reinterpret_cast<const uint4*>(xb + ch);
    if (has_inv) val = scale_x8(val, *reinterpret_cast<const uint4*>(ib + ch));
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
    if (live) {
      *reinterpret_cast<uint4*>(xb + ch) = val;
      s.ss[bf * s.gpad + u] = sv;
      s.os[bf * s.gpad + u] = ov;
    }
  }
  // this wavefront's own LDS writes, read back by other lanes of it
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int WAVES, int D>
__device__ __forceinline__ void stream_waves(const Lds& s, int wave) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, p = lane >> 4;
  const int P = gridDim.x, b = blockIdx.x;
  const int nl = n_layers(s);
  const uint32_t lane_code = 16u * lane, lane_scale = 2u * r, lane_zero = 4u * (r >> 3);
  const int zshift = 4 * (r & 7);

  struct Slot {
    uint4 c;
    uint32_t s, z;
  };
  Slot ring[D];

  Cursor C;
  C.li = 0;
  C.g = b;
  C.u = wave;
  C.tend = C.t = C.ng = 0;
  cursor_seek(s, C);
  Cursor Ld = C;
  __amdgpu_buffer_rsrc_t rw = make_rsrc(s.xs, 0);
  uint32_t soff = 0, zoff = 0, zskip = kNoLoad;
  int ld_li = -1;
  // load the unit under the load cursor into a slot and move the cursor on; past the
  // last unit the loads read nothing (offset kNoLoad)
  auto issue = [&](Slot& sl) {
    const bool live = Ld.li < nl;
    if (live && Ld.li != ld_li) {
      ld_li = Ld.li;
      rw = make_rsrc(LF(s, ld_li, packed), LF(s, ld_li, packed_bytes));
      soff = LF(s, ld_li, scales_off);
      zoff = LF(s, ld_li, zeros_off);
      zskip = LF(s, ld_li, asym) ? 0u : kNoLoad;  // the symmetric format has no zeros
    }
    const uint32_t unit = live ? static_cast<uint32_t>(uni(Ld.t * Ld.ng + Ld.u)) : 0u;
    const uint32_t skip = live ? 0u : kNoLoad;
    sl.c = buf_load16_stream(rw, lane_code + skip, unit * kUnitBytes);
    sl.s = buf_load2(rw, lane_scale + skip, soff + unit * (2 * kTileN));
    sl.z = buf_load4(rw, lane_zero + (skip | zskip), zoff + unit * 8);
    if (live) cursor_next<WAVES>(s, Ld, wave, P);
  };

#pragma unroll
  for (int i = 0; i < D; ++i) issue(ring[i]);

  // units this wavefront computes in all: a fixed trip count keeps the ring unrolled
  int total = 0;
  for (int li = 0; li < nl; ++li) {
    const int f = first_tile(s, li, b, P);
    if (f < 0) continue;
    const int te = LF(s, li, tile_begin) + LF(s, li, n_tiles);
    const int ng = LF(s, li, ng);
    total = uni(total + (te - f + P - 1) / P * ((ng - wave + WAVES - 1) / WAVES));
  }

  float yacc = 0.0f;
  int cur_li = -1, ord = -1, bf = 0;
  uint32_t tseq = 0;
  bool asym = false;
  // The only vector-memory instructions here are the ring's loads, three per slot and
  // issued in every slot of every pass (past the last unit they read nothing), so the
  // compiler's wait before a slot's use counts exactly the loads behind it. A wait that
  // runs out is recorded in LDS; the control wavefront reports it.
  for (int base = 0; base < total; base += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (base + i < total) {
        if (C.li != cur_li) {  // first unit of a layer: its input must be in LDS
          cur_li = C.li;
          ord = uni(ord + 1);
          bf = uni(ord % s.nbuf);
          asym = LF(s, cur_li, asym) != 0;
          const uint64_t t0 = now_ticks();
          while (lds_ld(s.landed + cur_li) == 0u) {
            __builtin_amdgcn_s_sleep(4);
            if (now_ticks() - t0 > kSpinTicks) {
              lds_st(s.err, 1u);
              break;
            }
          }
          lds_acquire();
          convert_input<WAVES>(s, cur_li, bf, wave);
        }
        const Slot& sl = ring[i];
        const _Float16* xg = s.xs + bf * s.kpad + C.u * kGroup + 32 * p;
        const uint32_t words[4] = {sl.c.x, sl.c.y, sl.c.z, sl.c.w};
        float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const Pairs4 pr = unpack_word_mfma(words[k]);
          typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
          const u32x4_t bw = {pr.p[0], pr.p[1], pr.p[2], pr.p[3]};
          const half8_t af = *reinterpret_cast<const half8_t*>(xg + 8 * k);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, __builtin_bit_cast(half8_t, bw), d, 0, 0, 0);
        }
        const float sc = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sl.s)));
        const float z = asym ? static_cast<float>((sl.z >> zshift) & 0xFu) : 8.0f;
        const int e = bf * s.gpad + C.u;
        yacc += sc * (d[0] - s.os[e] - z * s.ss[e]);

        if (C.u + WAVES >= C.ng) {  // this wavefront's last unit of the tile
          const uint32_t slot = tseq % kSlots, tag = tseq / kSlots + 1;
          const uint64_t t0 = now_ticks();
          while (lds_ld(s.gen + slot) != tag - 1) {  // the slot's previous tile is summed
            __builtin_amdgcn_s_sleep(1);
            if (now_ticks() - t0 > kSpinTicks) {
              lds_st(s.err, 1u);
              break;
            }
          }
          lds_acquire();
          // the four lanes of a column hold the same sum (every row of the product is the
          // single activation row), so all of them store it
          s.part[(slot * WAVES + wave) * kTileN + r] = yacc;
          lds_release();
          lds_st(s.arrive + slot * WAVES + wave, tag);
          yacc = 0.0f;
          tseq = uni(tseq + 1);
        }
        cursor_next<WAVES>(s, C, wave, P);
      }
      issue(ring[i]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load of the ring still in flight at exit
}

// -------------------------------------------------------------------- control wavefront
// LDS-direct load of `bytes` bytes (a multiple of 16) of a buffer into LDS at dst: one
// instruction moves 64 lanes x 16 bytes; lanes past the end fill zeros. AGENT makes the
// loads agent-scope (sc1). No register holds the data; the caller waits (wait_dma).
template <bool AGENT>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* dst, int bytes) {
  const int lane = threadIdx.x & 63;
  for (int off = 0; off < bytes; off += 1024) {
    const uint32_t voff = off + 16 * lane < bytes ? static_cast<uint32_t>(off + 16 * lane) : kNoLoad;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(static_cast<unsigned char*>(dst) + off), 16,
        static_cast<int>(voff), 0, 0, AGENT ? 16 : 0);
  }
}
__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's loads into LDS have landed
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// layer li's inv_s_c into buffer bf (it does not depend on any layer)
__device__ __forceinline__ void load_inv(const Lds& s, int li, int bf) {
  const uint16_t* inv = LF(s, li, inv);
  if (inv == nullptr) return;
  const int K = LF(s, li, K);
  dma_to_lds<false>(make_rsrc(inv, static_cast<uint32_t>(2 * K)), s.xinv + bf * s.kpad, 2 * K);
}

// Layer li's input into buffer bf: the caller's x with plain loads, another layer's
// output with agent-scope loads (it may have been written by another workgroup of this
// launch). The streaming wavefronts convert it once `landed` is set (publish_input).
__device__ __forceinline__ void load_input(const Lds& s, int li, int bf) {
  const int K = LF(s, li, K);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(LF(s, li, x), static_cast<uint32_t>(2 * K));
  if (LF(s, li, src) >= 0) {
    dma_to_lds<true>(rx, s.xs + bf * s.kpad, 2 * K);
  } else {
    dma_to_lds<false>(rx, s.xs + bf * s.kpad, 2 * K);
  }
}
__device__ __forceinline__ void publish_input(const Lds& s, int li) {
  lds_release();
  lds_st(s.landed + li, 1u);
}

// Whether every tile of layer li's source layer is complete (always, for a layer that
// reads the caller's x). Lanes 0..7 read the eight counters with agent-scope loads.
__device__ __forceinline__ bool source_done(const Lds& s, uint32_t* state, int li) {
  const int src = LF(s, li, src);
  if (src < 0) return true;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = state_rsrc(state);
  const uint32_t off = lane < kSub ? 4u * cnt_word(src, lane) : kNoLoad;
  const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(off), 0, 16);
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < kSub; ++j) sum += __builtin_amdgcn_readlane(v, j);
  return sum >= static_cast<uint32_t>(LF(s, src, n_tiles));
}

__device__ __forceinline__ void wait_source(const Lds& s, uint32_t* state, int li) {
  const uint64_t t0 = now_ticks();
  while (!source_done(s, state, li)) {
    __builtin_amdgcn_s_sleep(2);
    if (now_ticks() - t0 > kSpinTicks) {
      flag_error(state);
      return;
    }
  }
}

template <int WAVES>
__device__ __forceinline__ void control_wave(const Lds& s, uint32_t* state) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int P = gridDim.x, b = blockIdx.x;
  const int nbuf = s.nbuf;
  const __amdgpu_buffer_rsrc_t rs = state_rsrc(state);
  __builtin_amdgcn_s_setprio(3);
  // Layers with tiles here, in order: ordinal o is the o-th set bit of `mask`. Buffers:
  // ordinal o uses o % nbuf; a buffer is free again once the layer nbuf ordinals back is
  // summed (its streaming wavefronts are past it).
  uint32_t mask = 0;
  for (int j = 0; j < n_layers(s); ++j)
    if (first_tile(s, j, b, P) >= 0) mask |= 1u << j;
  const int n_ord = __builtin_popcount(mask);
  auto layer_of = [&](int o) {
    uint32_t m = mask;
    for (int j = 0; j < o; ++j) m &= m - 1;
    return static_cast<int>(__builtin_ctz(m));
  };
  int loaded = -1;   // ordinals whose input is in LDS: 0 .. loaded
  int inv_done = -1;
  // first, before the streaming wavefronts load any weights: inv_s_c of the first
  // buffers and the inputs of the leading layers that read the caller's x
  for (int o = 0; o < n_ord && o < nbuf; ++o) {
    load_inv(s, layer_of(o), o % nbuf);
    inv_done = o;
  }
  for (int o = 0; o < n_ord && o < nbuf; ++o) {
    const int l = layer_of(o);
    if (LF(s, l, src) >= 0) break;
    load_input(s, l, o % nbuf);
    loaded = o;
  }
  wait_dma();
  for (int o = 0; o <= loaded; ++o) publish_input(s, layer_of(o));

  uint32_t tseq = 0;
  for (int o = 0; o < n_ord; ++o) {
    const int li = layer_of(o);
    if (loaded < o) {  // this layer's input was not there yet
      wait_source(s, state, li);
      if (inv_done < o) {
        load_inv(s, li, o % nbuf);
        inv_done = o;
      }
      load_input(s, li, o % nbuf);
      wait_dma();
      publish_input(s, li);
      loaded = o;
    }
    // buffers of ordinals up to o + nbuf - 1 are free: their inv_s_c can go in now, and
    // the inputs of those layers that are already there
    for (int o2 = inv_done + 1; o2 < n_ord && o2 < o + nbuf; ++o2) {
      load_inv(s, layer_of(o2), o2 % nbuf);
      inv_done = o2;
    }
    {
      const int first = loaded + 1;
      for (int o2 = first; o2 < n_ord && o2 < o + nbuf; ++o2) {
        const int l2 = layer_of(o2);
        // a source at or after the current layer still has tiles of this workgroup to
        // come: no poll for it yet
        if (LF(s, l2, src) >= li || !source_done(s, state, l2)) break;
        load_input(s, l2, o2 % nbuf);
        loaded = o2;
      }
      if (loaded >= first) {
        wait_dma();
        for (int o2 = first; o2 <= loaded; ++o2) publish_input(s, layer_of(o2));
      }
    }
    const int tb = LF(s, li, tile_begin);
    const int te = tb + LF(s, li, n_tiles);
    const int N = LF(s, li, N);
    uint32_t* y32 = reinterpret_cast<uint32_t*>(LF(s, li, y));
    uint32_t returned = 0, count = 0;
    for (int g = first_tile(s, li, b, P); g < te; g = uni(g + P)) {
      const uint32_t slot = tseq % kSlots, tag = tseq / kSlots + 1;
      const uint64_t t0 = now_ticks();
      for (;;) {  // every streaming wavefront has delivered its partial sum of the tile
        const uint32_t got = __hip_atomic_load(s.arrive + slot * WAVES + (lane % WAVES), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
        constexpr uint64_t kAll = (uint64_t{1} << WAVES) - 1;  // lanes 0 .. WAVES - 1
        if ((__builtin_amdgcn_ballot_w64(got == tag) & kAll) == kAll) break;
        __builtin_amdgcn_s_sleep(1);
        if (now_ticks() - t0 > kSpinTicks) {
          flag_error(state);
          break;
        }
      }
      lds_acquire();
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += s.part[(slot * WAVES + w) * kTileN + r];
      lds_release();
      lds_st(s.gen + slot, tag);
      const uint32_t h = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
      const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(h), 1, 64));
      const int n = (g - tb) * kTileN + r;
      if (lane < kTileN && (r & 1) == 0 && n < N) {
        returned |= __hip_atomic_exchange(y32 + n / 2, h | (hi << 16), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
      }
      tseq = uni(tseq + 1);
      count = uni(count + 1);
    }
    // a layer that another reads: every output word of it has been performed at agent
    // scope (the atomics have returned) before its counter moves
    const bool consumed = (s.args->consumed >> li) & 1u;
    if (consumed) asm volatile("" ::"v"(returned) : "memory");
    if (consumed && count > 0) {
      (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(static_cast<int>(count), rs,
                                                           static_cast<int>(lane0_off(cnt_word(li, b % kSub))), 0, 16);
    }
  }
  if (lds_ld(s.err) != 0u) flag_error(state);
  // the last workgroup to finish puts the counters back to zero for the next launch
  const uint32_t before = __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, rs, static_cast<int>(lane0_off(kDoneWord)), 0, 16);
  if (__builtin_amdgcn_readlane(before, 0) == static_cast<uint32_t>(P - 1)) {
    const int n = n_layers(s);
    for (int w0 = 0; w0 < n * kSub; w0 += 64) {
      const int w = w0 + lane;
      const uint32_t off = w < n * kSub ? 4u * cnt_word(w / kSub, w % kSub) : kNoLoad;
      __builtin_amdgcn_raw_buffer_store_b32(0u, rs, static_cast<int>(off), 0, 16);
    }
    __builtin_amdgcn_raw_buffer_store_b32(0u, rs, static_cast<int>(lane0_off(kDoneWord)), 0, 16);
  }
}

template <int WAVES, int D>
__global__ void __launch_bounds__((WAVES + 1) * 64) chain_kernel(ChainArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Lds s;
  // the only kernel argument, at offset 0 of the kernel-argument segment
  s.args = (KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  {
    // One scalar load per 64-byte line of the arguments, all in flight together: the
    // per-layer fields read later (indexed by layer, one at a time) then hit the scalar
    // cache instead of each paying a round trip to the argument segment.
    typedef __attribute__((address_space(4))) const uint32_t KWord;
    KWord* w = (KWord*)(__builtin_amdgcn_kernarg_segment_ptr());
    uint32_t touch = 0;
#pragma unroll
    for (int i = 0; i < static_cast<int>(sizeof(ChainArgs) / 4); i += 16) touch ^= w[i];
    asm volatile("" ::"s"(touch));
  }
  s.nbuf = a.nbuf;
  s.kpad = a.kpad;
  s.gpad = a.kpad / kGroup;
  s.xs = reinterpret_cast<_Float16*>(smem);
  s.xinv = s.xs + s.nbuf * s.kpad;
  s.os = reinterpret_cast<float*>(s.xinv + s.nbuf * s.kpad);
  s.ss = s.os + s.nbuf * s.gpad;
  s.part = s.ss + s.nbuf * s.gpad;
  s.arrive = reinterpret_cast<uint32_t*>(s.part + kSlots * WAVES * kTileN);
  s.gen = s.arrive + kSlots * WAVES;
  s.landed = s.gen + kSlots;
  s.err = s.landed + kMaxChain;
  for (int i = threadIdx.x; i < kSlots * WAVES + kSlots + kMaxChain + 1; i += blockDim.x) s.arrive[i] = 0u;
  __syncthreads();
  uint32_t* state = s.args->state;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  if (wave == WAVES) {
    control_wave<WAVES>(s, state);
  } else {
    stream_waves<WAVES, D>(s, wave);
  }
}

size_t chain_lds_bytes(int kpad, int nbuf, int waves) {
  return 4ull * nbuf * kpad + 8ull * nbuf * (kpad / kGroup) + 4ull * kSlots * waves * kTileN +
         4ull * (kSlots * waves + kSlots + kMaxChain + 1);
}

// One workgroup per CU; the number of CUs per device is read once.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// 15 streaming wavefronts and a control wavefront (1024 threads): four wavefronts per
// SIMD hide each unit's LDS and matrix-core latency; a ring of 4 units per wavefront
// keeps 60 KiB of weights per CU in flight (measured over 8 / 12 / 15 wavefronts and
// rings of 4 to 12 units on the 7B block).
constexpr int kWaves = 15, kDepth = 4;

}  // namespace

size_t chain_state_bytes() { return kStateBytes; }
int chain_max_layers() { return kMaxChain; }
int chain_max_k() { return kMaxK; }
int chain_min_k() { return kMinK; }

hipError_t launch_chain(const awq_chain_layer* layers, int n, uint32_t* state, hipStream_t st) {
  ChainArgs a = {};
  int tiles = 0, kmax = 0;
  for (int i = 0; i < n; ++i) {
    const awq_chain_layer& l = layers[i];
    const PackedLayout L = make_layout(l.N, l.K, l.group, l.fmt);
    ChainLayerDev& d = a.L[i];
    d.x = l.src >= 0 ? layers[l.src].y : l.x;
    d.inv = l.inv_s_c;
    d.packed = static_cast<const uint8_t*>(l.packed);
    d.y = l.y;
    d.packed_bytes = static_cast<uint32_t>(L.total_bytes);
    d.scales_off = static_cast<uint32_t>(L.scales_off);
    d.zeros_off = static_cast<uint32_t>(L.zeros_off >= 0 ? L.zeros_off : 0);
    d.N = static_cast<int32_t>(l.N);
    d.K = static_cast<int32_t>(l.K);
    d.ng = static_cast<int32_t>(L.n_groups);
    d.n_tiles = static_cast<int32_t>(L.n_tiles);
    d.tile_begin = tiles;
    d.src = l.src;
    d.asym = l.fmt == AWQ_FMT_ASYM ? 1 : 0;
    if (l.src >= 0) a.consumed |= 1u << l.src;
    tiles += d.n_tiles;
    if (d.K > kmax) kmax = d.K;
  }
  a.state = state;
  a.n_layers = n;
  a.kpad = (kmax + 511) / 512 * 512;
  // as many inputs as fit beside each other (at least two: one in use, one loading)
  a.nbuf = kMaxBufs;
  while (a.nbuf > 2 && chain_lds_bytes(a.kpad, a.nbuf, kWaves) > static_cast<size_t>(kLdsLimit)) --a.nbuf;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const size_t lds = chain_lds_bytes(a.kpad, a.nbuf, kWaves);
  const void* fn = reinterpret_cast<const void*>(&chain_kernel<kWaves, kDepth>);
  static std::atomic<uint64_t> lds_done{0};
  hipError_t e = ensure_lds_limit(fn, kLdsLimit, lds_done);
  if (e != hipSuccess) return e;
  // every workgroup must be resident at once: the waits rely on it
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, (kWaves + 1) * 64, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((chain_kernel<kWaves, kDepth>), dim3(static_cast<unsigned>(cus)),
                     dim3((kWaves + 1) * 64), lds, st, a);
  return hipGetLastError();
}

}  // namespace awq
