// Measured ceilings for the W4A16 kernels on gfx950: what a plain streaming read of the
// same number of bytes reaches, what an empty launch costs, and how much ALU work the
// matrix cores leave room for.
//
// Decode time is bytes moved / bandwidth (edgesiliconlab ?p=2015, section "The
// Mathematics of Memory Bandwidth Saturation"). The HBM peak is a specification figure;
// at the few-megabyte sizes of one decode layer a launch also pays a fixed cost, so the
// benchmark reports, next to each decode kernel, a read-only kernel that streams the
// same number of bytes with the decode kernel's access pattern (one 16-byte load per
// lane, one 1 KiB block per wavefront load, non-temporal), and the per-launch cost of an
// empty kernel. Nothing here is part of the product path.
#include "../../include/awq_probe.h"

#include <hip/hip_runtime.h>

namespace {

constexpr uint32_t kMagic = 0x9E3779B9u;  // stored only if the data happen to XOR to it

// Workgroup b reads bytes [b C, (b + 1) C), C = THREADS / 64 * PER_WAVE KiB; wavefront w
// reads blocks w, w + waves, ... of 1 KiB, all PER_WAVE loads issued before the first
// use. Offsets past `bytes` read zeros without a memory access.
template <int THREADS, int PER_WAVE>
__global__ void __launch_bounds__(THREADS) stream_read_kernel(const unsigned char* buf, uint32_t bytes,
                                                             uint32_t* sink) {
  constexpr int kWaves = THREADS / 64;
  constexpr uint32_t kChunk = kWaves * PER_WAVE * 1024u;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(buf), 0, static_cast<int>(bytes), 0x00020000);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t base = blockIdx.x * kChunk;
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  u4 v[PER_WAVE];
#pragma unroll
  for (int d = 0; d < PER_WAVE; ++d) {
    const uint32_t off = base + (wave + kWaves * d) * 1024u;
    const uint32_t voff = off < bytes ? 16u * lane : 0x80000000u;
    v[d] = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff),
                                                 __builtin_amdgcn_readfirstlane(static_cast<int>(off < bytes ? off : 0)), 2);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int d = 0; d < PER_WAVE; ++d) acc ^= v[d][0] ^ v[d][1] ^ v[d][2] ^ v[d][3];
  if (acc == kMagic) sink[0] = acc;
}

__global__ void empty_kernel() {}

// Matrix-core / ALU co-issue: each iteration issues 8 independent 16 x 16 x 32 f16 matrix
// instructions, each followed by ALU instructions (packed binary16 multiplies on 8
// independent registers), placed in that order by scheduling groups. Timing it against
// ALU = 0 shows how many ALU instructions fit under one matrix instruction. out: one
// float per thread, a sum of the results (keeps them alive).
typedef _Float16 probe_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 probe_half2 __attribute__((ext_vector_type(2)));
typedef float probe_float4 __attribute__((ext_vector_type(4)));

template <int ALU>
__global__ void __launch_bounds__(256) mfma_alu_kernel(float* out, int iters) {
  probe_float4 acc[8];
  probe_half8 a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i] = probe_float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 8; ++e) a[i][e] = static_cast<_Float16>((threadIdx.x + 3 * i + e) & 7);
  }
  const probe_half8 b = a[3];
  probe_half2 h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = probe_half2{static_cast<_Float16>(i + 1), static_cast<_Float16>(threadIdx.x & 3)};
  }
  const probe_half2 hs = probe_half2{static_cast<_Float16>(1.0009765625f), static_cast<_Float16>(0.99951171875f)};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[s], b, acc[s], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < ALU; ++k) h[(s * ALU + k) & 7] = h[(s * ALU + k) & 7] * hs;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
      if (ALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, ALU, 0);  // then ALU ones
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sum += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3] + static_cast<float>(h[i][0]) +
           static_cast<float>(h[i][1]);
  }
  out[blockIdx.x * 256 + threadIdx.x] = sum;
}

template <int ALU>
int launch_mfma_alu(float* out, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_alu_kernel<ALU>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

template <int THREADS, int PER_WAVE>
int launch_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  constexpr size_t kChunk = static_cast<size_t>(THREADS / 64) * PER_WAVE * 1024;
  const unsigned blocks = static_cast<unsigned>((bytes + kChunk - 1) / kChunk);
  hipLaunchKernelGGL((stream_read_kernel<THREADS, PER_WAVE>), dim3(blocks), dim3(THREADS), 0, st,
                     static_cast<const unsigned char*>(buf), static_cast<uint32_t>(bytes), sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace

extern "C" {

int awq_probe_shapes(void) { return 4; }

int awq_probe_stream_read(const void* buf, size_t bytes, int shape, uint32_t* sink,
                          hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes >= (size_t{1} << 31)) return 1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return 3;
  switch (shape) {
    case 0: return launch_read<512, 4>(buf, bytes, sink, stream);   // 32 KiB per workgroup
    case 1: return launch_read<256, 4>(buf, bytes, sink, stream);   // 16 KiB
    case 2: return launch_read<1024, 4>(buf, bytes, sink, stream);  // 64 KiB
    case 3: return launch_read<256, 16>(buf, bytes, sink, stream);  // 64 KiB, 16 loads per wave
    default: return 1;
  }
}

int awq_probe_mfma_alu(float* out, int alu, int blocks, int iters, hipStream_t stream) {
  if (out == nullptr || blocks < 1 || blocks > 4096 || iters < 1) return 1;
  switch (alu) {
    case 0: return launch_mfma_alu<0>(out, blocks, iters, stream);
    case 1: return launch_mfma_alu<1>(out, blocks, iters, stream);
    case 2: return launch_mfma_alu<2>(out, blocks, iters, stream);
    case 3: return launch_mfma_alu<3>(out, blocks, iters, stream);
    case 4: return launch_mfma_alu<4>(out, blocks, iters, stream);
    default: return 1;
  }
}

int awq_probe_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
