// Achievable-peak probes for the rooflines of the triangle-multiplication
// kernels on gfx950, built as a library of its own (libtrimul_peaks.so) and
// driven by the benchmark's peaks mode:
//   - a matrix-core loop with no memory traffic: eight independent 32x32x16
//     bf16 accumulator chains per wave, two waves per SIMD, each wave timing
//     itself with the shader-clock counter (s_memtime) and the fixed-rate
//     real-time counter (s_memrealtime), which gives the clock it ran at;
//   - streaming kernels that read R and write W 16-byte units per element
//     (R:W = 1:0 read, 0:1 write, 1:1 copy, 1:2 the projection kernel's byte
//     mix, 3:2 the epilogue's), each plane accessed at consecutive addresses
//     by consecutive lanes.
// Nothing here is part of the triangle update; it only measures the chip.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kChains = 8;

__global__ __launch_bounds__(512) void peak_mfma(int iters, float *sink, unsigned long long *clk) {
  const int tid = threadIdx.x;
  // operands that the compiler cannot fold: built from the lane index
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((tid + e) & 7);
    b[e] = (__bf16)(float)((tid * 3 + e) & 7);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  // the results must be consumed before the end time is read
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + tid] = s;
  if ((tid & 63) == 0) {
    const int w = blockIdx.x * (blockDim.x / 64) + tid / 64;
    clk[2 * w] = t1 - t0;
    clk[2 * w + 1] = r1 - r0;
  }
}

// R source planes and W destination planes of `units` 16-byte elements each.
// Every thread takes U elements per step (all loads issued before the
// stores), striding over the grid; NT selects non-temporal (streaming) loads
// and stores, which bypass cache allocation for data used once.
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4 *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4 *p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int R, int W, int U, bool NT>
__global__ __launch_bounds__(256) void stream_rw(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                 int64_t units, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 keep = {0u, 0u, 0u, 0u};
  for (; u + (U - 1) * stride < units; u += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      v[q] = u32x4{(uint32_t)(u + q * stride), 1u, 2u, 3u};
#pragma unroll
      for (int r = 0; r < R; ++r) v[q] ^= ld16<NT>(src + r * units + u + q * stride);
    }
#pragma unroll
    for (int q = 0; q < U; ++q) {
#pragma unroll
      for (int w = 0; w < W; ++w) st16<NT>(dst + w * units + u + q * stride, v[q] + (uint32_t)w);
      if (W == 0) keep ^= v[q];
    }
  }
  for (; u < units; u += stride) {
    u32x4 v = u32x4{(uint32_t)u, 1u, 2u, 3u};
#pragma unroll
    for (int r = 0; r < R; ++r) v ^= ld16<NT>(src + r * units + u);
#pragma unroll
    for (int w = 0; w < W; ++w) st16<NT>(dst + w * units + u, v + (uint32_t)w);
    if (W == 0) keep ^= v;
  }
  // read-only form: keep the loads alive (the condition is practically never met)
  if (W == 0 && keep[0] == 0x9E3779B9u && keep[1] == 0x7F4A7C15u) sink[0] = keep[2];
}

// One-shot form: one element per thread, a grid that covers all elements
// (no stride loop; the dispatcher places every work-group).
template <int R, int W, bool NT>
__global__ __launch_bounds__(256) void stream_once(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                   int64_t units, uint32_t *sink) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  u32x4 v = u32x4{(uint32_t)u, 1u, 2u, 3u};
#pragma unroll
  for (int r = 0; r < R; ++r) v ^= ld16<NT>(src + r * units + u);
#pragma unroll
  for (int w = 0; w < W; ++w) st16<NT>(dst + w * units + u, v + (uint32_t)w);
  if (W == 0 && v[0] == 0x9E3779B9u && v[1] == 0x7F4A7C15u) sink[0] = v[2];
}

template <int R, int W, int U, bool NT>
hipError_t launch_stream(const void *src, void *dst, int64_t units, uint32_t *sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL((stream_rw<R, W, U, NT>), dim3(blocks), dim3(256), 0, s, static_cast<const u32x4 *>(src),
                     static_cast<u32x4 *>(dst), units, sink);
  return hipGetLastError();
}

// variant: bit 0 = non-temporal, bit 1 = 8 elements per thread and step (else
// 4); variants 4 and 5: the one-shot form (plain, non-temporal), whose grid
// size follows from `units` (`blocks` is ignored)
template <int R, int W>
hipError_t launch_variant(int variant, const void *src, void *dst, int64_t units, uint32_t *sink, int blocks,
                          hipStream_t s) {
  const int64_t once_blocks = (units + 255) / 256;
  switch (variant) {
    case 4:
      hipLaunchKernelGGL((stream_once<R, W, false>), dim3((unsigned)once_blocks), dim3(256), 0, s,
                         static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), units, sink);
      return hipGetLastError();
    case 5:
      hipLaunchKernelGGL((stream_once<R, W, true>), dim3((unsigned)once_blocks), dim3(256), 0, s,
                         static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), units, sink);
      return hipGetLastError();
    case 0: return launch_stream<R, W, 4, false>(src, dst, units, sink, blocks, s);
    case 1: return launch_stream<R, W, 4, true>(src, dst, units, sink, blocks, s);
    case 2: return launch_stream<R, W, 8, false>(src, dst, units, sink, blocks, s);
    case 3: return launch_stream<R, W, 8, true>(src, dst, units, sink, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" {

// Real-time counter rate of the current device in kHz (s_memrealtime ticks).
int peaks_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}

// Matrix-core loop: `blocks` work-groups of 8 waves, `iters` iterations of
// 8 bf16 32x32x16 products per wave (flop = blocks * 8 * iters * 8 * 32768).
// sink: blocks * 512 floats; clk: blocks * 8 * 2 values (shader-clock cycles,
// real-time ticks per wave).  Returns a hipError_t value.
int peaks_mfma(int blocks, int iters, float *sink, unsigned long long *clk, void *stream) {
  if (blocks <= 0 || iters <= 0 || !sink || !clk) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_mfma, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, sink, clk);
  return (int)hipGetLastError();
}

// Streaming kernel reading `r` planes of src and writing `w` planes of dst,
// each of `units` 16-byte elements (both pointers 16-byte aligned, src holding
// r * units and dst w * units elements).  (r, w) in {(1,0), (0,1), (1,1),
// (1,2), (3,2)}; variant 0..3 (bit 0 non-temporal, bit 1 eight elements per
// thread and step), 4..5 one element per thread over a covering grid (plain,
// non-temporal).  Returns a hipError_t value.
int peaks_stream(int r, int w, int variant, const void *src, void *dst, long long units, uint32_t *sink,
                 int blocks, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  if (units <= 0 || blocks <= 0 || !sink || variant < 0 || variant > 5) return (int)hipErrorInvalidValue;
  if (variant >= 4 && (units + 255) / 256 > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  if ((r > 0 && !src) || (w > 0 && !dst)) return (int)hipErrorInvalidValue;
  if (r == 1 && w == 0) return (int)launch_variant<1, 0>(variant, src, dst, units, sink, blocks, s);
  if (r == 0 && w == 1) return (int)launch_variant<0, 1>(variant, src, dst, units, sink, blocks, s);
  if (r == 1 && w == 1) return (int)launch_variant<1, 1>(variant, src, dst, units, sink, blocks, s);
  if (r == 1 && w == 2) return (int)launch_variant<1, 2>(variant, src, dst, units, sink, blocks, s);
  if (r == 3 && w == 2) return (int)launch_variant<3, 2>(variant, src, dst, units, sink, blocks, s);
  return (int)hipErrorInvalidValue;
}

}  // extern "C"
