// KB: data movement for the backward of the k-contraction.
//
// The contraction kernel computes, per channel d, x = A B^T from two
// k-contiguous operand planes.  Its gradients are dA = dX B and dB = dX^T A,
// which are again "operand times operand-transpose" products once dX, dX^T,
// B^T and A^T are available as operand planes.  This kernel produces them:
//   - from an fp32 tile in the x layout (see x_offset; the layout of the
//     contraction result and of its gradient dX): the same matrix as an
//     operand plane (operand_offset layout, element type T) and/or its
//     transpose;
//   - from an operand plane: its transpose.
// Work item: one 64 x 64 tile of one channel, staged in LDS as fp32, so that
// every global read and write is a run of at least 128 bytes.  Elements past
// the valid rows or columns are written as zeros: the contraction requires
// zero padding columns, and padding rows of a source are never copied.
// bf16 destinations are rounded to nearest-even (the rounding the forward
// contraction applies to its a and b operands).
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace trimul {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kStride = kTile + 1;    // LDS row stride (floats): column reads hit distinct banks
constexpr int kChanPerGroup = 8;      // channels one work-group walks through

__device__ __forceinline__ float load_elt(const bf16_t *p) { return bf16_to_f32(p->v); }
__device__ __forceinline__ float load_elt(const float *p) { return *p; }

// 16 bytes of T from 16 / sizeof(T) floats
__device__ __forceinline__ u32x4 pack16(const float *v, bf16_t) {
  return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}
__device__ __forceinline__ u32x4 pack16(const float *v, float) {
  return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}

template <typename T, bool kFromX>
__global__ __launch_bounds__(kThreads) void kb_relayout(RelayoutArgs p) {
  constexpr int E = sizeof(T);
  constexpr int EPV = 16 / E;               // elements per 16-byte vector
  constexpr int VPR = kTile / EPV;          // vectors per 64-element row
  constexpr int RPP = kThreads / VPR;       // rows per pass of the work-group
  __shared__ float tile[kTile * kStride];

  const int tid = threadIdx.x;
  const int64_t tiles_c = (p.cols + kTile - 1) / kTile;
  const int64_t tiles_r = (p.rows + kTile - 1) / kTile;
  const int64_t per_group = tiles_r * tiles_c;
  const int group = (int)(blockIdx.x / per_group);
  const int64_t t = blockIdx.x - (int64_t)group * per_group;
  const int64_t r0 = (t / tiles_c) * kTile, c0 = (t % tiles_c) * kTile;

  for (int dc = 0; dc < kChanPerGroup; ++dc) {
    const int d = group * kChanPerGroup + dc;
    // ---- load the 64 x 64 tile of channel d into LDS (row r, column c) ----
    if constexpr (kFromX) {
      // 16 row groups x 4 column groups of 4 x 16 x-blocks, 256 bytes of
      // channel d each; thread: block tid/4, floats 16*(tid%4) .. +15, i.e.
      // columns 4*(tid%4) .. +3 of the block, all 4 rows
      const int b = tid >> 2, qq = tid & 3;
      const int lr = 4 * (b >> 2), lc = 16 * (b & 3) + 4 * qq;
      const int64_t r = r0 + lr, c = c0 + lc;
      float v[16];
      const bool block_in = r < ((p.rows + 3) & ~int64_t(3)) && c < p.ldx;   // the block exists
      if (block_in) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(p.x + x_offset(r, c, d, p.ldx));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x4 w = src[u];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * u + e] = w[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = 0.f;
      }
      // float e of the 16: column lc + e/4, row lr + e%4
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = lr + (e & 3), cc = lc + (e >> 2);
        const bool ok = r0 + rr < p.rows && c0 + cc < p.cols;
        tile[rr * kStride + cc] = ok ? v[e] : 0.f;
      }
    } else {
      const T *src = static_cast<const T *>(p.src);
#pragma unroll
      for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int rr = pass * RPP + tid / VPR, cv = tid % VPR;
        const int64_t r = r0 + rr;
        const bool row_ok = r < p.rows;
        u32x4 w = u32x4{0, 0, 0, 0};
        if (row_ok) w = *reinterpret_cast<const u32x4 *>(src + operand_offset(r, c0 + cv * EPV, d, p.ld_src));
        const T *wt = reinterpret_cast<const T *>(&w);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int cc = cv * EPV + e;
          tile[rr * kStride + cc] = (row_ok && c0 + cc < p.cols) ? load_elt(wt + e) : 0.f;
        }
      }
    }
    __syncthreads();
    // ---- same orientation: rows r0.., columns c0.. of P ------------------
    if (p.p) {
      T *dst = static_cast<T *>(p.p);
#pragma unroll
      for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int rr = pass * RPP + tid / VPR, cv = tid % VPR;
        float v[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) v[e] = tile[rr * kStride + cv * EPV + e];
        *reinterpret_cast<u32x4 *>(dst + operand_offset(r0 + rr, c0 + cv * EPV, d, p.ld_p)) = pack16(v, T{});
      }
    }
    // ---- transposed: rows c0.., columns r0.. of Q ------------------------
    if (p.q) {
      T *dst = static_cast<T *>(p.q);
#pragma unroll
      for (int pass = 0; pass < kTile / RPP; ++pass) {
        const int cc = pass * RPP + tid / VPR, rv = tid % VPR;
        float v[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) v[e] = tile[(rv * EPV + e) * kStride + cc];
        *reinterpret_cast<u32x4 *>(dst + operand_offset(c0 + cc, r0 + rv * EPV, d, p.ld_q)) = pack16(v, T{});
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_relayout(const RelayoutArgs &a, bool from_x, int dtype, hipStream_t s) {
  if (a.rows <= 0 || a.cols <= 0) return hipSuccess;
  const int64_t tiles = ((a.rows + kTile - 1) / kTile) * ((a.cols + kTile - 1) / kTile);
  const int64_t grid = tiles * (kC / kChanPerGroup);
  if (dtype == TRIMUL_BF16) {
    if (from_x) hipLaunchKernelGGL((kb_relayout<bf16_t, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((kb_relayout<bf16_t, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  } else {
    if (from_x) hipLaunchKernelGGL((kb_relayout<float, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((kb_relayout<float, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace trimul
