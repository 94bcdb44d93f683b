// Shared device helpers for the gfx950 triangle-multiplication kernels:
// element types, 8-element k-fragments and the matrix-core wrappers built on
// them, bf16 rounding, the exp2-based logistic function and lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trimul {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Storage tag for bf16 data (raw 16-bit payload).
struct bf16_t {
  uint16_t v;
};

constexpr int kC = 128;  // hidden channels c
constexpr int kCz = 128; // pair channels c_z

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest even (the hardware conversion; no NaN inputs occur here).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
// Two values rounded to bf16 (round to nearest even) in one packed word, lo in
// the low half: a single packed conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Logistic function 1 / (1 + e^-t) from the identity e^u = 2^(u log2 e) on
// the hardware base-2 exponential and reciprocal.  For t -> -inf the
// exponential overflows to +inf and the reciprocal gives 0; for t -> +inf it
// underflows to 0 and the result is 1: no NaN for any finite t.
__device__ __forceinline__ float sigmoid_f32(float t) {
  const float kLog2e = 1.4426950408889634f;
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t * kLog2e));
}

// The same logistic function given u = -t log2 e instead of t: 1 / (1 + 2^u)
// (u = +inf gives 0, u = -inf gives 1).  Callers that can fold the factor
// -log2 e into an earlier scaling save the multiply.
__device__ __forceinline__ float sigmoid_of_exp2_arg(float u) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u));
}

__device__ __forceinline__ float rsqrt_f32(float v) { return __builtin_amdgcn_rsqf(v); }

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of the group receives the total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over each row of 16 lanes with DPP lane permutations (no LDS traffic):
// swap neighbours, swap neighbouring pairs, mirror inside each half-row of 8,
// mirror inside the row.  Every step adds two equal partial sums in either
// order, so all 16 lanes receive bit-identical totals.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}

// ---------------------------------------------------------------------------
// 8-element k-fragments: the operand one lane contributes to a 32x32 matrix
// product step over 16 k values (lane l holds row/col l % 32 and the k values
// 8*(l/32) .. 8*(l/32)+7).
// ---------------------------------------------------------------------------
template <typename T>
struct Frag;

template <>
struct Frag<bf16_t> {
  bf16x8 v;
  static constexpr int kBytes = 16;
  __device__ __forceinline__ void load(const void *p) {
    v = *reinterpret_cast<const bf16x8 *>(p);
  }
};

template <>
struct Frag<float> {
  f32x4 lo, hi;
  static constexpr int kBytes = 32;
  __device__ __forceinline__ void load(const void *p) {
    lo = reinterpret_cast<const f32x4 *>(p)[0];
    hi = reinterpret_cast<const f32x4 *>(p)[1];
  }
};

// acc[32x32] += A(32 x 16) * B(16 x 32) with both operands as k-fragments.
__device__ __forceinline__ void mma(f32x16 &acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}

// fp32 form: eight 32x32x2 steps.  Step t pairs lane-slot s = l/32 with k
// value 8*s + t, so the eight steps together cover k = 0..15 exactly once.
__device__ __forceinline__ void mma(f32x16 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[t], b.lo[t], acc, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[t], b.hi[t], acc, 0, 0, 0);
}

// Row index (within the 32x32 tile) of accumulator register r in lane l; the
// column is l % 32.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Layout of the contraction operands in HBM.  A logical operand plane set
// a[d][r][t] (channel d < 128, row r, column t < ld, ld a multiple of 64) is
// stored in blocks of kOpRows rows x kOpCols columns; the 128 channel blocks
// of one (row block, column block) are adjacent, each kOpRows * kOpCols
// elements, rows of a block contiguous.  The projection kernel writes one row
// of all 128 channels of a block per work item (a few pages), and the
// contraction kernel reads a whole 256 x 64 operand tile of one channel as one
// contiguous run.  Rows are padded to a multiple of kOpRows.
constexpr int kOpRows = 256;
constexpr int kOpCols = 64;
constexpr int64_t kOpBlock = (int64_t)kOpRows * kOpCols;   // elements per channel block

__device__ __forceinline__ int64_t operand_offset(int64_t r, int64_t t, int d, int64_t ld) {
  return (((r / kOpRows) * (ld / kOpCols) + t / kOpCols) * kC + d) * kOpBlock + (r % kOpRows) * kOpCols +
         (t % kOpCols);
}

// Layout of the contraction result x[d][i][j] of a tile in HBM: blocks of
// 4 rows x 16 columns with all 128 channels of a block adjacent, channel-major
// inside, element (ii, jj) of a block at 4*jj + ii.  One epilogue work item
// (4 rows x 16 columns) reads one contiguous 32 KB block; the contraction
// kernel writes 16-byte groups (4 rows of one column).  ldx = columns padded
// to a multiple of 16; rows padded to a multiple of 4.
__device__ __forceinline__ int64_t x_offset(int64_t i, int64_t j, int d, int64_t ldx) {
  return (((i >> 2) * (ldx >> 4) + (j >> 4)) * kC + d) * 64 + (j & 15) * 4 + (i & 3);
}

// XOR swizzle of 16-byte units inside an LDS row: unit u of row `row` is
// stored at unit u ^ (row % period).  Applied on both write and read, it
// spreads the 32 rows a k-fragment read touches over distinct banks.
template <int kPeriod>
__device__ __forceinline__ int swz(int row, int unit) {
  return unit ^ (row & (kPeriod - 1));
}

}  // namespace trimul
