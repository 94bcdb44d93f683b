// K3: the epilogue of the update for a tile of the pair grid,
//     out_ij = m_ij * sigmoid(W_out_gate LN_in(z_ij)) * (W_out_proj LN_out(x_ij))
// reading the channel-planar contraction result x[d][r][s] and the pair
// tensor, writing fp32 out[r][s][e].
//
// Work item: 64 consecutive columns s of one tile row r (64 pairs), 256
// threads.  x is read channel by channel (64 lanes = 256 contiguous bytes per
// channel), each wave holding 32 channels of all 64 pairs; the output
// LayerNorm statistics are combined across the four waves through LDS.  z is
// re-read (16 lanes per pair, 16-lane shuffle reductions) and re-normalised
// for the gate.  Both normalised operands go to LDS as matrix-core B
// operands; in bf16 mode each is split into hi + lo bf16 terms (hi = bf16(v),
// lo = bf16(v - hi)) and multiplied by the bf16 weights twice, so the
// products keep fp32-level accuracy.  Wave w computes output channels
// 32w .. 32w+31 of both the projection and the gate, so the final product is
// formed in registers, staged through LDS and stored as whole 512-byte pair
// rows.  Persistent over the work items; bf16 weight fragments stay in
// registers.
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kPairs = 64;
constexpr int kThreads = 256;
constexpr int kOutRowF = kCz + 4;  // staged output row (floats), padded against bank conflicts

template <typename T>
struct ZUnit;

template <>
struct ZUnit<bf16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const unsigned char *p) { v = *reinterpret_cast<const u32x4 *>(p); }
  __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ void to_f32(float (&f)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};

template <>
struct ZUnit<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const unsigned char *p) {
    lo = reinterpret_cast<const f32x4 *>(p)[0];
    hi = reinterpret_cast<const f32x4 *>(p)[1];
  }
  __device__ __forceinline__ void zero() { lo = f32x4{0, 0, 0, 0}; hi = lo; }
  __device__ __forceinline__ void to_f32(float (&f)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = lo[i]; f[4 + i] = hi[i]; }
  }
};

// LDS operand planes: bf16 mode keeps hi and lo planes [64][128] bf16 each;
// fp32 mode keeps one plane [64][128] fp32.  Rows are 256 / 512 bytes, units
// of 8 channels XOR-swizzled with period 16.
template <typename T>
struct Operand;

template <>
struct Operand<bf16_t> {
  static constexpr int ROWB = kC * 2, UNIT = 16, PLANE = kPairs * ROWB, BYTES = 2 * PLANE;
  __device__ static void put(unsigned char *base, int q, int unit, const float (&f)[8]) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float h0 = bf16_to_f32(f32_to_bf16(f[2 * i]));
      const float h1 = bf16_to_f32(f32_to_bf16(f[2 * i + 1]));
      h[i] = pack_bf16x2(h0, h1);
      l[i] = pack_bf16x2(f[2 * i] - h0, f[2 * i + 1] - h1);
    }
    const int off = q * ROWB + swz<16>(q, unit) * UNIT;
    *reinterpret_cast<u32x4 *>(base + off) = h;
    *reinterpret_cast<u32x4 *>(base + PLANE + off) = l;
  }
  // acc += W * v over 16 k values (both terms)
  __device__ static void mma_at(f32x16 &acc, const Frag<bf16_t> &w, const unsigned char *base, int q,
                                int unit) {
    const int off = q * ROWB + swz<16>(q, unit) * UNIT;
    Frag<bf16_t> h, l;
    h.load(base + off);
    l.load(base + PLANE + off);
    mma(acc, w, h);
    mma(acc, w, l);
  }
};

template <>
struct Operand<float> {
  static constexpr int ROWB = kC * 4, UNIT = 32, PLANE = kPairs * ROWB, BYTES = PLANE;
  __device__ static void put(unsigned char *base, int q, int unit, const float (&f)[8]) {
    const int off = q * ROWB + swz<16>(q, unit) * UNIT;
    reinterpret_cast<f32x4 *>(base + off)[0] = f32x4{f[0], f[1], f[2], f[3]};
    reinterpret_cast<f32x4 *>(base + off)[1] = f32x4{f[4], f[5], f[6], f[7]};
  }
  __device__ static void mma_at(f32x16 &acc, const Frag<float> &w, const unsigned char *base, int q,
                                int unit) {
    Frag<float> v;
    v.load(base + q * ROWB + swz<16>(q, unit) * UNIT);
    mma(acc, w, v);
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k3_epilogue(K3Args p) {
  constexpr int E = sizeof(T);
  constexpr bool kWeightsInRegs = (E == 2);
  using Op = Operand<T>;
  constexpr int kOpBytes = Op::BYTES;
  constexpr int kStageBytes = kPairs * kOutRowF * 4;
  constexpr int kLdsBytes = (2 * kOpBytes) > kStageBytes ? (2 * kOpBytes) : kStageBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ float red[4][kPairs];
  __shared__ float stat_mean[kPairs], stat_rstd[kPairs];
  unsigned char *const n_ops = lds;               // normalised x
  unsigned char *const z_ops = lds + kOpBytes;    // normalised z
  float *const stage = reinterpret_cast<float *>(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tiles_per_row = (p.n_cols + kPairs - 1) / kPairs;
  const int64_t n_tiles = p.n_rows * tiles_per_row;

  // LayerNorm parameters: x channels 32*wave .. +31 for this thread; z channel
  // group (tid & 15) for the gate path
  const int cg = tid & 15;
  float gz[8], bz[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { gz[i] = p.ln_in_w[cg * 8 + i]; bz[i] = p.ln_in_b[cg * 8 + i]; }

  const T *const Wo = static_cast<const T *>(p.w_out_proj);
  const T *const Wg = static_cast<const T *>(p.w_out_gate);
  auto wptr = [&](const T *W, int ks) -> const T * {
    const int row = 32 * wave + (lane & 31);
    return W + row * kC + 16 * ks + 8 * (lane >> 5);
  };
  Frag<T> wo[kWeightsInRegs ? 8 : 1], wg[kWeightsInRegs ? 8 : 1];
  if constexpr (kWeightsInRegs) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) { wo[ks].load(wptr(Wo, ks)); wg[ks].load(wptr(Wg, ks)); }
  }

  const unsigned char *zbytes = static_cast<const unsigned char *>(p.z);

  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int64_t r = tile / tiles_per_row;
    const int64_t s0 = (tile % tiles_per_row) * kPairs;
    const int64_t gi = p.row_off + r;                 // global row of the tile row

    // ---- x: this thread holds pair q = lane, channels 32*wave .. +31 ------
    const int q = lane;
    const bool qv = s0 + q < p.n_cols;
    float xv[32];
    const float *xp = p.x + (int64_t)(32 * wave) * p.n_rows * p.ldx + r * p.ldx + s0 + q;
#pragma unroll
    for (int c = 0; c < 32; ++c) xv[c] = qv ? xp[(int64_t)c * p.n_rows * p.ldx] : 0.f;

    // ---- z units for the gate: pairs 16s + tid/16, channels cg*8 .. +7 -----
    ZUnit<T> zr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int qq = 16 * s + (tid >> 4);
      if (s0 + qq < p.n_cols)
        zr[s].load(zbytes + ((gi * p.n + p.col_off + s0 + qq) * kCz + cg * 8) * E);
      else
        zr[s].zero();
    }

    // ---- output LayerNorm statistics (two passes, across the 4 waves) -----
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) sum += xv[c];
    red[wave][q] = sum;
    __syncthreads();
    if (tid < kPairs) stat_mean[tid] = (red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid]) * (1.0f / kC);
    __syncthreads();
    const float mean = stat_mean[q];
    float sq = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) { xv[c] -= mean; sq += xv[c] * xv[c]; }
    red[wave][q] = sq;
    __syncthreads();
    if (tid < kPairs)
      stat_rstd[tid] = rsqrt_f32((red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid]) * (1.0f / kC) + p.eps);
    __syncthreads();
    const float rstd = stat_rstd[q];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = 32 * wave + 8 * u + i;
        f[i] = xv[8 * u + i] * rstd * p.ln_out_w[c] + p.ln_out_b[c];
      }
      Op::put(n_ops, q, 4 * wave + u, f);
    }

    // ---- input LayerNorm of z (recomputed) for the gate --------------------
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float f[8];
      zr[s].to_f32(f);
      float zs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) zs += f[i];
      const float zm = group_sum<16>(zs) * (1.0f / kCz);
      float zq = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { f[i] -= zm; zq += f[i] * f[i]; }
      const float zr_std = rsqrt_f32(group_sum<16>(zq) * (1.0f / kCz) + p.eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * zr_std * gz[i] + bz[i];
      Op::put(z_ops, 16 * s + (tid >> 4), cg, f);
    }
    __syncthreads();

    // ---- projections on the matrix cores ----------------------------------
    f32x16 ay[2], ag[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) { ay[nt][e] = 0.f; ag[nt][e] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      Frag<T> fo, fg;
      if constexpr (kWeightsInRegs) { fo = wo[ks]; fg = wg[ks]; }
      else { fo.load(wptr(Wo, ks)); fg.load(wptr(Wg, ks)); }
      const int unit = 2 * ks + (lane >> 5);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int qq = 32 * nt + (lane & 31);
        Op::mma_at(ay[nt], fo, n_ops, qq, unit);
        Op::mma_at(ag[nt], fg, z_ops, qq, unit);
      }
    }
    __syncthreads();   // operands consumed; LDS becomes the output stage

    // ---- gate * projection * mask -> LDS stage -----------------------------
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int qq = 32 * nt + (lane & 31);
      const bool keep = (s0 + qq < p.n_cols) && p.mask[gi * p.n + p.col_off + s0 + qq] != 0;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g4 + i;
          v[i] = keep ? sigmoid_f32(ag[nt][e]) * ay[nt][e] : 0.f;
        }
        const int o = 32 * wave + acc_row(4 * g4, lane);
        *reinterpret_cast<f32x4 *>(stage + qq * kOutRowF + o) = v;
      }
    }
    __syncthreads();

    // ---- stage -> HBM: whole pair rows, 16 bytes per lane ------------------
    const int64_t nq = (p.n_cols - s0) < kPairs ? (p.n_cols - s0) : kPairs;
    float *orow = p.out + (r * p.n_cols + s0) * kCz;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = i * kThreads + tid;
      const int qq = u >> 5, o4 = (u & 31) * 4;
      if (qq < nq)
        *reinterpret_cast<f32x4 *>(orow + qq * kCz + o4) =
            *reinterpret_cast<const f32x4 *>(stage + qq * kOutRowF + o4);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_k3(const K3Args &a, int dtype, hipStream_t s) {
  const int64_t n_tiles = a.n_rows * ((a.n_cols + kPairs - 1) / kPairs);
  if (n_tiles <= 0) return hipSuccess;
  const int64_t cap = 2LL * device_cu_count();
  const int64_t grid = n_tiles < cap ? n_tiles : cap;
  if (dtype == TRIMUL_BF16)
    hipLaunchKernelGGL(k3_epilogue<bf16_t>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k3_epilogue<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace trimul
