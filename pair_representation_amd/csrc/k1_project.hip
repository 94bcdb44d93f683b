// K1: input LayerNorm, the four c_z -> c projections, sigmoid gates and the
// pair mask, producing the contraction operands
//     a = m * sigmoid(W_a_gate zh) * (W_a_proj zh),  b likewise,
// as channel-planar, k-contiguous planes  plane[d][r][t].  For the incoming
// direction the source pair of plane cell (r, t) is (t, r), so the planes come
// out transposed and the contraction kernel is the same for both directions.
//
// Work item: 64 consecutive plane columns t of one plane row r (64 pairs).
// 512 threads = 8 waves, two per SIMD, persistent over the work items with
// stride gridDim.x.
//  - z of the next item is prefetched into registers while the current one is
//    processed: every thread holds two 8-channel units (16 lanes per pair).
//  - LayerNorm statistics are 16-lane shuffle reductions; the normalised pairs
//    go to LDS (rounded to bf16 when the weights are bf16) with an XOR
//    swizzle, together with the 64 pair-mask bytes.
//  - Matrix-core product with pairs as rows: out[pair][col] = zh . W[col].
//    Wave w owns operand w/4 (a or b) and channels 32*(w%4) .. +31: its
//    32 projection columns and the 32 gate columns of the same channels land
//    in the same lanes, so the gated product is formed in registers.  bf16
//    weight fragments stay in registers for the whole pass.
//  - Each lane ends up with 4 consecutive pairs of one channel, stored as one
//    8-byte (bf16) or 16-byte (fp32) write.
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kPairs = 64;
constexpr int kThreads = 512;

template <typename T>
struct ZUnit;  // 8 channels of one pair as loaded from HBM

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

// Write 8 normalised channels (one unit) into an LDS row, rounded to T.
__device__ __forceinline__ void put_unit(unsigned char *dst, const float (&f)[8], bf16_t) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  *reinterpret_cast<u32x4 *>(dst) = w;
}
__device__ __forceinline__ void put_unit(unsigned char *dst, const float (&f)[8], float) {
  reinterpret_cast<f32x4 *>(dst)[0] = f32x4{f[0], f[1], f[2], f[3]};
  reinterpret_cast<f32x4 *>(dst)[1] = f32x4{f[4], f[5], f[6], f[7]};
}

// Four consecutive plane elements of one channel.
__device__ __forceinline__ void store4(bf16_t *p, const float (&v)[4]) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store4(float *p, const float (&v)[4]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k1_project(K1Args p) {
  constexpr int E = sizeof(T);
  constexpr int UNIT = 8 * E;          // bytes of one 8-channel unit
  constexpr int ROWB = kCz * E;        // bytes of one pair row in LDS
  constexpr bool kWeightsInRegs = (E == 2);
  __shared__ __attribute__((aligned(16))) unsigned char zh_lds[kPairs * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t mask_lds[kPairs];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int64_t tiles_per_row = p.ld / kPairs;
  const int64_t n_tiles = p.n_rows * tiles_per_row;

  // this thread's 8 channels of LayerNorm affine parameters
  const int cg = tid & 15;  // channel group (8 channels)
  float g8[8], b8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { g8[i] = p.ln_w[cg * 8 + i]; b8[i] = p.ln_b[cg * 8 + i]; }

  // this wave's operand and weight columns
  const int op = wave >> 2;        // 0: a, 1: b
  const int c0 = 32 * (wave & 3);  // first channel
  T *const out_plane = static_cast<T *>(op == 0 ? p.a_out : p.b_out);
  const T *const Wp = static_cast<const T *>(op == 0 ? p.w_a_proj : p.w_b_proj);
  const T *const Wg = static_cast<const T *>(op == 0 ? p.w_a_gate : p.w_b_gate);
  const bool active = out_plane != nullptr;   // wave-uniform

  // column tile nt: 0 -> projection rows c0..c0+31, 1 -> gate rows c0..c0+31
  auto wfrag_ptr = [&](int nt, int ks) -> const T * {
    const T *W = (nt == 0) ? Wp : Wg;
    return W + (c0 + (lane & 31)) * kCz + 16 * ks + 8 * (lane >> 5);
  };
  Frag<T> wreg[kWeightsInRegs ? 2 : 1][kWeightsInRegs ? 8 : 1];
  if constexpr (kWeightsInRegs) {
    if (active) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) wreg[nt][ks].load(wfrag_ptr(nt, ks));
    }
  }

  // source pair of plane cell (r, t); false past k_len
  auto src_pair = [&](int64_t r, int64_t t, int64_t &i, int64_t &j) -> bool {
    if (t >= p.k_len) return false;
    if (p.transposed) { i = p.k_off + t; j = p.row_base + r; }
    else { i = p.row_base + r; j = p.k_off + t; }
    return true;
  };

  const unsigned char *zbytes = static_cast<const unsigned char *>(p.z);
  ZUnit<T> raw[2];
  uint8_t mraw = 0;
  auto load_tile = [&](int64_t tile) {
    const int64_t r = tile / tiles_per_row;
    const int64_t t0 = (tile % tiles_per_row) * kPairs;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q = 32 * s + (tid >> 4);   // pair within the tile
      int64_t i, j;
      if (src_pair(r, t0 + q, i, j))
        raw[s].load(zbytes + ((i * p.n + j) * kCz + cg * 8) * E);
      else
        raw[s].zero();
    }
    if (tid < kPairs) {
      int64_t i, j;
      mraw = src_pair(r, t0 + tid, i, j) ? (p.mask[i * p.n + j] != 0) : 0;
    }
  };

  // Each work-group takes a contiguous range of work items: consecutive items
  // continue along the same plane row, so the 256 channel planes it writes
  // stay in the same few pages (scattering items over the grid makes nearly
  // every store miss the address-translation cache).
  const int64_t per_wg = (n_tiles + gridDim.x - 1) / gridDim.x;
  const int64_t tile_begin = blockIdx.x * per_wg;
  const int64_t tile_end = tile_begin + per_wg < n_tiles ? tile_begin + per_wg : n_tiles;
  int64_t tile = tile_begin;
  if (tile < tile_end) load_tile(tile);

  for (; tile < tile_end; ++tile) {
    const int64_t r = tile / tiles_per_row;
    const int64_t t0 = (tile % tiles_per_row) * kPairs;

    // ---- LayerNorm of the 64 pairs -> LDS --------------------------------
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float f[8];
      raw[s].to_f32(f);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += f[i];
      const float mean = group_sum<16>(sum) * (1.0f / kCz);
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { f[i] -= mean; sq += f[i] * f[i]; }
      const float rstd = rsqrt_f32(group_sum<16>(sq) * (1.0f / kCz) + p.eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * rstd * g8[i] + b8[i];
      const int q = 32 * s + (tid >> 4);
      put_unit(zh_lds + q * ROWB + swz<16>(q, cg) * UNIT, f, T{});
    }
    if (tid < kPairs) mask_lds[tid] = mraw;
    __syncthreads();

    // ---- prefetch the next work item ------------------------------------
    if (tile + 1 < tile_end) load_tile(tile + 1);

    // ---- projections on the matrix cores --------------------------------
    if (active) {
      f32x16 acc[2][2];   // [pair tile][proj, gate]
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.f;

#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        Frag<T> zf[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int q = 32 * mt + (lane & 31);
          const int unit = 2 * ks + (lane >> 5);
          zf[mt].load(zh_lds + q * ROWB + swz<16>(q, unit) * UNIT);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          Frag<T> wf;
          if constexpr (kWeightsInRegs) wf = wreg[nt][ks];
          else wf.load(wfrag_ptr(nt, ks));
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) mma(acc[mt][nt], zf[mt], wf);
        }
      }

      // ---- gate, mask, store: 4 consecutive pairs of channel d per lane ---
      const int d = c0 + (lane & 31);
      // operand layout: blocks of 256 rows x 64 columns, all channels of a
      // block adjacent (see operand_offset); this item is one row of block
      // (r / 256, t0 / 64), 128 contiguous bytes per channel
      T *const prow = out_plane + operand_offset(r, t0, d, p.ld);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int q0 = 32 * mt + acc_row(4 * g, lane);
          const uint32_t m4 = *reinterpret_cast<const uint32_t *>(mask_lds + q0);
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool keep = (m4 >> (8 * i)) & 0xff;
            v[i] = keep ? sigmoid_f32(acc[mt][1][4 * g + i]) * acc[mt][0][4 * g + i] : 0.f;
          }
          store4(prow + q0, v);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_k1(const K1Args &a, int dtype, hipStream_t s) {
  const int64_t n_tiles = a.n_rows * (a.ld / kPairs);
  if (n_tiles <= 0) return hipSuccess;
  // one resident work-group per CU, persistent over the work items
  const int64_t grid = n_tiles < device_cu_count() ? n_tiles : device_cu_count();
  if (dtype == TRIMUL_BF16)
    hipLaunchKernelGGL(k1_project<bf16_t>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k1_project<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace trimul
