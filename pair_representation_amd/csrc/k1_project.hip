// K1: input LayerNorm, the four c_z -> c projections, sigmoid gates and the
// pair mask, producing the contraction operands
//     a = m * sigmoid(W_a_gate zh) * (W_a_proj zh),  b likewise,
// as channel-planar, k-contiguous planes  plane[d][r][t]  (one 64-pair run of
// t per work item).  For the incoming direction the source pair of (r, t) is
// (t, r), so the planes come out transposed and the contraction kernel is the
// same for both directions.
//
// Work item: 64 consecutive plane columns t of one plane row r (64 pairs).
// 256 threads: every thread loads four 8-channel units of z (16 lanes per
// pair), the LayerNorm statistics are 16-lane shuffle reductions, and the
// normalised pairs go to LDS (bf16 when the weights are bf16) as the matrix-
// core B operand.  Wave w owns operand w/2 (a or b) and channels
// 64*(w%2) .. +63: projection rows and gate rows of the same channels land in
// the same lanes, so the gate product is formed in registers.  The kernel is
// persistent (one pass over the work items with stride gridDim.x); bf16 weight
// fragments stay in registers for the whole pass and the next item's z is
// prefetched while the current one is on the matrix cores.
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kPairs = 64;
constexpr int kThreads = 256;

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

__device__ __forceinline__ void store_elem(bf16_t *p, float v) { p->v = f32_to_bf16(v); }
__device__ __forceinline__ void store_elem(float *p, float v) { *p = v; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k1_project(K1Args p) {
  constexpr int E = sizeof(T);
  constexpr int UNIT = 8 * E;          // bytes of one 8-channel unit
  constexpr int ROWB = kCz * E;        // bytes of one pair row in LDS
  constexpr bool kWeightsInRegs = (E == 2);
  __shared__ __attribute__((aligned(16))) unsigned char zh_lds[kPairs * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tiles_per_row = p.ld / kPairs;
  const int64_t n_tiles = p.n_rows * tiles_per_row;

  // this thread's 8 channels of LayerNorm affine parameters
  const int cg = tid & 15;  // channel group (8 channels)
  float g8[8], b8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { g8[i] = p.ln_w[cg * 8 + i]; b8[i] = p.ln_b[cg * 8 + i]; }

  // this wave's operand and weight rows
  const int op = wave >> 1;        // 0: a, 1: b
  const int c0 = 64 * (wave & 1);  // first channel
  T *const out_plane = static_cast<T *>(op == 0 ? p.a_out : p.b_out);
  const T *const Wp = static_cast<const T *>(op == 0 ? p.w_a_proj : p.w_b_proj);
  const T *const Wg = static_cast<const T *>(op == 0 ? p.w_a_gate : p.w_b_gate);
  const bool active = out_plane != nullptr;   // wave-uniform

  // m-tile mt: 0,1 -> projection rows c0+32*mt ; 2,3 -> gate rows c0+32*(mt-2)
  auto wfrag_ptr = [&](int mt, int ks) -> const T * {
    const T *W = (mt < 2) ? Wp : Wg;
    const int row = c0 + 32 * (mt & 1) + (lane & 31);
    return W + row * kCz + 16 * ks + 8 * (lane >> 5);
  };
  Frag<T> wreg[kWeightsInRegs ? 4 : 1][kWeightsInRegs ? 8 : 1];
  if constexpr (kWeightsInRegs) {
    if (active) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) wreg[mt][ks].load(wfrag_ptr(mt, ks));
    }
  }

  // source pair of plane cell (r, t); returns false past k_len
  auto src_pair = [&](int64_t r, int64_t t, int64_t &i, int64_t &j) -> bool {
    if (t >= p.k_len) return false;
    if (p.transposed) { i = p.k_off + t; j = p.row_base + r; }
    else { i = p.row_base + r; j = p.k_off + t; }
    return true;
  };

  const unsigned char *zbytes = static_cast<const unsigned char *>(p.z);
  ZUnit<T> raw[4];
  auto load_tile = [&](int64_t tile) {
    const int64_t r = tile / tiles_per_row;
    const int64_t t0 = (tile % tiles_per_row) * kPairs;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int q = 16 * s + (tid >> 4);   // pair within the tile
      int64_t i, j;
      if (src_pair(r, t0 + q, i, j))
        raw[s].load(zbytes + ((i * p.n + j) * kCz + cg * 8) * E);
      else
        raw[s].zero();
    }
  };

  int64_t tile = blockIdx.x;
  if (tile < n_tiles) load_tile(tile);

  for (; tile < n_tiles; tile += gridDim.x) {
    const int64_t r = tile / tiles_per_row;
    const int64_t t0 = (tile % tiles_per_row) * kPairs;

    // ---- LayerNorm of the 64 pairs -> LDS --------------------------------
#pragma unroll
    for (int s = 0; s < 4; ++s) {
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
      const int q = 16 * s + (tid >> 4);
      put_unit(zh_lds + q * ROWB + swz<16>(q, cg) * UNIT, f, T{});
    }
    __syncthreads();

    // ---- prefetch the next work item ------------------------------------
    if (tile + gridDim.x < n_tiles) load_tile(tile + gridDim.x);

    // ---- projections on the matrix cores --------------------------------
    if (active) {
      f32x16 acc[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.f;

#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        Frag<T> bf[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int q = 32 * nt + (lane & 31);
          const int unit = 2 * ks + (lane >> 5);
          bf[nt].load(zh_lds + q * ROWB + swz<16>(q, unit) * UNIT);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          Frag<T> af;
          if constexpr (kWeightsInRegs) af = wreg[mt][ks];
          else af.load(wfrag_ptr(mt, ks));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) mma(acc[mt][nt], af, bf[nt]);
        }
      }

      // ---- gate, mask, store ---------------------------------------------
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int q = 32 * nt + (lane & 31);
        const int64_t t = t0 + q;
        int64_t i, j;
        bool keep = src_pair(r, t, i, j) && p.mask[i * p.n + j] != 0;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int d = c0 + 32 * mt + acc_row(e, lane);
            const float v = keep ? sigmoid_f32(acc[mt + 2][nt][e]) * acc[mt][nt][e] : 0.f;
            store_elem(out_plane + ((int64_t)d * p.n_rows + r) * p.ld + t, v);
          }
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
  // one resident work-group per CU (register-limited), persistent over items
  const int64_t grid = n_tiles < device_cu_count() ? n_tiles : device_cu_count();
  if (dtype == TRIMUL_BF16)
    hipLaunchKernelGGL(k1_project<bf16_t>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k1_project<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace trimul
