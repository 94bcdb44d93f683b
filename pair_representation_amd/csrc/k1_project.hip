// K1: input LayerNorm, the four c_z -> c projections, sigmoid gates and the
// pair mask, producing the contraction operands
//     a = m * sigmoid(W_a_gate zh) * (W_a_proj zh),  b likewise,
// in the blocked operand layout (see operand_offset).  For the incoming
// direction the source pair of plane cell (r, t) is (t, r), so the operands
// come out transposed and the contraction kernel is the same for both
// directions.
//
// Work item: 64 consecutive plane columns t of one plane row r (64 pairs).
// 512 threads = 8 waves, two per SIMD; each work-group walks a contiguous
// range of items, software-pipelined over three items:
//  - z of item i+2 is loaded into registers (16 lanes per pair, two 8-channel
//    units per thread) while item i is processed;
//  - the LayerNorm of item i+1 (16-lane DPP reductions, result rounded to the
//    weight type) is written to the other half of a double-buffered LDS tile,
//    its instructions interleaved with the matrix-core products of item i;
//  - matrix-core product with pairs as rows: out[pair][col] = zh . W[col].
//    Wave w owns operand w/4 (a or b) and channels 32*(w%4) .. +31: its
//    32 projection columns and the 32 gate columns of the same channels land
//    in the same lanes, so the gated, masked product is formed in registers
//    (bf16 weight fragments stay in registers for the whole pass);
//  - one barrier per item.
// Each lane ends up with 4 consecutive pairs of one channel; a wave stages
// its 32 channel rows of the item in LDS and writes each as whole 128-byte
// (bf16) lines, 16 bytes per lane.  z is read with non-temporal loads and
// the operands are written with non-temporal stores: this kernel touches
// neither again, and streaming them leaves the caches to other data.
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kPairs = 64;
constexpr int kThreads = 512;
constexpr int kRowGroup = 16;   // plane rows walked per column block

template <typename T>
struct ZUnit;  // 8 channels of one pair as loaded from HBM

template <>
struct ZUnit<bf16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const unsigned char *p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  }
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
// Eight values of one LDS operand row, or zeros where `keep` is false (a
// masked pair); the choice is made on the stored words.
__device__ __forceinline__ void put_unit(unsigned char *dst, const float (&f)[8], bool keep, bf16_t) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = keep ? pack_bf16x2(f[2 * i], f[2 * i + 1]) : 0u;
  *reinterpret_cast<u32x4 *>(dst) = w;
}
__device__ __forceinline__ void put_unit(unsigned char *dst, const float (&f)[8], bool keep, float) {
  reinterpret_cast<f32x4 *>(dst)[0] = keep ? f32x4{f[0], f[1], f[2], f[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
  reinterpret_cast<f32x4 *>(dst)[1] = keep ? f32x4{f[4], f[5], f[6], f[7]} : f32x4{0.f, 0.f, 0.f, 0.f};
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
  constexpr int OUTB = kPairs * E;     // bytes of one channel's output row of an item
  constexpr int OSTR = OUTB + 4 * E;   // padded staging stride (conflict-free writes)
  constexpr bool kWeightsInRegs = (E == 2);
  __shared__ __attribute__((aligned(16))) unsigned char zh_lds[2][kPairs * ROWB];
  __shared__ __attribute__((aligned(16))) unsigned char out_lds[kThreads / 64][32 * OSTR];

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
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) wreg[nt][ks].load(wfrag_ptr(nt, ks));
  }

  // Item order: groups of kRowGroup plane rows; inside a group, column block
  // by column block, and inside a column block row by row.  Each work-group
  // takes a contiguous range of items, so it writes kRowGroup consecutive
  // 128-byte rows of every channel block it touches one after the other
  // (2 KB runs per channel instead of scattered lines) and stays in a few
  // pages of the operand.
  const int64_t per_wg = (n_tiles + gridDim.x - 1) / gridDim.x;
  const int64_t tile_begin = blockIdx.x * per_wg;
  const int64_t tile_end = tile_begin + per_wg < n_tiles ? tile_begin + per_wg : n_tiles;
  if (tile_begin >= tile_end) return;

  // plane position of a work item: row r, first column t0, and the row group
  // [g0, g0 + gn) it belongs to; advanced in item order
  struct Pos {
    int64_t r, t0, g0, gn;
  };
  auto group_rows = [&](int64_t g0) { return p.n_rows - g0 < kRowGroup ? p.n_rows - g0 : (int64_t)kRowGroup; };
  auto pos_of = [&](int64_t tile) {
    const int64_t g0 = tile / (kRowGroup * tiles_per_row) * kRowGroup;
    const int64_t gn = group_rows(g0);
    const int64_t rem = tile - g0 * tiles_per_row;
    return Pos{g0 + rem % gn, rem / gn * kPairs, g0, gn};
  };
  auto next_pos = [&](Pos q) {
    if (++q.r == q.g0 + q.gn) {
      q.r = q.g0;
      q.t0 += kPairs;
      if (q.t0 == p.ld) {
        q.t0 = 0;
        q.g0 += kRowGroup;
        q.gn = group_rows(q.g0);
        q.r = q.g0;
      }
    }
    return q;
  };

  // Loads of z and mask for a work item.  Cells past k_len (and rows past the
  // last item, which the pipeline touches after the end of its range) read a
  // valid stand-in pair and count as masked, so the code stays branch-free.
  const unsigned char *zbytes = static_cast<const unsigned char *>(p.z);
  ZUnit<T> raw[2];
  uint8_t mbyte[2];   // mask bytes, tested only in the LayerNorm so that
  bool mvalid[2];     // issuing the loads never waits for them
  auto pair_index = [&](int64_t r, int64_t t, bool &valid) -> int64_t {
    valid = t < p.k_len && r < p.n_rows;
    const int64_t rr = r < p.n_rows ? r : p.n_rows - 1;
    const int64_t tt = t < p.k_len ? t : 0;
    const int64_t i = p.transposed ? p.k_off + tt : p.row_base + rr;
    const int64_t j = p.transposed ? p.row_base + rr : p.k_off + tt;
    return i * p.n + j;
  };
  // offsets of this thread's two units from the item's first pair
  // (consecutive plane columns are consecutive pairs, or pairs n apart when
  // the plane is transposed), in pairs (mask) and in bytes (z); used for
  // items that lie wholly in range, addressed as a wave-uniform base plus
  // these loop-invariant 32-bit offsets (at most 63 * 65535 pairs of 512
  // bytes, below 2^32)
  uint32_t poff[2], zoff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    poff[s] = (uint32_t)(32 * s + (tid >> 4)) * (uint32_t)(p.transposed ? p.n : 1);
    zoff[s] = (poff[s] * kCz + cg * 8) * E;
  }
  auto load_item = [&](Pos q) {
    if (q.r < p.n_rows && q.t0 + kPairs <= p.k_len) {
      bool valid;
      const int64_t base = pair_index(q.r, q.t0, valid);   // wave-uniform
      const unsigned char *zb = zbytes + base * (kCz * E);
      const uint8_t *mb = p.mask + base;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        raw[s].load(zb + zoff[s]);
        mbyte[s] = mb[poff[s]];
        mvalid[s] = true;
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int pr = 32 * s + (tid >> 4);   // pair within the item
        bool valid;
        const int64_t idx = pair_index(q.r, q.t0 + pr, valid);
        raw[s].load(zbytes + (idx * kCz + cg * 8) * E);
        mbyte[s] = p.mask[idx];
        mvalid[s] = valid;
      }
    }
  };

  // LayerNorm of the item held in `raw` -> LDS buffer `buf`.  A masked pair's
  // row is stored as zeros: its projections are then exactly 0 and so is the
  // gated product sigmoid(0) * 0, which applies the pair mask to a and b.
  auto layer_norm = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float f[8];
      raw[s].to_f32(f);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += f[i];
      const float mean = row_sum16(sum) * (1.0f / kCz);
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { f[i] -= mean; sq += f[i] * f[i]; }
      const float rstd = rsqrt_f32(row_sum16(sq) * (1.0f / kCz) + p.eps);
      const bool keep = mvalid[s] && mbyte[s] != 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * rstd * g8[i] + b8[i];
      const int pr = 32 * s + (tid >> 4);
      put_unit(zh_lds[buf] + pr * ROWB + swz<16>(pr, cg) * UNIT, f, keep, T{});
    }
  };

  f32x16 acc[2][2];   // [pair tile][proj, gate]
  // products of pair tile mt (pairs 32mt .. 32mt+31) with this wave's 32
  // projection and 32 gate columns
  auto products = [&](int buf, int mt) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      Frag<T> zf;
      const int q = 32 * mt + (lane & 31);
      zf.load(zh_lds[buf] + q * ROWB + swz<16>(q, 2 * ks + (lane >> 5)) * UNIT);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        Frag<T> wf;
        if constexpr (kWeightsInRegs) wf = wreg[nt][ks];
        else wf.load(wfrag_ptr(nt, ks));
        mma(acc[mt][nt], zf, wf);
      }
    }
  };
  // gated products of pair tile mt -> this wave's staging rows (row = channel
  // c0 + lane % 32; each lane holds 4 consecutive pairs per register group)
  unsigned char *const stage = out_lds[wave];
  auto gate = [&](int mt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = sigmoid_f32(acc[mt][1][4 * g + i]) * acc[mt][0][4 * g + i];
      const int q0 = 32 * mt + acc_row(4 * g, lane);
      store4(reinterpret_cast<T *>(stage + (lane & 31) * OSTR) + q0, v);
    }
  };
  // staging rows -> HBM: one 16-byte piece per lane, whole 128-byte (bf16)
  // or 256-byte (fp32) channel rows per group of lanes.  The operand layout
  // keeps the 64 columns of an item contiguous within each channel block.
  // (operand_offset is linear in the channel, and the 64 columns of an item
  // are one contiguous run per channel: a wave-uniform base plus a
  // loop-invariant lane offset)
  constexpr int LPR = OUTB / 16;     // lanes per channel row
  constexpr int RPI = 64 / LPR;      // rows per instruction
  const uint32_t st_lane = (uint32_t)(lane / LPR) * (uint32_t)kOpBlock + (lane % LPR) * (16 / E);
  auto store_out = [&](Pos q) {
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    T *const ob = out_plane + operand_offset(q.r, q.t0, c0, p.ld);   // wave-uniform
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + lane / LPR;
      const int piece = lane % LPR;
      const u32x2 *src = reinterpret_cast<const u32x2 *>(stage + row * OSTR + piece * 16);
      const u32x2 lo = src[0], hi = src[1];
      if (active)
        __builtin_nontemporal_store(u32x4{lo[0], lo[1], hi[0], hi[1]},
                                    reinterpret_cast<u32x4 *>(ob + (st_lane + (uint32_t)(i * RPI) * (uint32_t)kOpBlock)));
    }
  };

  // prologue: item 0 normalised into buffer 0, item 1 in registers
  Pos cur = pos_of(tile_begin);
  load_item(cur);
  layer_norm(0);
  Pos ahead = next_pos(cur);       // the item held in `raw`
  load_item(ahead);
  __syncthreads();

  // One barrier per item.  The matrix-core products of this item, the
  // LayerNorm of the next one (after the last item: a stand-in nobody reads)
  // and the loads of the one after are mutually independent.  The two waves
  // of a SIMD (w and w + 4) take them in opposite orders between the same
  // barriers, so one wave's products overlap the other's LayerNorm instead of
  // both waiting for the one matrix core at once.  Waves with no output run
  // the products on unused weights and skip the stores.
  for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
    const int buf = (int)((tile - tile_begin) & 1);
    // (each order is one straight-line block, gates and stores included, so
    // the compiler can interleave all of it)
    if (wave < 4) {
      products(buf, 0);
      products(buf, 1);
      layer_norm(buf ^ 1);
      ahead = next_pos(ahead);
      load_item(ahead);
      gate(0);
      gate(1);
      store_out(cur);
    } else {
      layer_norm(buf ^ 1);
      ahead = next_pos(ahead);
      load_item(ahead);
      products(buf, 0);
      products(buf, 1);
      gate(0);
      gate(1);
      store_out(cur);
    }
    cur = next_pos(cur);
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
