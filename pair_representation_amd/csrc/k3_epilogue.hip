// K3: the epilogue of the update for a tile of the pair grid,
//     out_ij = m_ij * sigmoid(W_out_gate LN_in(z_ij)) * (W_out_proj LN_out(x_ij))
// reading the contraction result x (blocks of 4 rows x 16 columns x 128
// channels, see x_offset) and the
// pair tensor, writing fp32 out[r][s][e].
//
// Work item: 32 pairs = 4 consecutive rows x 8 consecutive columns, pair
// index p = 4*jj + ii, which is also the order of one channel's 32 values in
// x (128 contiguous bytes).  256 threads = 4 waves (one per SIMD), persistent
// over the work items; the next item's x and z are prefetched into registers
// while the current one is processed.  Two work-groups share each compute
// unit and run out of step with each other, so the matrix-core phase of one
// overlaps the LayerNorm phases (short dependent chains of vector, LDS and
// cross-lane instructions) of the other on the same SIMD.
//  - x: thread (pair p = tid % 32, channel group tid / 32) holds 16 channels;
//    output LayerNorm statistics are combined over the 8 groups in LDS.
//  - z is re-read (16 lanes per pair, 16-lane DPP reductions) and
//    re-normalised for the gate.  x and z are read with non-temporal loads
//    (each is read once here).
//  - Both normalised operands go to LDS as matrix-core B operands; in bf16
//    mode each is split into hi + lo bf16 terms (hi = bf16(v),
//    lo = bf16(v - hi)) and multiplied by the bf16 weights twice, so the
//    products keep fp32-level accuracy.
//  - Wave w computes output channels 32*w .. +31 of both the projection
//    and the gate for the item's 32 pairs (pairs as the rows of the
//    products, channels as the columns), so the final product is formed in
//    registers and stored from there, each store instruction writing whole
//    128-byte lines (32 channels of two pairs).  bf16 weight fragments stay
//    in registers for the whole pass.
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kPairs = 32;
constexpr int kRows = 4, kCols = 8;   // work-item shape
constexpr int kThreads = 256;
constexpr int kGroups = kThreads / kPairs;   // x channel groups (8)
constexpr int kXPer = kC / kGroups;          // x channels per thread (16)
static_assert(kRows * kCols == kPairs && kThreads == 64 * 4, "one wave per SIMD");

template <typename T>
struct ZUnit;

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

// LDS operand planes: bf16 mode keeps hi and lo planes [32][128] bf16 each;
// fp32 mode keeps one plane [32][128] fp32.  Rows are 256 / 512 bytes, units
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
      // hi terms of both values from one packed rounding; unpacked exactly
      h[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
      const float h0 = __uint_as_float(h[i] << 16);
      const float h1 = __uint_as_float(h[i] & 0xffff0000u);
      l[i] = pack_bf16x2(f[2 * i] - h0, f[2 * i + 1] - h1);
    }
    const int off = q * ROWB + swz<16>(q, unit) * UNIT;
    *reinterpret_cast<u32x4 *>(base + off) = h;
    *reinterpret_cast<u32x4 *>(base + PLANE + off) = l;
  }
  // k-fragments of pair row q, 8-channel unit `unit`: hi and lo terms of the
  // normalised x (n) and z (z) operands
  struct Frags {
    Frag<bf16_t> nh, nl, zh, zl;
  };
  __device__ static void read(Frags &f, const unsigned char *n, const unsigned char *z, int q, int unit) {
    const int off = q * ROWB + swz<16>(q, unit) * UNIT;
    f.nh.load(n + off);
    f.nl.load(n + PLANE + off);
    f.zh.load(z + off);
    f.zl.load(z + PLANE + off);
  }
  // ay += n * Wo^T, ag += z * Wg^T over 16 k values (both terms): pairs are
  // the rows of the products, output channels the columns
  __device__ static void mma(f32x16 &ay, f32x16 &ag, const Frag<bf16_t> &wo, const Frag<bf16_t> &wg,
                             const Frags &f) {
    ::trimul::mma(ay, f.nh, wo);
    ::trimul::mma(ag, f.zh, wg);
    ::trimul::mma(ay, f.nl, wo);
    ::trimul::mma(ag, f.zl, wg);
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
  struct Frags {
    Frag<float> n, z;
  };
  __device__ static void read(Frags &f, const unsigned char *n, const unsigned char *z, int q, int unit) {
    const int off = q * ROWB + swz<16>(q, unit) * UNIT;
    f.n.load(n + off);
    f.z.load(z + off);
  }
  __device__ static void mma(f32x16 &ay, f32x16 &ag, const Frag<float> &wo, const Frag<float> &wg,
                             const Frags &f) {
    ::trimul::mma(ay, f.n, wo);
    ::trimul::mma(ag, f.z, wg);
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k3_epilogue(K3Args p) {
  constexpr int E = sizeof(T);
  constexpr bool kWeightsInRegs = (E == 2);
  using Op = Operand<T>;
  constexpr int kOpBytes = Op::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char n_ops[kOpBytes];   // normalised x
  __shared__ __attribute__((aligned(16))) unsigned char z_ops[kOpBytes];   // normalised z
  __shared__ __attribute__((aligned(8))) float2 part[kGroups][kPairs];    // per-group (mean, M2)
  __shared__ uint32_t mask_word;   // bit q: pair q of the item is kept

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int64_t rows4 = (p.n_rows + 3) / 4;
  const int64_t tiles_per_blk = (p.n_cols + kCols - 1) / kCols;
  const int64_t n_tiles = rows4 * tiles_per_blk;

  // x channels of this thread: xc0 .. xc0+15 of pair q
  const int q = tid % kPairs;
  const int grp = tid / kPairs;
  const int xc0 = kXPer * grp;
  float gx[kXPer], bx[kXPer];
#pragma unroll
  for (int c = 0; c < kXPer; ++c) { gx[c] = p.ln_out_w[xc0 + c]; bx[c] = p.ln_out_b[xc0 + c]; }
  // z units of this thread: pairs 16*s + tid/16, channel group tid & 15
  const int cg = tid & 15;
  // The gate operand is kept as -log2(e) * LN_in(z): the products then give
  // the argument of the base-2 exponential in the logistic function directly.
  constexpr float kNegLog2e = -1.4426950408889634f;
  float gz[8], bz[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { gz[i] = p.ln_in_w[cg * 8 + i]; bz[i] = p.ln_in_b[cg * 8 + i] * kNegLog2e; }

  // matrix-core rows (output channels) of this wave
  const int o0 = 32 * wave;
  const T *const Wo = static_cast<const T *>(p.w_out_proj);
  const T *const Wg = static_cast<const T *>(p.w_out_gate);
  auto wptr = [&](const T *W, int ks) -> const T * {
    return W + (o0 + (lane & 31)) * kC + 16 * ks + 8 * (lane >> 5);
  };
  Frag<T> wo[kWeightsInRegs ? 8 : 1], wg[kWeightsInRegs ? 8 : 1];
  if constexpr (kWeightsInRegs) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) { wo[ks].load(wptr(Wo, ks)); wg[ks].load(wptr(Wg, ks)); }
  }

  const unsigned char *zbytes = static_cast<const unsigned char *>(p.z);

  // ---- per-item loads (prefetched one item ahead) --------------------------
  // Pairs outside the tile read a valid stand-in pair and count as masked.
  float xv[kXPer];
  ZUnit<T> zr[2];
  uint8_t mbyte = 0;   // mask byte of pair q (tested only where it is used, so
  bool mvalid = false; // that issuing the prefetch never waits for it)
  auto pair_index = [&](int64_t blk, int64_t s0, int pr, bool &valid) -> int64_t {
    const int64_t r = blk * 4 + (pr & 3), col = s0 + (pr >> 2);
    valid = r < p.n_rows && col < p.n_cols;
    const int64_t rr = r < p.n_rows ? r : p.n_rows - 1;
    const int64_t cc = col < p.n_cols ? col : p.n_cols - 1;
    return (p.row_off + rr) * p.n + p.col_off + cc;
  };
  // position of a work item: row block (4 rows) and first column
  struct Pos {
    int64_t blk, s0;
  };
  auto advance = [&](Pos &ps) {
    ps.s0 += kCols;
    if (ps.s0 >= p.n_cols) { ps.s0 = 0; ++ps.blk; }
  };
  // pair offsets (relative to the item's first pair) of this thread's z
  // units and mask byte, used for items that lie wholly inside the tile
  int zoff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int pr = 16 * s + (tid >> 4);
    zoff[s] = (pr & 3) * (int)p.n + (pr >> 2);
  }
  const int moff = (q & 3) * (int)p.n + (q >> 2);
  // x: the item is one half (8 columns) of a 4 x 16 block of the x layout
  // (x_offset): 128 channels x 32 pairs, 128 contiguous bytes per channel,
  // pair q at 4*jj + ii
  auto load_x = [&](const Pos &ps) {
    const float *xp = p.x + x_offset(ps.blk * 4, ps.s0, xc0, p.ldx) + q;
#pragma unroll
    for (int c = 0; c < kXPer; ++c) xv[c] = __builtin_nontemporal_load(xp + c * 64);
  };
  // z and the mask byte
  auto load_zm = [&](const Pos &ps) {
    const int64_t blk = ps.blk, s0 = ps.s0;
    if (blk * 4 + kRows <= p.n_rows && s0 + kCols <= p.n_cols) {
      const int64_t base = (p.row_off + blk * 4) * p.n + p.col_off + s0;   // the item's first pair
#pragma unroll
      for (int s = 0; s < 2; ++s) zr[s].load(zbytes + ((base + zoff[s]) * kCz + cg * 8) * E);
      mbyte = p.mask[base + moff];
      mvalid = true;
    } else {
      bool valid;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int64_t idx = pair_index(blk, s0, 16 * s + (tid >> 4), valid);
        zr[s].load(zbytes + (idx * kCz + cg * 8) * E);
      }
      mbyte = p.mask[pair_index(blk, s0, q, valid)];
      mvalid = valid;
    }
  };
  auto load_item = [&](const Pos &ps) {
    load_x(ps);
    load_zm(ps);
  };

  // Each work-group takes a contiguous range of work items, so consecutive
  // items read consecutive 16 KB half-blocks of x and neighbouring columns
  // of z.
  const int64_t per_wg = (n_tiles + gridDim.x - 1) / gridDim.x;
  const int64_t tile_begin = blockIdx.x * per_wg;
  const int64_t tile_end = tile_begin + per_wg < n_tiles ? tile_begin + per_wg : n_tiles;
  int64_t tile = tile_begin;
  Pos cur{tile_begin / tiles_per_blk, (tile_begin % tiles_per_blk) * kCols};
  Pos nxt = cur;
  advance(nxt);
  if (tile < tile_end) load_item(cur);

  // Two barriers per item: (1) per-group LayerNorm partials written,
  // (2) normalised operands written.  The partials of the next item are
  // written after (2), when every wave has read the current ones; the
  // operands of the next item after its (1), when every wave has finished
  // this item's products.
  for (; tile < tile_end; ++tile, cur = nxt, advance(nxt)) {
    const int64_t blk = cur.blk, s0 = cur.s0;

    // ---- output LayerNorm: exact per-thread partials over 16 channels,
    //      merged per pair across the 8 groups (Chan et al.'s pairwise
    //      update of mean and sum of squared deviations) -----------------------
    {
      float sum = 0.f;
#pragma unroll
      for (int c = 0; c < kXPer; ++c) sum += xv[c];
      const float m = sum * (1.0f / kXPer);
      float m2 = 0.f;
#pragma unroll
      for (int c = 0; c < kXPer; ++c) { const float d = xv[c] - m; m2 += d * d; }
      part[grp][q] = make_float2(m, m2);
      // lanes q and q + 32 of wave 0 both hold pair q's mask byte
      const uint64_t kept = __ballot(mvalid && mbyte != 0);
      if (tid == 0) mask_word = (uint32_t)kept;
    }
    __syncthreads();   // (1)
    // the item's mask bits, read before (2): the next item's word is
    // written after it
    const uint32_t keep_bits = mask_word;
    const int pq = lane & 31;   // pair of this lane's operand fragments
    {
      float2 pg[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) pg[g] = part[g][q];
      float msum = 0.f;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) msum += pg[g].x;
      const float mean = msum * (1.0f / kGroups);
      float m2 = 0.f, dev = 0.f;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) { m2 += pg[g].y; const float d = pg[g].x - mean; dev += d * d; }
      const float var = (m2 + kXPer * dev) * (1.0f / kC);
      const float rstd = rsqrt_f32(var + p.eps);
#pragma unroll
      for (int u = 0; u < kXPer / 8; ++u) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (xv[8 * u + i] - mean) * rstd * gx[8 * u + i] + bx[8 * u + i];
        Op::put(n_ops, q, xc0 / 8 + u, f);
      }
    }

    // the next item's x (this item's is consumed): requested ahead of z and
    // the mask, so the prefetch goes out in two bursts
    if (tile + 1 < tile_end) load_x(nxt);

    // ---- input LayerNorm of z (recomputed) for the gate --------------------
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float f[8];
      zr[s].to_f32(f);
      float zs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) zs += f[i];
      const float zm = row_sum16(zs) * (1.0f / kCz);
      float zq = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { f[i] -= zm; zq += f[i] * f[i]; }
      const float zrs = rsqrt_f32(row_sum16(zq) * (1.0f / kCz) + p.eps) * kNegLog2e;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * zrs * gz[i] + bz[i];
      Op::put(z_ops, 16 * s + (tid >> 4), cg, f);
    }
    __syncthreads();   // (2)

    // ---- prefetch the rest of the next item --------------------------------
    if (tile + 1 < tile_end) load_zm(nxt);

    // ---- projections on the matrix cores ----------------------------------
    f32x16 ay, ag;
#pragma unroll
    for (int e = 0; e < 16; ++e) { ay[e] = 0.f; ag[e] = 0.f; }
    // operand fragments are read one k step ahead of the matrix-core
    // instructions that use them
    typename Op::Frags fr[2];
    Op::read(fr[0], n_ops, z_ops, pq, lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 1 < 8) Op::read(fr[(ks + 1) & 1], n_ops, z_ops, pq, 2 * (ks + 1) + (lane >> 5));
      Frag<T> fo, fg;
      if constexpr (kWeightsInRegs) { fo = wo[ks]; fg = wg[ks]; }
      else { fo.load(wptr(Wo, ks)); fg.load(wptr(Wg, ks)); }
      // keep the reads of step ks+1 ahead of this step's products
      __builtin_amdgcn_sched_barrier(0);
      Op::mma(ay, ag, fo, fg, fr[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- gate * projection * mask -> HBM ----------------------------------
    // Accumulator register e of a lane is output channel o0 + lane % 32 of
    // pair acc_row(e, lane) = 8 (e / 4) + 4 (lane / 32) + e % 4, i.e. row
    // e % 4 and column 2 (e / 4) + lane / 32 of the item: for each register
    // the two half-waves write the wave's 32 channels of one pair each, two
    // whole 128-byte lines, so the stores bypass the caches (the output is
    // not read again here) without partial-line writes.
    const uint32_t kb = keep_bits >> (4 * (lane >> 5));
    float *const obase = p.out + (blk * 4 * p.out_ld + s0 + (lane >> 5)) * kCz + o0 + (lane & 31);
    const int64_t row_stride = p.out_ld * kCz;
    const bool whole = blk * 4 + kRows <= p.n_rows && s0 + kCols <= p.n_cols;
    if (whole && keep_bits == 0xffffffffu) {
      // an item wholly inside the tile with every pair kept
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ii = e & 3;
        __builtin_nontemporal_store(sigmoid_of_exp2_arg(ag[e]) * ay[e],
                                    obase + ii * row_stride + 2 * (e >> 2) * kCz);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ii = e & 3, jj = 2 * (e >> 2) + (lane >> 5);
        const float gated = sigmoid_of_exp2_arg(ag[e]) * ay[e];
        const float v = ((kb >> (8 * (e >> 2) + (e & 3))) & 1u) ? gated : 0.f;
        if (whole || (blk * 4 + ii < p.n_rows && s0 + jj < p.n_cols))
          __builtin_nontemporal_store(v, obase + ii * row_stride + 2 * (e >> 2) * kCz);
      }
    }
  }
}

}  // namespace

hipError_t launch_k3(const K3Args &a, int dtype, hipStream_t s) {
  const int64_t n_tiles = ((a.n_rows + 3) / 4) * ((a.n_cols + kCols - 1) / kCols);
  if (n_tiles <= 0) return hipSuccess;
  const int64_t cap = 2 * (int64_t)device_cu_count();   // two work-groups per compute unit
  const int64_t grid = n_tiles < cap ? n_tiles : cap;
  if (dtype == TRIMUL_BF16)
    hipLaunchKernelGGL(k3_epilogue<bf16_t>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k3_epilogue<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace trimul
