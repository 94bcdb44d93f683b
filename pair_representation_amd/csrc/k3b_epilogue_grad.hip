// K3B: backward of a gated, masked pair of 128 x 128 linear maps after
// LayerNorm, on a grid of positions of the pair grid.  Epilogue mode: the
// backward of K3 for a tile (x = the contraction result, W_y = W_out_proj,
// W_t = W_out_gate, LN_x = the output and LN_z = the input LayerNorm).
// Projection mode: the backward of one side of K1 (x = z, LN_x = LN_z = the
// input LayerNorm, W_y / W_t = the side's projection / gate matrix, positions
// = the operand entries of a chunk, mapped to their source pairs).
//
// Forward, per pair: n = LN_x(x) = x^ g_x + b_x, y = W_y n,
// zh = LN_z(z) = z^ g_z + b_z, t = W_t zh, s = sigmoid(t), out = m s y.
// Given dout = dL/dout the kernel writes, per pair,
//   dy = m s dout,  dt = m y dout s (1 - s)
//   dn = W_y^T dy,  dx = LN backward of dn * g_x   (epilogue: the input of
//                                                  the contraction's backward)
//   dzh = W_t^T dt, dz = LN backward of dzh * g_z  (epilogue: the gate path's
//                                                  share of dL/dz)
// (projection mode: x^ = z^, so the normalised input is formed once, and one
// LayerNorm backward of dn * g + dzh * g is added to a global dL/dz)
// and, for the parameters, the sums over the grid's pairs
//   G = sum dy x^T,  S = sum dy,  H = sum dt z^T,  T = sum dt
// from which dW_y = G diag(g_x) + S b_x^T, dg_x = colsum(W_y * G),
// db_x = W_y^T S (W_t and LN_z likewise from H, T): the weight gradients
// become two 128 x 128 accumulators per work-group instead of six.
//
// Work item: 32 pairs = 4 rows x 8 columns as in K3 (pair p = 4*jj + ii, the
// order of one channel's values in the x layout).  One work-group of 4 waves
// per compute unit, persistent, with G and H held in the matrix-core
// accumulators of its waves for the whole pass (wave w: rows 32w .. +31 of
// both) and written once to a per-work-group slot; a second kernel sums the
// slots in a fixed order and forms the parameter gradients.
// Two thread layouts per item:
//  - row layout: thread (pair q = tid % 32, channel group tid / 32) holds 16
//    channels of x and z of pair q; LayerNorm statistics are combined over the
//    8 groups in LDS.  Wave w holds channels 32w .. +31, the rows its
//    matrix-core products produce.
//  - accumulator layout: lane l holds pair l % 32 and channels
//    32w + acc_row(e, l) of every 32 x 32 product; dy, dt, dn, dzh and the
//    LayerNorm backward live here, and dx, dz are stored from here.
// LDS: the normalised x and gate input, dy and dt as [pair][channel]
// matrix-core operands (bf16 mode: hi + lo bf16 terms, as in K3), and x^, z^,
// dy, dt as fp32 [channel][pair] planes, the operands of the G and H products
// (contraction over pairs; split into hi + lo bf16 terms when read in bf16
// mode, three products per step: hi = bf16(v), lo = bf16(v - hi) represent
// v to within 2^-16 |v|, and the dropped lo*lo term is as small).
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kPairs = 32;
constexpr int kCols = 8;                       // work item: 4 rows x 8 columns
constexpr int kThreads = 256;
constexpr int kGroups = kThreads / kPairs;     // channel groups of the row layout (8)
constexpr int kPer = kC / kGroups;             // channels per row-layout thread (16)
constexpr float kNegLog2e = -1.4426950408889634f;

// fp32 plane [128 rows][32 pairs]: 16-byte units of 4 pairs XOR-swizzled with
// the row's group of 8, so that the row layout's 16-row writes and the
// 32-row fragment reads spread over the banks.
__device__ __forceinline__ int pl(int row, int p) { return row * kPairs + (p ^ (((row >> 3) & 7) << 2)); }

// [pair][128 channel] matrix-core operand (B operand over channels):
// bf16 mode hi and lo planes, 16-byte units of 8 channels swizzled per pair
// row; fp32 mode one plane, 32-byte units.
template <typename T>
struct OpB;

template <>
struct OpB<bf16_t> {
  static constexpr int ROWB = kC * 2, PLANE = kPairs * ROWB, BYTES = 2 * PLANE;
  __device__ static int off(int q, int unit) { return q * ROWB + swz<16>(q, unit) * 16; }
  // channels 8 unit .. +7 of pair q
  __device__ static void put8(unsigned char *base, int q, int unit, const float (&f)[8]) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
      l[i] = pack_bf16x2(f[2 * i] - __uint_as_float(h[i] << 16), f[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
    }
    *reinterpret_cast<u32x4 *>(base + off(q, unit)) = h;
    *reinterpret_cast<u32x4 *>(base + PLANE + off(q, unit)) = l;
  }
  // channels ch4 .. ch4+3 of pair q (ch4 a multiple of 4)
  __device__ static void put4(unsigned char *base, int q, int ch4, const float (&f)[4]) {
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    u32x2 h, l;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      h[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
      l[i] = pack_bf16x2(f[2 * i] - __uint_as_float(h[i] << 16), f[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
    }
    const int o = off(q, ch4 >> 3) + (ch4 & 7) * 2;
    *reinterpret_cast<u32x2 *>(base + o) = h;
    *reinterpret_cast<u32x2 *>(base + PLANE + o) = l;
  }
  struct Fr {
    Frag<bf16_t> h, l;
  };
  __device__ static void read(Fr &f, const unsigned char *base, int q, int unit) {
    f.h.load(base + off(q, unit));
    f.l.load(base + PLANE + off(q, unit));
  }
  // acc += W * (hi + lo)
  __device__ static void mma_w(f32x16 &acc, const Frag<bf16_t> &w, const Fr &f) {
    ::trimul::mma(acc, w, f.h);
    ::trimul::mma(acc, w, f.l);
  }
};

template <>
struct OpB<float> {
  static constexpr int ROWB = kC * 4, PLANE = kPairs * ROWB, BYTES = PLANE;
  __device__ static int off(int q, int unit) { return q * ROWB + swz<16>(q, unit) * 32; }
  __device__ static void put8(unsigned char *base, int q, int unit, const float (&f)[8]) {
    reinterpret_cast<f32x4 *>(base + off(q, unit))[0] = f32x4{f[0], f[1], f[2], f[3]};
    reinterpret_cast<f32x4 *>(base + off(q, unit))[1] = f32x4{f[4], f[5], f[6], f[7]};
  }
  __device__ static void put4(unsigned char *base, int q, int ch4, const float (&f)[4]) {
    *reinterpret_cast<f32x4 *>(base + off(q, ch4 >> 3) + (ch4 & 7) * 4) = f32x4{f[0], f[1], f[2], f[3]};
  }
  struct Fr {
    Frag<float> v;
  };
  __device__ static void read(Fr &f, const unsigned char *base, int q, int unit) { f.v.load(base + off(q, unit)); }
  __device__ static void mma_w(f32x16 &acc, const Frag<float> &w, const Fr &f) { ::trimul::mma(acc, w, f.v); }
};

// k-fragment of an fp32 [channel][pair] plane: row `row`, pairs p0 .. p0+7
// (the operand of a contraction over pairs).  bf16 mode splits it into hi +
// lo terms; the product of two such fragments takes hi*hi + hi*lo + lo*hi.
template <typename T>
struct PFrag;

template <>
struct PFrag<bf16_t> {
  Frag<bf16_t> h, l;
  // returns the sum of the 8 values read
  __device__ float load(const float *plane, int row, int p0) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(plane + pl(row, p0));
    const f32x4 b = *reinterpret_cast<const f32x4 *>(plane + pl(row, p0 + 4));
    const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x4 hh, ll;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hh[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
      ll[i] = pack_bf16x2(f[2 * i] - __uint_as_float(hh[i] << 16), f[2 * i + 1] - __uint_as_float(hh[i] & 0xffff0000u));
    }
    h.v = __builtin_bit_cast(bf16x8, hh);
    l.v = __builtin_bit_cast(bf16x8, ll);
    return ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
  }
};

template <>
struct PFrag<float> {
  Frag<float> v;
  __device__ float load(const float *plane, int row, int p0) {
    v.lo = *reinterpret_cast<const f32x4 *>(plane + pl(row, p0));
    v.hi = *reinterpret_cast<const f32x4 *>(plane + pl(row, p0 + 4));
    return ((v.lo[0] + v.lo[1]) + (v.lo[2] + v.lo[3])) + ((v.hi[0] + v.hi[1]) + (v.hi[2] + v.hi[3]));
  }
};

__device__ __forceinline__ void mma_pp(f32x16 &acc, const PFrag<bf16_t> &a, const PFrag<bf16_t> &b) {
  mma(acc, a.h, b.h);
  mma(acc, a.h, b.l);
  mma(acc, a.l, b.h);
}
__device__ __forceinline__ void mma_pp(f32x16 &acc, const PFrag<float> &a, const PFrag<float> &b) {
  mma(acc, a.v, b.v);
}

// 16 channels of one pair of z, as loaded by the row layout
template <typename T>
struct ZRow;

template <>
struct ZRow<bf16_t> {
  u32x4 v[2];
  __device__ void load(const unsigned char *p) {
    v[0] = reinterpret_cast<const u32x4 *>(p)[0];
    v[1] = reinterpret_cast<const u32x4 *>(p)[1];
  }
  __device__ void to_f32(float (&f)[kPer]) const {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * u + 2 * i] = __uint_as_float(v[u][i] << 16);
        f[8 * u + 2 * i + 1] = __uint_as_float(v[u][i] & 0xffff0000u);
      }
  }
};

template <>
struct ZRow<float> {
  f32x4 v[4];
  __device__ void load(const unsigned char *p) {
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = reinterpret_cast<const f32x4 *>(p)[u];
  }
  __device__ void to_f32(float (&f)[kPer]) const {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) f[4 * u + i] = v[u][i];
  }
};

// mean and M2 (sum of squared deviations) of 16 values
__device__ __forceinline__ float2 moments16(const float (&v)[kPer]) {
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kPer; ++c) sum += v[c];
  const float m = sum * (1.0f / kPer);
  float m2 = 0.f;
#pragma unroll
  for (int c = 0; c < kPer; ++c) { const float d = v[c] - m; m2 += d * d; }
  return make_float2(m, m2);
}

// Chan et al.'s pairwise merge of 8 equal-size (mean, M2) partials into the
// mean and 1 / sqrt(var + eps) of the 128 values.
__device__ __forceinline__ float2 merge8(const float2 (&pg)[kGroups], float eps) {
  float msum = 0.f;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) msum += pg[g].x;
  const float mean = msum * (1.0f / kGroups);
  float m2 = 0.f, dev = 0.f;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) { m2 += pg[g].y; const float d = pg[g].x - mean; dev += d * d; }
  return make_float2(mean, rsqrt_f32((m2 + kPer * dev) * (1.0f / kC) + eps));
}

template <typename T, bool kProj>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k3b_epilogue_grad(K3BArgs p) {
  constexpr int E = sizeof(T);
  constexpr bool kWeightsInRegs = (E == 2);
  using Op = OpB<T>;
  __shared__ __attribute__((aligned(16))) unsigned char n_ops[Op::BYTES];    // LN_x(x)
  __shared__ __attribute__((aligned(16))) unsigned char z_ops[Op::BYTES];    // -log2(e) LN_z(z)
  __shared__ __attribute__((aligned(16))) unsigned char dy_ops[Op::BYTES];   // dy
  __shared__ __attribute__((aligned(16))) unsigned char dt_ops[Op::BYTES];   // dt
  __shared__ __attribute__((aligned(16))) float xh_pl[kC * kPairs];          // x^ [channel][pair]
  __shared__ __attribute__((aligned(16))) float zh_pl[kC * kPairs];          // z^
  __shared__ __attribute__((aligned(16))) float dy_pl[kC * kPairs];          // dy [channel][pair]
  __shared__ __attribute__((aligned(16))) float dt_pl[kC * kPairs];          // dt
  __shared__ __attribute__((aligned(16))) float4 part_f[kGroups][kPairs];    // per-group moments of x and z
  __shared__ __attribute__((aligned(16))) float4 part_b[4][kPairs];          // per-wave LN-backward sums
  __shared__ __attribute__((aligned(16))) float ln[4][kC];                   // g_x, b_x, g_z, b_z

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = tid & (kPairs - 1);   // pair of this thread in both layouts
  const int grp = tid / kPairs;
  const int c0 = kPer * grp;          // row-layout channels c0 .. c0+15
  const int o0 = 32 * wave;           // accumulator-layout rows 32w .. +31
  const int hl = lane >> 5;           // accumulator half: rows +4 of each group of 8

  for (int i = tid; i < kC; i += kThreads) {
    ln[0][i] = p.ln_x_w[i];
    ln[1][i] = p.ln_x_b[i];
    ln[2][i] = p.ln_z_w[i];
    ln[3][i] = p.ln_z_b[i];
  }

  const T *const Wo = static_cast<const T *>(p.w_y);
  const T *const Wg = static_cast<const T *>(p.w_t);
  const T *const WoT = static_cast<const T *>(p.wt);
  const T *const WgT = WoT + kC * kC;
  // A-operand fragment at k step ks of rows 32w .. +31 of a row-major 128 x 128
  auto wptr = [&](const T *W, int ks) -> const T * { return W + (o0 + (lane & 31)) * kC + 16 * ks + 8 * hl; };
  Frag<T> wo[kWeightsInRegs ? 8 : 1], wg[kWeightsInRegs ? 8 : 1], wot[kWeightsInRegs ? 8 : 1],
      wgt[kWeightsInRegs ? 8 : 1];
  if constexpr (kWeightsInRegs) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      wo[ks].load(wptr(Wo, ks));
      wg[ks].load(wptr(Wg, ks));
      wot[ks].load(wptr(WoT, ks));
      wgt[ks].load(wptr(WgT, ks));
    }
  }

  const int64_t rows4 = (p.n_rows + 3) / 4;
  const int64_t tiles_per_blk = (p.n_cols + kCols - 1) / kCols;
  const int64_t n_tiles = rows4 * tiles_per_blk;
  const unsigned char *zbytes = static_cast<const unsigned char *>(p.z);

  // ---- per-item loads, prefetched one item ahead ---------------------------
  // Positions outside the grid read a valid stand-in pair and are treated as
  // masked; their x and dout (padding of the x layout, unspecified) never
  // reach a sum.  Projection mode takes x from z (loaded once).
  float xv[kPer];
  ZRow<T> zr;
  f32x4 dv[4];
  uint8_t mbyte = 0;
  bool valid = false;
  struct Pos {
    int64_t blk, s0;
  };
  auto advance = [&](Pos &ps) {
    ps.s0 += kCols;
    if (ps.s0 >= p.n_cols) { ps.s0 = 0; ++ps.blk; }
  };
  // global pair index of grid position (r, c)
  auto pair_of = [&](int64_t r, int64_t c) -> int64_t {
    return p.transposed ? (p.col_off + c) * p.n + p.row_off + r : (p.row_off + r) * p.n + p.col_off + c;
  };
  // x, z and the mask byte (consumed before the second barrier of an item)
  auto load_xz = [&](const Pos &ps) {
    if constexpr (!kProj) {
      const float *xp = p.x + x_offset(ps.blk * 4, ps.s0, c0, p.ldx) + q;
#pragma unroll
      for (int c = 0; c < kPer; ++c) xv[c] = xp[c * 64];
    }
    const int64_t r = ps.blk * 4 + (q & 3), col = ps.s0 + (q >> 2);
    valid = r < p.n_rows && col < p.n_cols;
    const int64_t rr = r < p.n_rows ? r : p.n_rows - 1;
    const int64_t cc = col < p.n_cols ? col : p.n_cols - 1;
    const int64_t g = pair_of(rr, cc);
    zr.load(zbytes + (g * kCz + c0) * E);
    mbyte = p.mask[g];
  };
  // dL/dout (consumed when dy and dt are formed)
  auto load_dout = [&](const Pos &ps) {
    const int64_t r = ps.blk * 4 + (q & 3), col = ps.s0 + (q >> 2);
    const int64_t rr = r < p.n_rows ? r : p.n_rows - 1;
    const int64_t cc = col < p.n_cols ? col : p.n_cols - 1;
    if constexpr (kProj) {
      // the x layout: channel o of position (r, c) at x_offset(r, c, o) (the
      // item's block exists in the buffer, padding included)
      const float *dp = p.dout + x_offset(ps.blk * 4, ps.s0, o0, p.ldx) + q;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int i = 0; i < 4; ++i) dv[g4][i] = dp[acc_row(4 * g4 + i, lane) * 64];
    } else {
      const float *dp = p.dout + (rr * p.n_cols + cc) * kCz + o0 + 4 * hl;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) dv[g4] = *reinterpret_cast<const f32x4 *>(dp + 8 * g4);
    }
  };
  auto load_item = [&](const Pos &ps) {
    load_xz(ps);
    load_dout(ps);
  };

  f32x16 G[4], H[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) { G[b][e] = 0.f; H[b][e] = 0.f; }
  // S and T of row 32w + lane % 32 over the pairs this lane's G and H
  // operand fragments cover (half of each item's pairs; the lanes l and
  // l + 32 are combined at the end)
  float s_acc = 0.f, t_acc = 0.f;

  const int64_t per_wg = (n_tiles + gridDim.x - 1) / gridDim.x;
  const int64_t tile_begin = blockIdx.x * per_wg < n_tiles ? blockIdx.x * per_wg : n_tiles;
  const int64_t tile_end = tile_begin + per_wg < n_tiles ? tile_begin + per_wg : n_tiles;
  Pos cur{tile_begin / tiles_per_blk, (tile_begin % tiles_per_blk) * kCols};
  Pos nxt = cur;
  advance(nxt);
  if (tile_begin < tile_end) load_item(cur);
  __syncthreads();   // ln[] written

  // Four barriers per item: (1) moments written; (2) operands and planes of
  // x^, z^ written; (3) dy, dt written; (4) LN-backward sums written.  Each
  // LDS array is rewritten for the next item only after a barrier that every
  // reader of its current contents has passed.
  for (int64_t tile = tile_begin; tile < tile_end; ++tile, cur = nxt, advance(nxt)) {
    const int64_t blk = cur.blk, s0 = cur.s0;
    // lane-derived indices through a value the compiler cannot see through,
    // so that LDS addresses are formed where they are used instead of being
    // held in registers across the loop
    int lane_i = lane;
    asm volatile("" : "+v"(lane_i));
    const int lane = lane_i, q = lane_i & (kPairs - 1), hl = lane_i >> 5;
    const bool in_tile = valid, keep = valid && mbyte != 0;   // (the prefetch below reloads both)

    // ---- row layout: moments of x and z over this thread's 16 channels ----
    float zf[kPer];
    zr.to_f32(zf);
    if constexpr (kProj) {
#pragma unroll
      for (int c = 0; c < kPer; ++c) xv[c] = zf[c];
    }
    {
      // (projection mode: x is z and both LayerNorms are ln_in, so every
      // quantity of the z side below equals the x side's and is not redone)
      const float2 mx = moments16(xv), mz = kProj ? mx : moments16(zf);
      part_f[grp][q] = make_float4(mx.x, mx.y, mz.x, mz.y);
    }
    __syncthreads();   // (1)
    float rx, rz;      // 1 / sqrt(var + eps) of pair q's x and z
    {
      float2 px[kGroups], pz[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const float4 v = part_f[g][q];
        px[g] = make_float2(v.x, v.y);
        pz[g] = make_float2(v.z, v.w);
      }
      const float2 sx = merge8(px, p.eps), sz = kProj ? sx : merge8(pz, p.eps);
      rx = sx.y;
      rz = sz.y;
      // normalised values; zero for pairs that are not kept, whose x may be
      // unspecified padding
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        xv[c] = keep ? (xv[c] - sx.x) * rx : 0.f;
        zf[c] = kProj ? xv[c] : (keep ? (zf[c] - sz.x) * rz : 0.f);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float fn[8], fz[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = c0 + 8 * u + i;
          fn[i] = xv[8 * u + i] * ln[0][c] + ln[1][c];
          fz[i] = kProj ? fn[i] * kNegLog2e : (zf[8 * u + i] * ln[2][c] + ln[3][c]) * kNegLog2e;
        }
        Op::put8(n_ops, q, c0 / 8 + u, fn);
        Op::put8(z_ops, q, c0 / 8 + u, fz);
      }
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        xh_pl[pl(c0 + c, q)] = xv[c];
        if constexpr (!kProj) zh_pl[pl(c0 + c, q)] = zf[c];   // projection mode reads x^ for z^
      }
    }
    __syncthreads();   // (2)
    // the next item's x, z and mask (this item's are consumed)
    if (tile + 1 < tile_end) load_xz(nxt);

    // ---- accumulator layout: recompute y and the gate --------------------
    f32x16 a0, a1;   // y = W_y n and -log2(e) t, then dn and dzh
#pragma unroll
    for (int e = 0; e < 16; ++e) { a0[e] = 0.f; a1[e] = 0.f; }
    {
      typename Op::Fr fn[2], fz[2];
      Op::read(fn[0], n_ops, q, hl);
      Op::read(fz[0], z_ops, q, hl);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks + 1 < 8) {
          Op::read(fn[(ks + 1) & 1], n_ops, q, 2 * (ks + 1) + hl);
          Op::read(fz[(ks + 1) & 1], z_ops, q, 2 * (ks + 1) + hl);
        }
        Frag<T> fo, fg;
        if constexpr (kWeightsInRegs) { fo = wo[ks]; fg = wg[ks]; }
        else { fo.load(wptr(Wo, ks)); fg.load(wptr(Wg, ks)); }
        __builtin_amdgcn_sched_barrier(0);
        Op::mma_w(a0, fo, fn[ks & 1]);
        Op::mma_w(a1, fg, fz[ks & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // dy = m s dout, dt = m y dout s (1 - s); accumulate S, T
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float fy[4], ft[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * g4 + i;
        const float s = sigmoid_of_exp2_arg(a1[e]);
        const float d = dv[g4][i];
        fy[i] = keep ? s * d : 0.f;
        ft[i] = keep ? a0[e] * d * s * (1.f - s) : 0.f;
        const int o = o0 + acc_row(e, lane);
        dy_pl[pl(o, q)] = fy[i];
        dt_pl[pl(o, q)] = ft[i];
      }
      Op::put4(dy_ops, q, o0 + 8 * g4 + 4 * hl, fy);
      Op::put4(dt_ops, q, o0 + 8 * g4 + 4 * hl, ft);
    }
    // the next item's dL/dout (this item's is consumed)
    if (tile + 1 < tile_end) load_dout(nxt);
    // projection mode: this item's rows of the global dz are read here, so
    // that the read-modify-write at the end of the item finds them in
    // registers (each pair's row is touched by one item of one launch only)
    f32x4 dz_old[4];
    if constexpr (kProj) {
      if (in_tile) {
        const float *const dzr = p.dz + pair_of(blk * 4 + (q & 3), s0 + (q >> 2)) * kCz + o0 + 4 * hl;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) dz_old[g4] = *reinterpret_cast<const f32x4 *>(dzr + 8 * g4);
      }
    }
    __syncthreads();   // (3)

    // ---- G += dy x^T, H += dt z^T over the item's 32 pairs -----------------
    // (rows 32w .. +31: this wave's own dy, dt rows; columns: all 128)
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int p0 = 16 * ps + 8 * hl;
      PFrag<T> ay, at;
      s_acc += ay.load(dy_pl, o0 + (lane & 31), p0);
      t_acc += at.load(dt_pl, o0 + (lane & 31), p0);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        PFrag<T> bx, bz;
        bx.load(xh_pl, 32 * kb + (lane & 31), p0);
        if constexpr (kProj) bz = bx;
        else bz.load(zh_pl, 32 * kb + (lane & 31), p0);
        mma_pp(G[kb], ay, bx);
        mma_pp(H[kb], at, bz);
      }
    }

    // ---- dn = W_y^T dy, dzh = W_t^T dt (rows 32w .. +31, all 32 pairs) ------
#pragma unroll
    for (int e = 0; e < 16; ++e) { a0[e] = 0.f; a1[e] = 0.f; }
    {
      typename Op::Fr fy[2], ft[2];
      Op::read(fy[0], dy_ops, q, hl);
      Op::read(ft[0], dt_ops, q, hl);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (ks + 1 < 8) {
          Op::read(fy[(ks + 1) & 1], dy_ops, q, 2 * (ks + 1) + hl);
          Op::read(ft[(ks + 1) & 1], dt_ops, q, 2 * (ks + 1) + hl);
        }
        Frag<T> fo, fg;
        if constexpr (kWeightsInRegs) { fo = wot[ks]; fg = wgt[ks]; }
        else { fo.load(wptr(WoT, ks)); fg.load(wptr(WgT, ks)); }
        __builtin_amdgcn_sched_barrier(0);
        Op::mma_w(a0, fo, fy[ks & 1]);
        Op::mma_w(a1, fg, ft[ks & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- LayerNorm backward: per-pair sums over the 128 channels of
    //      g = dn * g_x and h = dzh * g_z; g and h are kept in this wave's
    //      own rows of the dy / dt planes (read back after the barrier) -------
    {
      float sg = 0.f, sgx = 0.f, sh = 0.f, shz = 0.f;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 vo = *reinterpret_cast<const f32x4 *>(&ln[0][o0 + 8 * g4 + 4 * hl]);
        const f32x4 vi = *reinterpret_cast<const f32x4 *>(&ln[2][o0 + 8 * g4 + 4 * hl]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g4 + i;
          const int k = o0 + acc_row(e, lane);
          const float g = a0[e] * vo[i], h = a1[e] * vi[i];
          if constexpr (kProj) {
            // one LayerNorm: only g + h and its sums are needed
            const float gh = g + h;
            sg += gh;
            sgx += gh * xh_pl[pl(k, q)];
            dy_pl[pl(k, q)] = gh;
          } else {
            sg += g;
            sgx += g * xh_pl[pl(k, q)];
            sh += h;
            shz += h * zh_pl[pl(k, q)];
            dy_pl[pl(k, q)] = g;
            dt_pl[pl(k, q)] = h;
          }
        }
      }
      sg += __shfl_xor(sg, 32, 64);
      sgx += __shfl_xor(sgx, 32, 64);
      sh += __shfl_xor(sh, 32, 64);
      shz += __shfl_xor(shz, 32, 64);
      if (hl == 0) part_b[wave][q] = make_float4(sg, sgx, sh, shz);
    }
    __syncthreads();   // (4)
    if (in_tile) {
      float4 t = part_b[0][q];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 v = part_b[w][q];
        t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
      }
      const float mg = t.x * (1.0f / kC), mgx = t.y * (1.0f / kC);
      const float mh = t.z * (1.0f / kC), mhz = t.w * (1.0f / kC);
      const int64_t r = blk * 4 + (q & 3), col = s0 + (q >> 2);
      if constexpr (kProj) {
        // one LayerNorm (x = z): dz = r (g + h - mean(g + h) - z^ mean((g + h) z^)),
        // added to the pair's row of the global dz (g + h and its sums sit in
        // the dy plane and in mg, mgx; mh = mhz = 0)
        float *const dzrow = p.dz + pair_of(r, col) * kCz + o0 + 4 * hl;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 vz = dz_old[g4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = o0 + acc_row(4 * g4 + i, lane);
            const float v = rz * (dy_pl[pl(k, q)] - mg - xh_pl[pl(k, q)] * mgx);
            vz[i] += keep ? v : 0.f;
          }
          *reinterpret_cast<f32x4 *>(dzrow + 8 * g4) = vz;
        }
      } else {
        float *const dzrow = p.dz + (r * p.n_cols + col) * kCz + o0 + 4 * hl;
        float *const dxp = p.dx + x_offset(blk * 4, s0, o0, p.ldx) + q;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 vz;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * g4 + i;
            const int k = o0 + acc_row(e, lane);
            // masked pairs: every term is zero (dn = dzh = 0, x^ = z^ = 0)
            const float dxv = rx * (dy_pl[pl(k, q)] - mg - xh_pl[pl(k, q)] * mgx);
            const float dzv = rz * (dt_pl[pl(k, q)] - mh - zh_pl[pl(k, q)] * mhz);
            dxp[acc_row(e, lane) * 64] = keep ? dxv : 0.f;
            vz[i] = keep ? dzv : 0.f;
          }
          *reinterpret_cast<f32x4 *>(dzrow + 8 * g4) = vz;
        }
      }
    }
  }

  // ---- this work-group's partial sums -> its slot ---------------------------
  float *const slot = p.part + (int64_t)blockIdx.x * kK3BSlotFloats;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int o = o0 + acc_row(e, lane);
      slot[o * kC + 32 * kb + (lane & 31)] = G[kb][e];
      slot[kC * kC + o * kC + 32 * kb + (lane & 31)] = H[kb][e];
    }
  s_acc += __shfl_xor(s_acc, 32, 64);
  t_acc += __shfl_xor(t_acc, 32, 64);
  if (hl == 0) {
    slot[2 * kC * kC + o0 + lane] = s_acc;
    slot[2 * kC * kC + kC + o0 + lane] = t_acc;
  }
}

// W^T of the two matrices into the workspace (element type kept).
template <typename T>
__global__ __launch_bounds__(256) void k3b_transpose(const T *wy, const T *wt_, T *wt) {
  const T *src = blockIdx.x == 0 ? wy : wt_;
  T *dst = wt + blockIdx.x * kC * kC;
  for (int i = threadIdx.x; i < kC * kC; i += 256) {
    const int o = i / kC, k = i % kC;
    dst[k * kC + o] = src[i];
  }
}

// Sum of the slots (fixed order) and the weight-matrix gradients
//   dW_y = G diag(g_x) + S b_x^T,  dW_t = H diag(g_z) + T b_z^T.
// Work-group (m, o): row o of G (m = 0) or H (m = 1); thread k: column k.
__global__ __launch_bounds__(kC) void k3b_reduce(K3BArgs p) {
  const int m = blockIdx.x / kC, o = blockIdx.x % kC, k = threadIdx.x;
  const float *src = p.part + m * kC * kC + o * kC + k;
  float acc = 0.f, sv = 0.f;
  for (int s = 0; s < p.n_parts; ++s) {
    acc += src[(int64_t)s * kK3BSlotFloats];
    sv += p.part[(int64_t)s * kK3BSlotFloats + 2 * kC * kC + m * kC + o];
  }
  p.tot[m * kC * kC + o * kC + k] = acc;
  if (k == 0) p.tot[2 * kC * kC + m * kC + o] = sv;
  const float *gam = m == 0 ? p.ln_x_w : p.ln_z_w;
  const float *bet = m == 0 ? p.ln_x_b : p.ln_z_b;
  float *dw = m == 0 ? p.g_w_y : p.g_w_t;
  const float v = acc * gam[k] + sv * bet[k];
  dw[o * kC + k] = p.grad_accumulate ? dw[o * kC + k] + v : v;
}

// LayerNorm parameter gradients: dgamma[k] = sum_o W[o][k] G[o][k],
// dbeta[k] = sum_o W[o][k] S[o] (W_y with G, S for LN_x; W_t with H, T for
// LN_z).  Epilogue mode: work-group m = 0 writes LN_x's, m = 1 LN_z's.
// Projection mode (LN_x = LN_z): one work-group writes the sum of both.
template <typename T>
__device__ __forceinline__ float elt(const T *w, int i);
template <>
__device__ __forceinline__ float elt<bf16_t>(const bf16_t *w, int i) { return bf16_to_f32(w[i].v); }
template <>
__device__ __forceinline__ float elt<float>(const float *w, int i) { return w[i]; }

template <typename T>
__device__ __forceinline__ void ln_sums(const K3BArgs &p, int m, int k, float &dg, float &db) {
  const T *W = static_cast<const T *>(m == 0 ? p.w_y : p.w_t);
  const float *Gt = p.tot + m * kC * kC;
  const float *St = p.tot + 2 * kC * kC + m * kC;
  for (int o = 0; o < kC; ++o) {
    const float w = elt<T>(W, o * kC + k);
    dg += w * Gt[o * kC + k];
    db += w * St[o];
  }
}

template <typename T, bool kProj>
__global__ __launch_bounds__(kC) void k3b_ln_grads(K3BArgs p) {
  const int m = blockIdx.x, k = threadIdx.x;
  float dg = 0.f, db = 0.f;
  ln_sums<T>(p, m, k, dg, db);
  if constexpr (kProj) ln_sums<T>(p, 1, k, dg, db);
  float *gw = (m == 0 && !kProj) ? p.g_ln_x_w : p.g_ln_z_w;
  float *gb = (m == 0 && !kProj) ? p.g_ln_x_b : p.g_ln_z_b;
  gw[k] = p.ln_accumulate ? gw[k] + dg : dg;
  gb[k] = p.ln_accumulate ? gb[k] + db : db;
}

template <typename T, bool kProj>
void launch_all(const K3BArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k3b_transpose<T>, dim3(2), dim3(256), 0, s, static_cast<const T *>(a.w_y),
                     static_cast<const T *>(a.w_t), static_cast<T *>(a.wt));
  hipLaunchKernelGGL((k3b_epilogue_grad<T, kProj>), dim3(a.n_parts), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(k3b_reduce, dim3(2 * kC), dim3(kC), 0, s, a);
  hipLaunchKernelGGL((k3b_ln_grads<T, kProj>), dim3(kProj ? 1 : 2), dim3(kC), 0, s, a);
}

}  // namespace

hipError_t launch_k3b(K3BArgs a, int dtype, bool projection, hipStream_t s) {
  const int64_t n_tiles = ((a.n_rows + 3) / 4) * ((a.n_cols + kCols - 1) / kCols);
  const int64_t slots = device_cu_count() < kK3BMaxParts ? device_cu_count() : kK3BMaxParts;
  a.n_parts = (int32_t)(n_tiles < slots ? (n_tiles > 0 ? n_tiles : 1) : slots);
  if (dtype == TRIMUL_BF16) {
    if (projection) launch_all<bf16_t, true>(a, s);
    else launch_all<bf16_t, false>(a, s);
  } else {
    if (projection) launch_all<float, true>(a, s);
    else launch_all<float, false>(a, s);
  }
  return hipGetLastError();
}

}  // namespace trimul
