// KA: window-batched sequence-local atom attention (page 1, section "Atom
// sequence local attention eficiente": AlphaFold3 restricts atom attention to
// local windows of 32 x 128, processed as a batch of windows).
//
// Query block w = atoms 32w .. 32w+31 attends to the 128 atoms centred on it,
// keys 32w - 48 .. 32w + 79 (those inside the sequence and not masked); per
// head, o_i = softmax_j(scale q_i.k_j + bias_ij) v_j, o_i = 0 when no key is
// left.  q, k, v are bf16 [batch][n][heads][32]; bias bf16
// [batch][windows][heads][32][128] (optional); out fp32 [batch][n][heads][32].
//
// Work-group = one (sequence, window), 4 waves; wave v takes heads v, v+4, ...
// (two waves per SIMD: the register budget is held to 256 per lane).  Per
// head, all global loads (Q, K, the bias row, V) are issued before any use, so
// a head costs one memory round trip; the first head's are issued together
// with the window's key-mask bytes, ahead of the barrier that publishes the
// key flags, so a work-group with one head per wave waits for memory once.
// Per head, on the matrix cores (bf16 32x32x16, fp32 accumulation):
//  - S^T = K Q^T for the 4 key blocks of 32: lane l holds query l % 32 and 16
//    keys of each block, so a query's 128 logits sit in two lanes (l, l ^ 32):
//    the softmax needs an in-lane reduction plus one lane swap;
//    Rows of a key block stand for permuted keys (kperm) so that lane (q, half)
//    holds keys 16 half .. +15 of each block;
//  - O = P V with the normalised probabilities as A operand straight from the
//    S^T registers: key block b, step s takes accumulator registers 8s .. 8s+7
//    of lane (q, half), i.e. keys 32b + 16 half + 8s .. +7; the B operand reads
//    the same keys of V from a transposed per-wave LDS copy (one 16-byte
//    read; the copy is written four keys of one dimension per 8-byte store).  P is
//    split into hi + lo bf16 terms (two products per step), so the output
//    keeps about 16 significant bits of P.
// Key validity (inside the sequence and unmasked) is computed once per
// work-group into LDS.  Keys outside the sequence read a clamped row (finite
// values) and get probability 0.
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kQ = 32;          // queries per window
constexpr int kK = 128;         // keys per window
constexpr int kKOff = -48;      // first key relative to 32w
constexpr int kD = 32;          // head dimension
constexpr int kWaves = 4;
constexpr int kVtStride = kK + 8;   // LDS row of V^T (bf16 elements): 272 bytes, spreads the d rows over banks

__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void ka_window_attention(KAArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kWaves][kD * kVtStride];   // V^T per wave: [d][key]
  __shared__ uint8_t key_ok[kK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wg = blockIdx.x;
  const int64_t b = wg / p.n_windows, w = wg % p.n_windows;
  const int64_t key0 = kQ * w + kKOff;
  const int q = lane & 31, hl = lane >> 5;
  const int64_t n = p.n_atoms;

  const bf16_t *Q = static_cast<const bf16_t *>(p.q);
  const bf16_t *Kp = static_cast<const bf16_t *>(p.k);
  const bf16_t *V = static_cast<const bf16_t *>(p.v);
  const bf16_t *Bias = static_cast<const bf16_t *>(p.bias);
  const int64_t H = p.heads;
  // element offset of (atom j, head h, dim 0) of sequence b
  auto row = [&](int64_t j, int64_t h) -> int64_t { return ((b * n + j) * H + h) * kD; };
  auto clampj = [&](int64_t j) -> int64_t { return j < 0 ? 0 : (j >= n ? n - 1 : j); };
  const float kLog2e = 1.4426950408889634f;
  const float sl = p.scale * kLog2e;
  uint16_t *const myvt = vt[wave];

  // A head's operands in registers: Q (B operand over d), K (A operand, 4
  // key blocks), this lane's bias row pieces, and V rows for the LDS copy.
  Frag<bf16_t> qf[2], kf[4][2];
  u32x4 braw[4][2];   // keys 32 bb + 16 hl + 8 j .. +7 of this lane's query
  u32x4 vraw[kK / 16];
  auto load_head = [&](int64_t h) {
    // The lane index passes through an opaque copy, so the lane-dependent
    // addresses are recomputed per head instead of being kept live across
    // the head loop (which would exceed the register budget).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lq = ln & 31, lh = ln >> 5;
    // Row r of a 32-key block of S^T stands for key kperm(r) = 16 ((r >> 2) & 1)
    // + 4 (r >> 3) + (r & 3): the 16 rows a lane holds (acc_row(e, l),
    // e = 0..15) are then keys 16 (l / 32) + e, so the lane's bias, key flags
    // and V operands are contiguous runs.
    const int kperm = 16 * ((lq >> 2) & 1) + 4 * (lq >> 3) + (lq & 3);
    const int64_t qi = kQ * w + lq;
    const int64_t qrow = row(qi < n ? qi : n - 1, h);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[ks].load(Q + qrow + 16 * ks + 8 * lh);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int64_t krow = row(clampj(key0 + 32 * bb + kperm), h);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) kf[bb][ks].load(Kp + krow + 16 * ks + 8 * lh);
    }
    const bf16_t *brow = Bias ? Bias + (((b * p.n_windows + w) * H + h) * kQ + lq) * kK : nullptr;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        braw[bb][j] = brow ? *reinterpret_cast<const u32x4 *>(brow + 32 * bb + 16 * lh + 8 * j) : u32x4{0u, 0u, 0u, 0u};
    // V: lane -> keys 64 (it / 4) + 4 (l / 4) + it % 4, dims 8 (l % 4) .. +7
#pragma unroll
    for (int it = 0; it < kK / 16; ++it)
      vraw[it] = *reinterpret_cast<const u32x4 *>(
          V + row(clampj(key0 + 64 * (it >> 2) + 4 * (ln >> 2) + (it & 3)), h) + 8 * (ln & 3));
  };

  // Key flags (inside the sequence and unmasked), once per work-group.  The
  // mask bytes are requested first and the first head's operands right after,
  // so both arrive within one memory round trip.
  bool jin = false;
  uint8_t mbyte = 1;
  if (threadIdx.x < kK) {
    const int64_t j = key0 + threadIdx.x;
    jin = j >= 0 && j < n;
    if (jin && p.mask) mbyte = p.mask[b * n + j];
  }
  if (wave < H) load_head(wave);
  if (threadIdx.x < kK) key_ok[threadIdx.x] = (jin && mbyte != 0) ? 1 : 0;
  __syncthreads();

  // Each wave owns its V^T copy, so no work-group barrier is needed inside the
  // loop: the wave's LDS operations execute in order, and compiler barriers
  // keep the copy's writes before its reads and this head's reads before the
  // next head's writes.  All global loads of a head are issued first.
  for (int64_t h = wave; h < H; h += kWaves) {
    // ---- loads (the first head's were issued before the key-flag barrier)
    if (h != wave) load_head(h);
    // ---- V^T of the window into LDS
    asm volatile("" ::: "memory");   // the previous head's V^T reads stay before these writes
    // (four consecutive keys of one dimension per 8-byte store)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int t = 64 * half + 4 * (lane >> 2), c = lane & 3;
      const u32x4 *v4 = vraw + 4 * half;   // keys t .. t+3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
        const u32x2 even{(v4[0][i] & 0xffffu) | (v4[1][i] << 16), (v4[2][i] & 0xffffu) | (v4[3][i] << 16)};
        const u32x2 odd{(v4[0][i] >> 16) | (v4[1][i] & 0xffff0000u), (v4[2][i] >> 16) | (v4[3][i] & 0xffff0000u)};
        *reinterpret_cast<u32x2 *>(myvt + (8 * c + 2 * i) * kVtStride + t) = even;
        *reinterpret_cast<u32x2 *>(myvt + (8 * c + 2 * i + 1) * kVtStride + t) = odd;
      }
    }
    asm volatile("" ::: "memory");   // the writes stay before the reads below
    // ---- S^T = K Q^T: 4 key blocks x 2 steps over d ------------------------
    f32x16 s[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[bb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) mma(s[bb], kf[bb][ks], qf[ks]);
    }
    // ---- logits (base-2 units), masked keys -> -inf; row max over 128 keys ---
    float mx = -__builtin_inff();
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 32 * bb + 16 * hl + e;   // key of register e (see kperm)
        const uint32_t word = braw[bb][e >> 3][(e & 7) >> 1];
        const float bv = __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
        const float l2 = key_ok[t] ? s[bb][e] * sl + bv * kLog2e : -__builtin_inff();
        s[bb][e] = l2;
        mx = fmaxf(mx, l2);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // ---- probabilities; a query with no key gets p = 0 ---------------------
    float sum = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = mx == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(s[bb][e] - mx);
        s[bb][e] = pe;
        sum += pe;
      }
    sum += __shfl_xor(sum, 32, 64);
    const float inv = sum > 0.f ? 1.0f / sum : 0.f;
    // ---- O = P V over 8 steps of 16 keys (P split into hi + lo) -------------
    f32x16 o;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 hh, ll;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float f0 = s[bb][8 * st + 2 * i] * inv, f1 = s[bb][8 * st + 2 * i + 1] * inv;
          hh[i] = pack_bf16x2(f0, f1);
          ll[i] = pack_bf16x2(f0 - __uint_as_float(hh[i] << 16), f1 - __uint_as_float(hh[i] & 0xffff0000u));
        }
        Frag<bf16_t> ph, pl, vf;
        ph.v = __builtin_bit_cast(bf16x8, hh);
        pl.v = __builtin_bit_cast(bf16x8, ll);
        // V at keys 32bb + 16hl + 8st .. +7 (registers 8st .. 8st+7 of the A
        // lanes with this half), dim q (this lane's column)
        vf.v = *reinterpret_cast<const bf16x8 *>(myvt + q * kVtStride + 32 * bb + 16 * hl + 8 * st);
        mma(o, ph, vf);
        mma(o, pl, vf);
      }
    // ---- out[b][32w + row][h][d = lane % 32] ---------------------------------
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t oi = kQ * w + acc_row(e, lane);
      if (oi < n) p.out[((b * n + oi) * H + h) * kD + q] = o[e];
    }
  }
}

}  // namespace

hipError_t launch_ka(const KAArgs &a, hipStream_t s) {
  const int64_t grid = a.batch * a.n_windows;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(ka_window_attention, dim3((unsigned)grid), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace trimul
