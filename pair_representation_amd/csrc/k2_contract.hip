// K2: the channel-batched k-contraction
//     x[d][i][j] (+)= sum over chunks, sum_t  a[d][i][t] * b[d][j][t]
// which is  x_ij = sum_k a_ik * b_jk  for outgoing operands and
// x_ij = sum_k a_ki * b_kj  for the transposed incoming operands.  Per channel
// d this is one "NT" matrix product (both operands k-contiguous).
//
// Work-group tile BM x BN of one channel, four waves in a 2 x 2 layout, each
// wave a (BM/2) x (BN/2) block of 32 x 32 matrix-core accumulators.  The
// k-loop walks the chunks in the order given (a ring's delivery order) and,
// inside each chunk, BK-wide k-tiles.  Global -> register -> LDS staging is
// double-buffered: the loads of k-tile t+1 are in flight while k-tile t is on
// the matrix cores, with one barrier per k-tile.  LDS rows are XOR-swizzled in
// 16-byte units so the k-fragment reads of 32 consecutive rows are free of
// bank conflicts.  Partial sums stay in registers across all chunks; the
// result is written (or added) once.
//
// Tile order: blocks are dealt round-robin to the 8 XCDs, so the linear block
// id is remapped so that each XCD receives a contiguous range of logical
// tiles; inside a channel, tiles go in groups of kGroupM tile-rows so that the
// concurrently running tiles of one XCD share operand panels in its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace trimul {

namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

template <typename T, int BM, int BN, int BK>
struct K2Cfg {
  static constexpr int E = sizeof(T);
  static constexpr int ROWB = BK * E;          // bytes per LDS row
  static constexpr int RU = ROWB / 16;         // 16-byte units per row
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MT = WM / 32, NT = WN / 32;
  static constexpr int KS = BK / 16;           // 16-wide k steps per k-tile
  static constexpr int UPF = Frag<T>::kBytes / 16;  // units per fragment
  static constexpr int A_LD = BM * RU / kThreads;   // 16-byte loads per thread
  static constexpr int B_LD = BN * RU / kThreads;
  static constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(RU == 8, "LDS rows are 8 units wide");
  static_assert(A_LD * kThreads == BM * RU && B_LD * kThreads == BN * RU, "load split");
};

template <typename T>
__device__ __forceinline__ void lds_frag(Frag<T> &f, const unsigned char *row_base, int row, int g) {
  constexpr int UPF = Frag<T>::kBytes / 16;
  u32x4 *dst = reinterpret_cast<u32x4 *>(&f);
#pragma unroll
  for (int u = 0; u < UPF; ++u)
    dst[u] = *reinterpret_cast<const u32x4 *>(row_base + swz<8>(row, g * UPF + u) * 16);
}

template <typename T, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads) void k2_contract(K2Args p) {
  using C = K2Cfg<T, BM, BN, BK>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- block -> (channel, tile row, tile col) --------------------------
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t per_ch = tiles_m * tiles_n;
  const int64_t total = per_ch * kC;
  const int64_t per_xcd = gridDim.x / kXcds;            // grid is a multiple of kXcds
  const int64_t logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (logical >= total) return;
  const int64_t d = logical / per_ch;
  const int64_t t = logical % per_ch;
  const int64_t group = t / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int64_t tm = first_m + (t % gm);
  const int64_t tn = (t % (kGroupM * tiles_n)) / gm;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  // ---- staged loads ---------------------------------------------------
  u32x4 ra[C::A_LD], rb[C::B_LD];
  auto gload = [&](int ci, int kt) {
    const int64_t ld = p.ch[ci].ld;
    const unsigned char *A = static_cast<const unsigned char *>(p.ch[ci].a) + d * p.M * ld * C::E;
    const unsigned char *B = static_cast<const unsigned char *>(p.ch[ci].b) + d * p.N * ld * C::E;
    const int64_t kb = (int64_t)kt * BK * C::E;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int u = i * kThreads + tid;
      const int row = u / C::RU, unit = u % C::RU;
      int64_t g = m0 + row;
      g = g < p.M ? g : p.M - 1;
      ra[i] = *reinterpret_cast<const u32x4 *>(A + g * ld * C::E + kb + unit * 16);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int u = i * kThreads + tid;
      const int row = u / C::RU, unit = u % C::RU;
      int64_t g = n0 + row;
      g = g < p.N ? g : p.N - 1;
      rb[i] = *reinterpret_cast<const u32x4 *>(B + g * ld * C::E + kb + unit * 16);
    }
  };
  auto lstore = [&](int buf) {
    unsigned char *sa = lds + buf * C::STAGE;
    unsigned char *sb = sa + BM * C::ROWB;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int u = i * kThreads + tid;
      const int row = u / C::RU, unit = u % C::RU;
      *reinterpret_cast<u32x4 *>(sa + row * C::ROWB + swz<8>(row, unit) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int u = i * kThreads + tid;
      const int row = u / C::RU, unit = u % C::RU;
      *reinterpret_cast<u32x4 *>(sb + row * C::ROWB + swz<8>(row, unit) * 16) = rb[i];
    }
  };

  f32x16 acc[C::MT][C::NT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.f;

  int total_kt = 0;
  for (int c = 0; c < p.n_chunks; ++c) total_kt += p.ch[c].ktiles;

  int ci = 0, kt = 0;  // position of the next k-tile to load
  auto advance = [&]() {
    if (++kt == p.ch[ci].ktiles) { ++ci; kt = 0; }
  };

  if (total_kt > 0) {
    gload(ci, kt);
    advance();
    lstore(0);
    __syncthreads();
  }

  for (int it = 0; it < total_kt; ++it) {
    const int buf = it & 1;
    const bool has_next = it + 1 < total_kt;
    if (has_next) gload(ci, kt);

    const unsigned char *sa = lds + buf * C::STAGE;
    const unsigned char *sb = sa + BM * C::ROWB;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int g = 2 * ks + (lane >> 5);  // 8-element group of this lane
      Frag<T> af[C::MT], bfr[C::NT];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const int row = wm * C::WM + mt * 32 + (lane & 31);
        lds_frag(af[mt], sa + row * C::ROWB, row, g);
      }
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        const int row = wn * C::WN + nt * 32 + (lane & 31);
        lds_frag(bfr[nt], sb + row * C::ROWB, row, g);
      }
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) mma(acc[mt][nt], af[mt], bfr[nt]);
    }

    if (has_next) {
      lstore(buf ^ 1);
      advance();
    }
    __syncthreads();
  }

  // ---- write / accumulate x -------------------------------------------
  float *X = p.x + d * p.M * p.ldx;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const int64_t col = n0 + wn * C::WN + nt * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * C::WM + mt * 32 + acc_row(e, lane);
        if (row < p.M && col < p.N) {
          float *dst = X + row * p.ldx + col;
          *dst = p.accumulate ? *dst + acc[mt][nt][e] : acc[mt][nt][e];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_k2(K2Args a, int dtype, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const int64_t bk = (dtype == TRIMUL_BF16) ? 64 : 32;
  const int64_t bm = (dtype == TRIMUL_BF16) ? 256 : 128;
  for (int c = 0; c < a.n_chunks; ++c) a.ch[c].ktiles = (int32_t)((a.ch[c].k_len + bk - 1) / bk);
  const int64_t tiles = ((a.M + bm - 1) / bm) * ((a.N + bm - 1) / bm) * kC;
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  if (dtype == TRIMUL_BF16)
    hipLaunchKernelGGL((k2_contract<bf16_t, 256, 256, 64>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k2_contract<float, 128, 128, 32>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace trimul
