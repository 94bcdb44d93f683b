// K2: the channel-batched k-contraction
//     x[d][i][j] (+)= sum over chunks, sum_t  a[d][i][t] * b[d][j][t]
// which is  x_ij = sum_k a_ik * b_jk  for outgoing operands and
// x_ij = sum_k a_ki * b_kj  for the transposed incoming operands.  Per channel
// d this is one "NT" matrix product (both operands k-contiguous).
//
// Work-group tile BM x BN of one channel, eight waves (two per SIMD) in a
// 2 x 4 layout, each wave a (BM/2) x (BN/4) block of 32 x 32 matrix-core
// accumulators; the two waves of a SIMD hide each other's LDS and barrier
// latency.  bf16: 256 x 384 x 64 (wave tile 128 x 96: 192 accumulator
// registers, two 80 KB LDS stages) or, when 384-wide tiles would pad much
// more of N, 256 x 256 x 64 (chosen per launch); fp32: 128 x 128 x 32.  The
// k-loop walks the chunks in the order given (a ring's delivery order) and,
// inside each chunk, BK-wide k-tiles.
//
// Operand staging: buffer loads that write LDS directly (no register
// staging), two LDS stages, one barrier per k-tile: the loads of k-tile t+1
// are in flight while k-tile t is on the matrix cores.  One wave per SIMD
// issues them.  Each load instruction fills 1 KB of LDS (64 lanes x 16 bytes
// at consecutive addresses), so the XOR swizzle of 16-byte units inside a row
// (unit u of row r stored at u ^ ((r / 2) % 8)) is applied on the global
// side: a lane fetches the logical unit that belongs in its LDS slot.  In the
// operand layout (see operand_offset) a k-tile of one channel is a contiguous
// 32 KB run per 256-row block; rows past the operand's end are padding rows
// of the last block and only feed output rows/columns that are never stored
// (in edge tiles, whole 32-row blocks of padding are skipped and the valid
// blocks are spread evenly over the waves).  k-fragments are read from LDS
// ahead of the matrix-core instructions that consume them: a whole 16-wide k
// step ahead (two register sets) for wave tiles of up to 8 blocks; for
// 128 x 96 wave tiles the A fragments are single-buffered, each re-read for
// the next step as soon as the products of the current step that use it have
// been issued.
//
// Tile order: blocks are dealt round-robin to the 8 XCDs, so the linear block
// id is remapped so that each XCD receives a contiguous range of logical
// tiles; inside a channel, tiles go in groups of group_m tile-rows so that the
// concurrently running tiles of one XCD share operand panels in its L2.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace trimul {

namespace {

constexpr int kThreads = 512;
constexpr int kLoadWaves = 4;   // waves that issue the operand loads (one per SIMD)
constexpr int kXcds = 8;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) void lds_void;

template <typename T, int BM, int BN, int BK>
struct K2Cfg {
  static constexpr int E = sizeof(T);
  static constexpr int ROWB = BK * E;          // bytes per LDS row
  static constexpr int RU = ROWB / 16;         // 16-byte units per row
  static constexpr int WM = BM / 2, WN = BN / 4;
  static_assert(kOpRows % 8 == 0 && BM <= kOpRows, "an A tile lies in one 256-row block");
  static_assert(BN <= 2 * kOpRows, "a B tile spans at most two 256-row blocks");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "tiles start at row 0 or 128 of a 256-row block");
  static_assert(kLoadWaves * 8 == 32, "load instruction i covers rows 32*i + 8*wave .. +7");
  static constexpr int MT = WM / 32, NT = WN / 32;
  static constexpr int KS = BK / 16;           // 16-wide k steps per k-tile
  static constexpr int A_I = BM * RU / (64 * kLoadWaves);   // 1 KB load instructions per loading wave (A)
  static constexpr int B_I = BN * RU / (64 * kLoadWaves);
  static constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(RU == 8, "LDS rows are 8 units wide");
  static_assert(A_I * 64 * kLoadWaves == BM * RU && B_I * 64 * kLoadWaves == BN * RU, "load split");
};

// Physical 16-byte unit of logical unit u in LDS row r.  A 128-byte row is
// half of the 256-byte window the 64 LDS banks cover, and a 16-byte-per-lane
// read serves 16 lanes per cycle: 16 consecutive rows at one logical unit
// must land on 16 distinct (row parity, unit) slots, hence the XOR with
// (r / 2) % 8 rather than r % 8.
__device__ __forceinline__ int k2_swz(int row, int unit) { return unit ^ ((row >> 1) & 7); }

template <typename T>
__device__ __forceinline__ void lds_frag(Frag<T> &f, const unsigned char *row_base, int row, int g) {
  constexpr int UPF = Frag<T>::kBytes / 16;
  u32x4 *dst = reinterpret_cast<u32x4 *>(&f);
#pragma unroll
  for (int u = 0; u < UPF; ++u)
    dst[u] = *reinterpret_cast<const u32x4 *>(row_base + k2_swz(row, g * UPF + u) * 16);
}

// Share of wave w (of `waves` along one side of the tile) in the 32-wide
// blocks of a tile that hold at least one valid row, given `valid` rows from
// the tile's start: a full tile gives every wave its own cap blocks; a tile
// at the ragged edge spreads its valid blocks as evenly as possible, so the
// busiest wave has as few as possible.  Returns the first block and the
// count (0 .. cap).
__device__ __forceinline__ void block_share(int valid, int cap, int waves, int w, int &first, int &count) {
  const int nb = valid >= cap * waves * 32 ? cap * waves : (valid + 31) / 32;
  const int per = nb / waves, extra = nb % waves;
  count = per + (w < extra ? 1 : 0);
  first = w * per + (w < extra ? w : extra);
}

// Rows of a tile covered by 32-row blocks that hold a valid row: valid rows
// rounded up to 32, at most cap.
__device__ __forceinline__ int row_extent(int valid, int cap) {
  const int r = (valid + 31) / 32 * 32;
  return r < cap ? r : cap;
}

__device__ __forceinline__ void wait_vm0() {
  // s_waitcnt vmcnt(0), other counters unconstrained
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <typename T, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads) void k2_contract(K2Args p) {
  using C = K2Cfg<T, BM, BN, BK>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (scalar): the per-instruction load descriptors derived from
  // it must live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  // ---- block -> (channel, tile row, tile col) --------------------------
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int per_ch = tiles_m * tiles_n;
  const int total = per_ch * kC;
  // Blocks are dispatched in order, round-robin over the XCDs, about
  // p.slots at a time (one per CU).  Block b of dispatch round s = b / slots
  // runs on XCD x = (b % slots) % 8; give that XCD the contiguous logical
  // tiles s*slots + x*(slots/8) + .., so each round works on ~one channel
  // (its operands stay in the shared last-level cache) and each XCD on a
  // compact group_m x 8 block of it (operand panels shared in its L2).
  const int slots = p.slots;
  const int round = blockIdx.x / slots;
  const int pos = blockIdx.x - round * slots;
  const int logical = round * slots + (pos % kXcds) * (slots / kXcds) + pos / kXcds;
  if (logical >= total) return;
  const int d = logical / per_ch;
  const int t = logical - d * per_ch;
  const int group_m = p.group_m;
  const int group = t / (group_m * tiles_n);
  const int first_m = group * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int tm = first_m + (t % gm);
  const int tn = (t % (group_m * tiles_n)) / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- direct-to-LDS loads --------------------------------------------
  // Only waves 0 .. kLoadWaves-1 (one per SIMD) issue loads: a wave stalls
  // while the texture path accepts its load instructions, and the other wave
  // of its SIMD keeps the matrix core busy meanwhile.  Load instruction i of
  // a loading wave fills LDS block q = i*kLoadWaves + wave (1 KB = 8 rows of
  // 128 bytes); lane l fills row q*8 + l/8, physical unit l%8, which holds
  // logical unit k2_swz(row, l%8) (the swizzle is an involution).
  const int lrow = lane >> 3;
  // Lane part of every load offset: row lrow of the 8-row group, logical
  // unit k2_swz(q*8 + lrow, lane % 8).  With q = i*kLoadWaves + wave and
  // kLoadWaves even, (q*8 + lrow)/2 % 8 = 4*(wave % 2) + lrow/2: the unit is
  // the same for every load instruction of a wave, and the rest of the
  // offset (row group, k) is wave-uniform (the scalar offset).
  static_assert(kLoadWaves % 2 == 0, "load groups of one wave share a swizzle");
  const int lane_off = lrow * kOpCols * (int)sizeof(T) + (((lane & 7) ^ (4 * (wave & 1) + (lrow >> 1))) * 16);
  // operand rows of this tile that any product uses: up to the end of the
  // last 32-row block holding a valid row (see the edge-tile skipping below)
  const int a_rows = row_extent((int)(p.M - m0), BM);
  const int b_rows = row_extent((int)(p.N - n0), BN);
  // The chunk whose k-tiles are being loaded, kept in registers: this
  // tile's operand blocks at the chunk's first k-tile, the distance between
  // 256-row blocks and the chunk's k-tile count.  Refreshed from the kernel
  // arguments only when the next chunk starts, so the k-loop issues no
  // scalar memory loads (which would also make every LDS wait a full one).
  const unsigned char *a_chunk = nullptr, *b_chunk = nullptr;
  int64_t blk_step = 0;
  int chunk_kt = 0;
  auto set_chunk = [&](int ci) __attribute__((always_inline)) {
    const K2Chunk &ch = p.ch[ci];
    const int64_t col_blocks = (int64_t)((uint64_t)ch.ld / kOpCols);   // ld: a positive multiple of 64
    blk_step = col_blocks * kC * kOpBlock * C::E;
    a_chunk = static_cast<const unsigned char *>(ch.a) +
              ((int64_t)(m0 / kOpRows) * col_blocks * kC + d) * kOpBlock * C::E;
    b_chunk = static_cast<const unsigned char *>(ch.b) +
              ((int64_t)(n0 / kOpRows) * col_blocks * kC + d) * kOpBlock * C::E;
    chunk_kt = ch.ktiles;
  };
  // Loads of k-tile kt of the current chunk into LDS stage buf.  With
  // `full` (every row of both operand tiles valid) no load is tested.
  auto issue_loads = [&](int kt, int buf, auto full) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full)::value;
    if (wave >= kLoadWaves) return;
    // The k-tile is one contiguous run of one channel block of each operand
    // (256 rows x 64 columns per block; a BK-wide k-tile is columns kk ..
    // kk+BK-1 of it, rows m0 % 256 ..); channel blocks of consecutive column
    // blocks are kC blocks apart.
    const int kcol = kt * BK;
    const int64_t cb_off = (int64_t)(kcol / kOpCols) * kC * kOpBlock * C::E;
    const int kk = kcol % kOpCols;
    // An A tile lies in one 256-row block; a B tile (384 rows) in at most
    // two consecutive ones.  Each 8-row load group lies in one block and is
    // addressed through that block's own buffer descriptor.
    const unsigned char *A = a_chunk + cb_off;
    const unsigned char *B = b_chunk + cb_off;
    unsigned char *sa = lds + buf * C::STAGE;
    unsigned char *sb = sa + BM * C::ROWB;
    // Load instruction i of this wave covers tile rows 32*i + 8*wave .. +7,
    // i.e. rows r0 + 32*i + 8*wave of the first block: with r0 (the tile's
    // first row inside its block, 0 or 128) a compile-time constant, the
    // block of every instruction is known at compile time.
    auto load_side = [&](auto r0c, auto ni, const unsigned char *base, unsigned char *dst, int valid_rows)
        __attribute__((always_inline)) {
      constexpr int r0 = decltype(r0c)::value;
      constexpr int NI = decltype(ni)::value;
      const __amdgpu_buffer_rsrc_t r_lo =
          __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)(kOpBlock * C::E), kRsrcWord3);
      const __amdgpu_buffer_rsrc_t r_hi =
          __builtin_amdgcn_make_buffer_rsrc((void *)(base + blk_step), (short)0, (int)(kOpBlock * C::E), kRsrcWord3);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int q = i * kLoadWaves + wave;
        if (!kFull && q * 8 >= valid_rows) continue;   // rows only skipped blocks would read
        constexpr int kBlockRows = kOpRows;
        const bool upper = r0 + 32 * i >= kBlockRows;   // folded per unrolled i
        const int r = (r0 + q * 8) % kBlockRows;
        const int soff = (r * kOpCols + kk) * C::E;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(upper ? r_hi : r_lo, (lds_void *)(dst + q * 1024), 16, lane_off,
                                                 soff, 0, 0);
      }
    };
    using R0 = std::integral_constant<int, 0>;
    using R128 = std::integral_constant<int, 128>;
    using NA = std::integral_constant<int, C::A_I>;
    using NB = std::integral_constant<int, C::B_I>;
    if (m0 % kOpRows == 0) load_side(R0{}, NA{}, A, sa, a_rows);
    else load_side(R128{}, NA{}, A, sa, a_rows);
    if (n0 % kOpRows == 0) load_side(R0{}, NB{}, B, sb, b_rows);
    else load_side(R128{}, NB{}, B, sb, b_rows);
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
    if (++kt == chunk_kt) {
      ++ci;
      kt = 0;
      if (ci < p.n_chunks) set_chunk(ci);
    }
  };

  using F = std::false_type;
  using Tr = std::true_type;
  if (total_kt > 0) {
    set_chunk(0);
    issue_loads(kt, 0, F{});
    advance();
    wait_vm0();
    __syncthreads();
  }

  // One k-tile from LDS stage `buf` on the matrix cores.  The k-fragments of
  // step ks+1 are read before the matrix-core instructions of step ks are
  // issued; scheduling barriers keep the compiler from sinking the reads next
  // to their consumers, so the LDS latency hides behind a whole step of
  // matrix-core work and the matrix core stays fed.
  //
  // In a tile at the ragged edge of the output, 32-row (32-column) blocks
  // that lie entirely past M (N) are padding: they are neither read nor
  // multiplied, and the valid blocks are spread evenly over the waves of
  // that side (wave-uniform counts), which makes the edge tiles of a ragged N
  // cheaper; full tiles take a path without these checks.
  int mb0, mt_act, nb0, nt_act;
  block_share((int)(p.M - m0), C::MT, 2, wm, mb0, mt_act);
  block_share((int)(p.N - n0), C::NT, 4, wn, nb0, nt_act);
  const int row0 = 32 * mb0, col0 = 32 * nb0;   // this wave's first row / column in the tile
  // The k-loop runs with compile-time block bounds MTA x NTA and, in the
  // checked form, skips blocks past the wave's own counts with wave-uniform
  // branches; see the dispatch after it.
  auto compute = [&](int buf, auto mta, auto nta, auto checked) __attribute__((always_inline)) {
    constexpr int MTA = decltype(mta)::value, NTA = decltype(nta)::value;
    constexpr bool kChecked = decltype(checked)::value;
    const unsigned char *sa = lds + buf * C::STAGE;
    const unsigned char *sb = sa + BM * C::ROWB;
    // Wave tiles of up to 8 blocks keep two register sets of A and B
    // fragments and read all of step ks+1 during step ks.  Larger ones (128 x
    // 96) do not fit in 256 registers that way: their A fragments are
    // single-buffered, each re-read for the next step right after the
    // products of the current step that use it have been issued.
    constexpr bool kRollA = C::MT * C::NT > 8;
    Frag<T> af[kRollA ? 1 : 2][C::MT], bfr[2][C::NT];
    const int g_lane = lane >> 5;   // which 8-element half of a 16-wide k step
    auto read_a = [&](int ks, int slot, int mt) __attribute__((always_inline)) {
      const int row = row0 + mt * 32 + (lane & 31);
      lds_frag(af[slot][mt], sa + row * C::ROWB, row, 2 * ks + g_lane);
    };
    auto read_b = [&](int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int nt = 0; nt < NTA; ++nt) {
        if (kChecked && nt >= nt_act) continue;
        const int row = col0 + nt * 32 + (lane & 31);
        lds_frag(bfr[slot][nt], sb + row * C::ROWB, row, 2 * ks + g_lane);
      }
    };
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
      if (!kChecked || mt < mt_act) read_a(0, 0, mt);
    read_b(0, 0);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int cur = ks & 1;
      const int aslot = kRollA ? 0 : cur;
      if (ks + 1 < C::KS) {
        read_b(ks + 1, cur ^ 1);
        if (!kRollA) {
#pragma unroll
          for (int mt = 0; mt < MTA; ++mt)
            if (!kChecked || mt < mt_act) read_a(ks + 1, aslot ^ 1, mt);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) {
        if (kChecked && mt >= mt_act) continue;
#pragma unroll
        for (int nt = 0; nt < NTA; ++nt)
          if (!kChecked || nt < nt_act) mma(acc[mt][nt], af[aslot][mt], bfr[cur][nt]);
        if (kRollA && ks + 1 < C::KS) read_a(ks + 1, 0, mt);
        if (kRollA) __builtin_amdgcn_sched_barrier(0);
      }
      if (!kRollA) __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto k_loop = [&](auto mta, auto nta, auto checked, auto loads_full) __attribute__((always_inline)) {
    for (int it = 0; it + 1 < total_kt; ++it) {
      const int buf = it & 1;
      issue_loads(kt, buf ^ 1, loads_full);
      advance();
      compute(buf, mta, nta, checked);
      wait_vm0();
      __syncthreads();
    }
    if (total_kt > 0) compute((total_kt - 1) & 1, mta, nta, checked);
  };
  // Dispatch.  Every wave runs exactly one k-loop, so its barriers pair
  // with the other waves'.
  //  - 128 x 96 wave tiles (384-wide tiles): full waves run the check-free
  //    loop, the others the checked loop, which multiplies exactly their own
  //    blocks (measured fastest at N = 3605, where edge waves have 1-2 blocks).
  //  - smaller wave tiles: straight-line loops with row blocks 1, 2 or MT and
  //    column blocks 1 or NT, a count in between rounded up (the extra blocks
  //    lie inside the tile, multiply stale LDS rows and are never written);
  //    the checked loop is slow when edge waves keep most of their blocks.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using IM = std::integral_constant<int, C::MT>;
  using IN = std::integral_constant<int, C::NT>;
  if constexpr (C::MT * C::NT > 8) {
    // tiles whose operand rows are all valid also load without tests
    const bool loads_full = a_rows >= BM && b_rows >= BN;
    if (mt_act == C::MT && nt_act == C::NT) {
      if (loads_full) k_loop(IM{}, IN{}, F{}, Tr{});
      else k_loop(IM{}, IN{}, F{}, F{});
    } else {
      k_loop(IM{}, IN{}, Tr{}, F{});
    }
  } else {
    auto k_loop_n = [&](auto mta) __attribute__((always_inline)) {
      if (nt_act == 1) k_loop(mta, I1{}, F{}, F{});
      else k_loop(mta, IN{}, F{}, F{});
    };
    if (mt_act == 0 || nt_act == 0) k_loop(I0{}, I0{}, F{}, F{});   // loads and barriers only
    else if (mt_act == 1) k_loop_n(I1{});
    else if (mt_act == 2) k_loop_n(std::conditional_t<(C::MT > 2), I2, IM>{});
    else k_loop_n(IM{});
  }

  // ---- write / accumulate x -------------------------------------------
  // The four accumulator registers 4g..4g+3 of a lane are rows 4k..4k+3 of
  // one column: one 16-byte group of the x layout (x_offset); 16 lanes cover
  // the 16 columns of a 256-byte block row.  Rows of the last 4-row group
  // past M hold products of padding rows and are ignored downstream.  Only
  // the wave's own blocks are written: in an edge tile the blocks past its
  // count belong to the next wave (or to padding).
  const int M4 = (int)((p.M + 3) & ~int64_t(3));
  const int N = (int)p.N;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    if (mt >= mt_act) continue;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      if (nt >= nt_act) continue;
      const int col = n0 + col0 + nt * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row4 = m0 + row0 + mt * 32 + acc_row(4 * g, lane);   // multiple of 4
        if (row4 < M4 && col < N) {
          f32x4 *dst = reinterpret_cast<f32x4 *>(p.x + x_offset(row4, col, d, p.ldx));
          f32x4 v = {acc[mt][nt][4 * g], acc[mt][nt][4 * g + 1], acc[mt][nt][4 * g + 2], acc[mt][nt][4 * g + 3]};
          if (p.accumulate) v += *dst;
          *dst = v;
        }
      }
    }
  }
}

}  // namespace

// bf16 tile width: 384 columns (wave tile 128 x 96, fewer operand bytes and
// LDS fragment reads per product) unless its last tile column would pad
// clearly more of N than 256-wide tiles do (the padding tiles still pay the
// full load stream of the k-loop).
static int64_t bf16_tile_cols(int64_t n) {
  const int64_t pad384 = (n + 383) / 384 * 384 - n, pad256 = (n + 255) / 256 * 256 - n;
  return (pad384 - pad256) * 100 > 3 * n ? 256 : 384;
}

hipError_t launch_k2(K2Args a, int dtype, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const int64_t bk = (dtype == TRIMUL_BF16) ? 64 : 32;
  const int64_t bm = (dtype == TRIMUL_BF16) ? 256 : 128;
  const int64_t bn = (dtype == TRIMUL_BF16) ? bf16_tile_cols(a.N) : 128;
  for (int c = 0; c < a.n_chunks; ++c) a.ch[c].ktiles = (int32_t)((a.ch[c].k_len + bk - 1) / bk);
  const int64_t tiles_m = (a.M + bm - 1) / bm;
  const int64_t tiles = tiles_m * ((a.N + bn - 1) / bn) * kC;
  // Tile-row groups of 4..6 that divide the tile rows evenly (a short last
  // group shares fewer operand panels), else 4.
  a.group_m = (tiles_m % 4 == 0) ? 4 : (tiles_m % 5 == 0) ? 5 : (tiles_m % 6 == 0) ? 6 : 4;
  // resident work-groups: one per CU for bf16 (128 or 160 KB of LDS), two for fp32
  const int per_cu = (dtype == TRIMUL_BF16) ? 1 : 2;
  a.slots = (device_cu_count() * per_cu + kXcds - 1) / kXcds * kXcds;
  const int64_t grid = (tiles + a.slots - 1) / a.slots * a.slots;
  if (dtype == TRIMUL_BF16 && bn == 384)
    hipLaunchKernelGGL((k2_contract<bf16_t, 256, 384, 64>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else if (dtype == TRIMUL_BF16)
    hipLaunchKernelGGL((k2_contract<bf16_t, 256, 256, 64>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k2_contract<float, 128, 128, 32>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace trimul
