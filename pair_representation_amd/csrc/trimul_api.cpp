// C ABI of the triangle multiplicative update: argument validation, workspace
// layout and the K1 -> K2 -> K3 launch sequence on the caller's stream.
// Every check runs before the first HIP call, so an invalid call enqueues
// nothing; see trimul.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.hpp"
#include "trimul.h"

namespace {

thread_local char g_last_error[512] = "";

trimul_status_t fail(trimul_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

trimul_status_t ok() {
  g_last_error[0] = '\0';
  return TRIMUL_OK;
}

constexpr int64_t kMaxN = 65535;
constexpr int64_t kKTile = 64;

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elt_bytes(int32_t dtype) { return dtype == TRIMUL_BF16 ? 2 : 4; }

trimul_status_t check_weights(const trimul_weights_t *w) {
  if (!w) return fail(TRIMUL_ERR_INVALID_ARG, "weights pointer is NULL");
  if (w->c_z != 128 || w->c != 128)
    return fail(TRIMUL_ERR_UNSUPPORTED, "c_z=%d c=%d: only c_z = c = 128 is supported", w->c_z, w->c);
  if (w->dtype != TRIMUL_F32 && w->dtype != TRIMUL_BF16)
    return fail(TRIMUL_ERR_UNSUPPORTED, "unknown dtype %d", w->dtype);
  if (!(w->ln_eps > 0.0f) || !(w->ln_eps < 1e30f))
    return fail(TRIMUL_ERR_INVALID_ARG, "ln_eps must be positive and finite");
  const void *ptrs[] = {w->ln_in_w, w->ln_in_b, w->w_a_proj, w->w_a_gate, w->w_b_proj,
                        w->w_b_gate, w->w_out_gate, w->ln_out_w, w->ln_out_b, w->w_out_proj};
  const char *names[] = {"ln_in_w", "ln_in_b", "w_a_proj", "w_a_gate", "w_b_proj",
                         "w_b_gate", "w_out_gate", "ln_out_w", "ln_out_b", "w_out_proj"};
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) return fail(TRIMUL_ERR_INVALID_ARG, "weight %s is NULL", names[i]);
    if (!aligned(ptrs[i], 16)) return fail(TRIMUL_ERR_ALIGNMENT, "weight %s is not 16-byte aligned", names[i]);
  }
  return TRIMUL_OK;
}

// Contraction result of a rows x cols tile: x[d][r/4][s][r%4], rows padded to
// a multiple of 4 and columns to a multiple of 16.
int64_t x_ld(int64_t cols) { return round_up(cols, 16); }
size_t xacc_bytes(int64_t rows, int64_t cols) {
  return (size_t)128 * round_up(rows, 4) * x_ld(cols) * sizeof(float);
}

// Operand chunk of `rows` rows and row length ld in the blocked operand layout
// (blocks of 256 rows x 64 columns, 128 channel blocks adjacent): rows are
// padded to a multiple of 256.
size_t operand_bytes(int64_t rows, int64_t ld, int32_t dtype) {
  return (size_t)128 * round_up(rows, 256) * ld * elt_bytes(dtype);
}

struct FullLayout {
  int64_t kp;       // padded k extent = row length of the operand planes
  size_t a_off, b_off, x_off, total;
};

FullLayout full_layout(int32_t dtype, int64_t n) {
  FullLayout L;
  L.kp = round_up(n, kKTile);
  const size_t plane = align256(operand_bytes(n, L.kp, dtype));
  L.a_off = 0;
  L.b_off = plane;
  L.x_off = 2 * plane;
  L.total = L.x_off + align256(xacc_bytes(n, n));
  return L;
}

trimul::K1Args k1_args(const trimul_weights_t *w, const void *z, const uint8_t *mask, int64_t n) {
  trimul::K1Args a{};
  a.z = z;
  a.mask = mask;
  a.n = n;
  a.ln_w = w->ln_in_w;
  a.ln_b = w->ln_in_b;
  a.eps = w->ln_eps;
  a.w_a_proj = w->w_a_proj;
  a.w_a_gate = w->w_a_gate;
  a.w_b_proj = w->w_b_proj;
  a.w_b_gate = w->w_b_gate;
  return a;
}

trimul::K3Args k3_args(const trimul_weights_t *w, const float *x, int64_t ldx, const void *z,
                       const uint8_t *mask, int64_t n, int64_t row_off, int64_t n_rows,
                       int64_t col_off, int64_t n_cols, float *out) {
  trimul::K3Args a{};
  a.x = x;
  a.ldx = ldx;
  a.z = z;
  a.mask = mask;
  a.n = n;
  a.row_off = row_off;
  a.n_rows = n_rows;
  a.col_off = col_off;
  a.n_cols = n_cols;
  a.out = out;
  a.out_ld = n_cols;
  a.ln_out_w = w->ln_out_w;
  a.ln_out_b = w->ln_out_b;
  a.ln_in_w = w->ln_in_w;
  a.ln_in_b = w->ln_in_b;
  a.eps = w->ln_eps;
  a.w_out_proj = w->w_out_proj;
  a.w_out_gate = w->w_out_gate;
  return a;
}

// Workspace of trimul_tile_backward: dx as an operand buffer (rows n_rows,
// row length ld_j = round_up(n_cols, 64)) and transposed (rows n_cols, row
// length ld_i = round_up(n_rows, 64)), then one chunk's transposed a (rows
// k_len, length ld_i) and transposed b (rows k_len, length ld_j), sized for the
// longest chunk.
struct BackwardLayout {
  int64_t ld_i, ld_j, kmax;
  size_t p_off, pt_off, at_off, bt_off, total;
};

BackwardLayout backward_layout(int32_t dtype, int64_t n_rows, int64_t n_cols, const trimul_kchunk_t *chunks,
                               int32_t n_chunks) {
  BackwardLayout L;
  L.ld_i = round_up(n_rows, kKTile);
  L.ld_j = round_up(n_cols, kKTile);
  L.kmax = 1;
  for (int i = 0; i < n_chunks; ++i) L.kmax = std::max<int64_t>(L.kmax, chunks[i].k_len);
  L.p_off = 0;
  L.pt_off = L.p_off + align256(operand_bytes(n_rows, L.ld_j, dtype));
  L.at_off = L.pt_off + align256(operand_bytes(n_cols, L.ld_i, dtype));
  L.bt_off = L.at_off + align256(operand_bytes(L.kmax, L.ld_i, dtype));
  L.total = L.bt_off + align256(operand_bytes(L.kmax, L.ld_j, dtype));
  return L;
}

trimul_status_t check_backward(const trimul_weights_t *w, int64_t n_rows, int64_t n_cols,
                               const trimul_kchunk_t *chunks, int32_t n_chunks) {
  trimul_status_t st = check_weights(w);
  if (st != TRIMUL_OK) return st;
  if (n_rows < 1 || n_rows > kMaxN || n_cols < 1 || n_cols > kMaxN)
    return fail(TRIMUL_ERR_INVALID_ARG, "tile %lld x %lld outside [1, %lld]^2", (long long)n_rows, (long long)n_cols,
                (long long)kMaxN);
  if (n_chunks < 1 || n_chunks > TRIMUL_MAX_CHUNKS)
    return fail(TRIMUL_ERR_INVALID_ARG, "n_chunks=%d outside [1, %d]", n_chunks, TRIMUL_MAX_CHUNKS);
  if (!chunks) return fail(TRIMUL_ERR_INVALID_ARG, "chunks is NULL");
  for (int i = 0; i < n_chunks; ++i) {
    const trimul_kchunk_t &c = chunks[i];
    if (c.k_len < 1 || c.k_len > kMaxN) return fail(TRIMUL_ERR_INVALID_ARG, "chunk %d: k_len=%lld", i, (long long)c.k_len);
    if (c.ld < c.k_len || c.ld % kKTile != 0)
      return fail(TRIMUL_ERR_INVALID_ARG, "chunk %d: ld=%lld must be a multiple of 64 and >= k_len", i, (long long)c.ld);
    if (!c.a || !c.b) return fail(TRIMUL_ERR_INVALID_ARG, "chunk %d: NULL operand", i);
    if (!aligned(c.a, 16) || !aligned(c.b, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "chunk %d: operands must be 16-byte aligned", i);
  }
  return TRIMUL_OK;
}

trimul_status_t hip_fail(hipError_t e, const char *what) {
  return fail(TRIMUL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// K1 launches for one operand chunk (arguments already validated): one
// launch writes both operands when their source rows coincide, else one per
// requested operand.
hipError_t enqueue_operands(const trimul_weights_t *w, trimul_dir_t dir, const void *z, const uint8_t *mask,
                            int64_t n, int64_t row_off, int64_t n_rows, int64_t col_off, int64_t n_cols,
                            int64_t k_off, int64_t k_len, int64_t ld, void *a_out, void *b_out, hipStream_t s) {
  trimul::K1Args k1 = k1_args(w, z, mask, n);
  k1.k_off = k_off;
  k1.k_len = k_len;
  k1.ld = ld;
  k1.transposed = dir == TRIMUL_INCOMING ? 1 : 0;
  if (a_out && b_out && row_off == col_off && n_rows == n_cols) {
    k1.row_base = row_off;
    k1.n_rows = n_rows;
    k1.a_out = a_out;
    k1.b_out = b_out;
    return trimul::launch_k1(k1, w->dtype, s);
  }
  if (a_out) {
    k1.row_base = row_off;
    k1.n_rows = n_rows;
    k1.a_out = a_out;
    k1.b_out = nullptr;
    const hipError_t e = trimul::launch_k1(k1, w->dtype, s);
    if (e != hipSuccess) return e;
  }
  if (b_out) {
    k1.row_base = col_off;
    k1.n_rows = n_cols;
    k1.a_out = nullptr;
    k1.b_out = b_out;
    return trimul::launch_k1(k1, w->dtype, s);
  }
  return hipSuccess;
}

trimul_status_t run_full(const trimul_weights_t *w, const void *z, const uint8_t *mask, float *out,
                         int64_t n, void *workspace, size_t workspace_bytes, void *stream,
                         bool incoming) {
  trimul_status_t st = check_weights(w);
  if (st != TRIMUL_OK) return st;
  if (n < 0 || n > kMaxN) return fail(TRIMUL_ERR_INVALID_ARG, "n=%lld out of range [0, %lld]", (long long)n, (long long)kMaxN);
  if (n == 0) return ok();
  if (!z || !mask || !out) return fail(TRIMUL_ERR_INVALID_ARG, "z, mask and out must be non-NULL");
  if (!workspace) return fail(TRIMUL_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(z, 16) || !aligned(out, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "z and out must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(TRIMUL_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  const FullLayout L = full_layout(w->dtype, n);
  if (workspace_bytes < L.total)
    return fail(TRIMUL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, L.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  void *a_pl = ws + L.a_off;
  void *b_pl = ws + L.b_off;
  float *x = reinterpret_cast<float *>(ws + L.x_off);

  trimul::K1Args k1 = k1_args(w, z, mask, n);
  k1.row_base = 0;
  k1.n_rows = n;
  k1.k_off = 0;
  k1.k_len = n;
  k1.ld = L.kp;
  k1.transposed = incoming ? 1 : 0;
  k1.a_out = a_pl;
  k1.b_out = b_pl;
  hipError_t e = trimul::launch_k1(k1, w->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "projection kernel launch");

  trimul::K2Args k2{};
  k2.ch[0].a = a_pl;
  k2.ch[0].b = b_pl;
  k2.ch[0].ld = L.kp;
  k2.ch[0].k_len = n;
  k2.n_chunks = 1;
  k2.accumulate = 0;
  k2.M = n;
  k2.N = n;
  k2.x = x;
  k2.ldx = x_ld(n);
  e = trimul::launch_k2(k2, w->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "contraction kernel launch");

  trimul::K3Args k3 = k3_args(w, x, x_ld(n), z, mask, n, 0, n, 0, n, out);
  e = trimul::launch_k3(k3, w->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "epilogue kernel launch");
  return ok();
}

// Blocks of the memory-bounded forward: rows R, columns C and k-chunk K of
// each step (0 or anything above n means n), and the workspace that holds
// one step: the a operand of R rows, the b operand of C rows (both with row
// length round_up(K, 64)) and the fp32 accumulator of an R x C tile.
struct ChunkedLayout {
  int64_t R, C, K, ldk;
  size_t a_off, b_off, x_off, total;
};

ChunkedLayout chunked_layout(int32_t dtype, int64_t n, int64_t row_block, int64_t col_block, int64_t k_block) {
  ChunkedLayout L;
  L.R = (row_block <= 0 || row_block > n) ? n : row_block;
  L.C = (col_block <= 0 || col_block > n) ? n : col_block;
  L.K = (k_block <= 0 || k_block > n) ? n : k_block;
  L.ldk = round_up(L.K, kKTile);
  L.a_off = 0;
  L.b_off = align256(operand_bytes(L.R, L.ldk, dtype));
  L.x_off = L.b_off + align256(operand_bytes(L.C, L.ldk, dtype));
  L.total = L.x_off + align256(xacc_bytes(L.R, L.C));
  return L;
}

trimul_status_t check_full_args(const trimul_weights_t *w, const void *z, const uint8_t *mask, float *out,
                                int64_t n, void *workspace) {
  trimul_status_t st = check_weights(w);
  if (st != TRIMUL_OK) return st;
  if (n < 0 || n > kMaxN) return fail(TRIMUL_ERR_INVALID_ARG, "n=%lld out of range [0, %lld]", (long long)n, (long long)kMaxN);
  if (n == 0) return TRIMUL_OK;
  if (!z || !mask || !out) return fail(TRIMUL_ERR_INVALID_ARG, "z, mask and out must be non-NULL");
  if (!workspace) return fail(TRIMUL_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(z, 16) || !aligned(out, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "z and out must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(TRIMUL_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  return TRIMUL_OK;
}

// The update one R x C output tile at a time; inside a tile the k range is
// walked in chunks of K: the chunk's operands (K1), then the contraction
// into the tile's accumulator (K2; the first chunk overwrites, the others
// add), and after the last chunk the epilogue (K3) writes the tile straight
// into out (row stride n).  When one chunk covers all of k the buffers still
// hold what a later tile needs: a (its rows, all of k) is kept across the
// column blocks of a row block, and with a single column block b (all
// columns, all of k) is built once for every row block.
trimul_status_t enqueue_chunked(const trimul_weights_t *w, trimul_dir_t dir, const void *z, const uint8_t *mask,
                                float *out, int64_t n, const ChunkedLayout &L, char *ws, hipStream_t s) {
  void *a_buf = ws + L.a_off;
  void *b_buf = ws + L.b_off;
  float *x = reinterpret_cast<float *>(ws + L.x_off);
  const bool one_k = L.K >= n;
  const bool one_c = L.C >= n;
  hipError_t e;
  for (int64_t r0 = 0; r0 < n; r0 += L.R) {
    const int64_t nr = std::min(L.R, n - r0);
    for (int64_t c0 = 0; c0 < n; c0 += L.C) {
      const int64_t nc = std::min(L.C, n - c0);
      for (int64_t k0 = 0; k0 < n; k0 += L.K) {
        const int64_t kl = std::min(L.K, n - k0);
        void *a_dst = (one_k && c0 > 0) ? nullptr : a_buf;
        void *b_dst = (one_k && one_c && r0 > 0) ? nullptr : b_buf;
        if (one_k && one_c && r0 == 0 && nr < n && nr % 256 == 0) {
          // First row tile, b built once at full width: a and b of the
          // tile's rows in one projection pass, then b of the other rows.
          // Those start on a 256-row operand block, so that part of the b
          // buffer is an operand buffer of its own.
          e = enqueue_operands(w, dir, z, mask, n, 0, nr, 0, nr, 0, kl, L.ldk, a_buf, b_buf, s);
          if (e == hipSuccess)
            e = enqueue_operands(w, dir, z, mask, n, 0, 0, nr, n - nr, 0, kl, L.ldk, nullptr,
                                 static_cast<char *>(b_buf) + operand_bytes(nr, L.ldk, w->dtype), s);
          if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
        } else if (a_dst || b_dst) {
          e = enqueue_operands(w, dir, z, mask, n, r0, nr, c0, nc, k0, kl, L.ldk, a_dst, b_dst, s);
          if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
        }
        trimul::K2Args k2{};
        k2.ch[0].a = a_buf;
        k2.ch[0].b = b_buf;
        k2.ch[0].ld = L.ldk;
        k2.ch[0].k_len = kl;
        k2.n_chunks = 1;
        k2.accumulate = k0 == 0 ? 0 : 1;
        k2.M = nr;
        k2.N = nc;
        k2.x = x;
        k2.ldx = x_ld(nc);
        e = trimul::launch_k2(k2, w->dtype, s);
        if (e != hipSuccess) return hip_fail(e, "contraction kernel launch");
      }
      trimul::K3Args k3 = k3_args(w, x, x_ld(nc), z, mask, n, r0, nr, c0, nc, out + (r0 * n + c0) * 128);
      k3.out_ld = n;
      e = trimul::launch_k3(k3, w->dtype, s);
      if (e != hipSuccess) return hip_fail(e, "epilogue kernel launch");
    }
  }
  return ok();
}

// Workspace of trimul_forward_chunked_noalloc: a file-scope device array, one
// copy per device.  In host code its name is a host-side stand-in, not a
// device address: only the address hipGetSymbolAddress returns (kept per
// device below) is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[TRIMUL_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
trimul_status_t scratch_address(char **out) {
  static std::mutex mu;
  static std::vector<void *> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    addr[dev] = p;
  }
  *out = static_cast<char *>(addr[dev]);
  return TRIMUL_OK;
}

}  // namespace

namespace trimul {

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

}  // namespace trimul

extern "C" {

size_t trimul_workspace_bytes(const trimul_weights_t *w, int64_t n) {
  if (!w || (w->dtype != TRIMUL_F32 && w->dtype != TRIMUL_BF16) || n < 0 || n > kMaxN) return 0;
  if (n == 0) return 0;
  return full_layout(w->dtype, n).total;
}

trimul_status_t trimul_outgoing(const trimul_weights_t *w, const void *z, const uint8_t *mask, float *out,
                                int64_t n, void *workspace, size_t workspace_bytes, void *stream) {
  return run_full(w, z, mask, out, n, workspace, workspace_bytes, stream, false);
}

trimul_status_t trimul_incoming(const trimul_weights_t *w, const void *z, const uint8_t *mask, float *out,
                                int64_t n, void *workspace, size_t workspace_bytes, void *stream) {
  return run_full(w, z, mask, out, n, workspace, workspace_bytes, stream, true);
}

size_t trimul_chunked_workspace_bytes(const trimul_weights_t *w, int64_t n, int64_t row_block, int64_t col_block,
                                      int64_t k_block) {
  if (!w || (w->dtype != TRIMUL_F32 && w->dtype != TRIMUL_BF16) || n < 1 || n > kMaxN) return 0;
  if (row_block < 0 || col_block < 0 || k_block < 0) return 0;
  return chunked_layout(w->dtype, n, row_block, col_block, k_block).total;
}

trimul_status_t trimul_forward_chunked(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                       const uint8_t *mask, float *out, int64_t n, int64_t row_block,
                                       int64_t col_block, int64_t k_block, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  trimul_status_t st = check_full_args(w, z, mask, out, n, workspace);
  if (st != TRIMUL_OK) return st;
  if (dir != TRIMUL_OUTGOING && dir != TRIMUL_INCOMING) return fail(TRIMUL_ERR_INVALID_ARG, "unknown direction %d", (int)dir);
  if (row_block < 0 || col_block < 0 || k_block < 0)
    return fail(TRIMUL_ERR_INVALID_ARG, "block sizes must be >= 0 (0 = n): %lld %lld %lld", (long long)row_block,
                (long long)col_block, (long long)k_block);
  if (n == 0) return ok();
  const ChunkedLayout L = chunked_layout(w->dtype, n, row_block, col_block, k_block);
  if (workspace_bytes < L.total)
    return fail(TRIMUL_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, L.total);
  return enqueue_chunked(w, dir, z, mask, out, n, L, static_cast<char *>(workspace), static_cast<hipStream_t>(stream));
}

trimul_status_t trimul_forward_chunked_noalloc(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                               const uint8_t *mask, float *out, int64_t n, int64_t row_block,
                                               int64_t col_block, int64_t k_block, void *stream) {
  // validation as trimul_forward_chunked, with the scratch array standing in
  // for the workspace (any non-NULL, 256-byte aligned pointer passes the
  // workspace checks)
  const void *placeholder = reinterpret_cast<const void *>(uintptr_t(256));
  trimul_status_t st = check_full_args(w, z, mask, out, n, const_cast<void *>(placeholder));
  if (st != TRIMUL_OK) return st;
  if (dir != TRIMUL_OUTGOING && dir != TRIMUL_INCOMING) return fail(TRIMUL_ERR_INVALID_ARG, "unknown direction %d", (int)dir);
  if (row_block < 0 || col_block < 0 || k_block < 0)
    return fail(TRIMUL_ERR_INVALID_ARG, "block sizes must be >= 0 (0 = n): %lld %lld %lld", (long long)row_block,
                (long long)col_block, (long long)k_block);
  if (n == 0) return ok();
  const ChunkedLayout L = chunked_layout(w->dtype, n, row_block, col_block, k_block);
  if (L.total > TRIMUL_NOALLOC_SCRATCH_BYTES)
    return fail(TRIMUL_ERR_WORKSPACE_TOO_SMALL,
                "blocks %lld x %lld x %lld need %zu bytes of workspace, more than the %zu-byte scratch array",
                (long long)L.R, (long long)L.C, (long long)L.K, L.total, (size_t)TRIMUL_NOALLOC_SCRATCH_BYTES);
  char *ws = nullptr;
  st = scratch_address(&ws);
  if (st != TRIMUL_OK) return st;
  return enqueue_chunked(w, dir, z, mask, out, n, L, ws, static_cast<hipStream_t>(stream));
}

size_t trimul_tile_xacc_bytes(const trimul_weights_t *w, int64_t n_rows, int64_t n_cols) {
  if (!w || n_rows < 0 || n_cols < 0) return 0;
  return xacc_bytes(n_rows, n_cols);
}

size_t trimul_tile_operand_bytes(const trimul_weights_t *w, int64_t rows, int64_t ld) {
  if (!w || (w->dtype != TRIMUL_F32 && w->dtype != TRIMUL_BF16) || rows < 0 || ld < 0) return 0;
  return operand_bytes(rows, ld, w->dtype);
}

trimul_status_t trimul_tile_operands(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                     const uint8_t *mask, int64_t n, int64_t row_off, int64_t n_rows,
                                     int64_t col_off, int64_t n_cols, int64_t k_off, int64_t k_len,
                                     int64_t ld, void *a_out, void *b_out, void *stream) {
  trimul_status_t st = check_weights(w);
  if (st != TRIMUL_OK) return st;
  if (dir != TRIMUL_OUTGOING && dir != TRIMUL_INCOMING) return fail(TRIMUL_ERR_INVALID_ARG, "unknown direction %d", (int)dir);
  if (n < 1 || n > kMaxN) return fail(TRIMUL_ERR_INVALID_ARG, "n=%lld out of range [1, %lld]", (long long)n, (long long)kMaxN);
  if (!z || !mask) return fail(TRIMUL_ERR_INVALID_ARG, "z and mask must be non-NULL");
  if (!a_out && !b_out) return fail(TRIMUL_ERR_INVALID_ARG, "a_out and b_out are both NULL");
  if (a_out && (row_off < 0 || n_rows < 1 || row_off + n_rows > n))
    return fail(TRIMUL_ERR_INVALID_ARG, "row range [%lld, +%lld) outside [0, %lld)", (long long)row_off, (long long)n_rows, (long long)n);
  if (b_out && (col_off < 0 || n_cols < 1 || col_off + n_cols > n))
    return fail(TRIMUL_ERR_INVALID_ARG, "col range [%lld, +%lld) outside [0, %lld)", (long long)col_off, (long long)n_cols, (long long)n);
  if (k_off < 0 || k_len < 1 || k_off + k_len > n)
    return fail(TRIMUL_ERR_INVALID_ARG, "k range [%lld, +%lld) outside [0, %lld)", (long long)k_off, (long long)k_len, (long long)n);
  if (ld < k_len || ld % kKTile != 0)
    return fail(TRIMUL_ERR_INVALID_ARG, "ld=%lld must be a multiple of 64 and >= k_len=%lld", (long long)ld, (long long)k_len);
  if (!aligned(z, 16) || (a_out && !aligned(a_out, 16)) || (b_out && !aligned(b_out, 16)))
    return fail(TRIMUL_ERR_ALIGNMENT, "z, a_out and b_out must be 16-byte aligned");

  hipError_t e = enqueue_operands(w, dir, z, mask, n, row_off, n_rows, col_off, n_cols, k_off, k_len, ld, a_out,
                                  b_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "projection kernel launch");
  return ok();
}

trimul_status_t trimul_tile(const trimul_weights_t *w, int64_t n, int64_t row_off, int64_t n_rows,
                            int64_t col_off, int64_t n_cols, const trimul_kchunk_t *chunks, int32_t n_chunks,
                            uint32_t flags, float *x_acc, const void *z, const uint8_t *mask, float *out_tile,
                            void *stream) {
  trimul_status_t st = check_weights(w);
  if (st != TRIMUL_OK) return st;
  if (n < 1 || n > kMaxN) return fail(TRIMUL_ERR_INVALID_ARG, "n=%lld out of range [1, %lld]", (long long)n, (long long)kMaxN);
  if (row_off < 0 || n_rows < 1 || row_off + n_rows > n)
    return fail(TRIMUL_ERR_INVALID_ARG, "row range [%lld, +%lld) outside [0, %lld)", (long long)row_off, (long long)n_rows, (long long)n);
  if (col_off < 0 || n_cols < 1 || col_off + n_cols > n)
    return fail(TRIMUL_ERR_INVALID_ARG, "col range [%lld, +%lld) outside [0, %lld)", (long long)col_off, (long long)n_cols, (long long)n);
  if (flags & ~(uint32_t)(TRIMUL_TILE_FIRST | TRIMUL_TILE_LAST))
    return fail(TRIMUL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (n_chunks < 0 || n_chunks > TRIMUL_MAX_CHUNKS)
    return fail(TRIMUL_ERR_INVALID_ARG, "n_chunks=%d outside [0, %d]", n_chunks, TRIMUL_MAX_CHUNKS);
  if (n_chunks == 0 && flags != TRIMUL_TILE_LAST)
    return fail(TRIMUL_ERR_INVALID_ARG, "n_chunks = 0 is only valid with TRIMUL_TILE_LAST alone");
  if (n_chunks > 0 && !chunks) return fail(TRIMUL_ERR_INVALID_ARG, "chunks is NULL");
  if (!x_acc) return fail(TRIMUL_ERR_INVALID_ARG, "x_acc is NULL");
  if (!aligned(x_acc, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "x_acc must be 16-byte aligned");
  const bool last = flags & TRIMUL_TILE_LAST;
  if (last) {
    if (!z || !mask || !out_tile) return fail(TRIMUL_ERR_INVALID_ARG, "z, mask and out_tile are required with TRIMUL_TILE_LAST");
    if (!aligned(z, 16) || !aligned(out_tile, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "z and out_tile must be 16-byte aligned");
  }
  std::vector<std::pair<int64_t, int64_t>> spans;
  for (int i = 0; i < n_chunks; ++i) {
    const trimul_kchunk_t &c = chunks[i];
    if (c.k_off < 0 || c.k_len < 1 || c.k_off + c.k_len > n)
      return fail(TRIMUL_ERR_INVALID_ARG, "chunk %d: k range [%lld, +%lld) outside [0, %lld)", i, (long long)c.k_off, (long long)c.k_len, (long long)n);
    if (c.ld < c.k_len || c.ld % kKTile != 0)
      return fail(TRIMUL_ERR_INVALID_ARG, "chunk %d: ld=%lld must be a multiple of 64 and >= k_len", i, (long long)c.ld);
    if (!c.a || !c.b) return fail(TRIMUL_ERR_INVALID_ARG, "chunk %d: NULL operand", i);
    if (!aligned(c.a, 16) || !aligned(c.b, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "chunk %d: operands must be 16-byte aligned", i);
    spans.emplace_back(c.k_off, c.k_off + c.k_len);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second)
      return fail(TRIMUL_ERR_INVALID_ARG, "chunks overlap at k=%lld", (long long)spans[i].first);
  if ((flags & TRIMUL_TILE_FIRST) && last) {
    int64_t cover = 0;
    for (auto &sp : spans) {
      if (sp.first != cover) return fail(TRIMUL_ERR_INVALID_ARG, "FIRST|LAST chunks leave k=%lld uncovered", (long long)cover);
      cover = sp.second;
    }
    if (cover != n) return fail(TRIMUL_ERR_INVALID_ARG, "FIRST|LAST chunks cover [0, %lld), not [0, %lld)", (long long)cover, (long long)n);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (n_chunks > 0) {
    trimul::K2Args k2{};
    for (int i = 0; i < n_chunks; ++i) {
      k2.ch[i].a = chunks[i].a;
      k2.ch[i].b = chunks[i].b;
      k2.ch[i].ld = chunks[i].ld;
      k2.ch[i].k_len = chunks[i].k_len;
    }
    k2.n_chunks = n_chunks;
    k2.accumulate = (flags & TRIMUL_TILE_FIRST) ? 0 : 1;
    k2.M = n_rows;
    k2.N = n_cols;
    k2.x = x_acc;
    k2.ldx = x_ld(n_cols);
    e = trimul::launch_k2(k2, w->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "contraction kernel launch");
  }
  if (last) {
    trimul::K3Args k3 = k3_args(w, x_acc, x_ld(n_cols), z, mask, n, row_off, n_rows, col_off, n_cols, out_tile);
    e = trimul::launch_k3(k3, w->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "epilogue kernel launch");
  }
  return ok();
}

size_t trimul_tile_backward_workspace_bytes(const trimul_weights_t *w, int64_t n_rows, int64_t n_cols,
                                            const trimul_kchunk_t *chunks, int32_t n_chunks) {
  if (check_backward(w, n_rows, n_cols, chunks, n_chunks) != TRIMUL_OK) return 0;
  return backward_layout(w->dtype, n_rows, n_cols, chunks, n_chunks).total;
}

trimul_status_t trimul_tile_backward(const trimul_weights_t *w, int64_t n_rows, int64_t n_cols,
                                     const trimul_kchunk_t *chunks, int32_t n_chunks, const float *dx,
                                     float *const *da_out, float *const *db_out, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  trimul_status_t st = check_backward(w, n_rows, n_cols, chunks, n_chunks);
  if (st != TRIMUL_OK) return st;
  if (!dx) return fail(TRIMUL_ERR_INVALID_ARG, "dx is NULL");
  if (!aligned(dx, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "dx must be 16-byte aligned");
  if (!da_out || !db_out) return fail(TRIMUL_ERR_INVALID_ARG, "da_out and db_out must be host arrays");
  for (int i = 0; i < n_chunks; ++i) {
    if (!da_out[i] || !db_out[i]) return fail(TRIMUL_ERR_INVALID_ARG, "chunk %d: NULL gradient output", i);
    if (!aligned(da_out[i], 16) || !aligned(db_out[i], 16))
      return fail(TRIMUL_ERR_ALIGNMENT, "chunk %d: gradient outputs must be 16-byte aligned", i);
  }
  const BackwardLayout L = backward_layout(w->dtype, n_rows, n_cols, chunks, n_chunks);
  if (!workspace) return fail(TRIMUL_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(TRIMUL_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(TRIMUL_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  void *P = ws + L.p_off, *Pt = ws + L.pt_off, *At = ws + L.at_off, *Bt = ws + L.bt_off;
  hipError_t e;
  // dx -> operand buffers P = dx (rows r, columns s) and Pt = dx^T
  trimul::RelayoutArgs r{};
  r.x = dx;
  r.ldx = x_ld(n_cols);
  r.rows = n_rows;
  r.cols = n_cols;
  r.p = P;
  r.ld_p = L.ld_j;
  r.q = Pt;
  r.ld_q = L.ld_i;
  e = trimul::launch_relayout(r, true, w->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "relayout kernel launch");
  for (int c = 0; c < n_chunks; ++c) {
    const trimul_kchunk_t &ch = chunks[c];
    // a^T: rows t < k_len, columns r < n_rows; b^T: rows t, columns s < n_cols
    trimul::RelayoutArgs ta{};
    ta.src = ch.a;
    ta.ld_src = ch.ld;
    ta.rows = n_rows;
    ta.cols = ch.k_len;
    ta.q = At;
    ta.ld_q = L.ld_i;
    e = trimul::launch_relayout(ta, false, w->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "transpose kernel launch");
    trimul::RelayoutArgs tb = ta;
    tb.src = ch.b;
    tb.rows = n_cols;
    tb.q = Bt;
    tb.ld_q = L.ld_j;
    e = trimul::launch_relayout(tb, false, w->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "transpose kernel launch");
    // da[r][t] = sum_s P[r][s] Bt[t][s];  db[s][t] = sum_r Pt[s][r] At[t][r]
    trimul::K2Args k2{};
    k2.n_chunks = 1;
    k2.accumulate = 0;
    k2.ch[0].a = P;
    k2.ch[0].b = Bt;
    k2.ch[0].ld = L.ld_j;
    k2.ch[0].k_len = n_cols;
    k2.M = n_rows;
    k2.N = ch.k_len;
    k2.x = da_out[c];
    k2.ldx = x_ld(ch.k_len);
    e = trimul::launch_k2(k2, w->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "contraction kernel launch (da)");
    k2.ch[0].a = Pt;
    k2.ch[0].b = At;
    k2.ch[0].ld = L.ld_i;
    k2.ch[0].k_len = n_rows;
    k2.M = n_cols;
    k2.x = db_out[c];
    e = trimul::launch_k2(k2, w->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "contraction kernel launch (db)");
  }
  return ok();
}

namespace {

struct EpilogueBackwardLayout {
  size_t wt_off, tot_off, part_off, total;
};

EpilogueBackwardLayout epilogue_backward_layout(int32_t dtype) {
  EpilogueBackwardLayout L;
  const size_t slot = align256((size_t)trimul::kK3BSlotFloats * sizeof(float));
  L.wt_off = 0;
  L.tot_off = align256((size_t)2 * 128 * 128 * elt_bytes(dtype));
  L.part_off = L.tot_off + slot;
  L.total = L.part_off + (size_t)trimul::kK3BMaxParts * slot;
  return L;
}

}  // namespace

size_t trimul_epilogue_backward_workspace_bytes(const trimul_weights_t *w) {
  if (check_weights(w) != TRIMUL_OK) return 0;
  return epilogue_backward_layout(w->dtype).total;
}

trimul_status_t trimul_epilogue_backward(const trimul_weights_t *w, int64_t n, int64_t row_off, int64_t n_rows,
                                         int64_t col_off, int64_t n_cols, const float *x_acc, const void *z,
                                         const uint8_t *mask, const float *dout, float *dx, float *dz,
                                         uint32_t flags, const trimul_epilogue_grads_t *grads, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  trimul_status_t st = check_weights(w);
  if (st != TRIMUL_OK) return st;
  if (n < 1 || n > kMaxN) return fail(TRIMUL_ERR_INVALID_ARG, "n=%lld out of range [1, %lld]", (long long)n, (long long)kMaxN);
  if (row_off < 0 || n_rows < 1 || row_off + n_rows > n)
    return fail(TRIMUL_ERR_INVALID_ARG, "row range [%lld, +%lld) outside [0, %lld)", (long long)row_off, (long long)n_rows, (long long)n);
  if (col_off < 0 || n_cols < 1 || col_off + n_cols > n)
    return fail(TRIMUL_ERR_INVALID_ARG, "col range [%lld, +%lld) outside [0, %lld)", (long long)col_off, (long long)n_cols, (long long)n);
  if (!x_acc || !z || !mask || !dout || !dx || !dz)
    return fail(TRIMUL_ERR_INVALID_ARG, "x_acc, z, mask, dout, dx and dz are required");
  if (!aligned(x_acc, 16) || !aligned(z, 16) || !aligned(dout, 16) || !aligned(dx, 16) || !aligned(dz, 16))
    return fail(TRIMUL_ERR_ALIGNMENT, "x_acc, z, dout, dx and dz must be 16-byte aligned");
  if (flags & ~(uint32_t)TRIMUL_GRAD_ACCUMULATE) return fail(TRIMUL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (!grads) return fail(TRIMUL_ERR_INVALID_ARG, "grads is NULL");
  float *const gp[] = {grads->w_out_proj, grads->w_out_gate, grads->ln_out_w, grads->ln_out_b, grads->ln_in_w, grads->ln_in_b};
  const char *gn[] = {"w_out_proj", "w_out_gate", "ln_out_w", "ln_out_b", "ln_in_w", "ln_in_b"};
  for (int i = 0; i < 6; ++i) {
    if (!gp[i]) return fail(TRIMUL_ERR_INVALID_ARG, "gradient %s is NULL", gn[i]);
    if (!aligned(gp[i], 16)) return fail(TRIMUL_ERR_ALIGNMENT, "gradient %s is not 16-byte aligned", gn[i]);
  }
  const EpilogueBackwardLayout L = epilogue_backward_layout(w->dtype);
  if (!workspace) return fail(TRIMUL_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(TRIMUL_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(TRIMUL_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);

  unsigned char *ws = static_cast<unsigned char *>(workspace);
  trimul::K3BArgs a{};
  a.x = x_acc;
  a.ldx = x_ld(n_cols);
  a.z = z;
  a.mask = mask;
  a.n = n;
  a.row_off = row_off;
  a.n_rows = n_rows;
  a.col_off = col_off;
  a.n_cols = n_cols;
  a.dout = dout;
  a.dx = dx;
  a.dz = dz;
  a.ln_x_w = w->ln_out_w;
  a.ln_x_b = w->ln_out_b;
  a.ln_z_w = w->ln_in_w;
  a.ln_z_b = w->ln_in_b;
  a.eps = w->ln_eps;
  a.w_y = w->w_out_proj;
  a.w_t = w->w_out_gate;
  a.wt = ws + L.wt_off;
  a.tot = reinterpret_cast<float *>(ws + L.tot_off);
  a.part = reinterpret_cast<float *>(ws + L.part_off);
  a.g_w_y = grads->w_out_proj;
  a.g_w_t = grads->w_out_gate;
  a.g_ln_x_w = grads->ln_out_w;
  a.g_ln_x_b = grads->ln_out_b;
  a.g_ln_z_w = grads->ln_in_w;
  a.g_ln_z_b = grads->ln_in_b;
  a.grad_accumulate = a.ln_accumulate = (flags & TRIMUL_GRAD_ACCUMULATE) ? 1 : 0;
  const hipError_t e = trimul::launch_k3b(a, w->dtype, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "epilogue backward kernel launch");
  return ok();
}

size_t trimul_tile_operands_backward_workspace_bytes(const trimul_weights_t *w) {
  return trimul_epilogue_backward_workspace_bytes(w);
}

trimul_status_t trimul_tile_operands_backward(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                              const uint8_t *mask, int64_t n, int64_t row_off, int64_t n_rows,
                                              int64_t col_off, int64_t n_cols, int64_t k_off, int64_t k_len,
                                              const float *da, const float *db, float *dz, uint32_t flags,
                                              const trimul_projection_grads_t *grads, void *workspace,
                                              size_t workspace_bytes, void *stream) {
  trimul_status_t st = check_weights(w);
  if (st != TRIMUL_OK) return st;
  if (dir != TRIMUL_OUTGOING && dir != TRIMUL_INCOMING) return fail(TRIMUL_ERR_INVALID_ARG, "unknown direction %d", (int)dir);
  if (n < 1 || n > kMaxN) return fail(TRIMUL_ERR_INVALID_ARG, "n=%lld out of range [1, %lld]", (long long)n, (long long)kMaxN);
  if (!da && !db) return fail(TRIMUL_ERR_INVALID_ARG, "da and db are both NULL");
  if (da && (row_off < 0 || n_rows < 1 || row_off + n_rows > n))
    return fail(TRIMUL_ERR_INVALID_ARG, "row range [%lld, +%lld) outside [0, %lld)", (long long)row_off, (long long)n_rows, (long long)n);
  if (db && (col_off < 0 || n_cols < 1 || col_off + n_cols > n))
    return fail(TRIMUL_ERR_INVALID_ARG, "col range [%lld, +%lld) outside [0, %lld)", (long long)col_off, (long long)n_cols, (long long)n);
  if (k_off < 0 || k_len < 1 || k_off + k_len > n)
    return fail(TRIMUL_ERR_INVALID_ARG, "k range [%lld, +%lld) outside [0, %lld)", (long long)k_off, (long long)k_len, (long long)n);
  if (flags & ~(uint32_t)TRIMUL_GRAD_ACCUMULATE) return fail(TRIMUL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (!z || !mask || !dz) return fail(TRIMUL_ERR_INVALID_ARG, "z, mask and dz are required");
  if (!aligned(z, 16) || !aligned(dz, 16) || (da && !aligned(da, 16)) || (db && !aligned(db, 16)))
    return fail(TRIMUL_ERR_ALIGNMENT, "z, dz, da and db must be 16-byte aligned");
  if (!grads) return fail(TRIMUL_ERR_INVALID_ARG, "grads is NULL");
  struct Need {
    bool on;
    float *ptr;
    const char *name;
  } need[] = {{da != nullptr, grads->w_a_proj, "w_a_proj"}, {da != nullptr, grads->w_a_gate, "w_a_gate"},
              {db != nullptr, grads->w_b_proj, "w_b_proj"}, {db != nullptr, grads->w_b_gate, "w_b_gate"},
              {true, grads->ln_in_w, "ln_in_w"}, {true, grads->ln_in_b, "ln_in_b"}};
  for (const Need &nd : need) {
    if (!nd.on) continue;
    if (!nd.ptr) return fail(TRIMUL_ERR_INVALID_ARG, "gradient %s is NULL", nd.name);
    if (!aligned(nd.ptr, 16)) return fail(TRIMUL_ERR_ALIGNMENT, "gradient %s is not 16-byte aligned", nd.name);
  }
  const EpilogueBackwardLayout L = epilogue_backward_layout(w->dtype);
  if (!workspace) return fail(TRIMUL_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(TRIMUL_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(TRIMUL_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);

  unsigned char *ws = static_cast<unsigned char *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool accumulate = (flags & TRIMUL_GRAD_ACCUMULATE) != 0;
  bool ln_accumulate = accumulate;
  for (int side = 0; side < 2; ++side) {
    const float *d = side == 0 ? da : db;
    if (!d) continue;
    trimul::K3BArgs a{};
    a.ldx = x_ld(k_len);
    a.z = z;
    a.mask = mask;
    a.n = n;
    a.row_off = side == 0 ? row_off : col_off;   // plane row r <-> residue row_off + r (col_off + s for b)
    a.n_rows = side == 0 ? n_rows : n_cols;
    a.col_off = k_off;                           // plane column t <-> residue k_off + t
    a.n_cols = k_len;
    a.transposed = dir == TRIMUL_INCOMING;       // incoming operands are stored transposed
    a.grad_accumulate = accumulate;
    a.ln_accumulate = ln_accumulate;
    a.dout = d;
    a.dz = dz;
    a.ln_x_w = a.ln_z_w = w->ln_in_w;
    a.ln_x_b = a.ln_z_b = w->ln_in_b;
    a.eps = w->ln_eps;
    a.w_y = side == 0 ? w->w_a_proj : w->w_b_proj;
    a.w_t = side == 0 ? w->w_a_gate : w->w_b_gate;
    a.wt = ws + L.wt_off;
    a.tot = reinterpret_cast<float *>(ws + L.tot_off);
    a.part = reinterpret_cast<float *>(ws + L.part_off);
    a.g_w_y = side == 0 ? grads->w_a_proj : grads->w_b_proj;
    a.g_w_t = side == 0 ? grads->w_a_gate : grads->w_b_gate;
    a.g_ln_z_w = grads->ln_in_w;
    a.g_ln_z_b = grads->ln_in_b;
    const hipError_t e = trimul::launch_k3b(a, w->dtype, true, s);
    if (e != hipSuccess) return hip_fail(e, "projection backward kernel launch");
    // the second side adds its input-LayerNorm share to the first's
    ln_accumulate = true;
  }
  return ok();
}

trimul_status_t trimul_atom_window_attention(int64_t batch, int64_t n_atoms, int32_t heads, int32_t head_dim,
                                             const void *q, const void *k, const void *v, const void *bias,
                                             const uint8_t *atom_mask, float scale, float *out, void *stream) {
  if (batch < 1 || n_atoms < 1) return fail(TRIMUL_ERR_INVALID_ARG, "batch=%lld n_atoms=%lld must be >= 1", (long long)batch, (long long)n_atoms);
  if (head_dim != 32) return fail(TRIMUL_ERR_UNSUPPORTED, "head_dim=%d: only 32 is supported", head_dim);
  if (heads < 1 || heads > 1024) return fail(TRIMUL_ERR_INVALID_ARG, "heads=%d outside [1, 1024]", heads);
  const int64_t n_windows = (n_atoms + 31) / 32;
  if (batch > (int64_t(1) << 40) / n_atoms || batch * n_windows > 0x7fffffff)
    return fail(TRIMUL_ERR_INVALID_ARG, "batch * n_atoms too large");
  if (!q || !k || !v || !out) return fail(TRIMUL_ERR_INVALID_ARG, "q, k, v and out are required");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || (bias && !aligned(bias, 16)))
    return fail(TRIMUL_ERR_ALIGNMENT, "q, k, v, bias and out must be 16-byte aligned");
  if (!(scale == scale) || scale > 1e30f || scale < -1e30f) return fail(TRIMUL_ERR_INVALID_ARG, "scale must be finite");
  trimul::KAArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.bias = bias;
  a.mask = atom_mask;
  a.out = out;
  a.batch = batch;
  a.n_atoms = n_atoms;
  a.n_windows = n_windows;
  a.heads = heads;
  a.scale = scale;
  const hipError_t e = trimul::launch_ka(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "window attention kernel launch");
  return ok();
}

const char *trimul_status_string(trimul_status_t s) {
  switch (s) {
    case TRIMUL_OK: return "ok";
    case TRIMUL_ERR_INVALID_ARG: return "invalid argument";
    case TRIMUL_ERR_UNSUPPORTED: return "unsupported configuration";
    case TRIMUL_ERR_ALIGNMENT: return "misaligned pointer";
    case TRIMUL_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TRIMUL_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *trimul_last_error(void) { return g_last_error; }

}  // extern "C"
