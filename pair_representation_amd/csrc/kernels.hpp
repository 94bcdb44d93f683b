// Kernel argument blocks and host-side launchers of the three kernels.
//   K1 (k1_project.hip)  input LayerNorm + gated a/b projections + mask,
//                        written as channel-planar k-contiguous operand planes
//   K2 (k2_contract.hip) channel-batched k-contraction on the matrix cores,
//                        streaming k-chunks in the given order
//   K3 (k3_epilogue.hip) output LayerNorm + output projection + output gate
//                        + pair mask, fp32 output
//   KB (kb_relayout.hip) layout copies and transposes for the contraction's
//                        gradients
//   K3B (k3b_epilogue_grad.hip) backward of the epilogue (dL/dx, the gate
//                        path's dL/dz, its parameter gradients) and of the
//                        projections (their dL/dz and parameter gradients)
//   KA (ka_window_attention.hip) window-batched atom attention (32 x 128)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "trimul.h"

namespace trimul {

struct K1Args {
  const void *z;          // [n][n][c_z] global pair tensor
  const uint8_t *mask;    // [n][n]
  int64_t n;
  int64_t row_base;       // source residue of plane row 0
  int64_t n_rows;         // plane rows
  int64_t k_off, k_len;   // source residues of plane columns 0 .. k_len-1
  int64_t ld;             // plane row length (multiple of 64); columns >= k_len get zeros
  int32_t transposed;     // 0: plane (r, t) <- pair (row_base+r, k_off+t); 1: pair (k_off+t, row_base+r)
  void *a_out;            // [c][n_rows][ld] or null
  void *b_out;            // [c][n_rows][ld] or null
  const float *ln_w, *ln_b;
  float eps;
  const void *w_a_proj, *w_a_gate, *w_b_proj, *w_b_gate;
};

struct K2Chunk {
  const void *a;          // [c][M][ld]
  const void *b;          // [c][N][ld]
  int64_t ld;
  int64_t k_len;          // residues in the chunk; columns k_len .. round_up(k_len, BK) must be 0
  int32_t ktiles;         // k-tiles of this chunk (filled by the launcher)
  int32_t pad_;
};

struct K2Args {
  K2Chunk ch[TRIMUL_MAX_CHUNKS];
  int32_t n_chunks;
  int32_t accumulate;     // 1: x += result, 0: x = result
  int32_t slots;          // work-groups resident at once (multiple of 8; set by the launcher)
  int32_t group_m;        // tile-rows per group of the tile order (set by the launcher)
  int64_t M, N;           // tile rows (a operand rows), tile cols (b operand rows)
  float *x;               // [c][round_up(M,4)/4][ldx][4] (4-row blocks), ldx = round_up(N,16)
  int64_t ldx;
};

struct K3Args {
  const float *x;         // [c][round_up(n_rows,4)/4][ldx][4] contraction result of the tile
  int64_t ldx;
  const void *z;          // [n][n][c_z] global
  const uint8_t *mask;    // [n][n] global
  int64_t n;
  int64_t row_off, n_rows, col_off, n_cols;
  float *out;             // [n_rows][out_ld][c_z]: pair (r, s) of the tile at out + (r * out_ld + s) * c_z
  int64_t out_ld;         // pairs between consecutive tile rows of out (>= n_cols)
  const float *ln_out_w, *ln_out_b, *ln_in_w, *ln_in_b;
  float eps;
  const void *w_out_proj;  // [c_z][c]
  const void *w_out_gate;  // [c_z][c_z]
};

// KB (kb_relayout.hip): 64 x 64 tile copies between the x layout and the
// operand layout, and operand-plane transposes, for the contraction's
// gradients (dA = dX B, dB = dX^T A).
struct RelayoutArgs {
  const float *x;         // fp32 source in the x layout (from_x), ldx its padded columns
  int64_t ldx;
  const void *src;        // operand-layout source of the element type (otherwise)
  int64_t ld_src;         // >= round_up(cols, 64)
  int64_t rows, cols;     // valid rows / columns of the source matrix
  void *p;                // [c][rows][ld_p] same orientation (operand layout) or null
  int64_t ld_p;           // >= round_up(cols, 64); columns cols .. round_up(cols, 64) get zeros
  void *q;                // [c][cols][ld_q] transpose (operand layout) or null
  int64_t ld_q;           // >= round_up(rows, 64); columns rows .. round_up(rows, 64) get zeros
};

// K3B (k3b_epilogue_grad.hip): backward of a gated, masked pair of 128 x 128
// linear maps after LayerNorm, on a grid of n_rows x n_cols positions:
//   out = m * sigmoid(W_t LN_z(z)) * (W_y LN_x(x))
// Epilogue mode: x = the contraction result, W_y = W_out_proj, W_t =
// W_out_gate, LN_x = the output LayerNorm, LN_z = the input LayerNorm.
// Projection mode: x = z (LN_x = LN_z = the input LayerNorm), W_y / W_t = one
// side's projection / gate matrices, out = that side's operand.
struct K3BArgs {
  const float *x;         // epilogue: the contraction result (x layout, ldx)
  int64_t ldx;            // row length of the x-layout buffers (x, dx; dout in projection mode)
  const void *z;          // [n][n][c_z] global
  const uint8_t *mask;    // [n][n] global
  int64_t n;
  int64_t row_off, n_rows, col_off, n_cols;   // position (r, c) is pair (row_off + r, col_off + c),
  int32_t transposed;                         // or (col_off + c, row_off + r) when transposed
  int32_t grad_accumulate;                    // matrix gradients: 1 add, 0 overwrite
  int32_t ln_accumulate;                      // LayerNorm-parameter gradients: 1 add, 0 overwrite
  const float *dout;      // dL/dout: epilogue [n_rows][n_cols][c_z]; projection x layout (ldx)
  float *dx;              // epilogue: dL/dx, x layout (may be x itself)
  float *dz;              // epilogue: [n_rows][n_cols][c_z] written; projection: [n][n][c_z] added to
  const float *ln_x_w, *ln_x_b, *ln_z_w, *ln_z_b;
  float eps;
  const void *w_y, *w_t;  // [128][128] in the element type
  void *wt;               // workspace: W_y^T, W_t^T (element type)
  float *part;            // workspace: kK3BMaxParts slots of kK3BSlotFloats
  float *tot;             // workspace: one slot, the sums over all work-groups
  int32_t n_parts;        // work-groups (set by the launcher)
  float *g_w_y, *g_w_t, *g_ln_x_w, *g_ln_x_b, *g_ln_z_w, *g_ln_z_b;   // projection: g_ln_x_* unused
};
// KA (ka_window_attention.hip): window-batched sequence-local atom attention.
struct KAArgs {
  const void *q, *k, *v;  // bf16 [batch][n_atoms][heads][32]
  const void *bias;       // bf16 [batch][n_windows][heads][32][128] or null
  const uint8_t *mask;    // [batch][n_atoms] (nonzero keeps the atom as a key) or null
  float *out;             // fp32 [batch][n_atoms][heads][32]
  int64_t batch, n_atoms, n_windows, heads;
  float scale;            // logit scale
};

// Slot of one work-group's partial sums: G [128][128], H [128][128], S [128], T [128].
constexpr int kK3BSlotFloats = 2 * 128 * 128 + 2 * 128;
constexpr int kK3BMaxParts = 256;

// Each launcher checks the launch with hipGetLastError.  dtype is
// TRIMUL_F32 or TRIMUL_BF16.
hipError_t launch_k1(const K1Args &a, int dtype, hipStream_t s);
hipError_t launch_k2(K2Args a, int dtype, hipStream_t s);
hipError_t launch_k3(const K3Args &a, int dtype, hipStream_t s);
hipError_t launch_relayout(const RelayoutArgs &a, bool from_x, int dtype, hipStream_t s);
hipError_t launch_k3b(K3BArgs a, int dtype, bool projection, hipStream_t s);
hipError_t launch_ka(const KAArgs &a, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace trimul
