/*
 * trimul.h -- C ABI of the MI355X (gfx950) triangle multiplicative update.
 *
 * The operation is the pair-representation layer that page 1 ("NVIDIA BioNeMo
 * escala modelagem biomolecular com context parallelism e quebra barreira de
 * memoria da GPU", section "Exemplo de codigo: triangle multiplication
 * CP-aware") builds as TriangleMultiplicationOutgoing(size_input_embed) and
 * calls as layer(x, mask).  The pages do not print its equations; this library
 * computes the AlphaFold3-style definition, per pair (i, j):
 *
 *   zh_ij  = LN(z_ij; ln_in_w, ln_in_b)
 *   a_ij   = m_ij * sigmoid(W_a_gate zh_ij) * (W_a_proj zh_ij)
 *   b_ij   = m_ij * sigmoid(W_b_gate zh_ij) * (W_b_proj zh_ij)
 *   x_ij   = sum_k a_ik * b_jk            (outgoing)
 *   x_ij   = sum_k a_ki * b_kj            (incoming)
 *   out_ij = m_ij * sigmoid(W_out_gate zh_ij) * (W_out_proj LN(x_ij; ln_out_w, ln_out_b))
 *
 * LN is LayerNorm over channels with biased variance; no linear map has a bias;
 * the output is the update only (no residual).  Page 1's section "2D tiling
 * da pair representation" splits the N x N grid into sub-blocks, one per
 * device, and its section "Sobreposicao de computacao e comunicacao" streams
 * the remote operand blocks around row and column rings while the local update
 * runs: trimul_tile_operands / trimul_tile are that per-device step, with the
 * k-contraction fed chunk by chunk in the order the ring delivers them.
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *    buffer; the library never allocates, frees or synchronizes.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *    default stream) and the call returns once enqueued.  Device faults
 *    surface at the caller's next synchronization.
 *  - All arguments are validated before the first HIP call; an invalid call
 *    enqueues nothing and returns a status code.  trimul_last_error() gives a
 *    message for the most recent failure on the calling thread.
 *  - Device pointers must be 16-byte aligned (the pair mask: any alignment);
 *    workspaces 256-byte aligned.
 *  - Supported widths: c_z = c = 128.  Supported sizes: 0 <= n <= 65535
 *    (n = 0 is a no-op).
 *  - Results are deterministic (no atomics; fixed summation order for a fixed
 *    chunk order).  Calls on different streams with different workspaces may
 *    run concurrently.
 *
 * Precision.  TRIMUL_F32: z, weights, a/b operands and every product in fp32
 * (matrix cores in fp32 mode).  TRIMUL_BF16: z and the five matrices are
 * bf16; LayerNorm statistics, sigmoid and all accumulation are fp32; the
 * normalised input and the a/b operands are rounded to bf16 (nearest-even)
 * for the bf16 matrix-core projection and contraction; the output LayerNorm
 * result and the normalised input feeding the output gate are split into two
 * bf16 terms (hi + lo, together within 2^-16 of the value) so the epilogue
 * products keep about 16 significant bits instead of bf16's 8.  The
 * output is fp32 in both modes.
 */
#ifndef TRIMUL_H
#define TRIMUL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TRIMUL_OK = 0,
  TRIMUL_ERR_INVALID_ARG = 1,         /* null pointer, bad size, range or flag        */
  TRIMUL_ERR_UNSUPPORTED = 2,         /* c_z or c other than 128, unknown dtype       */
  TRIMUL_ERR_ALIGNMENT = 3,           /* a pointer or leading dimension misaligned     */
  TRIMUL_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes < trimul_workspace_bytes()    */
  TRIMUL_ERR_HIP = 5                  /* a kernel launch or device query failed        */
} trimul_status_t;

typedef enum { TRIMUL_F32 = 0, TRIMUL_BF16 = 1 } trimul_dtype_t;
typedef enum { TRIMUL_OUTGOING = 0, TRIMUL_INCOMING = 1 } trimul_dir_t;

/* Flags of trimul_tile. */
enum { TRIMUL_TILE_FIRST = 1u, TRIMUL_TILE_LAST = 2u };
/* Flag of the backward entry points that produce parameter gradients
 * (trimul_epilogue_backward, trimul_tile_operands_backward): add them to the
 * grads buffers instead of overwriting them. */
enum { TRIMUL_GRAD_ACCUMULATE = 1u };

/* Largest number of k-chunks one trimul_tile call accepts. */
#define TRIMUL_MAX_CHUNKS 32

/* The layer's parameters (its state dict).  Matrices are row-major
 * (out_features, in_features), i.e. torch Linear.weight, in `dtype`
 * (fp32 or bf16); LayerNorm vectors are always fp32. */
typedef struct {
  int32_t c_z;                 /* pair channels; must be 128                   */
  int32_t c;                   /* hidden channels; must be 128                 */
  int32_t dtype;               /* trimul_dtype_t of z and of the matrices      */
  float ln_eps;                /* LayerNorm epsilon, > 0 (1e-5 usual)           */
  const float *ln_in_w;        /* [c_z] input LayerNorm gamma                   */
  const float *ln_in_b;        /* [c_z] input LayerNorm beta                    */
  const void *w_a_proj;        /* [c][c_z]                                      */
  const void *w_a_gate;        /* [c][c_z]                                      */
  const void *w_b_proj;        /* [c][c_z]                                      */
  const void *w_b_gate;        /* [c][c_z]                                      */
  const void *w_out_gate;      /* [c_z][c_z]                                    */
  const float *ln_out_w;       /* [c] output LayerNorm gamma                    */
  const float *ln_out_b;       /* [c] output LayerNorm beta                     */
  const void *w_out_proj;      /* [c_z][c]                                      */
} trimul_weights_t;

/* One k-chunk of the contraction for a tile: the operands of residues
 * k_off .. k_off+k_len-1, as two operand buffers
 *   a[d][r][t] = operand of (row_off + r, k_off + t),  r < n_rows, t < ld
 *   b[d][s][t] = operand of (col_off + s, k_off + t),  s < n_cols, t < ld
 * where "operand of (i, k)" is a_ik, b_jk for outgoing and a_ki, b_kj for
 * incoming (incoming operands are stored transposed so one layout serves
 * both).  Element type = the weights' dtype.  ld is a multiple of 64,
 * ld >= k_len, and columns k_len .. ld-1 must hold zeros (trimul_tile_operands
 * writes them).
 *
 * Operand layout: blocks of 256 rows x 64 columns; element [d][r][t] sits at
 *   ((r/256 * ld/64 + t/64) * 128 + d) * 16384 + (r%256) * 64 + t%64
 * i.e. the 128 channel blocks of one (row block, column block) are adjacent
 * and rows are padded to a multiple of 256 (padding rows are never read into
 * a stored result; trimul_tile_operand_bytes gives the size). */
typedef struct {
  int64_t k_off;
  int64_t k_len;
  int64_t ld;
  const void *a;
  const void *b;
} trimul_kchunk_t;

/* Bytes of workspace trimul_outgoing / trimul_incoming need for size n (the
 * buffers between the three steps of the layer of page 1, section "Exemplo de
 * codigo: triangle multiplication CP-aware"): the
 * a and b operands of all n rows with ld = round_up(n, 64) in the operand
 * layout of trimul_kchunk_t (element = dtype), and the fp32 contraction result
 * in the x_acc layout of trimul_tile for an n x n tile, each rounded up to 256
 * bytes.  Returns 0 for an invalid w or n. */
size_t trimul_workspace_bytes(const trimul_weights_t *w, int64_t n);

/* The full update over an n x n pair grid, outgoing direction: the layer that
 * page 1 builds as TriangleMultiplicationOutgoing(size_input_embed) and calls
 * as layer(x, mask) (section "Exemplo de codigo: triangle multiplication
 * CP-aware"), on one device that holds the whole grid.
 *   z    : [n][n][c_z] in w->dtype, pair-major (channels contiguous)
 *   mask : [n][n] uint8, nonzero = keep the pair
 *   out  : [n][n][c_z] fp32, fully overwritten (zeros at masked pairs)
 *   workspace : >= trimul_workspace_bytes(w, n) bytes, 256-byte aligned;
 *               contents on entry are ignored, on return unspecified.
 * Errors: TRIMUL_ERR_INVALID_ARG (NULL pointer, n outside [0, 65535]),
 * TRIMUL_ERR_UNSUPPORTED / _ALIGNMENT / _WORKSPACE_TOO_SMALL as named, all
 * detected before anything is enqueued; TRIMUL_ERR_HIP if a launch fails. */
trimul_status_t trimul_outgoing(const trimul_weights_t *w, const void *z, const uint8_t *mask,
                                float *out, int64_t n, void *workspace, size_t workspace_bytes,
                                void *stream);

/* The same for the incoming direction (x_ij = sum_k a_ki * b_kj), the
 * layer's other orientation (page 1, section "Exemplo de codigo: triangle
 * multiplication CP-aware", where the direction is the wrapper's parameter);
 * arguments, ownership and errors as trimul_outgoing. */
trimul_status_t trimul_incoming(const trimul_weights_t *w, const void *z, const uint8_t *mask,
                                float *out, int64_t n, void *workspace, size_t workspace_bytes,
                                void *stream);

/* Bytes of workspace trimul_forward_chunked needs: with R = row_block,
 * C = col_block, K = k_block (each 0 or > n meaning n),
 *   align256(c * round_up(R, 256) * round_up(K, 64) * elt)      a chunk
 * + align256(c * round_up(C, 256) * round_up(K, 64) * elt)      b chunk
 * + align256(c * round_up(R, 4) * round_up(C, 16) * 4)           tile accumulator
 * (elt = 2 for bf16, 4 for fp32; c = 128).  Returns 0 for an invalid w, n or
 * a negative block. */
size_t trimul_chunked_workspace_bytes(const trimul_weights_t *w, int64_t n, int64_t row_block,
                                      int64_t col_block, int64_t k_block);

/* The full update of trimul_outgoing / trimul_incoming (dir selects) in
 * bounded device memory: the in-architecture chunking that page 1 names as
 * the single-GPU workaround for pair grids beyond one device's memory
 * (section "O problema dos workarounds atuais").  The output is produced one
 * R x C tile at a time (row-major tile order); for each tile the k range is
 * streamed in chunks of K residues: the chunk's a and b operands are built
 * (input LayerNorm, gated projections, mask) and contracted into the tile's
 * fp32 accumulator, and after the last chunk the epilogue writes the tile
 * into out.  Besides z, mask and out, device memory is the workspace only
 * (trimul_chunked_workspace_bytes), independent of n when R, C and K are
 * fixed.  With K < n the a operand of a tile is rebuilt for every column
 * tile and the b operand for every row tile, so the projection work grows as
 * n/C + n/R passes over z; with K = n, a is built once per row tile (1 + n/R
 * passes, b still rebuilt for every row tile), and with C = n as well b is
 * built once per call (2 passes; 2 - R/n when R is a multiple of 256, the
 * first tile's a and b then coming from one pass).
 * Arguments as trimul_outgoing plus dir and the three block sizes (>= 0;
 * 0 = n); errors as trimul_outgoing.  Results agree with trimul_outgoing /
 * trimul_incoming up to the fp32 summation order over k. */
trimul_status_t trimul_forward_chunked(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                       const uint8_t *mask, float *out, int64_t n, int64_t row_block,
                                       int64_t col_block, int64_t k_block, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Size of the device scratch array that trimul_forward_chunked_noalloc uses
 * in place of a workspace argument (256 MiB). */
#define TRIMUL_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* trimul_forward_chunked without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace lives in a
 * library-owned device array of TRIMUL_NOALLOC_SCRATCH_BYTES: one copy per
 * device, created when the library's code is first loaded on that device
 * and held until the process ends.  Its device address is looked up once per
 * device on the first call made with that device current.  Nothing is
 * allocated or freed by the call (no hipMalloc / hipFree, no allocating
 * library routine).
 *   Blocks as trimul_forward_chunked; trimul_chunked_workspace_bytes(w, n,
 *   row_block, col_block, k_block) must not exceed
 *   TRIMUL_NOALLOC_SCRATCH_BYTES, else TRIMUL_ERR_WORKSPACE_TOO_SMALL (with a
 *   message naming both sizes) and nothing is enqueued.  With all blocks 0
 *   that is the whole-grid workspace: n <= 512 (bf16) or n <= 356 (fp32);
 *   e.g. 512 x 512 x 512 (bf16) or 512 x 512 x 256 (fp32) blocks fit and
 *   serve any n.
 *   Results are bitwise those of trimul_forward_chunked with the same
 *   blocks.  Every call on a device shares that device's array and leaves
 *   its contents behind (no kernel reads scratch it has not written in the
 *   same call): calls that overlap in time on one device (other streams,
 *   other threads) race and must be serialized by the caller.
 *   Errors: as trimul_forward_chunked; TRIMUL_ERR_HIP if the array's
 *   address cannot be obtained. */
trimul_status_t trimul_forward_chunked_noalloc(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                               const uint8_t *mask, float *out, int64_t n,
                                               int64_t row_block, int64_t col_block, int64_t k_block,
                                               void *stream);

/* Bytes of one operand buffer of trimul_tile_operands (one ring message of
 * page 1, section "Sobreposicao de computacao e comunicacao"):
 * c * round_up(rows, 256) * ld * elt. */
size_t trimul_tile_operand_bytes(const trimul_weights_t *w, int64_t rows, int64_t ld);

/* The operand chunk a device owning z contributes for one tile (page 1,
 * section "2D tiling da pair representation": each device holds one block of
 * the pair grid; section "Sobreposicao de computacao e comunicacao": the
 * operand blocks travel around the row or column ring): runs the
 * input LayerNorm, gated projections and mask on the source pairs and writes
 *   a_out[d][r][t] = operand a of (row_off + r, k_off + t),  r < n_rows
 *   b_out[d][s][t] = operand b of (col_off + s, k_off + t),  s < n_cols
 * for t < k_len, zeros for k_len <= t < ld (layout of trimul_kchunk_t).
 * Either output may be NULL (not computed), not both.  z and mask are the
 * global [n][n] tensors.  Ranges must lie inside [0, n); ld % 64 == 0,
 * ld >= k_len >= 1. */
trimul_status_t trimul_tile_operands(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                     const uint8_t *mask, int64_t n, int64_t row_off,
                                     int64_t n_rows, int64_t col_off, int64_t n_cols,
                                     int64_t k_off, int64_t k_len, int64_t ld, void *a_out,
                                     void *b_out, void *stream);

/* Bytes of the fp32 tile accumulator x_acc of trimul_tile (the contraction
 * result of one device's tile, page 1, section "2D tiling da pair
 * representation"):
 * c * round_up(n_rows, 4) * round_up(n_cols, 16) * 4. */
size_t trimul_tile_xacc_bytes(const trimul_weights_t *w, int64_t n_rows, int64_t n_cols);

/* One device's tile of the pair grid (page 1, section "2D tiling da pair
 * representation"), contracting the k-chunks in the order the ring delivers
 * them while the next ones are in flight (section "Sobreposicao de computacao
 * e comunicacao").  There is no direction argument: incoming operands arrive
 * already transposed (trimul_tile_operands writes them so), which makes the
 * contraction and the epilogue identical for both directions.
 * Rows row_off .. row_off+n_rows-1, cols
 * col_off .. col_off+n_cols-1.  Contracts the given chunks (host array, in
 * arrival order) into the fp32 accumulator x_acc, stored in blocks of 4 rows
 * x 16 columns with the 128 channels of a block adjacent, so that the
 * contraction writes 16-byte groups and the epilogue reads one contiguous
 * 32 KB block per 64 pairs:
 *   x_(row_off+r, col_off+s), channel d, sits at element
 *   ((r/4 * ldx/16 + s/16) * 128 + d) * 64 + (s%16) * 4 + r%4,
 *   ldx = round_up(n_cols, 16), r < round_up(n_rows, 4)
 * (trimul_tile_xacc_bytes bytes; entries of rows past n_rows or columns past
 * n_cols are unspecified and never read into a result), overwriting it when
 * flags has
 * TRIMUL_TILE_FIRST and adding to it otherwise;
 * the partial sums stay in registers across the chunks of one call.  With
 * TRIMUL_TILE_LAST the epilogue then writes
 *   out_tile[r][s][e] (fp32, [n_rows][n_cols][c_z])
 * from x_acc and the global z / mask (needed only with LAST).
 * Chunks of one call must lie in [0, n) and not overlap; when FIRST and LAST
 * are both set they must cover [0, n) exactly.  Coverage across calls is the
 * caller's responsibility.  n_chunks may be 0 only with LAST alone (epilogue
 * on an already complete x_acc). */
trimul_status_t trimul_tile(const trimul_weights_t *w, int64_t n, int64_t row_off,
                            int64_t n_rows, int64_t col_off, int64_t n_cols,
                            const trimul_kchunk_t *chunks /* (host) */, int32_t n_chunks,
                            uint32_t flags, float *x_acc, const void *z, const uint8_t *mask,
                            float *out_tile, void *stream);

/* Backward of the k-contraction of one tile: the gradients a training step
 * needs from trimul_tile's contraction (page 1, section "Pra quem e": the
 * layer is trained through custom autograd functions; sections "O problema
 * dos workarounds atuais" and "A pegadinha": training and fine-tuning need
 * the large crops the tiling makes possible).  Per channel d the contraction
 * is x = A B^T over the stored operands, so given
 *   dx = dL/dx of the tile (fp32, the x_acc layout of trimul_tile, rows
 *        n_rows, columns n_cols; entries past them are ignored)
 * it writes, for every chunk c (host array; the operands as passed to
 * trimul_tile, only a, b, k_len and ld are used),
 *   da_out[c][d][r][t] = sum_s dx[d][r][s] * b_c[d][s][t]     r < n_rows
 *   db_out[c][d][s][t] = sum_r dx[d][r][s] * a_c[d][r][t]     s < n_cols
 * for t < k_len: the gradients with respect to the stored operands (for
 * incoming, stored transposed, da_out[c][d][r][t] is the gradient of
 * a_(k_off+t, row_off+r)).  da_out and db_out are host arrays of n_chunks
 * device pointers, fp32 in the x_acc layout with rows r (s) and columns t:
 * trimul_tile_xacc_bytes(w, n_rows, k_len) and (w, n_cols, k_len) bytes each,
 * fully overwritten.  In bf16 mode dx is rounded to bf16 (nearest-even) for
 * the matrix-core products, as the forward rounds a and b; accumulation is
 * fp32.  workspace >= trimul_tile_backward_workspace_bytes(...) bytes,
 * 256-byte aligned (dx and its transpose as operand buffers, one chunk's
 * transposed operands); contents on entry are ignored. */
size_t trimul_tile_backward_workspace_bytes(const trimul_weights_t *w, int64_t n_rows, int64_t n_cols,
                                            const trimul_kchunk_t *chunks /* (host) */, int32_t n_chunks);

trimul_status_t trimul_tile_backward(const trimul_weights_t *w, int64_t n_rows, int64_t n_cols,
                                     const trimul_kchunk_t *chunks /* (host) */, int32_t n_chunks,
                                     const float *dx, float *const *da_out /* (host) */,
                                     float *const *db_out /* (host) */, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Parameter gradients of the epilogue, fp32: overwritten, or added to with
 * TRIMUL_GRAD_ACCUMULATE. */
typedef struct {
  float *w_out_proj;           /* [c_z][c]   dL/dW_out_proj                      */
  float *w_out_gate;           /* [c_z][c_z] dL/dW_out_gate                      */
  float *ln_out_w;             /* [c]        dL/d(output LayerNorm gamma)        */
  float *ln_out_b;             /* [c]        dL/d(output LayerNorm beta)         */
  float *ln_in_w;              /* [c_z]      the output gate's share of
                                              dL/d(input LayerNorm gamma)        */
  float *ln_in_b;              /* [c_z]      the same for beta                   */
} trimul_epilogue_grads_t;

/* Backward of the epilogue of one tile (the step trimul_tile runs with
 * TRIMUL_TILE_LAST): the rest of the training step around
 * trimul_tile_backward (page 1, section "Pra quem e": the layer is trained
 * through custom autograd functions).  With n = LN(x; ln_out), y = W_out_proj n,
 * zh = LN(z; ln_in), s = sigmoid(W_out_gate zh) and out = m s y, given
 *   dout = dL/dout_tile ([n_rows][n_cols][c_z] fp32, the layout of out_tile)
 * and the forward's inputs (x_acc as trimul_tile left it, the global z and
 * mask) it writes
 *   dx     = dL/dx in the x_acc layout (rows n_rows, columns n_cols; entries
 *            past them are not written): the dx of trimul_tile_backward.
 *            dx may be x_acc itself (each pair's x is read before its dx is
 *            written).
 *   dz     = [n_rows][n_cols][c_z] fp32: the output gate's share of
 *            dL/dz_(row_off+r, col_off+s) (through ln_in and W_out_gate; the
 *            a/b projections contribute the rest)
 *   grads  = sums over the tile's pairs (masked pairs contribute nothing),
 *            overwritten, or added to with flags = TRIMUL_GRAD_ACCUMULATE (a
 *            layer split into tiles sums the tiles' results)
 * Masked pairs get dx = dz = 0.  The weight-matrix gradients are formed as
 * dW_out_proj = G diag(ln_out_w) + S ln_out_b^T with G = sum dy LN0(x)^T and
 * S = sum dy (dy = m s dout, LN0 = LayerNorm before its affine map), the
 * LayerNorm parameter gradients from the same sums (sum over o of
 * W_out_proj[o][k] G[o][k], W_out_proj^T S), and the gate's from the same
 * construction.  Precision: as the forward epilogue (bf16 mode: the stored
 * bf16 matrices, every other operand of a matrix-core product split into two
 * bf16 terms; fp32 mode: fp32 products), fp32 accumulation, a fixed summation
 * order.  workspace >= trimul_epilogue_backward_workspace_bytes(w) bytes,
 * 256-byte aligned (transposed matrices, per-work-group partial sums);
 * contents on entry are ignored. */
size_t trimul_epilogue_backward_workspace_bytes(const trimul_weights_t *w);

trimul_status_t trimul_epilogue_backward(const trimul_weights_t *w, int64_t n, int64_t row_off,
                                         int64_t n_rows, int64_t col_off, int64_t n_cols,
                                         const float *x_acc, const void *z, const uint8_t *mask,
                                         const float *dout, float *dx, float *dz, uint32_t flags,
                                         const trimul_epilogue_grads_t *grads /* (host) */,
                                         void *workspace, size_t workspace_bytes, void *stream);

/* Parameter gradients of the a/b projections, fp32. */
typedef struct {
  float *w_a_proj;             /* [c][c_z] dL/dW_a_proj (used when da != NULL)  */
  float *w_a_gate;             /* [c][c_z] dL/dW_a_gate (used when da != NULL)  */
  float *w_b_proj;             /* [c][c_z] dL/dW_b_proj (used when db != NULL)  */
  float *w_b_gate;             /* [c][c_z] dL/dW_b_gate (used when db != NULL)  */
  float *ln_in_w;              /* [c_z] the projections' share of
                                        dL/d(input LayerNorm gamma)             */
  float *ln_in_b;              /* [c_z] the same for beta                       */
} trimul_projection_grads_t;

/* Backward of trimul_tile_operands: the step that turns the gradients of one
 * operand chunk into gradients of z and of the projection parameters (page 1,
 * section "Pra quem e": the layer is trained through custom autograd
 * functions).  With zh = LN(z; ln_in) and, per side s in {a, b},
 *   s = m * sigmoid(W_s_gate zh) * (W_s_proj zh)
 * at the source pair of each operand entry (layout of trimul_tile_operands:
 * a row r <-> residue row_off + r, b row s <-> col_off + s, column t <->
 * residue k_off + t; outgoing pairs (row, k), incoming (k, row)), given
 *   da = dL/da_chunk, fp32 in the x_acc layout with rows n_rows, columns
 *        k_len (trimul_tile_xacc_bytes(w, n_rows, k_len); as
 *        trimul_tile_backward writes it), or NULL (side a skipped)
 *   db = dL/db_chunk likewise with rows n_cols, or NULL (not both NULL)
 * it ADDS to dz ([n][n][c_z] fp32, the global pair tensor's gradient; the
 * caller zeroes it or passes the epilogue's share) the projections' share of
 * dL/dz at every source pair, and writes the parameter gradients (sums over
 * the chunk's entries; masked entries contribute nothing), or adds them with
 * TRIMUL_GRAD_ACCUMULATE.  grads->w_a_* are used only with da, w_b_* only with
 * db; ln_in_* receive both sides' shares.  Everything is linear in (da, db),
 * so several chunks, tiles or sides may be fed by separate calls.  The
 * parameter gradients use the same G/S construction as
 * trimul_epilogue_backward (both projections of a side share the one input
 * LayerNorm); precision as there (fixed summation order).  Calls on one
 * stream run in order; the same dz must not be updated by concurrent calls.
 * workspace >= trimul_tile_operands_backward_workspace_bytes(w) bytes,
 * 256-byte aligned; contents on entry are ignored. */
size_t trimul_tile_operands_backward_workspace_bytes(const trimul_weights_t *w);

trimul_status_t trimul_tile_operands_backward(const trimul_weights_t *w, trimul_dir_t dir, const void *z,
                                              const uint8_t *mask, int64_t n, int64_t row_off,
                                              int64_t n_rows, int64_t col_off, int64_t n_cols,
                                              int64_t k_off, int64_t k_len, const float *da,
                                              const float *db, float *dz, uint32_t flags,
                                              const trimul_projection_grads_t *grads /* (host) */,
                                              void *workspace, size_t workspace_bytes, void *stream);

/* Window-batched sequence-local atom attention (page 1, section "Atom sequence
 * local attention eficiente": AlphaFold3 restricts atom attention to local
 * windows of 32 x 128, processed as a batch of windows).  Per sequence b, the
 * atoms are split into query blocks of 32 (block w = atoms 32w .. 32w+31, the
 * last one possibly partial); block w attends to the 128 atoms centred on it,
 * keys 32w - 48 .. 32w + 79, of which those inside the sequence and unmasked
 * take part.  Per head h:
 *   out_i = sum_j softmax_j(scale * q_i . k_j + bias[b][w][h][i - 32w][j - 32w + 48]) v_j
 * and out_i = 0 for a query whose window has no key left.
 *   q, k, v   : [batch][n_atoms][heads][head_dim] bf16, head_dim = 32
 *   bias      : [batch][ceil(n_atoms / 32)][heads][32][128] bf16 (the pair
 *               bias of each window: query row, key column), or NULL
 *   atom_mask : [batch][n_atoms] uint8, nonzero keeps the atom as a key, or NULL
 *   scale     : logit scale (1 / sqrt(head_dim) is the usual choice)
 *   out       : [batch][n_atoms][heads][head_dim] fp32, fully overwritten
 * Logits, softmax and accumulation are fp32; the probabilities enter the
 * bf16 matrix-core product with V as two bf16 terms (hi + lo).  Needs no
 * workspace. */
trimul_status_t trimul_atom_window_attention(int64_t batch, int64_t n_atoms, int32_t heads, int32_t head_dim,
                                             const void *q, const void *k, const void *v, const void *bias,
                                             const uint8_t *atom_mask, float scale, float *out, void *stream);

/* Static description of a status code. */
const char *trimul_status_string(trimul_status_t s);

/* Message for the most recent failing call on this thread ("" if none). */
const char *trimul_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TRIMUL_H */
