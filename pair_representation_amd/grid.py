"""The 2D-tiled form on one GPU: every device step of an s_rows x s_cols grid.

Page 1 ("NVIDIA BioNeMo escala modelagem biomolecular com context parallelism e
quebra barreira de memoria da GPU"), section "2D tiling da pair representation":
the N x N pair grid is split into one block per device.  Section "Sobreposicao
de computacao e comunicacao": the operand blocks a device needs for its
k-contraction travel around its row ring (outgoing) or its column ring
(incoming) and are contracted as they arrive, the device's own block first.

Here the devices are emulated one after another on one GPU.  For tile (p, q)
(rows I_p, columns J_q):
  outgoing  x_ij = sum_k a_ik b_jk: the k-blocks are the column blocks J_r, held
            by the devices (p, r) of the row ring, arriving in the order
            r = q, q+1, ..., q-1 (mod s_cols);
  incoming  x_ij = sum_k a_ki b_kj: the k-blocks are the row blocks I_r, held by
            the devices (r, q) of the column ring, arriving in the order
            r = p, p+1, ..., p-1 (mod s_rows).
Each arriving block is produced by trimul_tile_operands (what its owner would
send) and contracted by one trimul_tile call (FIRST on the first block, LAST on
the final one), exactly as a device would do it; the only other step is
placing each tile of the result into the full output.

An s x 1 split produces the output in row blocks with one block's contraction
result resident; it still builds a full-height b operand per block.  The
memory-bounded forward proper, which bounds a, b and the accumulator by
tiling the output in both directions and streaming k in chunks, is the
library's trimul_forward_chunked (binding: forward_chunked).

emulate_backward runs the same grid's backward (the training step the pages
make the point of the tiling): each tile's gradients from the library's three
backward entry points, summed over the tiles.

This module is host logic over the C ABI: it plans, allocates and calls; all
arithmetic of the method runs in the library's kernels.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

from . import (C_Z, EPILOGUE_GRAD_SHAPES, INCOMING, OUTGOING, PROJECTION_GRAD_SHAPES, TILE_FIRST, TILE_LAST, Weights,
               epilogue_backward, new_operand, new_xacc, tile, tile_backward, tile_operands, tile_operands_backward)


def split(n: int, parts: int) -> List[Tuple[int, int]]:
    """Contiguous near-equal blocks (offset, length) of range(n); the first
    n % parts blocks are one longer."""
    if parts < 1 or parts > max(n, 1):
        raise ValueError(f"cannot split {n} into {parts} blocks")
    base, extra = divmod(n, parts)
    out, off = [], 0
    for i in range(parts):
        ln = base + (1 if i < extra else 0)
        out.append((off, ln))
        off += ln
    return out


def ring_order(own: int, s: int) -> List[int]:
    """Arrival order of the s blocks on a ring, the device's own block first."""
    return [(own + t) % s for t in range(s)]


@dataclass
class TilePlan:
    p: int
    q: int
    row_off: int
    n_rows: int
    col_off: int
    n_cols: int
    k_blocks: List[Tuple[int, int]] = field(default_factory=list)   # (k_off, k_len) in arrival order


def plan(n: int, direction: int, s_rows: int, s_cols: int = None) -> List[TilePlan]:
    """The tiles of an s_rows x s_cols grid and, for each, its k-blocks in ring
    arrival order."""
    s_cols = s_rows if s_cols is None else s_cols
    rows, cols = split(n, s_rows), split(n, s_cols)
    tiles = []
    for p, (r0, rn) in enumerate(rows):
        for q, (c0, cn) in enumerate(cols):
            if direction == OUTGOING:
                kb = [cols[r] for r in ring_order(q, s_cols)]
            elif direction == INCOMING:
                kb = [rows[r] for r in ring_order(p, s_rows)]
            else:
                raise ValueError("direction must be OUTGOING or INCOMING")
            tiles.append(TilePlan(p, q, r0, rn, c0, cn, kb))
    return tiles


def emulate(z, mask, w: Weights, direction: int, s_rows: int, s_cols: int = None, out=None):
    """Run every device step of the grid on this GPU and assemble the full
    update [n, n, 128] fp32.  Each k-block is contracted by its own
    trimul_tile call, in the tile's ring order."""
    import torch

    n = z.shape[0]
    if out is None:
        out = torch.empty((n, n, 128), dtype=torch.float32, device=z.device)
    for t in plan(n, direction, s_rows, s_cols):
        ld = (max(kl for _, kl in t.k_blocks) + 63) // 64 * 64
        x = new_xacc(t.n_rows, t.n_cols, z.device)
        a = new_operand(t.n_rows, ld, w.torch_dtype, z.device)
        b = new_operand(t.n_cols, ld, w.torch_dtype, z.device)
        last = len(t.k_blocks) - 1
        out_tile = None
        for i, (k_off, k_len) in enumerate(t.k_blocks):
            # the block the ring delivers (its owner's K1) ...
            tile_operands(w, direction, z, mask, t.row_off, t.n_rows, t.col_off, t.n_cols, k_off, k_len, ld,
                          a_out=a, b_out=b)
            # ... contracted on arrival (the next block reuses the buffers:
            # calls on one stream run in order)
            flags = (TILE_FIRST if i == 0 else 0) | (TILE_LAST if i == last else 0)
            out_tile = tile(w, n, t.row_off, t.n_rows, t.col_off, t.n_cols, [(k_off, k_len, a, b)], flags, x,
                            z, mask)
        out[t.row_off:t.row_off + t.n_rows, t.col_off:t.col_off + t.n_cols].copy_(out_tile)
    return out


def emulate_backward(z, mask, w: Weights, direction: int, dout, s_rows: int, s_cols: int = None):
    """The grid's backward, every device step on this GPU: the gradients of
    L = sum(dout * layer(z)) with respect to z and all ten parameters.

    Each tile recomputes its forward state as a device would (its operand
    blocks in ring order, the contraction result), then runs
      - the epilogue's backward on its own pairs (its share of the gate path's
        dL/dz and of the epilogue's parameter gradients),
      - the contraction's backward over its blocks (dL/da, dL/db per block),
      - the projections' backward of each block, which adds dL/dz at the
        blocks' source pairs (owned by other devices of its ring: on a real
        grid these partial sums travel back around the ring).
    Parameter gradients are summed over all tiles by the library
    (GRAD_ACCUMULATE).  Two passes: every tile's gate-path dL/dz is placed
    before any projection backward adds to those pairs.  Returns
    (dz [n, n, 128] fp32, grads dict keyed by parameter name)."""
    import torch

    n = z.shape[0]
    dev = z.device
    f32 = torch.float32
    dz = torch.zeros((n, n, C_Z), dtype=f32, device=dev)
    g_epi = {k: torch.zeros(shp, dtype=f32, device=dev) for k, shp in EPILOGUE_GRAD_SHAPES.items()}
    g_proj = {k: torch.zeros(shp, dtype=f32, device=dev) for k, shp in PROJECTION_GRAD_SHAPES.items()
              if not k.startswith("ln_in")}
    g_proj["ln_in_w"], g_proj["ln_in_b"] = g_epi["ln_in_w"], g_epi["ln_in_b"]
    tiles = plan(n, direction, s_rows, s_cols)

    def forward_state(t):
        ld = (max(kl for _, kl in t.k_blocks) + 63) // 64 * 64
        blocks = []
        for k_off, k_len in t.k_blocks:
            a, b = tile_operands(w, direction, z, mask, t.row_off, t.n_rows, t.col_off, t.n_cols, k_off, k_len, ld)
            blocks.append((k_off, k_len, a, b))
        x = new_xacc(t.n_rows, t.n_cols, dev)
        tile(w, n, t.row_off, t.n_rows, t.col_off, t.n_cols, blocks, TILE_FIRST, x)
        return blocks, x

    dxs = []
    for t in tiles:                       # pass 1: epilogue backward per tile
        _, x = forward_state(t)
        dout_t = dout[t.row_off:t.row_off + t.n_rows, t.col_off:t.col_off + t.n_cols].contiguous()
        dx, dz_t, _ = epilogue_backward(w, n, t.row_off, t.n_rows, t.col_off, t.n_cols, x, z, mask, dout_t,
                                        grads=g_epi, accumulate=True)
        dz[t.row_off:t.row_off + t.n_rows, t.col_off:t.col_off + t.n_cols].copy_(dz_t)   # placement
        dxs.append(dx)
    for t, dx in zip(tiles, dxs):         # pass 2: contraction and projections
        blocks, _ = forward_state(t)
        da, db = tile_backward(w, t.n_rows, t.n_cols, blocks, dx)
        for (k_off, k_len, _, _), dai, dbi in zip(blocks, da, db):
            tile_operands_backward(w, direction, z, mask, t.row_off, t.n_rows, t.col_off, t.n_cols, k_off, k_len,
                                   da=dai, db=dbi, dz=dz, grads=g_proj, accumulate=True)
    grads = dict(g_epi)
    grads.update(g_proj)
    return dz, grads


def step_model(n: int, s: int, tflops: float, link_gbs: float, c: int = 128, elt_bytes: int = 2) -> dict:
    """Per ring step of an s x s grid: the contraction of one operand block
    pair against the transfer of one block over one link.  Returns both
    times, which one bounds the step, and the tile size n/s above which the
    step is compute-bound (2 (n/s)^3 c / F = (n/s)^2 c b / BW, so
    n/s = F b / (2 BW))."""
    t = n / s
    t_comp = 2.0 * t ** 3 * c / (tflops * 1e12)
    t_comm = t * t * c * elt_bytes / (link_gbs * 1e9)
    return {"tile": t, "compute_s": t_comp, "transfer_s": t_comm,
            "bound": "compute" if t_comp >= t_comm else "transfer",
            "crossover_tile": tflops * 1e12 * elt_bytes / (2.0 * link_gbs * 1e9)}
