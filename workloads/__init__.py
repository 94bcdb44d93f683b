"""Seeded synthetic inputs for the triangle multiplicative update.

This package produces input data only: pair tensors, pair masks and layer
weights.  It holds none of the update's arithmetic, and it is the one piece of
code that both the HIP path's callers (tests, benchmark) and the float64
oracle consume, so that both sides see bit-identical inputs.

Workloads (sizes from the pages, values synthetic):

* ``n64_f32``     -- N=64 single chain, fp32, all pairs valid.
* ``n768_pad``    -- N=768, the Boltz-2 training crop named on page 1
                     ("Os numeros"); the last 10% of residues (77) are
                     padding with mask 0.
* ``n3605_4ch``   -- N=3605 in 4 chains (1200/1000/800/605 residues), the
                     complex folded on 4 GPUs in page 1's "Os numeros"; each
                     ordered pair of distinct chains gets one c_z-vector offset
                     drawn from N(0, 0.5^2), added to its inter-chain block.
* ``n6500_2ch``   -- N=6500 in 2 chains of 3250, the PPI size of page 1's
                     "Quem ja ta usando"; 3% of residues (195) masked out at
                     random.
* ``n10000_tile`` -- N=10000, the 10,000-residue grid of page 1's "2D tiling
                     da pair representation", split 2 x 2: one device's tile
                     is rows 0-4999 x cols 0-4999, and its k-contraction
                     streams in 8 chunks of 1250 residues.
* ``n14000_chunked`` -- N=14000, a grid whose whole-grid workspace does not
                     fit beside z and the output on one device (page 1's
                     "O problema dos workarounds atuais": chunking is the
                     single-GPU workaround); run in the memory-bounded form
                     with 3584-row output blocks (14 contraction tiles) at
                     full width and k in one chunk, so both operands are
                     built once; 2% random residues masked out.

Every workload uses c_z = c = 128, z ~ N(0, 1), Xavier-normal weights (one
draw per logical matrix), LayerNorm gamma = 1 and beta = 0.

Random streams: the pair tensor is drawn in blocks of ``ROW_BLOCK`` rows; block
b uses its own generator seeded from (seed, "z", b), so any row block can be
regenerated alone.  z is drawn as float32 standard normals with torch's
generator on the target device (so large tensors are made on the GPU) and
cast round-to-nearest-even to the storage dtype; consumers that need z on the
host copy the stored tensor, so the values are identical by construction.
Weights, offsets and masks are drawn with numpy in float64 on the host.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

ROW_BLOCK = 64

_TAG_Z, _TAG_W, _TAG_MASK, _TAG_OFF, _TAG_LN = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    dtype: str                      # storage/compute dtype of z and weights: "bf16" or "f32"
    seed: int
    c_z: int = 128
    c: int = 128
    chains: tuple = ()              # chain lengths; empty = single chain
    chain_offset_std: float = 0.0   # std of the per-(chain, chain) offset vectors
    pad_fraction: float = 0.0       # trailing residues with mask 0
    masked_fraction: float = 0.0    # random residues with mask 0
    tile: dict = field(default_factory=dict)  # tiled form: rows, cols, chunk, n_chunks
    chunked: dict = field(default_factory=dict)  # memory-bounded form: row_block, col_block, k_block


WORKLOADS = {
    "n64_f32": Workload("n64_f32", 64, "f32", seed=1),
    "n768_pad": Workload("n768_pad", 768, "bf16", seed=2, pad_fraction=0.10),
    "n3605_4ch": Workload("n3605_4ch", 3605, "bf16", seed=3, chains=(1200, 1000, 800, 605),
                          chain_offset_std=0.5),
    "n6500_2ch": Workload("n6500_2ch", 6500, "bf16", seed=4, chains=(3250, 3250),
                          masked_fraction=0.03),
    "n10000_tile": Workload("n10000_tile", 10000, "bf16", seed=5,
                            tile={"row_off": 0, "n_rows": 5000, "col_off": 0, "n_cols": 5000,
                                  "chunk": 1250, "n_chunks": 8}),
    "n14000_chunked": Workload("n14000_chunked", 14000, "bf16", seed=6, masked_fraction=0.02,
                               chunked={"row_block": 3584, "col_block": 0, "k_block": 0}),
}


def _seed(*key):
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, np.uint32)[0])


def _rng(*key):
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([int(k) for k in key])))


def torch_dtype(dtype):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

def make_weights(c_z=128, c=128, seed=0, dtype="bf16", random_ln=False):
    """Layer weights as CPU torch tensors in storage precision.

    Matrices (out_features, in_features): w_a_proj, w_a_gate, w_b_proj,
    w_b_gate [c, c_z]; w_out_gate [c_z, c_z]; w_out_proj [c_z, c].  Each is
    Xavier-normal on its own shape, std = sqrt(2 / (fan_in + fan_out)), drawn
    in float64 and rounded to the storage dtype.  LayerNorm vectors are fp32:
    gamma = 1, beta = 0, or with ``random_ln`` gamma ~ 1 + N(0, 0.1^2) and
    beta ~ N(0, 0.1^2).
    """
    shapes = {
        "w_a_proj": (c, c_z), "w_a_gate": (c, c_z), "w_b_proj": (c, c_z), "w_b_gate": (c, c_z),
        "w_out_gate": (c_z, c_z), "w_out_proj": (c_z, c),
    }
    td = torch_dtype(dtype)
    out = {}
    for idx, (name, (fo, fi)) in enumerate(shapes.items()):
        std = np.sqrt(2.0 / (fi + fo))
        v = _rng(seed, _TAG_W, idx).standard_normal((fo, fi)) * std
        out[name] = torch.from_numpy(v).to(torch.float32).to(td).contiguous()
    if random_ln:
        r = _rng(seed, _TAG_LN)
        out["ln_in_w"] = torch.from_numpy(1.0 + 0.1 * r.standard_normal(c_z)).float()
        out["ln_in_b"] = torch.from_numpy(0.1 * r.standard_normal(c_z)).float()
        out["ln_out_w"] = torch.from_numpy(1.0 + 0.1 * r.standard_normal(c)).float()
        out["ln_out_b"] = torch.from_numpy(0.1 * r.standard_normal(c)).float()
    else:
        out["ln_in_w"] = torch.ones(c_z, dtype=torch.float32)
        out["ln_in_b"] = torch.zeros(c_z, dtype=torch.float32)
        out["ln_out_w"] = torch.ones(c, dtype=torch.float32)
        out["ln_out_b"] = torch.zeros(c, dtype=torch.float32)
    return out


def weights_f64(wts):
    """The same weights as float64 numpy arrays (exact copies of the stored values)."""
    return {k: v.detach().to("cpu", torch.float64).numpy() for k, v in wts.items()}


# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------

def residue_mask(wl: Workload):
    """uint8 [N] residue mask: 1 = valid residue."""
    r = np.ones(wl.n, dtype=np.uint8)
    if wl.pad_fraction > 0:
        n_pad = int(np.ceil(wl.pad_fraction * wl.n))
        r[wl.n - n_pad:] = 0
    if wl.masked_fraction > 0:
        n_m = int(round(wl.masked_fraction * wl.n))
        idx = _rng(wl.seed, _TAG_MASK).choice(wl.n, size=n_m, replace=False)
        r[idx] = 0
    return r


def pair_mask_from_residues(r_rows, r_cols=None):
    """uint8 pair mask m_ij = r_i * r_j."""
    r_rows = np.asarray(r_rows, dtype=np.uint8)
    r_cols = r_rows if r_cols is None else np.asarray(r_cols, dtype=np.uint8)
    return np.ascontiguousarray(np.outer(r_rows, r_cols).astype(np.uint8))


def random_pair_mask(n, seed, keep=0.9):
    """uint8 [n, n] pair mask with independent Bernoulli(keep) entries (tests)."""
    return (_rng(seed, _TAG_MASK, 7).random((n, n)) < keep).astype(np.uint8)


# ---------------------------------------------------------------------------
# pair tensor
# ---------------------------------------------------------------------------

def chain_ids(wl: Workload):
    if not wl.chains:
        return np.zeros(wl.n, dtype=np.int64)
    assert sum(wl.chains) == wl.n
    return np.repeat(np.arange(len(wl.chains)), wl.chains)


def chain_offsets(wl: Workload):
    """[n_chains, n_chains, c_z] offsets: N(0, std^2) vectors for ordered pairs of
    distinct chains, zero on the diagonal (intra-chain blocks)."""
    nc = max(1, len(wl.chains))
    off = np.zeros((nc, nc, wl.c_z))
    if wl.chain_offset_std > 0:
        r = _rng(wl.seed, _TAG_OFF)
        for p in range(nc):
            for q in range(nc):
                if p != q:
                    off[p, q] = wl.chain_offset_std * r.standard_normal(wl.c_z)
    return off


def make_pair_tensor(n, c_z, seed, dtype, device, chains=None, offsets=None, rows=None):
    """z [len(rows) or n, n, c_z] in storage dtype on ``device``.

    Row block b (rows [64b, 64b+64)) is drawn from its own generator, so
    ``rows=range(r0, r1)`` with r0 a multiple of 64 reproduces those rows of
    the full tensor (on the same device type).  ``chains`` (int array [n]) and
    ``offsets`` ([nc, nc, c_z]) add the inter-chain offset vectors before the
    cast.
    """
    dev = torch.device(device)
    r0, r1 = (0, n) if rows is None else (rows[0], rows[-1] + 1)
    assert r0 % ROW_BLOCK == 0
    z = torch.empty((r1 - r0, n, c_z), dtype=torch_dtype(dtype), device=dev)
    if offsets is not None:
        off_t = torch.as_tensor(offsets, dtype=torch.float32, device=dev)
        ch_t = torch.as_tensor(chains, dtype=torch.long, device=dev)
    for b0 in range(r0, r1, ROW_BLOCK):
        b1 = min(r1, b0 + ROW_BLOCK)
        g = torch.Generator(device=dev)
        g.manual_seed(_seed(seed, _TAG_Z, b0 // ROW_BLOCK))
        blk = torch.randn((min(n, b0 + ROW_BLOCK) - b0, n, c_z), generator=g, device=dev,
                          dtype=torch.float32)[: b1 - b0]
        if offsets is not None:
            blk += off_t[ch_t[b0:b1]][:, ch_t]
        z[b0 - r0:b1 - r0] = blk.to(z.dtype)
    return z


def make_inputs(wl: Workload, device="cpu", random_ln=False):
    """(z, mask, weights) for a workload; z and mask on ``device``."""
    offsets = chain_offsets(wl) if wl.chain_offset_std > 0 else None
    z = make_pair_tensor(wl.n, wl.c_z, wl.seed, wl.dtype, device,
                         chains=chain_ids(wl) if offsets is not None else None, offsets=offsets)
    mask = torch.from_numpy(pair_mask_from_residues(residue_mask(wl))).to(device)
    w = make_weights(wl.c_z, wl.c, wl.seed, wl.dtype, random_ln=random_ln)
    return z, mask, w


def make_small(n, c_z=128, c=128, seed=0, dtype="bf16", device="cpu", random_ln=True,
               mask_keep=0.9):
    """Test-sized inputs: random pair mask (Bernoulli keep), random LN affine."""
    z = make_pair_tensor(n, c_z, seed, dtype, device)
    mask = torch.from_numpy(random_pair_mask(n, seed, mask_keep) if mask_keep < 1
                            else np.ones((n, n), np.uint8)).to(device)
    w = make_weights(c_z, c, seed, dtype, random_ln=random_ln)
    return z, mask, w
