"""The 2D-tiled form emulated on one GPU: every tile of an s_rows x s_cols grid,
each contracting its k-blocks one call at a time in its own ring order,
assembled into the full update.

Bars (max |diff| / rms(ref)):
  against the whole-grid entry point (same kernels, one k pass): only the
  order of fp32 summation over k differs                        <= 1e-4
  against the Q-mode oracle                                      <= 1e-2
"""

import pytest
import torch

import oracle
import pair_representation_amd as pra
from pair_representation_amd import grid
import workloads as wl
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu

DIRS = {"outgoing": pra.OUTGOING, "incoming": pra.INCOMING}


@pytest.fixture(scope="module")
def dev():
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


@pytest.fixture(scope="module")
def case(dev):
    n = 300
    z, mask, wts = wl.make_small(n, seed=21, dtype="bf16", device="cpu", random_ln=True, mask_keep=0.9)
    w = pra.Weights(wts, pra.BF16, device=dev)
    host = dict(z=z.double().numpy(), mask=mask.numpy(), w=wl.weights_f64(wts))
    return n, z.to(dev), mask.to(dev), w, host


@pytest.mark.parametrize("direction", list(DIRS))
@pytest.mark.parametrize("s_rows,s_cols", [(2, 2), (3, 3), (3, 1), (2, 3)])
def test_grid_emulation_matches_whole_grid(case, direction, s_rows, s_cols):
    n, z, mask, w, _ = case
    print(f"[case] grid {s_rows}x{s_cols} {direction} n={n}", flush=True)
    d = DIRS[direction]
    full = (pra.outgoing if d == pra.OUTGOING else pra.incoming)(z, mask, w)
    emu = grid.emulate(z, mask, w, d, s_rows, s_cols)
    torch.cuda.synchronize()
    e = rel_err(emu.double().cpu().numpy(), full.double().cpu().numpy())
    print(f"  vs whole grid {e:.3e}", flush=True)
    assert e <= 1e-4
    m = mask.bool()
    assert (emu[~m] == 0).all()


@pytest.mark.parametrize("direction", list(DIRS))
def test_grid_emulation_vs_oracle(case, direction):
    n, z, mask, w, host = case
    print(f"[case] grid 3x3 {direction} vs Q-oracle n={n}", flush=True)
    emu = grid.emulate(z, mask, w, DIRS[direction], 3)
    torch.cuda.synchronize()
    ref = oracle.trimul(host["z"], host["mask"], host["w"], direction, quant=True)
    e = rel_err(emu.double().cpu().numpy(), ref)
    print(f"  vs Q-oracle {e:.3e}", flush=True)
    assert e <= 1e-2


@pytest.mark.parametrize("direction", list(DIRS))
@pytest.mark.parametrize("s_rows", [2, 3, 5])
def test_row_block_mode_vs_oracle(case, direction, s_rows):
    """The s x 1 split (output produced one row block at a time, each block's
    k-blocks contracted in ring order) against the Q-mode oracle, not against
    the library's own whole-grid path."""
    n, z, mask, w, host = case
    print(f"[case] grid {s_rows}x1 {direction} vs Q-oracle n={n}", flush=True)
    emu = grid.emulate(z, mask, w, DIRS[direction], s_rows, 1)
    torch.cuda.synchronize()
    ref = oracle.trimul(host["z"], host["mask"], host["w"], direction, quant=True)
    e = rel_err(emu.double().cpu().numpy(), ref)
    print(f"  vs Q-oracle {e:.3e}", flush=True)
    assert e <= 1e-2
    assert (emu[~mask.bool()] == 0).all()


@pytest.mark.parametrize("direction", list(DIRS))
@pytest.mark.parametrize("s_rows,s_cols", [(2, 2), (3, 2), (3, 1)])
def test_grid_backward_matches_oracle(dev, direction, s_rows, s_cols):
    """The grid's backward (grid.emulate_backward: each tile's share from the
    three backward entry points, summed over tiles; 3 x 1 is the memory-bounded
    row-block mode) in fp32 mode against
    oracle.trimul_vjp: dL/dz and all ten parameter gradients, bar 1e-4 (the
    forward's fp32 bar; the k-blocks only change the fp32 summation order)."""
    import numpy as np
    n = 71
    print(f"[case] grid backward {s_rows}x{s_cols} {direction} n={n}", flush=True)
    z, mask, wts = wl.make_small(n, seed=31, dtype="f32", device="cpu", random_ln=True, mask_keep=0.85)
    w = pra.Weights(wts, pra.F32, device=dev)
    dout = np.random.default_rng(32).standard_normal((n, n, pra.C_Z))
    dz, grads = grid.emulate_backward(z.to(dev), mask.to(dev), w, DIRS[direction],
                                      torch.from_numpy(dout).float().to(dev), s_rows, s_cols)
    torch.cuda.synchronize()
    ref = oracle.trimul_vjp(z.double().numpy(), mask.numpy(), wl.weights_f64(wts), direction, dout)
    errs = {"z": rel_err(dz.double().cpu().numpy(), ref["z"])}
    for k in oracle.WEIGHT_KEYS:
        errs[k] = rel_err(grads[k].double().cpu().numpy(), ref[k])
    print("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= 1e-4, (k, v)
