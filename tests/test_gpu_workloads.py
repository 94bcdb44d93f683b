"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times.

n64_f32 and n768_pad are compared on the whole output tensor.  The larger
grids are compared on a sample of rows x cols (about 48 x 48 residues = 2,304
pairs x 128 channels), which the oracle computes exactly from the operand rows
(outgoing) or columns (incoming) of just those residues; the sample holds the
first and last residue, chain boundaries +-1, masked residues, tile and chunk
edges, and seeded random residues.  The whole output is also checked for
finiteness, exact zeros at masked pairs, and an rms within 5% of the sample's.
"""

import gc

import numpy as np
import pytest
import torch

import oracle
import pair_representation_amd as pra
import workloads as wl
from tests.gpu_util import device_getters, rel_err, sample_indices, whole_tensor_checks as _whole_tensor_checks

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
BF16_EXACT_TOL = 5e-2   # bf16 path vs the exact oracle (the operand rounding alone: 3.6e-2 at N=768)
F32_TOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _weights(work, dev):
    wts = wl.make_weights(work.c_z, work.c, work.seed, work.dtype)
    return pra.Weights(wts, pra.BF16 if work.dtype == "bf16" else pra.F32, device=dev), wl.weights_f64(wts)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_n64_f32_full(dev, direction):
    work = wl.WORKLOADS["n64_f32"]
    print(f"[case] {work.name} {direction}", flush=True)
    z, mask, wts = wl.make_inputs(work, "cpu")
    w = pra.Weights(wts, pra.F32, device=dev)
    fn = pra.outgoing if direction == "outgoing" else pra.incoming
    got = fn(z.to(dev), mask.to(dev), w).cpu().double().numpy()
    ref = oracle.trimul(z.double().numpy(), mask.numpy(), wl.weights_f64(wts), direction)
    e = rel_err(got, ref)
    print(f"  vs exact {e:.3e}")
    assert e <= F32_TOL


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_n768_pad_full(dev, direction):
    work = wl.WORKLOADS["n768_pad"]
    print(f"[case] {work.name} {direction}", flush=True)
    z, mask, wts = wl.make_inputs(work, "cpu")
    w = pra.Weights(wts, pra.BF16, device=dev)
    fn = pra.outgoing if direction == "outgoing" else pra.incoming
    got = fn(z.to(dev), mask.to(dev), w).cpu().double().numpy()
    ref = oracle.trimul_blockwise(z.double().numpy(), mask.numpy(), wl.weights_f64(wts), direction, quant=True)
    e = rel_err(got, ref)
    exact = oracle.trimul_blockwise(z.double().numpy(), mask.numpy(), wl.weights_f64(wts), direction)
    e_exact = rel_err(got, exact)
    print(f"  vs Q-oracle {e:.3e}  vs exact {e_exact:.3e}")
    assert e <= BF16_TOL
    assert e_exact <= BF16_EXACT_TOL
    assert np.all(got[mask.numpy() == 0] == 0)
    valid = 768 - 77
    assert np.all(got[valid:] == 0) and np.all(got[:, valid:] == 0)


def _boundaries(work):
    b = []
    acc = 0
    for L in work.chains[:-1]:
        acc += L
        b += [acc - 1, acc]
    return b


@pytest.mark.parametrize("name", ["n3605_4ch", "n6500_2ch"])
def test_large_sampled(dev, name):
    work = wl.WORKLOADS[name]
    z, mask, _ = wl.make_inputs(work, dev)
    w, w64 = _weights(work, dev)
    res = wl.residue_mask(work)
    masked = list(np.flatnonzero(res == 0)[:6])
    rows = sample_indices(work.n, 101, 48, _boundaries(work) + masked)
    cols = sample_indices(work.n, 202, 48, _boundaries(work) + masked[::-1])
    gz, gm = device_getters(z, mask)
    ws = pra.new_workspace(w, work.n, dev)
    for direction in ("outgoing", "incoming"):
        print(f"[case] {name} {direction} n={work.n}", flush=True)
        fn = pra.outgoing if direction == "outgoing" else pra.incoming
        out = fn(z, mask, w, workspace=ws)
        torch.cuda.synchronize()
        got = out[torch.as_tensor(rows, device=dev)][:, torch.as_tensor(cols, device=dev)]
        got = got.double().cpu().numpy()
        ref = oracle.trimul_sampled(gz, gm, work.n, w64, direction, rows, cols, quant=True)
        e = rel_err(got, ref)
        print(f"  sampled {len(rows)}x{len(cols)} vs Q-oracle {e:.3e}", flush=True)
        assert e <= BF16_TOL
        _whole_tensor_checks(out, mask, ref, gm(rows, cols))
        del out
        _free()
    del z, mask, ws
    _free()


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_n10000_tile_sampled(dev, direction):
    work = wl.WORKLOADS["n10000_tile"]
    t = work.tile
    print(f"[case] {work.name} {direction}", flush=True)
    z, mask, _ = wl.make_inputs(work, dev)
    w, w64 = _weights(work, dev)
    d = pra.OUTGOING if direction == "outgoing" else pra.INCOMING
    ld = (t["chunk"] + 63) // 64 * 64
    chunks = []
    for c in range(t["n_chunks"]):
        k_off = c * t["chunk"]
        a, b = pra.tile_operands(w, d, z, mask, t["row_off"], t["n_rows"], t["col_off"], t["n_cols"],
                                 k_off, t["chunk"], ld)
        chunks.append((k_off, t["chunk"], a, b))
    x = pra.new_xacc(t["n_rows"], t["n_cols"], dev)
    out = pra.tile(w, work.n, t["row_off"], t["n_rows"], t["col_off"], t["n_cols"], chunks,
                   pra.TILE_FIRST | pra.TILE_LAST, x, z, mask)
    torch.cuda.synchronize()
    edges = [0, 1249, 1250, 2499, 2500, 3749, 3750, 4999]
    rows = sample_indices(t["n_rows"], 303, 48, edges) + t["row_off"]
    cols = sample_indices(t["n_cols"], 404, 48, edges) + t["col_off"]
    got = out[torch.as_tensor(rows - t["row_off"], device=dev)][:, torch.as_tensor(cols - t["col_off"], device=dev)]
    gz, gm = device_getters(z, mask)
    ref = oracle.trimul_sampled(gz, gm, work.n, w64, direction, rows, cols, quant=True)
    e = rel_err(got.double().cpu().numpy(), ref)
    print(f"  sampled {len(rows)}x{len(cols)} vs Q-oracle {e:.3e}", flush=True)
    assert e <= BF16_TOL
    _whole_tensor_checks(out, mask[:t["n_rows"], :t["n_cols"]], ref, gm(rows, cols))
    del z, mask, chunks, x, out
    _free()


def test_whole_grid_near_device_limit(dev):
    """The whole-grid entry points at the largest N (a multiple of 256) whose
    workspace fits beside z, mask and out in the device's free memory (8 GiB
    kept back): both directions on a 24 x 24 sample of residues (first, last,
    masked, random) against the Q-oracle, plus whole-tensor checks."""
    _free()
    free, _ = torch.cuda.mem_get_info(dev)
    wts = wl.make_weights(128, 128, 11, "bf16")
    w, w64 = pra.Weights(wts, pra.BF16, device=dev), wl.weights_f64(wts)
    io = lambda m: m * m * (128 * 2 + 1 + 128 * 4)
    n = 256
    while io(n + 256) + pra.workspace_bytes(w, n + 256) <= free - (8 << 30):
        n += 256
    work = wl.Workload("n_device_limit", n, "bf16", seed=11, masked_fraction=0.02)
    print(f"[case] whole grid at n={n} ({(io(n) + pra.workspace_bytes(w, n)) / 1e9:.0f} GB of "
          f"{free / 1e9:.0f} GB free)", flush=True)
    assert n >= 4096
    z, mask, _ = wl.make_inputs(work, dev)
    masked = list(np.flatnonzero(wl.residue_mask(work) == 0)[:4])
    rows = sample_indices(n, 111, 24, masked)
    cols = sample_indices(n, 222, 24, masked[::-1])
    gz, gm = device_getters(z, mask)
    ws = pra.new_workspace(w, n, dev)
    for direction in ("outgoing", "incoming"):
        fn = pra.outgoing if direction == "outgoing" else pra.incoming
        out = fn(z, mask, w, workspace=ws)
        torch.cuda.synchronize()
        got = out[torch.as_tensor(rows, device=dev)][:, torch.as_tensor(cols, device=dev)].double().cpu().numpy()
        ref = oracle.trimul_sampled(gz, gm, n, w64, direction, rows, cols, quant=True)
        e = rel_err(got, ref)
        print(f"  {direction}: sampled {len(rows)}x{len(cols)} vs Q-oracle {e:.3e}", flush=True)
        assert e <= BF16_TOL
        _whole_tensor_checks(out, mask, ref, gm(rows, cols))
        del out
        _free()
    del z, mask, ws
    _free()


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_f32_n1000_sampled(dev, direction):
    """The fp32 path over many contraction tiles (8 x 8 of 128, ragged):
    n = 1000 with random LayerNorm affine and a random pair mask, on a 32 x 32
    sample against the exact oracle (fp32 bar 1e-4)."""
    n = 1000
    print(f"[case] f32 n={n} {direction}", flush=True)
    z, mask, wts = wl.make_small(n, seed=77, dtype="f32", device="cpu", random_ln=True, mask_keep=0.9)
    w = pra.Weights(wts, pra.F32, device=dev)
    zd, md = z.to(dev), mask.to(dev)
    fn = pra.outgoing if direction == "outgoing" else pra.incoming
    out = fn(zd, md, w)
    torch.cuda.synchronize()
    rows = sample_indices(n, 303, 32, [127, 128, 255, 256, 895, 896])
    cols = sample_indices(n, 404, 32, [127, 128, 511, 512, 999])
    got = out[torch.as_tensor(rows, device=dev)][:, torch.as_tensor(cols, device=dev)].double().cpu().numpy()
    gz, gm = oracle.array_getters(z.double().numpy(), mask.numpy())
    ref = oracle.trimul_sampled(gz, gm, n, wl.weights_f64(wts), direction, rows, cols)
    e = rel_err(got, ref)
    print(f"  sampled {len(rows)}x{len(cols)} vs exact oracle {e:.3e}", flush=True)
    assert e <= F32_TOL
    assert np.all(got[gm(rows, cols) == 0] == 0)
    del out, zd, md
    _free()
