"""The memory-bounded forward (trimul_forward_chunked): R x C output tiles,
each contracting k in chunks of K, in a workspace that does not grow with
the whole grid.

Bars (max |diff| / rms(ref)):
  bf16 against the Q-mode oracle                                   <= 1e-2
  fp32 against the exact oracle                                    <= 1e-4
  against the whole-grid entry point (only the fp32 summation order over
  k differs)                                                       <= 1e-4
At N = 14000 the whole-grid entry point cannot run (its workspace alone is
201 GB, with z and out 351 GB of the 288 GB); the chunked path runs in
88 GB of workspace (3584-row tiles, k in one chunk) or 57 GB (3500-row
tiles, k in two chunks) and is checked against the oracle on sampled pairs.
"""

import numpy as np
import pytest
import torch

import oracle
import pair_representation_amd as pra
import workloads as wl
from tests.gpu_util import device_getters, rel_err, sample_indices, whole_tensor_checks

pytestmark = pytest.mark.gpu

DIRS = {"outgoing": pra.OUTGOING, "incoming": pra.INCOMING}


@pytest.fixture(scope="module")
def dev():
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


def _case(n, dtype, seed, dev):
    z, mask, wts = wl.make_small(n, seed=seed, dtype=dtype, device="cpu", random_ln=True, mask_keep=0.9)
    w = pra.Weights(wts, pra.BF16 if dtype == "bf16" else pra.F32, device=dev)
    host = dict(z=z.double().numpy(), mask=mask.numpy(), w=wl.weights_f64(wts))
    return z.to(dev), mask.to(dev), w, host


@pytest.mark.parametrize("direction", list(DIRS))
@pytest.mark.parametrize("blocks", [(64, 0, 50), (100, 77, 128), (300, 300, 300), (257, 33, 299), (1, 300, 64),
                                    (64, 77, 0), (64, 0, 0), (100, 300, 300), (256, 0, 0)])
def test_chunked_bf16_vs_oracle(dev, direction, blocks):
    n = 300
    R, C, K = blocks
    print(f"[case] chunked bf16 {direction} n={n} blocks {blocks}", flush=True)
    z, mask, w, h = _case(n, "bf16", 41, dev)
    got = pra.forward_chunked(z, mask, w, DIRS[direction], R, C, K)
    full = (pra.outgoing if direction == "outgoing" else pra.incoming)(z, mask, w)
    torch.cuda.synchronize()
    ref = oracle.trimul(h["z"], h["mask"], h["w"], direction, quant=True)
    e = rel_err(got.double().cpu().numpy(), ref)
    e_full = rel_err(got.double().cpu().numpy(), full.double().cpu().numpy())
    print(f"  vs Q-oracle {e:.3e}, vs whole grid {e_full:.3e}", flush=True)
    assert e <= 1e-2
    assert e_full <= 1e-4
    assert (got[~mask.bool()] == 0).all()


@pytest.mark.parametrize("direction", list(DIRS))
def test_chunked_f32_vs_exact_oracle(dev, direction):
    n = 131
    print(f"[case] chunked f32 {direction} n={n}", flush=True)
    z, mask, w, h = _case(n, "f32", 42, dev)
    got = pra.forward_chunked(z, mask, w, DIRS[direction], 50, 64, 40)
    torch.cuda.synchronize()
    ref = oracle.trimul(h["z"], h["mask"], h["w"], direction)
    e = rel_err(got.double().cpu().numpy(), ref)
    print(f"  vs exact oracle {e:.3e}", flush=True)
    assert e <= 1e-4


def test_chunked_workspace_formula(dev):
    """The workspace is the sum of the three pieces the header states and does
    not depend on n once the blocks are fixed."""
    z, mask, w, _ = _case(8, "bf16", 43, dev)
    def pieces(R, C, K, e=2):
        a256 = lambda v: (v + 255) // 256 * 256
        r = lambda v, m: (v + m - 1) // m * m
        return (a256(128 * r(R, 256) * r(K, 64) * e) + a256(128 * r(C, 256) * r(K, 64) * e)
                + a256(128 * r(R, 4) * r(C, 16) * 4))
    for n, R, C, K in ((5000, 512, 512, 512), (14000, 512, 512, 512), (14000, 3500, 0, 7000), (14000, 3584, 0, 0),
                       (100, 0, 0, 0)):
        R2, C2, K2 = (v if 0 < v <= n else n for v in (R, C, K))
        assert pra.chunked_workspace_bytes(w, n, R, C, K) == pieces(R2, C2, K2)
    with pytest.raises(pra.TrimulError):
        pra.forward_chunked(z, mask, w, pra.OUTGOING, 4, 4, 4,
                            workspace=torch.empty(pieces(4, 4, 4) - 256, dtype=torch.uint8, device=dev))


@pytest.mark.parametrize("direction", list(DIRS))
@pytest.mark.parametrize("blocks", ["workload", (3500, 0, 7000), "planned"])
def test_chunked_beyond_whole_grid_memory(dev, direction, blocks):
    """The n14000_chunked workload: the whole-grid path would need 351 GB with
    z and out; the chunked path runs in z + out + 88 GB with the workload's
    blocks (3584-row tiles, full width, k in one chunk: each operand built
    once) and in z + out + 57 GB with 3500-row tiles and k in two chunks of
    7000 (operands rebuilt per tile and chunk).  Checked on sampled pairs
    against the Q-oracle (rows and columns at tile and chunk boundaries, first
    and last, random), plus finiteness, exact zeros at masked pairs and the
    sample's rms.  A third case takes the blocks plan_chunked picks for the
    device's free memory."""
    work = wl.WORKLOADS["n14000_chunked"]
    n = work.n
    free, total = torch.cuda.mem_get_info(dev)
    wts = wl.make_weights(work.c_z, work.c, work.seed, work.dtype)
    w = pra.Weights(wts, pra.BF16, device=dev)
    io = n * n * (128 * 2 + 1 + 128 * 4)                  # z, mask, out
    if blocks == "workload":
        blocks = (work.chunked["row_block"], work.chunked["col_block"], work.chunked["k_block"])
    elif blocks == "planned":
        # the tallest tiles the free memory allows beside z, mask and out (2 GiB kept back)
        blocks = pra.plan_chunked(w, n, free - io - (2 << 30))
    R, C, K = blocks
    print(f"[case] {work.name} {direction} blocks {(R, C, K)}", flush=True)
    need = io + pra.chunked_workspace_bytes(w, n, R, C, K)
    # the whole-grid path cannot hold its workspace beside z and out here
    assert io + pra.workspace_bytes(w, n) > total
    if free < need:
        pytest.skip(f"needs {need / 1e9:.0f} GB of device memory, {free / 1e9:.0f} GB free")
    z, mask, _ = wl.make_inputs(work, dev)
    r = wl.residue_mask(work)
    out = pra.forward_chunked(z, mask, w, DIRS[direction], R, C, K)
    torch.cuda.synchronize()
    print("  computed", flush=True)
    masked = np.flatnonzero(r == 0)[:4]
    edges = sorted({e for b in (R, K) if 0 < b < n for m in range(b, n, b) for e in (m - 1, m)})
    must = [0, n - 1] + edges + list(masked)
    rows = sample_indices(n, 61, count=24, must=must)
    cols = sample_indices(n, 62, count=24, must=must)
    gz, gm = device_getters(z, mask)
    ref = oracle.trimul_sampled(gz, gm, n, wl.weights_f64(wts), direction, rows, cols, quant=True)
    got = out[torch.as_tensor(rows, device=dev)][:, torch.as_tensor(cols, device=dev)].double().cpu().numpy()
    e = rel_err(got, ref)
    print(f"  sampled {len(rows)}x{len(cols)} vs Q-oracle {e:.3e}", flush=True)
    assert e <= 1e-2
    whole_tensor_checks(out, mask, ref, gm(rows, cols))
    del out, z
    torch.cuda.empty_cache()
