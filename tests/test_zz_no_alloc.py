"""trimul_forward_chunked_noalloc: the allocation-free variant of
trimul_forward_chunked, whose workspace is a library-owned device array.

Called through the C ABI (the binding passes pointers only) and checked
against trimul_forward_chunked with the same blocks on the same inputs:
bitwise equal (the same kernels in the same order, only the workspace
address differs).  Two calls in a row, the second on a smaller input, so
stale contents of the shared array from the first call cannot leak into the
second.  Also: the first call against the Q-mode oracle, blocks whose
workspace exceeds the array rejected before anything runs, and any n served
by blocks that fit.
"""

import numpy as np
import pytest
import torch

import oracle
import pair_representation_amd as pra
import workloads as wl
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("direction", [pra.OUTGOING, pra.INCOMING])
def test_noalloc_matches_chunked_two_calls(dev, dtype, direction):
    name = "outgoing" if direction == pra.OUTGOING else "incoming"
    # first call: whole grid in one block; second: smaller n, several blocks
    for n, blocks, seed in ((300, (0, 0, 0), 51), (130, (64, 100, 50), 52)):
        print(f"[case] noalloc {dtype} {name} n={n} blocks {blocks}", flush=True)
        z, mask, w, h = _case(n, dtype, seed, dev)
        assert pra.chunked_workspace_bytes(w, n, *blocks) <= pra.NOALLOC_SCRATCH_BYTES
        got = pra.forward_chunked_noalloc(z, mask, w, direction, *blocks)
        want = pra.forward_chunked(z, mask, w, direction, *blocks)
        torch.cuda.synchronize()
        assert torch.equal(got, want), float((got - want).abs().max())
        ref = oracle.trimul(h["z"], h["mask"], h["w"], name, quant=(dtype == "bf16"))
        e = rel_err(got.double().cpu().numpy(), ref)
        print(f"  bitwise equal to the chunked entry point; vs oracle {e:.3e}", flush=True)
        assert e <= (1e-2 if dtype == "bf16" else 1e-4)


def test_noalloc_any_n_with_blocks_that_fit(dev):
    n = 1100
    blocks = (512, 512, 512)
    print(f"[case] noalloc bf16 n={n} blocks {blocks}", flush=True)
    z, mask, w, _ = _case(n, "bf16", 53, dev)
    assert pra.workspace_bytes(w, n) > pra.NOALLOC_SCRATCH_BYTES
    assert pra.chunked_workspace_bytes(w, n, *blocks) <= pra.NOALLOC_SCRATCH_BYTES
    got = pra.forward_chunked_noalloc(z, mask, w, pra.OUTGOING, *blocks)
    want = pra.forward_chunked(z, mask, w, pra.OUTGOING, *blocks)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_noalloc_rejects_blocks_beyond_scratch(dev):
    n = 600
    z, mask, w, _ = _case(n, "bf16", 54, dev)
    assert pra.chunked_workspace_bytes(w, n, 0, 0, 0) > pra.NOALLOC_SCRATCH_BYTES
    out = torch.full((n, n, pra.C_Z), 7.0, device=dev)
    with pytest.raises(pra.TrimulError) as ei:
        pra.forward_chunked_noalloc(z, mask, w, pra.OUTGOING, 0, 0, 0, out=out)
    assert ei.value.status == pra.ERR_WORKSPACE_TOO_SMALL
    assert str(pra.NOALLOC_SCRATCH_BYTES) in ei.value.message
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was enqueued
