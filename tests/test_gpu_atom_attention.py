"""GPU parity of window-batched sequence-local atom attention
(trimul_atom_window_attention) against oracle.atom_attention, through the C ABI.

q, k, v and the bias are bf16 and the oracle gets their exact values.  Logits
are fp32 sums of 32 exact products, the softmax is fp32 (hardware exp2 and
reciprocal), and P enters the product with V as hi + lo bf16 terms (together
within 2^-16 of P): the bar is 1e-4 of the output's rms.
"""

import numpy as np
import pytest
import torch

from oracle import atom_attention as aa
import pair_representation_amd as pra
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bf16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).float().to(torch.bfloat16).to(dev)


@pytest.mark.parametrize("bsz,n,heads,with_bias,mask_mode", [
    (1, 1, 1, True, "none"),          # one atom
    (2, 31, 3, True, "random"),       # one partial window
    (2, 33, 4, False, "random"),      # a window of one query
    (1, 100, 6, True, "none"),        # heads beyond one round of 4 waves
    (3, 257, 4, True, "random"),
    (2, 200, 4, True, "holes"),       # whole windows without keys
])
def test_window_attention_matches_oracle(dev, bsz, n, heads, with_bias, mask_mode):
    print(f"[case] atom attention b={bsz} n={n} heads={heads} bias={with_bias} mask={mask_mode}", flush=True)
    r = np.random.default_rng(n * 7 + heads)
    q, k, v = (r.standard_normal((bsz, n, heads, 32)) * 0.8 for _ in range(3))
    bias = r.standard_normal((bsz, aa.n_windows(n), heads, 32, 128)) if with_bias else None
    mask = None
    if mask_mode == "random":
        mask = (r.random((bsz, n)) < 0.8).astype(np.uint8)
    elif mask_mode == "holes":
        mask = np.ones((bsz, n), np.uint8)
        mask[:, 40:] = 0                  # blocks 3.. see no key (block 3's window starts at atom 48)
    tq, tk, tv = bf16(q, dev), bf16(k, dev), bf16(v, dev)
    tb = None if bias is None else bf16(bias, dev)
    tm = None if mask is None else torch.from_numpy(mask).to(dev)
    out = pra.atom_window_attention(tq, tk, tv, tb, tm)
    torch.cuda.synchronize()
    back = lambda t: None if t is None else t.double().cpu().numpy()
    ref = aa.window_attention(back(tq), back(tk), back(tv), back(tb), mask)
    got = out.double().cpu().numpy()
    e = rel_err(got, ref)
    print(f"  max|diff|/rms {e:.2e}", flush=True)
    assert e <= TOL
    if mask_mode == "holes":
        assert np.all(got[:, 96:] == 0) and np.any(got[:, :96] != 0)
    assert np.all(np.isfinite(got))


def test_window_attention_full_size_sampled(dev):
    """The benchmarked shape (8 sequences of 28840 atoms, 4 heads, pair bias,
    90% of atoms kept): 24 sampled windows per sequence, the first and last
    included, against the oracle on a slice that holds each window's keys."""
    bsz, n, heads = 8, 28840, 4
    nw = aa.n_windows(n)
    print(f"[case] atom attention full size b={bsz} n={n}", flush=True)
    g = torch.Generator(device=dev).manual_seed(5)
    tq, tk, tv = (torch.randn((bsz, n, heads, 32), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    tb = torch.randn((bsz, nw, heads, 32, 128), generator=g, device=dev).to(torch.bfloat16)
    tm = (torch.rand((bsz, n), generator=g, device=dev) < 0.9).to(torch.uint8)
    out = pra.atom_window_attention(tq, tk, tv, tb, tm)
    torch.cuda.synchronize()
    r = np.random.default_rng(6)
    errs = []
    for b in range(bsz):
        ws = sorted(set([0, 1, nw - 2, nw - 1] + list(r.integers(0, nw, 20))))
        for w in ws:
            lo, hi = max(0, 32 * (w - 2)), min(n, 32 * (w + 3))   # holds keys 32w-48 .. 32w+79
            wl = w - lo // 32
            sl = lambda t: t[b:b + 1, lo:hi].double().cpu().numpy()
            bias = torch.zeros((1, aa.n_windows(hi - lo), heads, 32, 128), dtype=torch.float64)
            bias[0, wl] = tb[b, w].double().cpu()
            ref = aa.window_attention(sl(tq), sl(tk), sl(tv), bias.numpy(), tm[b:b + 1, lo:hi].cpu().numpy())
            qs = slice(32 * w - lo, min(32 * w + 32, n) - lo)
            got = out[b, lo:hi].double().cpu().numpy()[qs]
            errs.append(rel_err(got, ref[0, qs]))
    print(f"  worst window max|diff|/rms {max(errs):.2e} over {len(errs)} windows", flush=True)
    assert max(errs) <= TOL
    assert torch.isfinite(out).all()
