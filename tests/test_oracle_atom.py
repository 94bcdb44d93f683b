"""CPU pins of the window-batched atom attention oracle
(oracle.atom_attention): an independent scalar-loop spelling, torch's
scaled-dot-product attention on a window whose 128 keys all exist, and
closed forms (one key left, uniform logits, per-row bias shifts, no key left,
locality of a window)."""

import numpy as np
import torch

from oracle import atom_attention as aa
from oracle import bruteforce


def _case(seed, bsz=2, n=150, heads=3, d=8, keep=0.85, with_bias=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((bsz, n, heads, d))
    k = r.standard_normal((bsz, n, heads, d))
    v = r.standard_normal((bsz, n, heads, d))
    bias = r.standard_normal((bsz, aa.n_windows(n), heads, 32, 128)) if with_bias else None
    mask = (r.random((bsz, n)) < keep).astype(np.uint8)
    return q, k, v, bias, mask


def test_matches_scalar_loops():
    for n in (1, 31, 33, 100):
        q, k, v, bias, mask = _case(n, bsz=2, n=n, heads=2, d=4)
        got = aa.window_attention(q, k, v, bias, mask)
        want = np.array(bruteforce.window_attention_loops(q, k, v, bias, mask))
        assert np.max(np.abs(got - want)) < 1e-12, n


def test_full_window_matches_torch_sdpa():
    """Window 2 of a 200-atom sequence: queries 64..95, keys 16..143, all in
    the sequence; with no mask this is ordinary attention with the window's
    bias as an additive mask."""
    q, k, v, bias, _ = _case(3, bsz=1, n=200, heads=4, d=16)
    got = aa.window_attention(q, k, v, bias, None)[0, 64:96]                  # [32, h, d]
    tq = torch.from_numpy(q[0, 64:96]).permute(1, 0, 2)                      # [h, 32, d]
    tk = torch.from_numpy(k[0, 16:144]).permute(1, 0, 2)
    tv = torch.from_numpy(v[0, 16:144]).permute(1, 0, 2)
    tb = torch.from_numpy(bias[0, 2])                                        # [h, 32, 128]
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tb).permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - want)) < 1e-12


def test_single_key_and_no_key():
    q, k, v, bias, _ = _case(5, bsz=1, n=96, heads=2, d=4)
    mask = np.zeros((1, 96), np.uint8)
    mask[0, 40] = 1                       # only atom 40 is a key: inside the windows of blocks 0, 1, 2
    o = aa.window_attention(q, k, v, bias, mask)
    for i in range(96):
        w = i // 32
        if 32 * w - 48 <= 40 < 32 * w + 80:
            assert np.max(np.abs(o[0, i] - v[0, 40])) < 1e-12
        else:
            assert np.max(np.abs(o[0, i])) == 0
    assert np.max(np.abs(aa.window_attention(q, k, v, bias, np.zeros((1, 96), np.uint8)))) == 0


def test_uniform_logits_give_window_mean():
    q, _, v, _, mask = _case(7, bsz=1, n=130, heads=2, d=4)
    k = np.zeros_like(q)
    o = aa.window_attention(q, k, v, None, mask)
    for i in (0, 31, 32, 64, 129):
        w = i // 32
        keys = [j for j in range(32 * w - 48, 32 * w + 80) if 0 <= j < 130 and mask[0, j]]
        assert np.max(np.abs(o[0, i] - v[0, keys].mean(axis=0))) < 1e-12


def test_bias_row_shift_invariance():
    q, k, v, bias, mask = _case(9)
    shift = np.random.default_rng(10).standard_normal(bias.shape[:-1])[..., None]
    a = aa.window_attention(q, k, v, bias, mask)
    b = aa.window_attention(q, k, v, bias + shift, mask)
    assert np.max(np.abs(a - b)) < 1e-12


def test_window_locality():
    """Atoms outside a block's 128-key window do not affect its outputs."""
    q, k, v, bias, mask = _case(11, bsz=1, n=300)
    o = aa.window_attention(q, k, v, bias, mask)
    k2, v2 = k.copy(), v.copy()
    k2[0, 200:], v2[0, 200:] = 7.0, -3.0              # block 1's keys are atoms -16 .. 111
    o2 = aa.window_attention(q, k2, v2, bias, mask)
    assert np.array_equal(o[0, 32:64], o2[0, 32:64])
    assert np.max(np.abs(o[0, 160:192] - o2[0, 160:192])) > 1e-3   # block 5 (keys 112 .. 239) sees them
