"""GPU parity of the epilogue's backward (trimul_epilogue_backward) against
the oracle's gradients (oracle.finish_vjp), through the C ABI.

The inputs are exact in the storage dtype (z and the two matrices bf16 in bf16
mode) and the oracle gets those exact values.  In bf16 mode each non-weight
operand of a matrix-core product is split into hi = bf16(v) and
lo = bf16(v - hi) (|v - hi| <= 2^-8 |v|, so the pair represents v to within
2^-16 |v|) and the lo*lo term is dropped: one product is off by at most about
3 * 2^-16 = 4.6e-5 of its size, and typically far less; accumulation is fp32.
Bars, as max |diff| / rms(ref):
  dx, dz (each entry a sum of 128 such products)           1e-4
  parameter gradients                                      3e-4
the latter because a gradient summed over few pairs is close to a rank-1
outer product, whose largest entries are 10-25 times its rms, and each entry
carries its product's relative error (measured: 1.0e-4 for one pair, under
5e-5 otherwise).  fp32 mode is well inside both.

x_acc is filled with NaN outside the tile's pairs: the padding of the
accumulator layout must never reach a gradient.
"""

import numpy as np
import pytest
import torch

import oracle
import pair_representation_amd as pra
import workloads as wl
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu

C = 128
TOL = {"x": 1e-4, "z": 1e-4}
TOL_PARAM = 3e-4
NAMES = ("w_out_proj", "w_out_gate", "ln_out_w", "ln_out_b", "ln_in_w", "ln_in_b")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def planar_to_xacc(planar, fill=float("nan")):
    """Accumulator-layout tensor holding planar [128, rows, cols]; the padding
    entries get ``fill`` (layout only)."""
    _, rows, cols = planar.shape
    rb, cb = (rows + 3) // 4, (cols + 15) // 16
    full = torch.full((C, rb * 4, cb * 16), fill, dtype=torch.float32, device=planar.device)
    full[:, :rows, :cols] = planar
    return full.reshape(C, rb, 4, cb, 16).permute(1, 3, 0, 4, 2).contiguous()


def setup(dtype, n, seed, dev, mask_keep=0.8):
    z, mask, wts = wl.make_small(n, seed=seed, dtype=dtype, device="cpu", mask_keep=mask_keep)
    w = pra.Weights(wts, pra.BF16 if dtype == "bf16" else pra.F32, device=dev)
    wref = {k: v.double().numpy() for k, v in wts.items()}
    return z, mask, w, wref


def run_case(dev, dtype, n, row_off, n_rows, col_off, n_cols, seed, in_place=False):
    z, mask, w, wref = setup(dtype, n, seed, dev)
    r = np.random.default_rng(seed + 100)
    # x like a contraction result: a per-pair offset and scale, so both
    # LayerNorm statistics matter
    x = (r.standard_normal((n_rows, n_cols, C)) * r.uniform(0.5, 3.0, (n_rows, n_cols, 1))
         + r.standard_normal((n_rows, n_cols, 1)))
    x = np.float32(x).astype(np.float64)
    dout = np.float32(r.standard_normal((n_rows, n_cols, C))).astype(np.float64)
    x_acc = planar_to_xacc(torch.from_numpy(np.moveaxis(x, 2, 0)).float().to(dev))
    zd, md = z.to(dev), mask.to(dev)
    dout_d = torch.from_numpy(dout).float().to(dev)
    dx_buf = x_acc if in_place else None
    dx, dz, g = pra.epilogue_backward(w, n, row_off, n_rows, col_off, n_cols, x_acc, zd, md, dout_d, dx=dx_buf)
    torch.cuda.synchronize()
    zt = z[row_off:row_off + n_rows, col_off:col_off + n_cols].double().numpy()
    mt = mask[row_off:row_off + n_rows, col_off:col_off + n_cols].numpy()
    ref = oracle.finish_vjp(x, zt, mt, wref, dout, eps=1e-5)
    got = {"x": np.moveaxis(pra.xacc_to_planar(dx, n_rows, n_cols).double().cpu().numpy(), 0, 2),
           "z": dz.double().cpu().numpy()}
    for k in NAMES:
        got[k] = g[k].double().cpu().numpy()
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    print(f"  errors: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    # masked pairs: exact zeros
    keep = mt != 0
    assert np.all(got["x"][~keep] == 0) and np.all(got["z"][~keep] == 0)
    for k, v in errs.items():
        assert v <= TOL.get(k, TOL_PARAM), (k, v)
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,row_off,n_rows,col_off,n_cols", [
    (1, 0, 1, 0, 1),          # one pair
    (20, 3, 5, 7, 9),         # ragged in both directions, inside one work item
    (48, 0, 48, 0, 48),       # whole grid, whole work items
    (90, 10, 37, 2, 85),      # several items per work-group, ragged tails
    (300, 0, 300, 0, 300),    # more work items than work-groups
])
def test_epilogue_backward_matches_oracle(dev, dtype, n, row_off, n_rows, col_off, n_cols):
    print(f"[case] epilogue backward {dtype} n={n} rows {row_off}+{n_rows} cols {col_off}+{n_cols}", flush=True)
    run_case(dev, dtype, n, row_off, n_rows, col_off, n_cols, seed=n + n_rows + 3 * n_cols)


def test_epilogue_backward_in_place_and_deterministic(dev):
    """dx written over x_acc equals dx written elsewhere; two calls give
    bit-identical parameter gradients (fixed summation order)."""
    print("[case] epilogue backward in place", flush=True)
    a = run_case(dev, "bf16", 70, 5, 50, 0, 70, seed=5)
    b = run_case(dev, "bf16", 70, 5, 50, 0, 70, seed=5, in_place=True)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_epilogue_backward_full_size_sparse_dout(dev):
    """The whole 3605-residue grid as one tile, bf16, as the benchmark runs it.
    dout is nonzero only on a sample of pairs (corners and edges included), so
    the parameter gradients are sums over those pairs alone and the oracle
    computes them exactly; dx and dz are checked on the sample and are zero on
    other sampled pairs."""
    n = 3605
    print(f"[case] epilogue backward full size n={n}", flush=True)
    _, _, wts = wl.make_small(4, seed=3, dtype="bf16", device="cpu")
    w = pra.Weights(wts, pra.BF16, device=dev)
    wref = {k: v.double().numpy() for k, v in wts.items()}
    g = torch.Generator(device=dev).manual_seed(11)
    z = torch.randn((n, n, C), generator=g, device=dev).to(torch.bfloat16)
    mask = (torch.rand((n, n), generator=g, device=dev) < 0.9).to(torch.uint8)
    x_acc = torch.randn(pra.xacc_shape(n, n), generator=g, device=dev) * 2.0 + 0.3
    r = np.random.default_rng(12)
    m = 1500
    I = np.concatenate([[0, 0, n - 1, n - 1], r.integers(0, n, m)])
    J = np.concatenate([[0, n - 1, 0, n - 1], r.integers(0, n, m)])
    flat = np.unique(I * n + J)
    I, J = flat // n, flat % n
    It, Jt = torch.as_tensor(I, device=dev), torch.as_tensor(J, device=dev)
    dvals = torch.randn((len(I), C), generator=g, device=dev)
    dout = torch.zeros((n, n, C), dtype=torch.float32, device=dev)
    dout[It, Jt] = dvals
    dx, dz, grads = pra.epilogue_backward(w, n, 0, n, 0, n, x_acc, z, mask, dout)
    torch.cuda.synchronize()
    xpl = pra.xacc_to_planar(x_acc, n, n)
    dxpl = pra.xacc_to_planar(dx, n, n)
    xs = xpl[:, It, Jt].T.double().cpu().numpy()                 # [m, 128]
    zs = z[It, Jt].double().cpu().numpy()
    ms = mask[It, Jt].cpu().numpy()
    ref = oracle.finish_vjp(xs, zs, ms, wref, dvals.double().cpu().numpy(), eps=1e-5)
    got = {"x": dxpl[:, It, Jt].T.double().cpu().numpy(), "z": dz[It, Jt].double().cpu().numpy()}
    for k in NAMES:
        got[k] = grads[k].double().cpu().numpy()
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    print("  errors: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= TOL.get(k, TOL_PARAM), (k, v)
    # pairs with dout = 0 get exactly zero gradients
    I0 = torch.as_tensor(r.integers(0, n, 400), device=dev)
    J0 = torch.as_tensor(r.integers(0, n, 400), device=dev)
    zero = (dout[I0, J0].abs().sum(dim=1) == 0)
    assert torch.all(dz[I0, J0][zero] == 0) and torch.all(dxpl[:, I0, J0].T[zero] == 0)
