"""GPU parity of the projections' backward (trimul_tile_operands_backward)
against oracle.project_vjp, and of the whole layer's gradient (the autograd
function composing the three backward entry points) against the oracle's
gradients, through the C ABI.

Bars (max |diff| / rms(ref)):
  projections' backward: dz 1e-4, parameter gradients 3e-4 (the hi/lo split
  of every non-weight matrix-core operand, as for the epilogue's backward);
  whole layer, fp32 mode vs oracle.trimul_vjp: 1e-4, the forward's fp32 bar;
  whole layer, bf16 mode: against the oracle steps composed with the same
  rounding points the bf16 path has (a and b rounded to bf16 by the forward
  projection, whose input is rounded too; dL/dx rounded to bf16 for the
  contraction's backward): 1e-2, the forward's bf16 bar against the Q-mode
  oracle, for the same reason -- an entry whose fp32 and float64 values fall
  on either side of a bf16 rounding boundary differs by one bf16 ulp (2^-7 of
  it) between the two; plus for dL/dz, returned in z's bf16 dtype, the bound
  of that rounding, 2^-8 max|ref| / rms(ref).
"""

import numpy as np
import pytest
import torch

import oracle
import pair_representation_amd as pra
from pair_representation_amd import autograd as pag
import workloads as wl
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu

C = 128
NAMES = ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate", "ln_in_w", "ln_in_b")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def planar_to_xacc(planar, fill=float("nan")):
    _, rows, cols = planar.shape
    rb, cb = (rows + 3) // 4, (cols + 15) // 16
    full = torch.full((C, rb * 4, cb * 16), fill, dtype=torch.float32, device=planar.device)
    full[:, :rows, :cols] = planar
    return full.reshape(C, rb, 4, cb, 16).permute(1, 3, 0, 4, 2).contiguous()


def source(z, m, direction, base, rows, k_off, k_len):
    """z and mask at the source pairs of an operand chunk: [rows, k_len, ...]."""
    if direction == "outgoing":
        return z[base:base + rows, k_off:k_off + k_len], m[base:base + rows, k_off:k_off + k_len]
    return (np.swapaxes(z[k_off:k_off + k_len, base:base + rows], 0, 1),
            np.swapaxes(m[k_off:k_off + k_len, base:base + rows], 0, 1))


def scatter_add(dz, g, direction, base, rows, k_off, k_len):
    if direction == "outgoing":
        dz[base:base + rows, k_off:k_off + k_len] += g
    else:
        dz[k_off:k_off + k_len, base:base + rows] += np.swapaxes(g, 0, 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("n,row_off,n_rows,col_off,n_cols,k_off,k_len,sides,accumulate", [
    (1, 0, 1, 0, 1, 0, 1, "ab", False),
    (40, 3, 17, 20, 9, 5, 30, "ab", False),
    (70, 0, 70, 0, 70, 0, 70, "ab", True),
    (90, 10, 37, 50, 33, 40, 45, "a", True),
    (90, 10, 37, 50, 33, 40, 45, "b", False),
])
def test_tile_operands_backward_matches_oracle(dev, dtype, direction, n, row_off, n_rows, col_off, n_cols, k_off,
                                               k_len, sides, accumulate):
    print(f"[case] operands backward {dtype} {direction} n={n} a {row_off}+{n_rows} b {col_off}+{n_cols} "
          f"k {k_off}+{k_len} sides {sides} acc {accumulate}", flush=True)
    seed = n + 7 * n_rows + 3 * k_len + len(sides)
    z, mask, wts = wl.make_small(n, seed=seed, dtype=dtype, device="cpu", mask_keep=0.8)
    w = pra.Weights(wts, pra.BF16 if dtype == "bf16" else pra.F32, device=dev)
    wref = {k: v.double().numpy() for k, v in wts.items()}
    zn, mn = z.double().numpy(), mask.numpy()
    r = np.random.default_rng(seed)
    d = pra.OUTGOING if direction == "outgoing" else pra.INCOMING
    da = np.float32(r.standard_normal((n_rows, k_len, C))).astype(np.float64) if "a" in sides else None
    db = np.float32(r.standard_normal((n_cols, k_len, C))).astype(np.float64) if "b" in sides else None
    dz0 = np.float32(r.standard_normal((n, n, C))).astype(np.float64)
    g0 = {k: np.float32(r.standard_normal(shp)).astype(np.float64) for k, shp in pra.PROJECTION_GRAD_SHAPES.items()}
    to_x = lambda t: planar_to_xacc(torch.from_numpy(np.moveaxis(t, 2, 0)).float().to(dev))
    dz = torch.from_numpy(dz0).float().to(dev)
    grads = {k: torch.from_numpy(v).float().to(dev) for k, v in g0.items()}
    pra.tile_operands_backward(w, d, z.to(dev), mask.to(dev), row_off, n_rows, col_off, n_cols, k_off, k_len,
                               da=None if da is None else to_x(da), db=None if db is None else to_x(db), dz=dz,
                               grads=grads, accumulate=accumulate)
    torch.cuda.synchronize()
    # reference: each side's pairs through the oracle, the other side's gradient zero
    want_dz = dz0.copy()
    want = {k: (g0[k].copy() if accumulate else np.zeros_like(g0[k])) for k in g0}
    for side, dgrad, base, rows in (("a", da, row_off, n_rows), ("b", db, col_off, n_cols)):
        if dgrad is None:
            if not accumulate:
                want[f"w_{side}_proj"], want[f"w_{side}_gate"] = g0[f"w_{side}_proj"], g0[f"w_{side}_gate"]
            continue
        zs, ms = source(zn, mn, direction, base, rows, k_off, k_len)
        zero = np.zeros_like(dgrad)
        ref = oracle.project_vjp(zs, ms, wref, dgrad if side == "a" else zero, dgrad if side == "b" else zero)
        scatter_add(want_dz, ref["z"], direction, base, rows, k_off, k_len)
        for k in (f"w_{side}_proj", f"w_{side}_gate", "ln_in_w", "ln_in_b"):
            want[k] = want[k] + ref[k]
    got_dz = dz.double().cpu().numpy()
    e_dz = rel_err(got_dz - dz0, want_dz - dz0)
    errs = {k: rel_err(grads[k].double().cpu().numpy(), want[k]) for k in want}
    print(f"  dz {e_dz:.2e}  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    assert e_dz <= 1e-4
    for k, v in errs.items():
        assert v <= 3e-4, (k, v)


def _params(wts, dev):
    """fp32 master parameters (the matrices hold bf16-exact values in bf16
    mode; the layer casts them to the storage dtype and returns fp32
    gradients)."""
    return {k: wts[k].to(dev).float().contiguous().requires_grad_(True) for k in pag.PARAM_NAMES}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("n", [37, 130])
def test_layer_autograd_matches_oracle(dev, dtype, direction, n):
    """loss = sum(dout * layer(z)) backpropagated through TriMul: dL/dz and all
    ten parameters' gradients."""
    print(f"[case] layer autograd {dtype} {direction} n={n}", flush=True)
    z, mask, wts = wl.make_small(n, seed=n + 1, dtype=dtype, device="cpu", mask_keep=0.85)
    r = np.random.default_rng(n + 2)
    dout = np.float32(r.standard_normal((n, n, C))).astype(np.float64)
    params = _params(wts, dev)
    zd = z.to(dev).requires_grad_(True)
    out = pag.trimul(zd, mask.to(dev), params, pra.OUTGOING if direction == "outgoing" else pra.INCOMING)
    out.backward(torch.from_numpy(dout).float().to(dev))
    torch.cuda.synchronize()
    wref = {k: v.double().numpy() for k, v in wts.items()}
    zn, mn = z.double().numpy(), mask.numpy()
    if dtype == "f32":
        ref = oracle.trimul_vjp(zn, mn, wref, direction, dout)
    else:
        # the oracle's steps with the bf16 path's rounding points
        a, b = oracle.project(zn, mn, wref, quant=True)
        x = oracle.contract(a, b, direction)
        ge = oracle.finish_vjp(x, zn, mn, wref, dout)
        dxq = oracle.bf16_round(ge["x"])
        if direction == "outgoing":
            da, db = oracle.contract_rows_vjp(a, b, dxq)
        else:
            dat, dbt = oracle.contract_rows_vjp(np.swapaxes(a, 0, 1), np.swapaxes(b, 0, 1), dxq)
            da, db = np.swapaxes(dat, 0, 1), np.swapaxes(dbt, 0, 1)
        gp = oracle.project_vjp(zn, mn, wref, da, db)
        ref = {"z": ge["z"] + gp["z"], "ln_in_w": ge["ln_in_w"] + gp["ln_in_w"],
               "ln_in_b": ge["ln_in_b"] + gp["ln_in_b"]}
        for k in ("w_a_proj", "w_a_gate", "w_b_proj", "w_b_gate"):
            ref[k] = gp[k]
        for k in ("w_out_gate", "ln_out_w", "ln_out_b", "w_out_proj"):
            ref[k] = ge[k]
    got = {"z": zd.grad.double().cpu().numpy()}
    for k in pag.PARAM_NAMES:
        got[k] = params[k].grad.double().cpu().numpy()
    # dL/dz comes back in z's dtype: in bf16 mode rounded to nearest-even,
    # each entry off by at most 2^-8 of its size on top of the bar
    tol = {k: (1e-2 if dtype == "bf16" else 1e-4) for k in got}
    if dtype == "bf16":
        tol["z"] += 2.0 ** -8 * np.max(np.abs(ref["z"])) / np.sqrt(np.mean(ref["z"] ** 2))
    errs = {k: rel_err(got[k], ref[k]) for k in got}
    print("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= tol[k], (k, v)


def test_layer_autograd_second_backward_is_identical(dev):
    """Two backward passes through one graph (retain_graph) give the same
    gradients: the backward leaves the saved forward state untouched."""
    print("[case] layer autograd twice", flush=True)
    n = 45
    z, mask, wts = wl.make_small(n, seed=77, dtype="bf16", device="cpu")
    params = _params(wts, dev)
    zd = z.to(dev).requires_grad_(True)
    out = pag.trimul(zd, mask.to(dev), params, pra.OUTGOING)
    g = torch.randn_like(out)
    out.backward(g, retain_graph=True)
    first = [zd.grad.clone()] + [params[k].grad.clone() for k in pag.PARAM_NAMES]
    for t in [zd] + [params[k] for k in pag.PARAM_NAMES]:
        t.grad = None
    out.backward(g)
    second = [zd.grad] + [params[k].grad for k in pag.PARAM_NAMES]
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)
