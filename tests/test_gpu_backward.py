"""GPU parity of the contraction's backward (trimul_tile_backward) against the
oracle's gradients (oracle.contract_rows_vjp), through the C ABI.

The operands are exact in the storage dtype; in bf16 mode the library rounds
dx to bf16 (nearest-even) for the matrix-core products, so the reference uses
the same rounding (oracle.bf16_round) and the remaining difference is fp32
accumulation order: the bar is the contraction kernel's, 1e-5 of the rms."""

import numpy as np
import pytest
import torch

import oracle
import pair_representation_amd as pra
import workloads as wl
from tests.gpu_util import rel_err

pytestmark = pytest.mark.gpu

C = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def planar_to_xacc(planar):
    """Accumulator-layout tensor holding planar [128, rows, cols] (layout only)."""
    _, rows, cols = planar.shape
    rb, cb = (rows + 3) // 4, (cols + 15) // 16
    full = torch.zeros((C, rb * 4, cb * 16), dtype=torch.float32, device=planar.device)
    full[:, :rows, :cols] = planar
    return full.reshape(C, rb, 4, cb, 16).permute(1, 3, 0, 4, 2).contiguous()


def weights(dtype, dev):
    _, _, wts = wl.make_small(4, seed=1, dtype=dtype, device="cpu")
    return pra.Weights(wts, pra.BF16 if dtype == "bf16" else pra.F32, device=dev)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_rows,n_cols,k_lens", [
    (1, 1, [1]),
    (40, 300, [77]),
    (256, 256, [256]),
    (300, 129, [200, 315]),
    (150, 533, [64, 70, 33]),
    (277, 21, [100]),
    (513, 400, [130]),
])
def test_tile_backward_matches_oracle(dev, dtype, n_rows, n_cols, k_lens):
    """Several chunks of unequal length, ragged edges past 64-, 256- and
    384-wide blocks, 1 x 1 tiles: every gradient entry against float64."""
    print(f"[case] backward {dtype} {n_rows}x{n_cols} chunks {k_lens}", flush=True)
    r = np.random.default_rng(n_rows * 31 + n_cols + len(k_lens))
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    w = weights(dtype, dev)
    a_l, b_l, chunks = [], [], []
    k_off = 0
    for k_len in k_lens:
        ld = (k_len + 63) // 64 * 64
        a = r.standard_normal((C, n_rows, k_len))
        b = r.standard_normal((C, n_cols, k_len))
        if dtype == "bf16":
            a, b = oracle.bf16_round(a), oracle.bf16_round(b)
        A = torch.zeros((C, n_rows, ld), dtype=td)
        B = torch.zeros((C, n_cols, ld), dtype=td)
        A[:, :, :k_len] = torch.from_numpy(a).to(td)
        B[:, :, :k_len] = torch.from_numpy(b).to(td)
        chunks.append((k_off, k_len, pra.planar_to_operand(A.to(dev)), pra.planar_to_operand(B.to(dev))))
        a_l.append(a)
        b_l.append(b)
        k_off += k_len
    dx = r.standard_normal((C, n_rows, n_cols))
    dx_x = planar_to_xacc(torch.from_numpy(dx).float().to(dev))
    da, db = pra.tile_backward(w, n_rows, n_cols, chunks, dx_x)
    torch.cuda.synchronize()
    dxq = np.float32(dx).astype(np.float64)
    if dtype == "bf16":
        dxq = oracle.bf16_round(dxq)
    for i, k_len in enumerate(k_lens):
        ra, rb = oracle.contract_rows_vjp(np.moveaxis(a_l[i], 0, 2), np.moveaxis(b_l[i], 0, 2),
                                          np.moveaxis(dxq, 0, 2))
        ga = pra.xacc_to_planar(da[i], n_rows, k_len).cpu().double().numpy()
        gb = pra.xacc_to_planar(db[i], n_cols, k_len).cpu().double().numpy()
        ea = rel_err(ga, np.moveaxis(ra, 2, 0))
        eb = rel_err(gb, np.moveaxis(rb, 2, 0))
        print(f"  chunk {i} (k_len {k_len}): da {ea:.3e}  db {eb:.3e}", flush=True)
        assert ea <= 1e-5 and eb <= 1e-5


def test_tile_backward_full_size_sampled(dev):
    """The whole 3605-residue grid as one tile and one chunk, bf16, in the
    launch configuration the benchmark times; 48 sampled rows, columns and k
    entries of both gradients against float64 (each needs only a slice of dx
    and of one operand)."""
    n = 3605
    ld = (n + 63) // 64 * 64
    print(f"[case] backward full size n={n}", flush=True)
    w = weights("bf16", dev)
    g = torch.Generator(device=dev).manual_seed(7)
    A = torch.zeros((C, n, ld), dtype=torch.bfloat16, device=dev)
    B = torch.zeros((C, n, ld), dtype=torch.bfloat16, device=dev)
    A[:, :, :n] = torch.randn((C, n, n), generator=g, device=dev).to(torch.bfloat16)
    B[:, :, :n] = torch.randn((C, n, n), generator=g, device=dev).to(torch.bfloat16)
    dx = torch.randn((C, n, n), generator=g, device=dev)
    Ab, Bb = pra.planar_to_operand(A), pra.planar_to_operand(B)
    dx_x = planar_to_xacc(dx)
    da, db = pra.tile_backward(w, n, n, [(0, n, Ab, Bb)], dx_x)
    torch.cuda.synchronize()
    r = np.random.default_rng(11)
    I = np.sort(r.choice(n, 48, replace=False)); I[0], I[-1] = 0, n - 1
    J = np.sort(r.choice(n, 48, replace=False)); J[0], J[-1] = 0, n - 1
    K = np.sort(r.choice(n, 48, replace=False)); K[0], K[-1] = 0, n - 1
    It, Jt, Kt = (torch.as_tensor(v, device=dev) for v in (I, J, K))
    dxI = oracle.bf16_round(dx.index_select(1, It).double().cpu().numpy())      # [c, |I|, n]
    dxJ = oracle.bf16_round(dx.index_select(2, Jt).double().cpu().numpy())      # [c, n, |J|]
    aK = A.index_select(2, Kt).double().cpu().numpy()                            # [c, n, |K|]
    bK = B.index_select(2, Kt).double().cpu().numpy()
    # the oracle's gradients on the slices: da[I, K] needs dx[I, :] and b[:, K]
    # only, db[J, K] needs dx[:, J] and a[:, K] only (the other operand is
    # irrelevant to the gradient asked for, so zeros stand in for it)
    rows = lambda t: np.moveaxis(t, 0, 2)                                        # [c, r, s] -> [r, s, c]
    ref_da, _ = oracle.contract_rows_vjp(np.zeros((len(I), len(K), C)), rows(bK), rows(dxI))
    _, ref_db = oracle.contract_rows_vjp(rows(aK), np.zeros((len(J), len(K), C)), rows(dxJ))
    ref_da, ref_db = np.moveaxis(ref_da, 2, 0), np.moveaxis(ref_db, 2, 0)        # [c, |I|, |K|], [c, |J|, |K|]
    got_da = pra.xacc_to_planar(da[0], n, n).index_select(1, It).index_select(2, Kt).double().cpu().numpy()
    got_db = pra.xacc_to_planar(db[0], n, n).index_select(1, Jt).index_select(2, Kt).double().cpu().numpy()
    ea, eb = rel_err(got_da, ref_da), rel_err(got_db, ref_db)
    print(f"  sampled da {ea:.3e}  db {eb:.3e}", flush=True)
    assert ea <= 1e-5 and eb <= 1e-5
    full = pra.xacc_to_planar(da[0], n, n)
    assert torch.isfinite(full).all()
