"""Helpers shared by the GPU parity tests (no arithmetic of the method)."""

import numpy as np
import torch


def rel_err(got, ref):
    """max |got - ref| / rms(ref), both as float64 arrays."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got - ref)))


def device_getters(z_dev, mask_dev):
    """get_z / get_mask callables for the oracle's sampled evaluation that copy
    the requested rows x cols of device tensors to the host."""
    def pick(t, ri, ci):
        # the smaller index set first, so the intermediate copy stays small
        ri_t = torch.as_tensor(np.asarray(ri), device=t.device, dtype=torch.long)
        ci_t = torch.as_tensor(np.asarray(ci), device=t.device, dtype=torch.long)
        if len(ri_t) <= len(ci_t):
            return t.index_select(0, ri_t).index_select(1, ci_t)
        return t.index_select(1, ci_t).index_select(0, ri_t)

    def get_z(ri, ci):
        return pick(z_dev, ri, ci).to(torch.float64).cpu().numpy()

    def get_mask(ri, ci):
        return pick(mask_dev, ri, ci).cpu().numpy()

    return get_z, get_mask


def sample_indices(n, seed, count=48, must=()):
    """Sorted unique residues: the first and last, the given ones (clipped to
    [0, n)), and seeded random ones up to ``count``."""
    s = {0, n - 1}
    s.update(int(m) for m in must if 0 <= m < n)
    r = np.random.default_rng(seed)
    while len(s) < min(count, n):
        s.add(int(r.integers(0, n)))
    return np.array(sorted(s))


def whole_tensor_checks(out, mask_dev, sample_out, sample_mask, rows_per_step=512):
    """Finite everywhere, exact zeros at masked pairs, and the rms over kept
    pairs within 5% of the sample's rms over its kept pairs; the output is
    scanned in row blocks so no temporary of its full size is made."""
    sq = 0.0
    kept = 0
    for r0 in range(0, out.shape[0], rows_per_step):
        o = out[r0:r0 + rows_per_step]
        assert bool(torch.isfinite(o).all())
        m = mask_dev[r0:r0 + rows_per_step] != 0
        if bool((~m).any()):
            assert torch.count_nonzero(o[~m]).item() == 0
        sq += torch.sum(o[m].double() ** 2).item()
        kept += int(m.sum().item()) * o.shape[-1]
    rms_full = (sq / kept) ** 0.5
    s = sample_out[np.asarray(sample_mask) != 0]
    rms_s = float(np.sqrt(np.mean(s ** 2)))
    print(f"  rms over kept pairs: full {rms_full:.4f} sample {rms_s:.4f}")
    assert abs(rms_full / rms_s - 1) < 0.05
