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
    def get_z(ri, ci):
        ri_t = torch.as_tensor(np.asarray(ri), device=z_dev.device, dtype=torch.long)
        ci_t = torch.as_tensor(np.asarray(ci), device=z_dev.device, dtype=torch.long)
        return z_dev.index_select(0, ri_t).index_select(1, ci_t).to(torch.float64).cpu().numpy()

    def get_mask(ri, ci):
        ri_t = torch.as_tensor(np.asarray(ri), device=mask_dev.device, dtype=torch.long)
        ci_t = torch.as_tensor(np.asarray(ci), device=mask_dev.device, dtype=torch.long)
        return mask_dev.index_select(0, ri_t).index_select(1, ci_t).cpu().numpy()

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
