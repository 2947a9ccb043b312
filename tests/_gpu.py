"""Shared helpers for the GPU parity tests (not collected by pytest)."""

import numpy as np
import torch

import workloads as wl

# Tolerances for the fp16 outputs against the float64 oracle: max-abs 2e-3
# and relative L2 1e-3, the stated bound for fp16 inputs with fp32
# accumulation.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def dev():
    return torch.device("cuda:0")


def to_dev(a, device=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device or dev())


def to_host(t):
    return t.detach().cpu().numpy()


def device_pools(case, layer=0, device=None):
    """(k_pool, v_pool) on the device: the case's host pools if it has them,
    else seeded device fills."""
    device = device or dev()
    if case.k_pool is not None:
        return to_dev(case.k_pool, device), to_dev(case.v_pool, device)
    return (wl.device_pool(torch, case, layer, 0, device),
            wl.device_pool(torch, case, layer, 1, device))


def assert_close(out, ref, what=""):
    """fp16 GPU output (tensor or array) against a float64 reference, over
    the rows where the reference is defined."""
    got = to_host(out).astype(np.float64) if isinstance(out, torch.Tensor) else \
        np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rows = ~np.isnan(ref).any(axis=tuple(range(1, ref.ndim)))
    got, ref = got[rows], ref[rows]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref)) or 1.0
    rel = float(np.linalg.norm(got - ref)) / denom
    worst = np.unravel_index(int(err.argmax()), err.shape) if err.size else None
    print(f"[{what}] rows={int(rows.sum())} max_abs={max_abs:.3e} rel_l2={rel:.3e} worst={worst}",
          flush=True)
    assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs} at {worst}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel}"
    return max_abs, rel
