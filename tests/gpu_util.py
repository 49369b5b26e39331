"""Helpers for the GPU tests: host<->device copies of bit patterns, case banners."""
import sys

import numpy as np

# A bound on the additions along any path of the kernels' fp32 sum trees:
# two fma chains of 4V (bf16) or 2V (fp32) terms per lane, their sum, a
# 6-level wave tree and G - 1 sequential wave totals, with V <= 16 and
# G <= 16 (at most 54).  The strict checks use min(this, the generic bound).
KERNEL_DEPTH = 64


def depth_for(cols: int) -> int:
    from oracle.check import default_depth
    return min(default_depth(cols), KERNEL_DEPTH)


def announce(*parts):
    """Name the case before a GPU step (flushed, so a lost box still shows it)."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def dev_bits(a: np.ndarray):
    """uint16 bf16 bits -> torch.bfloat16 tensor on cuda:0."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def host_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def sample_rows(rows: int, n: int, seed: int, must=()) -> np.ndarray:
    """Sorted row sample: first/last rows, rows in `must`, and random rows."""
    rng = np.random.default_rng(seed)
    pick = set([0, rows - 1]) | set(int(m) for m in must)
    pick |= set(rng.choice(rows, size=min(n, rows), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def unit_norm_ok(y, skip_rows=None, tol=2.0 ** -8):
    """Every row of a bf16 tensor has length 1 within tol (GPU-side property)."""
    import torch
    n = y.float().pow(2).sum(dim=1).sqrt()
    if skip_rows is not None and len(skip_rows):
        keep = torch.ones_like(n, dtype=torch.bool)
        keep[torch.as_tensor(skip_rows, device=n.device)] = False
        n = n[keep]
    return bool(((n - 1).abs() <= tol).all().item())
