"""Shared helpers for the GPU parity tests (comparison metric, tolerances)."""
import numpy as np
import torch

# Tolerances on max|gpu - oracle| / max|oracle|, per element type of q/k/v/o.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| in fp64 (gpu values upcast exactly)."""
    g = gpu.detach().to("cpu", torch.float64).numpy() if isinstance(gpu, torch.Tensor) \
        else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if not np.all(np.isfinite(g)):
        return float("inf")
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / den) if den > 0 else float(np.max(np.abs(g)))


def assert_close(name, gpu, ref, tol):
    e = rel_err(gpu, ref)
    print(f"  {name}: rel err {e:.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: relative error {e:.3e} exceeds {tol:.1e}"
    return e


class RelErrAccum:
    """max |gpu - ref| / max |ref| accumulated over pieces of one output that
    are compared one after another (the same metric as rel_err over their
    union)."""

    def __init__(self, name):
        self.name, self.num, self.den, self.count, self.finite = name, 0.0, 0.0, 0, True

    def add(self, gpu, ref):
        g = gpu.detach().to("cpu", torch.float64).numpy() if isinstance(gpu, torch.Tensor) \
            else np.asarray(gpu, np.float64)
        r = np.asarray(ref, np.float64)
        assert g.shape == r.shape, (g.shape, r.shape)
        if not np.all(np.isfinite(g)):
            self.finite = False
            return
        self.num = max(self.num, float(np.max(np.abs(g - r))) if g.size else 0.0)
        self.den = max(self.den, float(np.max(np.abs(r))) if r.size else 0.0)
        self.count += g.size

    def check(self, tol):
        assert self.finite, f"{self.name}: non-finite GPU values"
        e = self.num / self.den if self.den > 0 else self.num
        print(f"  {self.name}: rel err {e:.3e} over {self.count} values (tol {tol:.0e})",
              flush=True)
        assert e <= tol, f"{self.name}: relative error {e:.3e} exceeds {tol:.1e}"
        return e
