"""Helpers of the GPU parity tests: device copies of seeded inputs, tolerance checks."""
import numpy as np
import torch

TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}
# tolerances on max |gpu - oracle| relative to the RMS of the oracle output
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def dev(a, dtype="fp32"):
    """numpy values (already representable in dtype) -> device tensor of that dtype (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(TDT[dtype])


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rms(a):
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def assert_close_rms(got, want, tol, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    scale = rms(want)
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol} x RMS {scale:.3e} (ratio {err / max(scale, 1e-30):.2e})"
    return err / max(scale, 1e-30)


def print_case(*args):
    print("[case]", *args, flush=True)
