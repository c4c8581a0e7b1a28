"""Helpers of the GPU parity tests: device copies of seeded inputs, tolerance checks."""
import numpy as np
import torch

TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}
# Tolerance on max |gpu - oracle| relative to the RMS of the oracle output, against the exact (fp64,
# unrounded) oracle: the stated bars for fp32 and bf16 layer outputs.  (The storage-precision oracle -- the
# tensors handed between operators rounded to the model dtype -- is reported beside it; end to end it agrees
# only up to rounding flips that the norms amplify, so single operators are checked against it element-wise.)
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
    if err > tol * scale:
        idx = np.unravel_index(int(np.argmax(np.abs(got - want))), got.shape)
        raise AssertionError(f"{what}: max|err| {err:.3e} > {tol} x RMS {scale:.3e} (ratio {err / max(scale, 1e-30):.2e}) "
                             f"at {tuple(int(i) for i in idx)}: got {got[idx]:.6g} want {want[idx]:.6g}")
    return err / max(scale, 1e-30)


def print_case(*args):
    print("[case]", *args, flush=True)


def assert_close_elem(got, want, dtype, what=""):
    """Element-wise bound for one rounding of the result to the output dtype: |got - want| <= u |want| + 1e-5 RMS.
    bf16: u = 2^-7 = one unit in the last place at worst (a fp32 result next to a rounding midpoint may round
    to the other neighbour of the exact value); fp32: u = 2e-6 (a few fp32 operations)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    u = 2.0 ** -7 if dtype == "bf16" else 2e-6
    bound = u * np.abs(want) + 1e-5 * rms(want)     # absolute term: fp32 sums with cancellation
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off; worst {float(np.max(np.abs(got - want) - bound)):.3e}"


def assert_close_attention(got, want, want_abs, dtype, what=""):
    """Element-wise bound for the attention kernel's output.

    bf16: one rounding of the result (as ``assert_close_elem``) plus the error of the probabilities.  The
    kernel feeds each probability p_k to the P.V product as a hi + lo pair of bf16 values, 16 significant
    bits, so p_k carries a relative error of at most 2^-17 (scores and exp2 add far less).  The output error
    is then at most eps * sum_k p_k |v_k| / sum_k p_k, which is the attention of the same q and K over |V|
    (``want_abs``); eps = 2^-15 leaves a factor of 4.  Against the row's RMS this term is not small for a
    prompt row spread over hundreds of keys, whose output (a mean of many values) is much smaller than the
    values themselves.  fp32 rows: ``assert_close_elem``."""
    if dtype != "bf16":
        return assert_close_elem(got, want, dtype, what)
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    want_abs = np.asarray(want_abs, np.float64)
    assert got.shape == want.shape == want_abs.shape, (what, got.shape, want.shape, want_abs.shape)
    bound = 2.0 ** -7 * np.abs(want) + 2.0 ** -15 * want_abs + 1e-6 * rms(want)
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off; worst {float(np.max(np.abs(got - want) - bound)):.3e}"
