"""Shared helpers of the test suite: moving seeded inputs to the GPU and back,
and the error metric.  No arithmetic of the method lives here."""
import numpy as np

from manifold_constrained_residuals_amd import inputs as I


def to_dev(a, torch):
    """storage array (fp32, or uint16 bf16 bits) -> torch tensor on cuda:0"""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def to_host(t, torch):
    """torch tensor -> exact fp64 numpy array"""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return I.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def rel_inf(gpu, ref):
    """max |gpu - ref| / max |ref| over the tensor (inf-norm relative error)"""
    gpu = np.asarray(gpu, np.float64); ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    num = np.abs(gpu - ref).max()
    return num / den if den > 0 else num


def assert_close(name, gpu, ref, tol):
    e = rel_inf(gpu, ref)
    assert np.isfinite(gpu).all(), f"{name}: non-finite GPU values"
    assert e <= tol, f"{name}: rel inf-norm error {e:.3e} > {tol:.1e}"
    return e


TOL = {"f32": 1e-5, "bf16": 1e-2}


def proj_ref(z_ref, bias, alpha, n):
    """The unscaled normalised projection p / r from the oracle's fp64 logits:
    z = alpha_g p / r + b, so p / r = (z - b) / alpha_g (alpha_g nonzero in every test
    workload; the fp64 subtraction loses nothing that matters at 1e-5)."""
    a = np.repeat(np.asarray(alpha, np.float64), [n, n, n * n])
    return (np.asarray(z_ref, np.float64) - np.asarray(bias, np.float64)[None, :]) / a[None, :]
