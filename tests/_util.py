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


def dalpha_bound(z_gpu, z_ref, dz_gpu, dz_ref, bias, alpha, n):
    """Per logit group: the error of dalpha_g = sum dz (z - b) / alpha_g that the z and dz
    errors alone carry into it (each of those is checked on its own), to first and
    second order: sum (|dz| |dz_err| ... ) over tokens and the group's logits."""
    zd = np.abs(np.asarray(z_gpu, np.float64) - z_ref)
    dzd = np.abs(np.asarray(dz_gpu, np.float64) - dz_ref)
    term = np.abs(dz_ref) * zd + dzd * np.abs(z_ref - bias) + dzd * zd
    grp = np.array([0] * n + [1] * n + [2] * (n * n))
    return np.array([term[:, grp == g].sum() for g in range(3)]) / np.abs(np.asarray(alpha, np.float64))


def assert_dalpha(gpu, ref, bound, tol):
    """dalpha within tol (inf-norm relative), or within twice the error its inputs
    z and dz carry (plus its own fp32 rounding): the reduction itself adds none."""
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    allowed = np.maximum(tol * np.abs(ref).max(), 2.0 * bound + 2.0 ** -23 * np.abs(ref))
    assert np.isfinite(gpu).all(), "dalpha: non-finite GPU values"
    assert (err <= allowed).all(), f"dalpha: error {err} > allowed {allowed}"
