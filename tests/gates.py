"""Value gates for the LoRA delta parity tests.

G1 (contract): max |y_gpu - y_ref| <= 1e-2 * max |y_ref|.
G2 (delta-sensitive, elementwise):
    |y_gpu - y_ref| <= 1e-2 * max |s d_ref| + 0.5 ulp_out(y_ref)
G1 alone is loose when the base y dominates the delta (Tiny: s d has a max of
about 0.13 next to |y| up to 4), so every parity test applies both.  The
expected error is far inside them: fp32 accumulation over at most 8192 terms
(relative error ~1e-6 of the delta) plus one rounding of y to the output type
(half an ulp, which G2 allows on top).
"""
import numpy as np


def half_ulp(y_ref: np.ndarray, dtype) -> np.ndarray:
    mag = np.abs(y_ref).astype(dtype)
    return 0.5 * np.spacing(mag).astype(np.float64)


def check_gates(y_gpu, y_ref, sd_ref, dtype, label=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert np.isfinite(y_gpu).all(), f"{label}: non-finite output (a page outside the batch was read?)"
    err = np.abs(y_gpu - y_ref)
    g1 = 1e-2 * np.abs(y_ref).max()
    assert err.max() <= g1, f"{label}: G1 failed, max err {err.max():.3e} > {g1:.3e}"
    g2 = 1e-2 * np.abs(sd_ref).max() + half_ulp(y_ref, dtype)
    bad = err > g2
    assert not bad.any(), (f"{label}: G2 failed at {int(bad.sum())} elements, worst excess "
                           f"{(err - g2).max():.3e}")
    return float(err.max())


def check_forward_gates(y_gpu, h_ref, sd_ref, base_abs, k, dtype, label=""):
    """Gates of the base-plus-delta product h = x W + s d.

    Unlike the delta, whose base y is an exact input, the base part x W is
    computed here: k fp16 products (exact in fp32) summed in fp32 in some
    order.  Any order of n additions errs by at most gamma_n * sum |terms|,
    gamma_n = n u / (1 - n u) with u = 2^-24, so G2 gains that term per element
    (base_abs = |x| |W|, elementwise, computed in fp64):
        |y_gpu - h_ref| <= 1e-2 * max |s d_ref| + 0.5 ulp_out(h_ref) + gamma_k * base_abs
    G1 is unchanged.
    """
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert np.isfinite(y_gpu).all(), f"{label}: non-finite output (a page outside the batch was read?)"
    err = np.abs(y_gpu - h_ref)
    g1 = 1e-2 * np.abs(h_ref).max()
    assert err.max() <= g1, f"{label}: G1 failed, max err {err.max():.3e} > {g1:.3e}"
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    g2 = 1e-2 * np.abs(sd_ref).max() + half_ulp(h_ref, dtype) + gamma * np.asarray(base_abs, np.float64)
    bad = err > g2
    assert not bad.any(), (f"{label}: G2 failed at {int(bad.sum())} elements, worst excess "
                           f"{(err - g2).max():.3e}")
    return float(err.max())
