"""Helpers shared by the GPU parity tests: tolerances and comparisons.

The tolerances are the stated bars: max-abs 1e-2 for fp32-accumulated bf16
attention, relative RMSE 5e-2 for the fp8 path, bit-exact for the page
gather and the quantiser's codes. A bf16 *output* adds its own rounding: half
a bf16 ulp of the reference value, which alone exceeds 1e-2 once |O| >= 4, so
bf16-output checks allow 1e-2 + ulp/2 of the reference element.
"""

import sys

import numpy as np
import torch

ATOL = 1e-2
FP8_REL_RMSE = 5e-2
# The MFMA kernels normalise by l, the fp32 sum of the unrounded P, so their
# LSE = m + log l carries fp32 rounding only: the scores' accumulation over d
# bf16 products (d * 2^-24 of sum |q_k k_k| * scale, under 6e-5 for N(0,1)
# inputs at d <= 128), l added tile by tile (about (N/64 + 5) * 2^-24
# relative in the worst case, with rounding errors of random sign growing
# like its square root), and one rounding each in exp2 and log2. Over the
# GPU suite the worst measured error was 1.75e-6 (MFMA prefill paths, heads
# up to 2^18 keys) and 1.5e-6 (decode); 1e-4 keeps a margin of about 50x
# and fails a real loss of precision (a normaliser of bf16-rounded weights
# alone would be off by up to 2e-3).
LSE_TOL_MFMA = 1e-4
# The fp8 matrix cores multiply E4M3 codes exactly but accumulate the raw code
# products (up to 448^2 each) in fp32 before the block scales apply, so a score
# carries the fp32 rounding of sums far larger than itself. With the outlier
# workloads (LSE near 130) this measured 3.3e-4 of |LSE|; the fp8 paths' LSE is
# held to 2e-3 of max(1, |LSE|).
LSE_REL_TOL_FP8 = 2e-3


def check_lse(got, ref, tol=None, what=""):
    """max |LSE_gpu - LSE_ref| over the finite rows <= tol (default
    LSE_TOL_MFMA); rows with no visible key must be -inf on both sides. The
    error is printed so a run's log records the margin."""
    tol = LSE_TOL_MFMA if tol is None else tol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    live = np.isfinite(ref)
    assert np.all(got[~live] == -np.inf), f"{what}: LSE of a row with no key"
    err = float(np.max(np.abs(got[live] - ref[live]))) if live.any() else 0.0
    say(f"LSE max abs err {err:.3g} (tol {tol:.3g}) {what}")
    assert err <= tol, f"{what}: LSE max abs err {err:.3g} > {tol:.3g}"
    return err


def check_lse_fp8(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    live = np.isfinite(ref)
    assert np.all(got[~live] == -np.inf)
    err = np.abs(got[live] - ref[live]) / np.maximum(1.0, np.abs(ref[live]))
    assert err.max() <= LSE_REL_TOL_FP8, f"fp8 LSE relative error {err.max():.3g}"
    return float(err.max())


def say(*a):
    """Print a progress line and flush (so a GPU run shows what it was doing)."""
    print(*a, flush=True)
    sys.stdout.flush()


def half_ulp_bf16(ref):
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_close(got, ref, out_bf16, what=""):
    """max |got - ref| <= 1e-2 (+ half a bf16 ulp of ref for bf16 outputs)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = ATOL + (half_ulp_bf16(ref) if out_bf16 else 0.0)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"{what}: max err {err.max():.3g} at {worst} (ref {ref[worst]:.4g}, tol {tol if np.isscalar(tol) else tol[worst]:.3g})"
    return float(err.max())


def rel_rmse(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.sum((got - ref) ** 2) / np.sum(ref ** 2)))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def cuda(t):
    return t.contiguous().to("cuda")


def sample_rows(N, seed, extra=24):
    """Edge rows (tile boundaries, first, last) plus a seeded random sample."""
    fixed = {0, 1, 2, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 2, N - 1}
    rng = np.random.default_rng(seed)
    rnd = set(rng.integers(0, N, size=extra).tolist())
    return sorted(r for r in fixed | rnd if 0 <= r < N)
