"""Comparison helpers shared by the GPU parity tests."""
import math

import numpy as np
import torch

# Tolerances (see the design notes: readings of the stated tolerances).
BF16_ABS = 2e-2          # max abs error on O, dQ, dK, dV for bf16 inputs, fp32 accumulation
BF16_LSE_ABS = 1e-3      # LSE of bf16 inputs (float32 output)
F32_REL = 1e-5           # normwise relative error, float32 tiny configuration
# A bf16 output carries the rounding of its final cast, at most half an ulp:
# 2^-8 of the value's magnitude. It is allowed on top of the computation error.
BF16_CAST = 2.0 ** -8


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def max_abs(gpu, ref):
    return float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0


def check_bf16(name, gpu, ref, tol=BF16_ABS):
    """max |gpu - ref| <= tol + 2^-8 |ref| elementwise (the bf16 output cast)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "%s has non-finite values" % name
    excess = np.abs(gpu - ref) - (tol + BF16_CAST * np.abs(ref))
    worst = float(np.max(excess)) if excess.size else -1.0
    assert worst <= 0.0, "%s: max abs err %.4g exceeds %.3g + 2^-8|ref| (worst excess %.3g)" % (
        name, max_abs(gpu, ref), tol, worst)
    return max_abs(gpu, ref)


def check_abs(name, gpu, ref, tol):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(gpu), fin), "%s: non-finite pattern differs" % name
    err = max_abs(gpu[fin], ref[fin])
    assert err <= tol, "%s: max abs err %.4g > %.3g" % (name, err, tol)
    return err


def check_rel(name, gpu, ref, tol=F32_REL):
    """Normwise relative error max|gpu - ref| / max|ref| (elementwise relative
    error is undefined near zero)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    den = float(np.max(np.abs(ref)))
    err = max_abs(gpu, ref) / (den if den > 0 else 1.0)
    assert err <= tol, "%s: normwise rel err %.3g > %.1g" % (name, err, tol)
    return err


def default_scale(d):
    return 1.0 / math.sqrt(d)


# Long sequences: an output row that averages thousands of terms is far
# smaller than the absolute bar (|O| of a late row of a 64K causal sequence
# is ~0.01), so the long-context samples are also held to a per-row
# normwise relative bound. bf16 rounding of P, dS and the output gives
# about 2^-9 relative error per row; a missing or doubled chunk pair or key
# tile changes a row by a sizeable fraction of its own norm.
LONG_ROW_REL = 1e-2


def check_rows_rel(name, gpu, ref, tol=LONG_ROW_REL):
    """Per-row normwise relative error max_c|gpu - ref| / max_c|ref| over the
    last axis, for every row."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    den = np.max(np.abs(ref), axis=-1)
    err = np.max(np.abs(gpu - ref), axis=-1) / np.where(den > 0, den, 1.0)
    worst = float(np.max(err)) if err.size else 0.0
    assert worst <= tol, "%s: per-row normwise rel err %.3g > %.1g (row %s)" % (
        name, worst, tol, np.unravel_index(int(np.argmax(err)), err.shape))
    return worst
