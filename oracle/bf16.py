"""bfloat16 and float16 storage rounding for the oracle (test infrastructure only).

The pages never define a low-precision format; the C++/CUDA page (section 3.4,
mixed precision) describes fp32 master weights with low-precision activations,
and the workload names bfloat16.  The reading used here: a value stored as bf16
is the bf16 number nearest to the exact value, ties to even (IEEE round to
nearest even on an 8-bit significand), NaN stays NaN, values past the largest
finite bf16 become infinity.

The rounding is applied directly to the float64 value (no intermediate float32
rounding), which is the mathematical definition of "nearest bf16 value".
"""

import numpy as np

_BF16_MAX = float(np.float64((2.0 - 2.0 ** -7) * 2.0 ** 127))


def round_bf16(x):
    """Return float64 array holding the nearest-even bfloat16 value of ``x``.

    bf16 keeps 8 significant bits (7 stored).  A float64 keeps 53, so the
    45 low significand bits are rounded away: add half an ulp of the kept
    part (minus one if the kept lsb is 0, which makes ties go to even) and
    clear the low bits.  Exponents of bf16 and float32 agree; results below
    the normal range of bf16 (|x| < 2**-126) are rounded on the bf16 subnormal
    grid (step 2**-133) explicitly.  Non-finite inputs pass through.
    """
    a = np.asarray(x, dtype=np.float64)
    u = np.ascontiguousarray(a).view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = u + np.uint64((1 << 44) - 1) + lsb
    u = u & ~np.uint64((1 << 45) - 1)
    r = u.view(np.float64).reshape(a.shape)
    with np.errstate(invalid="ignore", over="ignore"):
        big = np.abs(r) > _BF16_MAX
        if big.any():
            r[big] = np.copysign(np.inf, a[big])
        tiny = np.abs(a) < 2.0 ** -126
        if tiny.any():
            step = 2.0 ** -133
            r[tiny] = np.round(a[tiny] / step) * step   # np.round: half to even
        bad = ~np.isfinite(a)
        if bad.any():
            r[bad] = a[bad]
    return r


def round_fp16(x):
    """Return float64 array holding the nearest-even IEEE binary16 value of ``x``.

    The C++/CUDA page (section 3.4) runs activations and gradients in FP16 with
    fp32 master weights.  binary16 keeps 11 significant bits, exponents down to
    2**-14 (subnormal step 2**-24) and a largest finite value of 65504; values
    at or past the midpoint 65520 become infinity.  NumPy's float64 -> float16
    cast rounds the float64 value once, to nearest with ties to even (no
    intermediate float32 rounding); it serves as the step here.
    """
    a = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return a.astype(np.float16).astype(np.float64)
