"""bf16 <-> float64 conversions for the oracle (test infrastructure only).

bf16 is the upper 16 bits of an IEEE-754 binary32 value, so widening a bf16
bit pattern to float64 is exact.  Rounding float64 to bf16 is done directly
(one rounding, nearest-even), not through float32.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Widen bf16 bit patterns (uint16 array) to float64, exactly."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"bf16 bits must be uint16, got {bits.dtype}")
    u32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN payloads widen as NaN
        return u32.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to the nearest bf16 (ties to even); return uint16 bits.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and the binary32
    exponent range.  Values below the smallest normal (2**-126) are quantised
    to multiples of the smallest subnormal, 2**-133.  Overflow gives +-inf,
    NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = x[finite]
    mant, expo = np.frexp(xf)                     # xf = mant * 2**expo, 0.5 <= |mant| < 1
    quantum_exp = np.maximum(expo - 8, -133)      # 8 significant bits, subnormal floor
    q = np.ldexp(1.0, quantum_exp)
    r = np.rint(xf / q) * q                       # np.rint rounds half to even
    big = np.abs(r) >= np.ldexp(1.0, 128)
    r[big] = np.copysign(np.inf, r[big])
    out[finite] = r
    out[~finite] = x[~finite]
    f32 = out.astype(np.float32)                  # exact: r has <= 8 significant bits
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = np.uint16(0x7FC0)
    return bits


def as_f64(a):
    """Float64 view of an oracle input: uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)
