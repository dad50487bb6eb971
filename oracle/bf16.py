"""bf16 rounding for the oracle (test infrastructure only).

bf16 keeps float32's 8 exponent bits and 7 explicit mantissa bits.  A float64
value is rounded once, directly, to the nearest bf16 value with ties to even
(no intermediate float32 step, so there is no double rounding).
"""
from __future__ import annotations

import numpy as np


def round_f64(v) -> np.ndarray:
    """Nearest bf16 value (returned as float64), ties to even."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = (v != 0) & np.isfinite(v)
    m, ex = np.frexp(v[nz])             # v = m * 2**ex, 0.5 <= |m| < 1
    # bf16 normal numbers hold 8 significant bits: ulp = 2**(ex - 8).
    # Below the smallest normal exponent the ulp stays at 2**-133.
    ulp_exp = np.maximum(ex - 8, -133)
    q = np.ldexp(v[nz], -ulp_exp)       # exact: power-of-two scaling
    q = np.rint(q)                      # round half to even
    out[nz] = np.ldexp(q, ulp_exp)
    out[~np.isfinite(v)] = v[~np.isfinite(v)]
    # signed zero: keep the sign of the input
    out = np.where((out == 0) & np.signbit(v), -0.0, out)
    return out


def to_bits(v) -> np.ndarray:
    """Round float64 to bf16 and return the bit patterns as uint16."""
    r = round_f64(v).astype(np.float32)   # exact: r is a bf16 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def from_bits(b) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Distance in bf16 ulps between two bit-pattern arrays (ordered-integer
    mapping, so it is exact across zero and across binades)."""
    def key(x):
        x = np.asarray(x, dtype=np.uint16).astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(key(a_bits) - key(b_bits))
