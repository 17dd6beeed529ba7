"""Element formats, decoded from their bit fields (test infrastructure only).

The pages name the stored parts only: NVFP4 weights as U8 bytes of E2M1 codes
with F8_E4M3 block scales, kept in their stored form [FP4-Local checkpoints on
DGX Spark, §4 Round 1, #489], and MXFP8 as E4M3 blocks of 32 with an E8M0 scale
[same page, §4 Round 1, #521]. They print no bit layout, so the layouts are
taken from the OCP Microscaling Formats (MX) v1.0 specification:

* E2M1: sign | 2 exponent bits | 1 mantissa bit, exponent bias 1, no inf/NaN.
* E4M3 ("fn" variant, the safetensors F8_E4M3): sign | 4 exponent bits | 3
  mantissa bits, bias 7, no infinities, S.1111.111 is NaN, max 448.
* E8M0: an unsigned biased exponent, 2^(c-127); 0xFF is NaN.

Packing of two E2M1 codes in a byte is not stated on the pages either; the
reading taken is: element 2j in the low nibble of byte j, element 2j+1 in the
high nibble.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code."""
    code = int(code) & 0xF
    s = -1.0 if code >> 3 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:                      # subnormal: 2^(1-bias) * m/2, bias 1
        mag = m * 0.5
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return s * mag


def e4m3_value(code: int) -> float:
    """Value of one E4M3 ("fn") byte; NaN for S.1111.111."""
    code = int(code) & 0xFF
    s = -1.0 if code >> 7 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = 2.0 ** (-6) * (m / 8.0)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return s * mag


def e8m0_value(code: int) -> float:
    """Value of one E8M0 byte; NaN for 0xFF."""
    code = int(code) & 0xFF
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


# 256-entry float64 tables, built from the scalar definitions above.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> float64 [..., K]: byte j holds element 2j in its low
    nibble and element 2j+1 in its high nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = E2M1_TABLE[packed & 0x0F]
    hi = E2M1_TABLE[packed >> 4]
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


_BF16_MAX_EXP = 128  # values >= 2^128 after rounding are +-inf


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16, to nearest with ties to even, in ONE
    step from float64 (no float32 intermediate); returns float64 values that
    are exactly representable in bfloat16 (or +-inf / NaN).

    bfloat16 keeps 8 significant bits and float32's exponent range: normal
    numbers down to 2^-126, subnormals in steps of 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                      # |x| in [2^(e-1), 2^e)
    q_exp = np.maximum(e, -125) - 8          # quantum: 2^(e-1-7), floor 2^-133
    scaled = np.ldexp(xf, -q_exp)            # exact (power-of-two scaling)
    r = np.ldexp(np.rint(scaled), q_exp)     # np.rint: round half to even, exact here
    r = np.where(np.abs(r) >= 2.0 ** _BF16_MAX_EXP, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """bf16_rne() as uint16 bit patterns."""
    r = bf16_rne(x)
    f32 = r.astype(np.float32)               # exact: bfloat16 values are float32 values
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    return bits


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |v| (the quantum of v's binade)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(v == 0, 2.0 ** -133, v))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)
