"""Exact decoding of stored elements to float64, and the OCP E4M3FN codec.

Test infrastructure only (see the package docstring): nothing in the HIP
library imports or mirrors this file.

Stored tensors are handed to the oracle as their raw bits:

=========  ===========  ==================================================
name       numpy bits   meaning
=========  ===========  ==================================================
f32        uint32       IEEE binary32
f16        uint16       IEEE binary16
bf16       uint16       the upper 16 bits of an IEEE binary32
fp8_e4m3   uint8        OCP 8-bit float E4M3FN (no infinities)
int8       int8         two's-complement integer code (scaled per block)
=========  ===========  ==================================================

Every value of these formats is exactly representable in float64, so the
decode below is exact.

Why fp8 at all: the ybb.press page ("vLLM 与 LLM 推理部署实战", §6.2 "KV Cache
量化与分页调度联合优化") states that storing the KV cache in INT8 or FP8 halves
the bytes per token, and the intelliparadigm page (§6.1 "混合精度配置") names an
fp8 K cache.  Neither page fixes the fp8 variant, rounding or overflow rule; the
readings taken here are: OCP E4M3FN, round-to-nearest-even, finite overflow and
infinities saturate to the largest finite magnitude 448, NaN keeps its sign and
becomes the NaN code.  The saturation rule is a convention the pages do not fix
("parity unpinned" for inputs beyond 448 in magnitude); everything else is
pinned by the tests against closed forms and torch's CPU cast.

INT8 (the same ybb.press §6.2 sentence): the pages fix no scale granularity or
rounding.  The reading taken: symmetric codes in [-127, 127], one float32
scale per (block, KV head) for K and one for V, code = round-half-even of
float32(x) / float32(scale) (one correctly rounded float32 division), clamped
to [-127, 127]; NaN stores 0.  The value of a code is code * scale.
"""

from __future__ import annotations

import numpy as np

STORAGE_DTYPES = {
    "f32": np.uint32,
    "f16": np.uint16,
    "bf16": np.uint16,
    "fp8_e4m3": np.uint8,
    "int8": np.int8,
}


def e4m3_value_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes, as float64 (NaN for 0x7F/0xFF).

    Written from the format definition: 1 sign bit, 4 exponent bits with bias
    7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2**-6; the
    all-ones exponent with all-ones mantissa is NaN and there is no infinity.
    """
    values = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            values[code] = np.nan
        elif exp_field == 0:
            values[code] = sign * (mant / 8.0) * 2.0 ** (-6)
        else:
            values[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return values


_E4M3 = e4m3_value_table()
# Non-negative finite codes 0x00..0x7E in increasing order of value.
_POS_VALUES = _E4M3[:0x7F].copy()
_MAX_FINITE = _POS_VALUES[-1]  # 448


def e4m3_encode(x_f32: np.ndarray) -> np.ndarray:
    """Encode float32 values to E4M3FN codes (uint8).

    Nearest representable value by plain search over the 127 non-negative
    finite codes; a tie goes to the code whose mantissa is even; magnitudes
    above 448 (and infinities) saturate to 448; NaN maps to 0x7F with the
    input's sign bit.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    flat = x.reshape(-1).astype(np.float64)
    sign = np.signbit(flat).astype(np.uint8) << 7
    mag = np.abs(flat)
    codes = np.zeros(flat.shape, dtype=np.uint8)
    nan = np.isnan(flat)
    finite_mag = np.where(nan, 0.0, np.minimum(mag, _MAX_FINITE))
    # Index of the first table value >= mag; the nearest value is either it or
    # its predecessor.
    hi = np.searchsorted(_POS_VALUES, finite_mag, side="left")
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_hi = np.abs(_POS_VALUES[hi] - finite_mag)
    d_lo = np.abs(finite_mag - _POS_VALUES[lo])
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    # On a tie pick the even code (even mantissa, because the code's low bit
    # is the mantissa's low bit).
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    chosen = np.where(pick_hi, hi, lo).astype(np.uint8)
    codes[:] = chosen
    codes[nan] = 0x7F
    codes |= sign
    return codes.reshape(x.shape)


def decode_elements(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode raw stored bits of the given element type exactly to float64."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        widened = bits.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return widened.view(np.float32).astype(np.float64)
    if dtype == "fp8_e4m3":
        return _E4M3[bits.astype(np.uint8)]
    if dtype == "int8":
        return bits.astype(np.uint8).view(np.int8).astype(np.float64)
    raise ValueError(f"unknown element type {dtype!r}")


def int8_encode(x_f32: np.ndarray, scale_f32) -> np.ndarray:
    """Symmetric INT8 code of float32 values under a float32 scale (see the
    module docstring): round half to even of x / scale, clamped to ±127, NaN -> 0."""
    x = np.asarray(x_f32, dtype=np.float32)
    q = x / np.asarray(scale_f32, dtype=np.float32)        # one float32 division
    q = np.where(np.isnan(q), np.float32(0), q)
    return np.clip(np.rint(q), -127, 127).astype(np.int8)
