"""Storage-dtype arithmetic of the oracle.

A reduction step stores ``round_dtype(widen(a) + widen(b))``:

* fp32: one IEEE-754 binary32 addition, round to nearest even. numpy's float32
  add is exactly that. Subnormals are kept (numpy does not flush them).
* bf16: both operands widened exactly to fp32 (bf16 is the top half of a
  binary32), added in fp32, and the fp32 sum rounded to bf16 to nearest even.
  This is the reading taken for "bf16 inputs with fp32 accumulate": every value
  that is stored, including values in flight between ranks, is bf16.
* int32: two's-complement addition that wraps.

bf16 rounding is written from the format's definition (drop the low 16 bits of
the binary32 pattern, rounding to the nearest representable value, ties to the
one with an even last bit). It is pinned against torch's CPU cast and against a
brute-force nearest search in the tests.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even). Returns uint16 bits.

    The kept half is the high 16 bits. The dropped half ``lo`` is compared with the
    midpoint 0x8000: above rounds up, below rounds down, equal rounds to make the
    kept half even. Adding ``0x7FFF + lsb`` and shifting right by 16 does exactly
    this, and a carry out of the mantissa moves correctly into the exponent (up to
    infinity). NaNs are returned quiet with their sign.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(f)
    if nan.any():
        sign = (u >> np.uint64(16)).astype(np.uint32) & np.uint32(0x8000)
        rounded = np.where(nan, sign | np.uint32(0x7FC0), rounded)
    return rounded.astype(np.uint16)


def add_stored(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """One reduction step on stored values: round_dtype(widen(a) + widen(b))."""
    if dtype == "f32":
        return (np.asarray(a, np.float32) + np.asarray(b, np.float32)).astype(np.float32)
    if dtype == "bf16":
        s = bf16_to_f32(a) + bf16_to_f32(b)  # float32 + float32 -> float32, RNE
        return f32_to_bf16_rne(s)
    if dtype == "i32":
        s = np.asarray(a, np.int32).astype(np.int64) + np.asarray(b, np.int32).astype(np.int64)
        return wrap_i32(s)
    raise ValueError(f"unknown dtype {dtype!r}")


def wrap_i32(v: np.ndarray) -> np.ndarray:
    """Two's-complement wrap of int64 values into int32."""
    v = np.asarray(v, dtype=np.int64)
    return ((v + 2**31) % 2**32 - 2**31).astype(np.int32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored data."""
    if dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x).astype(np.float64)


def storage_np(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "i32": np.int32}[dtype]


def scaled_error(y: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray, dtype: str) -> float:
    """max_i |y_i - s_i| / sum_r |x_{r,i}|.

    ``exact`` is the float64 sum s, ``abs_sum`` the float64 sum of magnitudes of the
    addends. The denominator is the scale of the standard forward-error bound of
    recursive summation, so the ratio stays bounded where sums cancel. Columns whose
    addends are all zero must give exactly zero.
    """
    yv = to_f64(y, dtype)
    err = np.abs(yv - exact)
    zero = abs_sum == 0
    if zero.any() and np.any(yv[zero] != 0):
        return float("inf")
    denom = np.where(zero, 1.0, abs_sum)
    if err.size == 0:
        return 0.0
    return float(np.max(err / denom))


def elementwise_rel_error(y: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray, dtype: str,
                          floor: float = 1e-3) -> float:
    """max |y - s| / |s| over elements with |s| >= floor * sum|x| (reported beside scaled_error)."""
    yv = to_f64(y, dtype)
    keep = np.abs(exact) >= floor * abs_sum
    keep &= abs_sum > 0
    if not keep.any():
        return 0.0
    return float(np.max(np.abs(yv[keep] - exact[keep]) / np.abs(exact[keep])))
