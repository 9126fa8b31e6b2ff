"""Asymmetric group-wise INT4 quantization (reference, fp64 / exact).

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this module.

Source passage
--------------
* Q-TensorFormer model card, section 6 "Adaptive KV Cache Quantization &
  Attention-Sink Eviction", asymmetric group-wise INT4 formula: over a group
  of values the step is (max - min) / 15 and the offset is the minimum; a
  value minus the offset, divided by the step, is rounded to the nearest
  integer and clamped to [0, 15]; the reconstruction is code * step + offset.

Readings taken where the passage is open
----------------------------------------
* Group: g consecutive values of one row (one token of one head); a row of d
  values has d / g groups, each with its own step s and offset z.  The page
  gives no group size; g is a parameter (a multiple of 16 dividing d).
* z = min of the group (exact in binary32); s = RN32(RN32(max - min) / 15),
  IEEE binary32 subtraction and division.
* code = clamp(rne(RN32(RN32(x - z) / s)), 0, 15): binary32 subtraction and
  division, then the nearest integer with ties to even (the rounding bracket
  on the page has no tie rule).
* A group whose step is +0 (all values equal, or a range so small that
  range / 15 underflows) gets step +0 and all codes 0; it reconstructs to z.
* Reconstruction: RN32(RN32(code * s) + z); an fp16 output is RN16 of that
  binary32 value.
* Storage: codes two per byte, the even-indexed value of a pair in the low
  nibble (LSB-first, as the QJL sign bits); steps and offsets binary32,
  [rows, d / g] each.
* Non-finite input is outside the domain, and so is a group whose range
  max - min overflows binary32 (its step would be infinite): the reference
  raises for both.

Why fp64 gives the binary32 results exactly: every operand is binary32 (or
binary16 widened exactly); one fp64 operation followed by a cast to binary32
is correctly rounded, since 53 >= 2*24 + 2 (Figueroa, "When is double
rounding innocuous?", 1995).  Products code * s need 4 + 24 bits and are
exact in fp64.
"""
from __future__ import annotations

import numpy as np

LEVELS = 15.0           # codes 0 .. 15
CODE_LO, CODE_HI = 0, 15


def _widen(x: np.ndarray) -> np.ndarray:
    if x.dtype not in (np.float32, np.float16):
        raise TypeError(f"expected float32/float16 input, got {x.dtype}")
    xw = x.astype(np.float64)
    if not np.all(np.isfinite(xw)):
        raise ValueError("non-finite input is outside the quantizer's domain")
    return xw


def _check_group(d: int, g: int) -> None:
    if g <= 0 or g % 16 != 0 or d % g != 0:
        raise ValueError(f"group size {g} must be a positive multiple of 16 dividing d = {d}")


def group_params(x: np.ndarray, g: int) -> tuple[np.ndarray, np.ndarray]:
    """Steps s and offsets z, float32 [R, d / g], for x [R, d]."""
    xw = _widen(x)
    R, d = xw.shape
    _check_group(d, g)
    grp = xw.reshape(R, d // g, g)
    mx = grp.max(axis=2)
    mn = grp.min(axis=2)
    with np.errstate(over="ignore"):
        rng = (mx - mn).astype(np.float32)                   # RN32(max - min)
    if not np.all(np.isfinite(rng)):
        raise ValueError("a group's range max - min overflows binary32")
    s = (rng.astype(np.float64) / LEVELS).astype(np.float32)  # RN32(range / 15)
    z = mn.astype(np.float32)                                 # exact
    return s, z


def quantize_int4(x: np.ndarray, g: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """x [R, d] (fp32 or fp16) -> (codes uint8 [R, d / 2] two per byte,
    steps float32 [R, d / g], offsets float32 [R, d / g])."""
    xw = _widen(x)
    R, d = xw.shape
    s, z = group_params(x, g)
    grp = xw.reshape(R, d // g, g)
    diff = (grp - z.astype(np.float64)[:, :, None]).astype(np.float32)   # RN32(x - z)
    live = s != 0
    codes = np.zeros((R, d // g, g), dtype=np.int64)
    t = (diff[live].astype(np.float64) / s[live].astype(np.float64)[:, None]).astype(np.float32)
    codes[live] = np.clip(np.rint(t), CODE_LO, CODE_HI).astype(np.int64)
    return pack_nibbles(codes.reshape(R, d)), s, z


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """codes [R, d] in 0..15 -> bytes [R, d / 2]; element 2j in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """bytes [R, d / 2] -> codes [R, d] (uint8, 0..15)."""
    R, h = packed.shape
    out = np.empty((R, 2 * h), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def dequantize_int4(packed: np.ndarray, s: np.ndarray, z: np.ndarray, g: int,
                    out_dtype: str = "f32") -> np.ndarray:
    """x_hat = RN32(RN32(code * s) + z) [R, d]; fp16 output is RN16 of it."""
    codes = unpack_nibbles(packed).astype(np.float64)
    R, d = codes.shape
    _check_group(d, g)
    c = codes.reshape(R, d // g, g)
    prod = (c * s.astype(np.float64)[:, :, None]).astype(np.float32)           # exact, then RN32
    x32 = (prod.astype(np.float64) + z.astype(np.float64)[:, :, None]).astype(np.float32)
    x32 = x32.reshape(R, d)
    if out_dtype == "f32":
        return x32
    if out_dtype == "f16":
        with np.errstate(over="ignore"):                     # RN16 overflows to inf
            return x32.astype(np.float16)
    raise ValueError(f"out_dtype must be 'f32' or 'f16', got {out_dtype}")


def storage_bits_per_element(g: int) -> float:
    """4-bit codes plus a binary32 step and offset per group of g."""
    return 4.0 + 64.0 / g
