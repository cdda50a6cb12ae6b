"""Encoders that turn fp32 draws into the stored element formats.

These are used only to manufacture inputs: the key/value cache contents and the
queries that the paged decode reads.  Nothing here takes part in the attention
arithmetic.  Decoding (bytes back to numbers) lives separately in the oracle
and, on the GPU, in the kernels.

Formats
-------
* bf16: the upper 16 bits of an IEEE binary32, rounded to nearest-even.
* fp8 e4m3 ("fn" variant of the OCP 8-bit floating point specification):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
  S.1111.111 is NaN, largest finite magnitude 448, smallest subnormal 2^-9.
  The first page (TensorRT-LLM concept page, "key mechanisms" section) says FP8
  data is widened back to 16 bits before the matrix product accumulates; the
  encoder here produces those stored bytes.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); return uint16 bits.

    NaN inputs become the canonical quiet NaN 0x7FC0 with the input's sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    # No overflow for non-NaN inputs (largest is 0xFF800000); NaNs are replaced below.
    with np.errstate(over="ignore"):
        rounded = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    nan = np.isnan(x)
    if nan.any():
        sign = (u >> np.uint32(16)) & np.uint32(0x8000)
        rounded = np.where(nan, sign | np.uint32(0x7FC0), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (used by the generators only)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Encode float32 values as e4m3fn bytes, nearest-even, saturating to +-448.

    Works in float64, where every step below is exact: the exponent is found
    with frexp, scaling by a power of two is exact, and rint rounds half to even.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    nan = np.isnan(y)
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)
    # frexp: a = f * 2**ex with f in [0.5, 1); the leading binary digit is 2**(ex-1).
    _, ex = np.frexp(a)
    ex = ex.astype(np.int64) - 1
    normal = a >= 2.0 ** -6
    # Normal numbers: 1.mmm * 2**ex, ex in [-6, 8]; quantum 2**(ex-3).
    ex_n = np.clip(ex, -6, 8)
    q_n = np.rint(a / np.exp2(ex_n - 3)).astype(np.int64)  # in [8, 16]
    bump = q_n >= 16
    ex_n = ex_n + bump
    q_n = np.where(bump, q_n // 2, q_n)                    # mantissa carry
    code_n = ((ex_n + 7) << 3) | (q_n - 8)
    # Subnormals (and zero): m * 2**-9, m in [0, 8]; m == 8 is the smallest normal 0x08.
    q_s = np.rint(a / 2.0 ** -9).astype(np.int64)
    code_s = q_s
    code = np.where(normal, code_n, code_s)
    code = np.minimum(code, 0x7E)                          # saturate at 448
    out = code.astype(np.uint8) | sign
    out = np.where(nan, np.uint8(0x7F), out)
    return out.astype(np.uint8)


def e4m3_page_scales(x: np.ndarray) -> np.float32:
    """Per-(page, head) scale: amax / 448 in fp32 (1.0 when the block is all zero)."""
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def int8_encode(y: np.ndarray) -> np.ndarray:
    """Encode float32 values as symmetric int8 bytes (two's complement):
    nearest integer, half to even (numpy rint), clamped to [-127, 127]."""
    q = np.rint(np.asarray(y, dtype=np.float32))
    return np.clip(q, -127, 127).astype(np.int8).view(np.uint8)


INT8_MAX = np.float32(127.0)


def int4_encode(y: np.ndarray) -> np.ndarray:
    """Encode float32 values as symmetric int4 nibble codes (two's complement,
    0..15, one per byte): nearest integer, half to even, clamped to [-7, 7]."""
    q = np.clip(np.rint(np.asarray(y, dtype=np.float32)), -7, 7).astype(np.int8)
    return (q.view(np.uint8) & 0xF).astype(np.uint8)


INT4_MAX = np.float32(7.0)
