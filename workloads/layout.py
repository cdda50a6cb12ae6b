"""Place logical per-sequence K/V tokens into the physical page pool.

The first page (TensorRT-LLM concept page, "key mechanisms" section) describes
the cache as fixed-size pages drawn from a shared pool, with a per-sequence page
table mapping logical token positions to physical pages; it gives no byte
layout.  The layout used by this library is defined in ``include/pkv.h``; this
module is the input generator's own rendering of that definition, used to build
pools in host memory.  It does no attention arithmetic.

For one (page, kv head) chunk of ``P`` tokens by ``D`` elements, with
``E = 16 / element_bytes`` elements per 16-byte group:

* K element (j, d) sits at ``((d // E) * P + j) * E + d % E``.
* V tokens come in blocks of ``TB = 4 * E`` tokens.  Token j has
  ``blk = j // TB``, ``r = j % TB``, ``sub = r // 16``, ``c = (r % 16) // 4``,
  ``i = r % 4``, ``e = 4 * sub + i``; V element (j, d) sits at
  ``blk * TB * D + (c * D + d) * E + e``.

The chunk for (page pg, head g) starts at element ``(pg * Hkv + g) * P * D``.
"""
from __future__ import annotations

import numpy as np

ELEM_BITS = {"f32": 32, "bf16": 16, "fp8": 8, "i8": 8, "i4": 4}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "i8": 1}          # whole-byte formats
NP_DTYPE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "i8": np.uint8, "i4": np.uint8}
# Poison for slots that hold no token: a quiet NaN in each storage format;
# int8 and int4 have no NaN, so theirs is the most negative code (-128, -8),
# which the quantisers never write.  int4 elements are nibble codes (0..15,
# two's complement); a pool packs two per byte, the even element in the low
# nibble.
POISON = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F), "i8": np.uint8(0x80),
          "i4": np.uint8(0x8)}


def elems_per_16b(kv_dtype: str) -> int:
    return 128 // ELEM_BITS[kv_dtype]


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] nibble codes -> [..., n] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] nibble codes."""
    b = np.asarray(b, dtype=np.uint8)
    return np.stack([b & 0xF, b >> 4], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])


def v_block_tokens(kv_dtype: str) -> int:
    return 4 * elems_per_16b(kv_dtype)


def k_chunk_index(P: int, D: int, kv_dtype: str) -> np.ndarray:
    """[P, D] array: position of K element (j, d) inside its chunk."""
    E = elems_per_16b(kv_dtype)
    j = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    return ((d // E) * P + j) * E + d % E


def v_chunk_index(P: int, D: int, kv_dtype: str) -> np.ndarray:
    """[P, D] array: position of V element (j, d) inside its chunk."""
    E = elems_per_16b(kv_dtype)
    TB = 4 * E
    if P % TB:
        raise ValueError(f"page size {P} is not a multiple of the {TB}-token V block")
    j = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    blk, r = j // TB, j % TB
    sub, c, i = r // 16, (r % 16) // 4, r % 4
    e = 4 * sub + i
    return blk * TB * D + (c * D + d) * E + e


def empty_pool(num_pages: int, Hkv: int, P: int, D: int, kv_dtype: str) -> np.ndarray:
    """A pool filled with poison: [num_pages, Hkv, P*D] elements (int4: P*D/2
    bytes of packed nibbles)."""
    if kv_dtype == "i4":
        return np.full((num_pages, Hkv, P * D // 2), 0x88, dtype=np.uint8)
    return np.full((num_pages, Hkv, P * D), POISON[kv_dtype], dtype=NP_DTYPE[kv_dtype])


def pack_sequence(pool: np.ndarray, pages: np.ndarray, tokens: np.ndarray, P: int,
                  index: np.ndarray, kv_dtype: str) -> None:
    """Write logical tokens [L, Hkv, D] of one sequence into ``pool`` at ``pages``.

    Slots of the last page past L are set to poison.
    """
    L, Hkv, D = tokens.shape
    npg = len(pages)
    assert npg * P >= L, (npg, P, L)
    if npg == 0:
        return
    padded = np.full((npg * P, Hkv, D), POISON[kv_dtype], dtype=NP_DTYPE[kv_dtype])
    padded[:L] = tokens
    chunks = padded.reshape(npg, P, Hkv, D).transpose(0, 2, 1, 3).reshape(npg, Hkv, P * D)
    out = np.empty_like(chunks)
    out[..., index.reshape(-1)] = chunks
    if kv_dtype == "i4":
        out = pack_nibbles(out)
    pool[np.asarray(pages, dtype=np.int64)] = out
