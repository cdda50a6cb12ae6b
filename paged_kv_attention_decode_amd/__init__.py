"""Paged KV-cache decode attention for MI355X (gfx950): Python binding of libpkv.so.

Argument marshalling only.  Every step runs in the HIP kernels of
``csrc/``; tensors are torch tensors used as device memory, and work is
queued on torch's current HIP stream.  The functions mirror the C ABI in
``include/pkv.h`` (same names without the ``pkv_`` prefix).
"""
from __future__ import annotations

import ctypes

from ._native import NativeLibraryMissing, lib  # noqa: F401

F32, BF16, FP8_E4M3, INT8, INT4 = 0, 1, 2, 3, 4
_DTYPE_CODE = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "i8": INT8, "i4": INT4}


class PkvError(RuntimeError):
    def __init__(self, fn: str, code: int):
        L = lib()
        msg = L.pkv_last_error().decode() or L.pkv_strerror(code).decode()
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def _code(dtype) -> int:
    return _DTYPE_CODE[dtype] if isinstance(dtype, str) else int(dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise PkvError(fn, rc)


def kv_append(k_new, v_new, kv_dtype, block_tables, seq_lens, k_pool, v_pool,
              num_kv_heads, head_dim, page_size, stream=None):
    """Write each sequence's new token (position seq_lens[b]-1) into its page."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("kv_append", lib().pkv_kv_append(
        _ptr(k_new), _ptr(v_new), _code(kv_dtype), _ptr(block_tables), MP, _ptr(seq_lens), B,
        _ptr(k_pool), _ptr(v_pool), NP, num_kv_heads, head_dim, page_size, _stream(stream)))


def kv_append_fp8(k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool, k_scales, v_scales,
                  num_kv_heads, head_dim, page_size, stream=None):
    """Quantise each sequence's new bf16/f32 K/V row into its fp8 page, keeping the
    per-(page, kv head) scales at amax / 448 (earlier tokens re-encoded when a
    scale grows)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("kv_append_fp8", lib().pkv_kv_append_fp8(
        _ptr(k_new), _ptr(v_new), _code(new_dtype), _ptr(block_tables), MP, _ptr(seq_lens), B,
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), NP, num_kv_heads, head_dim, page_size,
        _stream(stream)))


def kv_append_int4(k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool, k_scales, v_scales,
                   num_kv_heads, head_dim, page_size, stream=None):
    """As kv_append_fp8 for a symmetric int4 cache (page scales amax / 7, two codes
    per byte)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("kv_append_int4", lib().pkv_kv_append_int4(
        _ptr(k_new), _ptr(v_new), _code(new_dtype), _ptr(block_tables), MP, _ptr(seq_lens), B,
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), NP, num_kv_heads, head_dim, page_size,
        _stream(stream)))


def kv_append_int8(k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool, k_scales, v_scales,
                   num_kv_heads, head_dim, page_size, stream=None):
    """As kv_append_fp8 for a symmetric int8 cache (page scales amax / 127)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("kv_append_int8", lib().pkv_kv_append_int8(
        _ptr(k_new), _ptr(v_new), _code(new_dtype), _ptr(block_tables), MP, _ptr(seq_lens), B,
        _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), NP, num_kv_heads, head_dim, page_size,
        _stream(stream)))


def decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim) -> int:
    return int(lib().pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim))


def paged_attn_decode(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, seq_lens,
                      num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype,
                      workspace, partition_tokens=0, stream=None):
    """softmax(scale * q K^T) V over each sequence's pages (f32 or bf16 cache)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("paged_attn_decode", lib().pkv_paged_attn_decode(
        _ptr(q), _code(q_dtype), _ptr(k_pool), _ptr(v_pool), _code(kv_dtype), _ptr(block_tables),
        MP, _ptr(seq_lens), B, NP, num_q_heads, num_kv_heads, head_dim, page_size, float(scale),
        int(partition_tokens), _ptr(out), _code(out_dtype), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def paged_attn_decode_fp8(q, q_dtype, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens,
                          num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype,
                          workspace, partition_tokens=0, stream=None):
    """As paged_attn_decode for an fp8 e4m3 cache with per-(page, kv head) scales."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("paged_attn_decode_fp8", lib().pkv_paged_attn_decode_fp8(
        _ptr(q), _code(q_dtype), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), MP, _ptr(seq_lens), B, NP, num_q_heads, num_kv_heads, head_dim,
        page_size, float(scale), int(partition_tokens), _ptr(out), _code(out_dtype), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def paged_attn_decode_int4(q, q_dtype, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens,
                           num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype,
                           workspace, partition_tokens=0, stream=None):
    """As paged_attn_decode for a symmetric int4 cache with per-(page, kv head) scales."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("paged_attn_decode_int4", lib().pkv_paged_attn_decode_int4(
        _ptr(q), _code(q_dtype), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), MP, _ptr(seq_lens), B, NP, num_q_heads, num_kv_heads, head_dim,
        page_size, float(scale), int(partition_tokens), _ptr(out), _code(out_dtype), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def paged_attn_decode_int8(q, q_dtype, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens,
                           num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype,
                           workspace, partition_tokens=0, stream=None):
    """As paged_attn_decode for a symmetric int8 cache with per-(page, kv head) scales."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("paged_attn_decode_int8", lib().pkv_paged_attn_decode_int8(
        _ptr(q), _code(q_dtype), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales), _ptr(v_scales),
        _ptr(block_tables), MP, _ptr(seq_lens), B, NP, num_q_heads, num_kv_heads, head_dim,
        page_size, float(scale), int(partition_tokens), _ptr(out), _code(out_dtype), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_step(q, q_dtype, k_new, v_new, k_pool, v_pool, kv_dtype, block_tables, seq_lens,
                num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype, workspace,
                k_scales=None, v_scales=None, partition_tokens=0, stream=None):
    """kv_append + decode in one launch (k_new/v_new become token seq_lens[b]-1)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("decode_step", lib().pkv_decode_step(
        _ptr(q), _code(q_dtype), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _code(kv_dtype),
        _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), MP, _ptr(seq_lens), B, NP, num_q_heads,
        num_kv_heads, head_dim, page_size, float(scale), int(partition_tokens), _ptr(out),
        _code(out_dtype), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def decode_step_quant(q, q_dtype, k_new, v_new, new_dtype, k_pool, v_pool, kv_dtype, k_scales, v_scales,
                      block_tables, seq_lens, num_q_heads, num_kv_heads, head_dim, page_size, scale, out,
                      out_dtype, workspace, partition_tokens=0, stream=None):
    """Quantising append of bf16 / fp32 rows into an fp8 / int8 / int4 cache
    (dynamic page scales) fused into the decode of that cache."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("decode_step_quant", lib().pkv_decode_step_quant(
        _ptr(q), _code(q_dtype), _ptr(k_new), _ptr(v_new), _code(new_dtype), _ptr(k_pool), _ptr(v_pool),
        _code(kv_dtype), _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), MP, _ptr(seq_lens), B, NP,
        num_q_heads, num_kv_heads, head_dim, page_size, float(scale), int(partition_tokens), _ptr(out),
        _code(out_dtype), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_step_noalloc(q, q_dtype, k_new, v_new, k_pool, v_pool, kv_dtype, block_tables, seq_lens,
                        num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype,
                        k_scales=None, v_scales=None, partition_tokens=0, stream=None):
    """decode_step with the library's static per-device scratch as its workspace
    (no allocation; calls that overlap on one device race)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("decode_step_noalloc", lib().pkv_decode_step_noalloc(
        _ptr(q), _code(q_dtype), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _code(kv_dtype),
        _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), MP, _ptr(seq_lens), B, NP, num_q_heads,
        num_kv_heads, head_dim, page_size, float(scale), int(partition_tokens), _ptr(out),
        _code(out_dtype), _stream(stream)))


def kv_append_chunk(k_new, v_new, kv_dtype, cu_new, block_tables, seq_lens, k_pool, v_pool,
                    num_kv_heads, head_dim, page_size, stream=None):
    """Write each sequence's chunk of new tokens (rows cu_new[b] .. cu_new[b+1] of
    k_new / v_new) into positions seq_lens[b] - C_b .. seq_lens[b] - 1."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("kv_append_chunk", lib().pkv_kv_append_chunk(
        _ptr(k_new), _ptr(v_new), _code(kv_dtype), _ptr(cu_new), int(k_new.shape[0]), _ptr(block_tables), MP,
        _ptr(seq_lens), B, _ptr(k_pool), _ptr(v_pool), NP, num_kv_heads, head_dim, page_size, _stream(stream)))


def paged_prefill(q, q_dtype, cu_q, k_pool, v_pool, kv_dtype, block_tables, seq_lens,
                  num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype, stream=None):
    """Causal attention of each sequence's chunk of query rows (rows cu_q[b] ..
    cu_q[b+1] of q) over its pages (bf16 cache)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("paged_prefill", lib().pkv_paged_prefill(
        _ptr(q), _code(q_dtype), _ptr(cu_q), int(q.shape[0]), _ptr(k_pool), _ptr(v_pool), _code(kv_dtype),
        _ptr(block_tables), MP, _ptr(seq_lens), B, NP, num_q_heads, num_kv_heads, head_dim, page_size,
        float(scale), _ptr(out), _code(out_dtype), _stream(stream)))


def paged_prefill_fp8(q, q_dtype, cu_q, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens,
                      num_q_heads, num_kv_heads, head_dim, page_size, scale, out, out_dtype, stream=None):
    """paged_prefill over an fp8-e4m3 cache with per-(page, kv head) scales."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("paged_prefill_fp8", lib().pkv_paged_prefill_fp8(
        _ptr(q), _code(q_dtype), _ptr(cu_q), int(q.shape[0]), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales),
        _ptr(v_scales), _ptr(block_tables), MP, _ptr(seq_lens), B, NP, num_q_heads, num_kv_heads, head_dim,
        page_size, float(scale), _ptr(out), _code(out_dtype), _stream(stream)))


def alloc_pages(seq_lens, block_tables, page_size, free_pages, free_count, stream=None):
    """Give each sequence the page its newest token opens, from the device free-page
    stack free_pages[0 .. free_count[0] - 1] (updated in place)."""
    B, MP = block_tables.shape
    _check("alloc_pages", lib().pkv_alloc_pages(
        _ptr(seq_lens), B, _ptr(block_tables), MP, page_size, _ptr(free_pages), _ptr(free_count),
        int(free_pages.numel()), _stream(stream)))


def release_pages(release, seq_lens, block_tables, page_size, num_pages, free_pages, free_count, stream=None):
    """Push the pages of sequences marked in ``release`` back onto the stack."""
    B, MP = block_tables.shape
    _check("release_pages", lib().pkv_release_pages(
        _ptr(release), _ptr(seq_lens), B, _ptr(block_tables), MP, page_size, num_pages, _ptr(free_pages),
        _ptr(free_count), int(free_pages.numel()), _stream(stream)))


def debug_gather(k_pool, v_pool, kv_dtype, block_tables, seq_lens, num_kv_heads, head_dim,
                 page_size, k_out, v_out, stream=None):
    """Copy cached tokens to contiguous [B, Hkv, MP*P, D] rows (tests of the address path)."""
    B, MP = block_tables.shape
    NP = k_pool.shape[0]
    _check("debug_gather", lib().pkv_debug_gather(
        _ptr(k_pool), _ptr(v_pool), _code(kv_dtype), _ptr(block_tables), MP, _ptr(seq_lens), B, NP,
        num_kv_heads, head_dim, page_size, _ptr(k_out), _ptr(v_out), _stream(stream)))


def debug_read_probe(buf, out, stream=None):
    """Read every byte of ``buf`` once with 16-byte nontemporal loads (measures
    the streaming-read rate; ``out`` is a one-element int32 device tensor)."""
    _check("debug_read_probe", lib().pkv_debug_read_probe(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(out), _stream(stream)))


def version() -> int:
    return int(lib().pkv_version())
