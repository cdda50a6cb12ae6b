"""Seeded synthetic workloads for paged decode attention.

The pages name no dataset, trace or model weights; their serving loop (first
page, "runtime execution model") batches sequences of very different lengths,
hands the engine their page tables, and frees pages of finished requests for
reuse.  The five workloads below reproduce those shapes with random data.

Random streams
--------------
``seed`` drives one ``numpy.random.default_rng(seed)`` for lengths, page
placement and allocator churn, in that order.  Bulk tensors come from child
streams keyed by ``[seed, tag, index]`` so that any one sequence can be
regenerated on its own:

* q: ``[seed, 1]``            -> [B, Hq, D]
* K of sequence b: ``[seed, 2, b]``  -> [L_b, Hkv, D]
* V of sequence b: ``[seed, 3, b]``  -> [L_b, Hkv, D]
* new K/V of decode step s: ``[seed, 4, s]`` -> k_new then v_new, [B, Hkv, D] each

All draws are float32 standard normals, scaled where a workload says so, then
stored as fp32, bf16 (nearest-even), fp8 e4m3 or symmetric int8 with one fp32
scale per (page, kv head) equal to amax/448 (fp8) or amax/127 (int8) over the
valid tokens of that page.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import codec, layout

# ----------------------------------------------------------------------------
# Workload container
# ----------------------------------------------------------------------------


@dataclass
class Step:
    """One decode iteration of an in-flight batch: append one token, then decode."""
    seq_lens: np.ndarray          # int32 [B], counts the token appended this step
    k_new: np.ndarray             # [B, Hkv, D] stored format
    v_new: np.ndarray


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    num_pages: int
    max_pages: int
    kv_dtype: str                 # "f32" | "bf16" | "fp8" | "i8" | "i4"
    q_dtype: str                  # "f32" | "bf16"
    out_dtype: str                # "f32" | "bf16"
    scale: np.float32
    partition_tokens: int         # 0 = library's choice
    seq_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray      # int32 [B, max_pages], -1 where unused
    q: np.ndarray                 # [B, Hq, D] stored format
    k_pool: np.ndarray            # [num_pages, Hkv, P*D] stored format
    v_pool: np.ndarray
    k_scales: Optional[np.ndarray] = None   # float32 [num_pages, Hkv]
    v_scales: Optional[np.ndarray] = None
    steps: List[Step] = field(default_factory=list)
    # format of the steps' k_new / v_new rows: the cache format (copied into the
    # pages), or bf16 rows for an fp8 cache (quantised on write)
    new_dtype: Optional[str] = None

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def kv_bytes(self, seq_lens: Optional[np.ndarray] = None) -> int:
        """Bytes of K and V that a decode over ``seq_lens`` must read."""
        L = self.seq_lens if seq_lens is None else seq_lens
        bits = layout.ELEM_BITS[self.kv_dtype]
        return int(np.sum(L.astype(np.int64))) * self.Hkv * self.D * bits // 8 * 2


# ----------------------------------------------------------------------------
# Draw helpers
# ----------------------------------------------------------------------------


def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _child(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng([seed, *key])


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return codec.f32_to_bf16_bits(x)
    raise ValueError(dtype)


def draw_q(seed: int, B: int, Hq: int, D: int, dtype: str, mult: float = 1.0) -> np.ndarray:
    x = _child(seed, 1).standard_normal((B, Hq, D), dtype=np.float32)
    if mult != 1.0:
        x = x * np.float32(mult)
    return _store(x, dtype)


def draw_seq_f32(seed: int, tag: int, b: int, L: int, Hkv: int, D: int) -> np.ndarray:
    return _child(seed, tag, b).standard_normal((L, Hkv, D), dtype=np.float32)


def quantize_fp8_pages(x: np.ndarray, P: int):
    """x: [L, Hkv, D] fp32 -> (bytes [L, Hkv, D], scales [npages, Hkv]).

    Each (logical page, head) gets scale = fp32(amax/448) over its valid tokens
    (1.0 if that block is all zero); bytes = e4m3(fp32(x / scale)).
    """
    L, Hkv, D = x.shape
    npg = -(-L // P)
    padded = np.zeros((npg * P, Hkv, D), dtype=np.float32)
    padded[:L] = x
    amax = np.abs(padded).reshape(npg, P, Hkv, D).max(axis=(1, 3))
    scales = np.where(amax == 0, np.float32(1.0),
                      (amax / np.float32(codec.E4M3_MAX)).astype(np.float32)).astype(np.float32)
    per_tok = np.repeat(scales, P, axis=0)[:L]                 # [L, Hkv]
    y = (x / per_tok[:, :, None]).astype(np.float32)
    return codec.e4m3_encode(y), scales


def quantize_int8_pages(x: np.ndarray, P: int):
    """x: [L, Hkv, D] fp32 -> (int8 bytes [L, Hkv, D], scales [npages, Hkv]).

    Each (logical page, head) gets scale = fp32(amax/127) over its valid tokens
    (1.0 if that block is all zero); bytes = rint(fp32(x / scale)) clamped to +-127.
    """
    L, Hkv, D = x.shape
    npg = -(-L // P)
    padded = np.zeros((npg * P, Hkv, D), dtype=np.float32)
    padded[:L] = x
    amax = np.abs(padded).reshape(npg, P, Hkv, D).max(axis=(1, 3))
    scales = np.where(amax == 0, np.float32(1.0),
                      (amax / codec.INT8_MAX).astype(np.float32)).astype(np.float32)
    per_tok = np.repeat(scales, P, axis=0)[:L]
    y = (x / per_tok[:, :, None]).astype(np.float32)
    return codec.int8_encode(y), scales


def quantize_int4_pages(x: np.ndarray, P: int):
    """x: [L, Hkv, D] fp32 -> (int4 nibble codes [L, Hkv, D], scales [npages, Hkv]).

    Each (logical page, head) gets scale = fp32(amax/7) over its valid tokens
    (1.0 if that block is all zero); codes = rint(fp32(x / scale)) clamped to +-7.
    """
    L, Hkv, D = x.shape
    npg = -(-L // P)
    padded = np.zeros((npg * P, Hkv, D), dtype=np.float32)
    padded[:L] = x
    amax = np.abs(padded).reshape(npg, P, Hkv, D).max(axis=(1, 3))
    scales = np.where(amax == 0, np.float32(1.0),
                      (amax / codec.INT4_MAX).astype(np.float32)).astype(np.float32)
    per_tok = np.repeat(scales, P, axis=0)[:L]
    y = (x / per_tok[:, :, None]).astype(np.float32)
    return codec.int4_encode(y), scales


QUANTIZERS = {"fp8": quantize_fp8_pages, "i8": quantize_int8_pages, "i4": quantize_int4_pages}
SCALED = tuple(QUANTIZERS)


def seq_tokens(seed: int, b: int, L: int, Hkv: int, D: int, kv_dtype: str, P: int):
    """Logical K, V (stored format) and, for fp8, logical-page scales of sequence b."""
    kf = draw_seq_f32(seed, 2, b, L, Hkv, D)
    vf = draw_seq_f32(seed, 3, b, L, Hkv, D)
    if kv_dtype in SCALED:
        quant = QUANTIZERS[kv_dtype]
        k, ks = quant(kf, P)
        v, vs = quant(vf, P)
        return k, v, ks, vs
    return _store(kf, kv_dtype), _store(vf, kv_dtype), None, None


# ----------------------------------------------------------------------------
# Page placement
# ----------------------------------------------------------------------------


def pages_needed(L: np.ndarray, P: int) -> np.ndarray:
    return (L.astype(np.int64) + P - 1) // P


def place_permuted(rng: np.random.Generator, L: np.ndarray, P: int, num_pages: int,
                   max_pages: int) -> np.ndarray:
    """Sequence b takes the next ceil(L_b/P) entries of one random permutation."""
    perm = rng.permutation(num_pages).astype(np.int32)
    need = pages_needed(L, P)
    bt = np.full((len(L), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


class PageAllocator:
    """Free-page stack over a shared pool; freed pages are pushed back for reuse."""

    def __init__(self, order: np.ndarray):
        self.free = [int(p) for p in order[::-1]]   # pop() yields order[0] first
        self.num_pages = len(order)

    def pop(self) -> int:
        if not self.free:
            raise RuntimeError("page pool exhausted")
        return self.free.pop()

    def push(self, pages) -> None:
        self.free.extend(int(p) for p in pages)

    @property
    def used(self) -> int:
        return self.num_pages - len(self.free)


def round_robin_alloc(alloc: PageAllocator, need: List[int], stop_used: Optional[int] = None):
    """Give one page per round to every sequence that still needs pages.

    Stops early once ``alloc.used`` reaches ``stop_used``.  Returns page lists.
    """
    tables = [[] for _ in need]
    progress = True
    while progress:
        progress = False
        for i, n in enumerate(need):
            if len(tables[i]) < n:
                if stop_used is not None and alloc.used >= stop_used:
                    return tables
                tables[i].append(alloc.pop())
                progress = True
    return tables


def lognormal_lengths(rng: np.random.Generator, n: int, median: float, sigma: float,
                      lo: int, hi: int) -> np.ndarray:
    x = np.exp(rng.normal(math.log(median), sigma, size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


# ----------------------------------------------------------------------------
# Assembly
# ----------------------------------------------------------------------------


def _assemble(name, seed, B, Hq, Hkv, D, P, num_pages, kv_dtype, q_dtype, out_dtype,
              scale, partition_tokens, L, bt, q_mult=1.0, pool_lens=None, quant_lens=None):
    """Draw q/K/V and pack the pools.  ``pool_lens`` (default L) is how many tokens
    of each sequence are resident in the pool.  A scaled cache is quantised per
    page over the first ``quant_lens`` (default pool_lens) tokens: with
    quant_lens = L, the page scales come from every token a page will hold, so
    tokens past pool_lens, packed later, fit the same scales."""
    max_pages = bt.shape[1]
    pool_lens = L if pool_lens is None else pool_lens
    quant_lens = pool_lens if quant_lens is None else quant_lens
    q = draw_q(seed, B, Hq, D, q_dtype, q_mult)
    kpool = layout.empty_pool(num_pages, Hkv, P, D, kv_dtype)
    vpool = layout.empty_pool(num_pages, Hkv, P, D, kv_dtype)
    kidx = layout.k_chunk_index(P, D, kv_dtype)
    vidx = layout.v_chunk_index(P, D, kv_dtype)
    ks = vs = None
    if kv_dtype in SCALED:
        ks = np.full((num_pages, Hkv), np.nan, dtype=np.float32)
        vs = np.full((num_pages, Hkv), np.nan, dtype=np.float32)
    def fill(b):
        n = int(pool_lens[b])
        pages = bt[b, :int(pages_needed(np.array([n]), P)[0])]
        nq = int(quant_lens[b]) if kv_dtype in SCALED else n
        k, v, kls, vls = seq_tokens(seed, b, nq, Hkv, D, kv_dtype, P)
        layout.pack_sequence(kpool, pages, k[:n], P, kidx, kv_dtype)
        layout.pack_sequence(vpool, pages, v[:n], P, vidx, kv_dtype)
        if kv_dtype in SCALED and nq:
            all_pages = bt[b, :int(pages_needed(np.array([nq]), P)[0])]
            ks[all_pages] = kls
            vs[all_pages] = vls

    # Sequences own disjoint pages, so they can be drawn and placed concurrently;
    # each draws from its own child stream, so the result does not depend on order.
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(fill, range(B)))
    return Workload(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P,
                    num_pages=num_pages, max_pages=max_pages, kv_dtype=kv_dtype,
                    q_dtype=q_dtype, out_dtype=out_dtype, scale=np.float32(scale),
                    partition_tokens=partition_tokens, seq_lens=L.astype(np.int32),
                    block_tables=bt, q=q, k_pool=kpool, v_pool=vpool,
                    k_scales=ks, v_scales=vs)


def tiny_fp32(seed: int = 1) -> Workload:
    """4 sequences of {1,17,64,130} tokens, 8 q heads = 8 kv heads, D 64, pages of 16,
    a 64-page pool assigned through one seeded permutation; all fp32."""
    rng = np.random.default_rng(seed)
    L = np.array([1, 17, 64, 130], dtype=np.int32)
    P, NP = 16, 64
    bt = place_permuted(rng, L, P, NP, max_pages=int(pages_needed(L, P).max()))
    return _assemble("tiny_fp32", seed, 4, 8, 8, 64, P, NP, "f32", "f32", "f32",
                     np.float32(1.0 / math.sqrt(64)), 0, L, bt)


def llama3_8b_bf16(seed: int = 2, B: int = 64) -> Workload:
    """Llama-3-8B-shaped layer: B 64, 32 q heads / 8 kv heads, D 128, pages of 64,
    lengths uniform in [128, 4096], pages shuffled across a pool of 1.25x need."""
    rng = np.random.default_rng(seed)
    L = rng.integers(128, 4096, size=B, endpoint=True).astype(np.int32)
    P = 64
    need = int(pages_needed(L, P).sum())
    NP = int(math.ceil(1.25 * need))
    bt = place_permuted(rng, L, P, NP, max_pages=4096 // P)
    return _assemble("llama3_8b_bf16", seed, B, 32, 8, 128, P, NP, "bf16", "bf16", "bf16",
                     np.float32(1.0 / math.sqrt(128)), 0, L, bt)


def inflight_bf16(seed: int = 3, B: int = 256, n_steps: int = 16,
                  max_len: int = 32768) -> Workload:
    """In-flight batch: lognormal lengths (median 1024, sigma 1, clipped to
    [1, max_len]), 32/8 heads, D 128, pages of 128, a pool fragmented by seeded
    alloc/free churn, and ``n_steps`` decode iterations that each append one token
    per sequence (taking a fresh page when the last one is full) before decoding.

    Churn: pool = 2 * sum(ceil((L+n_steps)/P)) pages in random order on a free
    stack; 2B dummy sequences take pages round-robin until 60% of the pool is in
    use; a random half of them is freed; the B real sequences take their pages
    round-robin; the remaining dummies are freed.
    """
    return _inflight("inflight_bf16", seed, B, n_steps, max_len, "bf16")


def inflight_fp8(seed: int = 3, B: int = 256, n_steps: int = 16, max_len: int = 32768) -> Workload:
    """The in-flight batch above (same seed, lengths, churn and draws) with an fp8
    e4m3 cache: resident pages quantised with per-(page, kv head) scale amax/448,
    and each step's new K/V rows given in bf16, to be quantised on write with
    dynamic page scales (the cache format the fp8 append produces)."""
    return _inflight("inflight_fp8", seed, B, n_steps, max_len, "fp8")


def _inflight(name, seed, B, n_steps, max_len, kv_dtype) -> Workload:
    rng = np.random.default_rng(seed)
    P = 128
    L0 = lognormal_lengths(rng, B, 1024.0, 1.0, 1, max_len)
    NP = int(2 * pages_needed(L0 + n_steps, P).sum())
    alloc = PageAllocator(rng.permutation(NP))
    dummy_len = lognormal_lengths(rng, 2 * B, 1024.0, 1.0, 1, max_len)
    dummy = round_robin_alloc(alloc, [int(x) for x in pages_needed(dummy_len, P)],
                              stop_used=int(0.6 * NP))
    freed = rng.permutation(len(dummy))[: len(dummy) // 2]
    for i in freed:
        alloc.push(dummy[i])
        dummy[i] = []
    real = round_robin_alloc(alloc, [int(x) for x in pages_needed(L0, P)])
    for i in range(len(dummy)):
        alloc.push(dummy[i])
    max_pages = int(pages_needed(np.array([max_len + n_steps]), P)[0])
    # Decode steps: step s appends the token at position L0 + s.
    tables = [list(t) for t in real]
    step_lens = []
    for s in range(n_steps):
        for b in range(B):
            if (int(L0[b]) + s) % P == 0:
                tables[b].append(alloc.pop())
        step_lens.append((L0 + s + 1).astype(np.int32))
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    for b, t in enumerate(tables):
        bt[b, :len(t)] = t
    wl = _assemble(name, seed, B, 32, 8, 128, P, NP, kv_dtype, "bf16", "bf16",
                   np.float32(1.0 / math.sqrt(128)), 0, step_lens[-1], bt, pool_lens=L0)
    wl.new_dtype = "bf16"
    for s in range(n_steps):
        r = _child(seed, 4, s)
        kn = r.standard_normal((B, 8, 128), dtype=np.float32)
        vn = r.standard_normal((B, 8, 128), dtype=np.float32)
        wl.steps.append(Step(seq_lens=step_lens[s], k_new=_store(kn, "bf16"),
                             v_new=_store(vn, "bf16")))
    wl.seq_lens = L0.astype(np.int32)   # resident tokens before step 0
    return wl


def long_splitkv_bf16(seed: int = 4, B: int = 8, L: int = 131072) -> Workload:
    """Long context: B sequences of L tokens, 64 q heads / 8 kv heads (group 8),
    D 128, pages of 128, 512-token partitions merged by log-sum-exp; q drawn as
    3*N(0,1) so that logits q.k/sqrt(128) have standard deviation about 3."""
    rng = np.random.default_rng(seed)
    P = 128
    Ls = np.full(B, L, dtype=np.int32)
    NP = int(pages_needed(Ls, P).sum())
    bt = place_permuted(rng, Ls, P, NP, max_pages=int(pages_needed(Ls, P).max()))
    return _assemble("long_splitkv_bf16", seed, B, 64, 8, 128, P, NP, "bf16", "bf16", "bf16",
                     np.float32(1.0 / math.sqrt(128)), 512, Ls, bt, q_mult=3.0)


def inflight_int8(seed: int = 3, B: int = 256, n_steps: int = 16, max_len: int = 32768) -> Workload:
    """The in-flight batch with a symmetric int8 cache (per-(page, kv head) scale
    amax/127) and bf16 new rows, quantised on write with dynamic page scales."""
    return _inflight("inflight_int8", seed, B, n_steps, max_len, "i8")


def int4_kv(seed: int = 5, B: int = 128) -> Workload:
    """The fp8 workload's lengths and draws (B 128, lengths uniform in [1024,
    8192], 32/8 heads, D 128) with a symmetric int4 cache (scale amax/7 per
    (page, kv head), two codes per byte) on pages of 128 tokens (int4 tiles are
    128 tokens); q bf16, out bf16."""
    wl = fp8_kv(seed, B, kv_dtype="i4", P=128)
    wl.name = "int4_kv"
    return wl


def inflight_int4(seed: int = 3, B: int = 256, n_steps: int = 16, max_len: int = 32768) -> Workload:
    """The in-flight batch with a symmetric int4 cache and bf16 new rows,
    quantised on write with dynamic page scales (amax / 7)."""
    return _inflight("inflight_int4", seed, B, n_steps, max_len, "i4")


def int8_kv(seed: int = 5, B: int = 128) -> Workload:
    """The fp8 workload's shape and draws (B 128, lengths uniform in [1024, 8192],
    32/8 heads, D 128, pages of 64) with a symmetric int8 cache, scale amax/127
    per (page, kv head); q bf16, out bf16."""
    wl = fp8_kv(seed, B, kv_dtype="i8")
    wl.name = "int8_kv"
    return wl


def fp8_kv(seed: int = 5, B: int = 128, kv_dtype: str = "fp8", P: int = 64) -> Workload:
    """fp8 e4m3 cache: B 128, lengths uniform in [1024, 8192], 32/8 heads, D 128,
    pages of 64, per-(page, kv head) scale amax/448; q bf16, out bf16."""
    rng = np.random.default_rng(seed)
    L = rng.integers(1024, 8192, size=B, endpoint=True).astype(np.int32)
    need = int(pages_needed(L, P).sum())
    NP = int(math.ceil(1.25 * need))
    bt = place_permuted(rng, L, P, NP, max_pages=8192 // P)
    return _assemble("fp8_kv", seed, B, 32, 8, 128, P, NP, kv_dtype, "bf16", "bf16",
                     np.float32(1.0 / math.sqrt(128)), 0, L, bt)


def custom(seed: int, lens, Hq: int, Hkv: int, D: int, P: int, kv_dtype: str,
           out_dtype: Optional[str] = None, num_pages: Optional[int] = None,
           q_mult: float = 1.0, partition_tokens: int = 0, scale: Optional[float] = None,
           extra_table_cols: int = 0) -> Workload:
    """Small edge-case workloads for tests: given lengths, random page placement."""
    rng = np.random.default_rng(seed)
    L = np.asarray(lens, dtype=np.int32)
    need = int(pages_needed(L, P).sum())
    NP = num_pages if num_pages is not None else max(1, int(math.ceil(1.25 * need)) + 1)
    mp = max(1, int(pages_needed(L, P).max()) if len(L) else 1) + extra_table_cols
    bt = place_permuted(rng, L, P, NP, max_pages=mp)
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    out_dtype = out_dtype or q_dtype
    sc = np.float32(1.0 / math.sqrt(D)) if scale is None else np.float32(scale)
    return _assemble(f"custom_{kv_dtype}", seed, len(L), Hq, Hkv, D, P, NP, kv_dtype,
                     q_dtype, out_dtype, sc, partition_tokens, L, bt, q_mult=q_mult)


CONFIGS = {
    "tiny_fp32": tiny_fp32,
    "llama3_8b_bf16": llama3_8b_bf16,
    "inflight_bf16": inflight_bf16,
    "long_splitkv_bf16": long_splitkv_bf16,
    "fp8_kv": fp8_kv,
    "inflight_fp8": inflight_fp8,
    "int8_kv": int8_kv,
    "inflight_int8": inflight_int8,
    "int4_kv": int4_kv,
    "inflight_int4": inflight_int4,
}


# ----------------------------------------------------------------------------
# Chunked prefill
# ----------------------------------------------------------------------------
#
# A batch of sequences that each bring a chunk of C_b new tokens on top of
# L_b - C_b cached ones: the pools hold the cached tokens, k_new / v_new the
# chunk's rows (tokens L_b - C_b .. L_b - 1 of the same per-sequence draws, so
# appending them gives the pool of all L_b tokens), q one row per chunk token
# from child stream [seed, 5].  Rows of all chunks are packed back to back;
# cu_q[b] .. cu_q[b+1] are sequence b's.


@dataclass
class PrefillWorkload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    num_pages: int
    max_pages: int
    kv_dtype: str                 # "f32" | "bf16" | "fp8"
    q_dtype: str
    out_dtype: str
    scale: np.float32
    seq_lens: np.ndarray          # int32 [B], cached tokens + chunk
    chunk_lens: np.ndarray        # int32 [B]
    cu_q: np.ndarray              # int32 [B + 1]
    block_tables: np.ndarray      # int32 [B, max_pages]
    q: np.ndarray                 # [T, Hq, D] stored format
    k_pool: np.ndarray            # cached tokens only
    v_pool: np.ndarray
    k_new: np.ndarray             # [T, Hkv, D] stored format, the chunks' rows
    v_new: np.ndarray
    k_scales: Optional[np.ndarray] = None   # fp8: [NP, Hkv] page scales (of the full pages)
    v_scales: Optional[np.ndarray] = None

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def T(self) -> int:
        return int(self.cu_q[-1])

    def attended(self) -> int:
        """(query token, key token) pairs the causal chunks attend to, per head."""
        L = self.seq_lens.astype(np.int64)
        C = self.chunk_lens.astype(np.int64)
        first = np.maximum(L - C + 1, 0)           # keys seen by the chunk's first row
        return int(np.sum(C * first + C * (C - 1) // 2))

    def flops(self) -> int:
        """2 flops per multiply-add of q.k and of p.v, per attended pair and head."""
        return 4 * self.attended() * self.Hq * self.D

    def kv_bytes(self) -> int:
        """K and V bytes of all L_b tokens (each read at least once)."""
        bits = layout.ELEM_BITS[self.kv_dtype]
        return int(np.sum(self.seq_lens.astype(np.int64))) * self.Hkv * self.D * bits // 8 * 2


def prefill_case(name: str, seed: int, ctx_lens, chunk_lens, Hq: int, Hkv: int, D: int, P: int,
                 kv_dtype: str = "bf16", out_dtype: Optional[str] = None, slack: float = 1.25,
                 q_mult: float = 1.0, extra_table_cols: int = 0) -> PrefillWorkload:
    """Sequences with ``ctx_lens`` cached tokens and chunks of ``chunk_lens``.

    fp8 cache: every sequence's L tokens are quantised per page (amax / 448 of
    the tokens each page holds once the chunk is in), the pool holds the first
    L - C tokens' bytes, the scales are those of the full pages, and k_new /
    v_new are the chunk tokens' bytes (the chunk append copies them)."""
    if kv_dtype not in ("f32", "bf16", "fp8"):
        raise ValueError("chunked prefill workloads are fp32, bf16 or fp8")
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    C = np.asarray(chunk_lens, dtype=np.int32)
    L = (ctx + C).astype(np.int32)
    B = len(L)
    need = int(pages_needed(L, P).sum())
    NP = max(1, int(math.ceil(slack * need)))
    mp = max(1, int(pages_needed(L, P).max()) if B else 1) + extra_table_cols
    bt = place_permuted(rng, L, P, NP, max_pages=mp)
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    sc = np.float32(1.0 / math.sqrt(D))
    base = _assemble(name, seed, B, Hq, Hkv, D, P, NP, kv_dtype, q_dtype, out_dtype or q_dtype,
                     sc, 0, L, bt, pool_lens=ctx, quant_lens=L)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(C)
    T = int(cu[-1])
    qf = _child(seed, 5).standard_normal((T, Hq, D), dtype=np.float32)
    if q_mult != 1.0:
        qf = qf * np.float32(q_mult)
    if kv_dtype in SCALED:
        kn = np.zeros((T, Hkv, D), dtype=np.uint8)
        vn = np.zeros((T, Hkv, D), dtype=np.uint8)
        for b in range(B):
            k, v, _, _ = seq_tokens(seed, b, int(L[b]), Hkv, D, kv_dtype, P)
            kn[cu[b]:cu[b + 1]] = k[ctx[b]:]
            vn[cu[b]:cu[b + 1]] = v[ctx[b]:]
    else:
        kn = np.zeros((T, Hkv, D), dtype=np.float32)
        vn = np.zeros((T, Hkv, D), dtype=np.float32)
        for b in range(B):
            n = int(L[b])
            kn[cu[b]:cu[b + 1]] = draw_seq_f32(seed, 2, b, n, Hkv, D)[ctx[b]:]
            vn[cu[b]:cu[b + 1]] = draw_seq_f32(seed, 3, b, n, Hkv, D)[ctx[b]:]
        kn, vn = _store(kn, kv_dtype), _store(vn, kv_dtype)
    return PrefillWorkload(name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P, num_pages=NP,
                           max_pages=bt.shape[1], kv_dtype=kv_dtype, q_dtype=q_dtype,
                           out_dtype=base.out_dtype, scale=sc, seq_lens=L, chunk_lens=C, cu_q=cu,
                           block_tables=bt, q=_store(qf, q_dtype), k_pool=base.k_pool,
                           v_pool=base.v_pool, k_new=kn, v_new=vn,
                           k_scales=base.k_scales, v_scales=base.v_scales)


def chunked_prefill_bf16(seed: int = 6, B: int = 16, chunk: int = 512) -> PrefillWorkload:
    """Llama-3-8B-shaped chunked prefill: 16 sequences, each a 512-token chunk on
    top of U{0..7680} cached tokens, 32/8 heads, D 128, pages of 64, bf16."""
    rng = np.random.default_rng([seed, 0])
    ctx = rng.integers(0, 7680, size=B, endpoint=True).astype(np.int32)
    return prefill_case("chunked_prefill_bf16", seed, ctx, np.full(B, chunk, np.int32), 32, 8, 128, 64)


def chunked_prefill_fp8(seed: int = 6, B: int = 16, chunk: int = 512) -> PrefillWorkload:
    """The chunked-prefill workload above (same draws and lengths) over an fp8
    e4m3 cache with per-(page, kv head) scales amax / 448."""
    rng = np.random.default_rng([seed, 0])
    ctx = rng.integers(0, 7680, size=B, endpoint=True).astype(np.int32)
    return prefill_case("chunked_prefill_fp8", seed, ctx, np.full(B, chunk, np.int32), 32, 8, 128, 64,
                        kv_dtype="fp8", out_dtype="bf16")


PREFILL_CONFIGS = {
    "chunked_prefill_bf16": chunked_prefill_bf16,
    "chunked_prefill_fp8": chunked_prefill_fp8,
}
