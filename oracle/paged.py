"""numpy fp64 oracle for paged decode attention (vectorised twin of pkv_oracle.c),
the quantising appends, and causal chunked prefill over the same pages.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline, never by the product path.  It shares no code with
the HIP library, nor with the C oracle beside it: format decoders, layout
offsets and arithmetic are written out again here.

Definition followed (first page, TensorRT-LLM concept page: "key mechanisms"
for pages and the page table, "compile-time graph optimization" for the
page-table lookup on cache reads and writes, "runtime execution model" for
decode reading and updating the pages): with g = h // (Hq // Hkv) and
L = seq_lens[b], token t of sequence b lives in slot t % P of page
block_tables[b, t // P]; the output is softmax(scale * q K^T) V over those
L tokens, computed in fp64 after exact widening of the stored elements, with
fp8 elements multiplied by their (page, kv head) scale.  L = 0 gives zeros.
"""
from __future__ import annotations

import math

import numpy as np

ELEM_BITS = {"f32": 32, "bf16": 16, "fp8": 8, "i8": 8, "i4": 4}
SCALED = ("fp8", "i8", "i4")      # formats with per-(page, kv head) scales


def pool_elems(pool: np.ndarray, kv_dtype: str) -> int:
    """Elements per (page, kv head) chunk of a pool array (int4: two per byte)."""
    return pool.shape[-1] * (2 if kv_dtype == "i4" else 1)


def read_elems(pool: np.ndarray, idx, kv_dtype: str) -> np.ndarray:
    """Stored elements pool[..., idx] by element index (int4: the nibble codes)."""
    if kv_dtype != "i4":
        return pool[idx]
    *lead, e = idx
    b = pool[tuple(lead) + (e // 2,)]
    return ((b >> (4 * (e % 2))) & 0xF).astype(np.uint8)


def write_elems(pool: np.ndarray, idx, vals, kv_dtype: str) -> None:
    """pool[..., idx] = vals by element index (int4: nibble codes, the byte's other
    nibble kept).  For int4 the even elements are written first, then the odd
    ones: each byte holds one of each, so neither pass assigns a byte twice."""
    if kv_dtype != "i4":
        pool[idx] = vals
        return
    *lead, e = idx
    e = np.asarray(e)
    shape = np.broadcast(*lead, e).shape
    vals = np.broadcast_to(np.asarray(vals, dtype=np.uint8) & 0xF, shape)
    full = [np.broadcast_to(np.asarray(x), shape) for x in lead] + [np.broadcast_to(e, shape)]
    for parity in (0, 1):
        m = full[-1] % 2 == parity
        sel = tuple(x[m] for x in full[:-1]) + (full[-1][m] // 2,)
        old = pool[sel]
        if parity == 0:
            pool[sel] = (old & 0xF0) | vals[m]
        else:
            pool[sel] = (old & 0x0F) | (vals[m] << 4)


# ---------------------------------------------------------------- decoding ----

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64: the pattern is the upper half of a binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    """All 256 OCP e4m3fn codes: bias 7, subnormal m * 2**-9, S.1111.111 = NaN."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            v = math.nan
        elif e == 0:
            v = m * 2.0 ** -9
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[code] = -v if s else v
    return t


E4M3_TABLE = _e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "fp8":
        return e4m3_to_f64(x)
    if dtype == "i8":                       # two's complement bytes
        return np.asarray(x).view(np.int8).astype(np.float64)
    if dtype == "i4":                       # two's complement nibble codes
        c = np.asarray(x, dtype=np.int64) & 0xF
        return ((c ^ 8) - 8).astype(np.float64)
    raise ValueError(dtype)


# ------------------------------------------------------------------ layout ----

def _offsets(P: int, D: int, kv_dtype: str):
    """Element offsets inside one (page, head) chunk, as [P, D] arrays (K, V)."""
    E = 128 // ELEM_BITS[kv_dtype]
    TB = 4 * E
    j = np.arange(P).reshape(P, 1)
    d = np.arange(D).reshape(1, D)
    k = (d // E * P + j) * E + d % E
    blk, r = j // TB, j % TB
    v = blk * (TB * D) + ((r % 16) // 4 * D + d) * E + (4 * (r // 16) + r % 4)
    return k, v


def gather(k_pool, v_pool, kv_dtype, block_tables, seq_lens, P, b):
    """Stored K, V elements of sequence b in logical order: [Hkv, L, D] each."""
    NP, Hkv = k_pool.shape[:2]
    D = pool_elems(k_pool, kv_dtype) // P
    L = max(int(seq_lens[b]), 0)
    koff, voff = _offsets(P, D, kv_dtype)
    t = np.arange(L)
    pages = np.asarray(block_tables[b])[t // P].astype(np.int64)
    if L and (pages.min() < 0 or pages.max() >= NP):
        raise IndexError("page id out of range")
    slot = t % P
    hh = np.arange(Hkv)[:, None, None]
    k = read_elems(k_pool, (pages[None, :, None], hh, koff[slot][None, :, :]), kv_dtype)
    v = read_elems(v_pool, (pages[None, :, None], hh, voff[slot][None, :, :]), kv_dtype)
    return k, v, pages


def decode_row_group(q_rows, k, v, scale):
    """fp64 attention of G query rows [G, D] over keys/values [L, D]."""
    s = float(scale) * (q_rows @ k.T)                     # [G, L]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def decode(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables, seq_lens, Hq, P, scale,
           k_scales=None, v_scales=None, batches=None):
    """fp64 [B, Hq, D] outputs (rows of sequences not in ``batches`` stay zero)."""
    B = len(seq_lens)
    NP, Hkv = k_pool.shape[:2]
    D = pool_elems(k_pool, kv_dtype) // P
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    qf = widen(q, q_dtype).reshape(B, Hq, D)
    for b in (range(B) if batches is None else batches):
        if int(seq_lens[b]) <= 0:
            continue
        k, v, pages = gather(k_pool, v_pool, kv_dtype, block_tables, seq_lens, P, b)
        kf, vf = widen(k, kv_dtype), widen(v, kv_dtype)
        if kv_dtype in SCALED:
            kf = kf * np.asarray(k_scales, np.float64)[pages].T[:, :, None]
            vf = vf * np.asarray(v_scales, np.float64)[pages].T[:, :, None]
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G] = decode_row_group(qf[b, g * G:(g + 1) * G], kf[g], vf[g], scale)
    return out


def append(k_new, v_new, kv_dtype, block_tables, seq_lens, k_pool, v_pool, P):
    """In place: token L-1 of each sequence (L = seq_lens[b] >= 1) into its page slot.
    int4 rows k_new[b][g] are packed (D/2 bytes, element 2i in the low nibble)."""
    NP, Hkv = k_pool.shape[:2]
    D = pool_elems(k_pool, kv_dtype) // P
    koff, voff = _offsets(P, D, kv_dtype)
    if kv_dtype == "i4":
        k_new = np.stack([np.asarray(k_new) & 0xF, np.asarray(k_new) >> 4], -1).reshape(len(seq_lens), Hkv, D)
        v_new = np.stack([np.asarray(v_new) & 0xF, np.asarray(v_new) >> 4], -1).reshape(len(seq_lens), Hkv, D)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        t = L - 1
        pg = int(block_tables[b][t // P])
        if not 0 <= pg < NP:
            raise IndexError("page id out of range")
        hh = np.arange(Hkv)[:, None]
        write_elems(k_pool, (pg, hh, koff[t % P][None, :]), k_new[b], kv_dtype)
        write_elems(v_pool, (pg, hh, voff[t % P][None, :]), v_new[b], kv_dtype)


# ------------------------------------------------- split-KV partitions -------

def partition_partials(q_rows, k, v, scale, part):
    """Per partition of ``part`` tokens: normalised output and log-sum-exp.

    Returns (o [S, G, D], lse [S, G]); lse_s = m_s + ln sum exp(s_t - m_s).
    """
    L = k.shape[0]
    outs, lses = [], []
    for t0 in range(0, L, part):
        s = float(scale) * (q_rows @ k[t0:t0 + part].T)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        outs.append((w @ v[t0:t0 + part]) / l)
        lses.append((m + np.log(l))[:, 0])
    return np.stack(outs), np.stack(lses)


def merge_partials(o, lse):
    """Combine partition results: weights exp(lse_s - max lse), normalised."""
    M = lse.max(axis=0, keepdims=True)
    w = np.exp(lse - M)                                   # [S, G]
    return (w[:, :, None] * o).sum(axis=0) / w.sum(axis=0)[:, None]


# ------------------------------------- fp8 append with dynamic page scales ----
#
# Source: the concept page's "compile-time graph optimization" section inserts
# a dynamic scaling-factor computation where data enters an FP8 product; the
# yololab page ("FP8 與極致量化") gives FP8 as the way to halve the bandwidth a
# model needs.  Applied here where new K/V data enter the fp8 cache.  Reading
# (the pages fix no granularity or update rule): one fp32 scale per (page, kv
# head), real value = decoded byte * scale, set to amax / 448 by the page's
# first token; a later token keeps the scale if its largest element still
# rounds to a finite code without clipping (|x| / scale <= 464, the midpoint
# between 448 and the next binade step, which rounds down to 448), otherwise
# the scale grows to its amax / 448 and the page's earlier tokens are
# re-encoded under it.  Every step below is one fp32 operation rounded to
# nearest even, so the result is a unique byte image.

E4M3_FINITE_MAX = 448.0
E4M3_NO_CLIP = 464.0        # largest |x| / scale that still rounds to +-448


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn code: the nearest finite e4m3 value, a tie going to
    the even code (even significand), magnitudes above 448 saturating to 448,
    NaN -> 0x7F; the sign of x (also of -0) is kept.  Written as a search over
    the 127 non-negative finite codes, which increase with their value."""
    x = np.asarray(x, dtype=np.float32)
    pos = E4M3_TABLE[:127]
    a = np.abs(np.where(np.isnan(x), np.float32(0), x)).astype(np.float64)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - pos[lo], pos[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a >= E4M3_FINITE_MAX, 126, code).astype(np.uint8)
    code = code | (np.signbit(x).astype(np.uint8) << np.uint8(7))
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def int8_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> symmetric int8 byte: round to the nearest integer, a tie going
    to the even one, then clamp to [-127, 127] (-128 is not used)."""
    q = np.clip(np.rint(np.asarray(x, dtype=np.float32).astype(np.float64)), -127, 127)
    return q.astype(np.int8).view(np.uint8)


def int8_to_f64(codes: np.ndarray) -> np.ndarray:
    return np.asarray(codes, dtype=np.uint8).view(np.int8).astype(np.float64)


# Per format: (largest code value, largest |x| / scale that still rounds into
# range without clipping, encoder, exact decoder).  int8 rounds 127.5 to 128
# (ties to even), which clamps to 127: still within half a step, so 127.5 is
# the no-clip bound there, as 464 (the midpoint above 448) is for e4m3.
def int4_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> symmetric int4 nibble code: nearest integer, ties to even,
    clamped to [-7, 7] (-8 is not used), as a two's complement nibble 0..15."""
    q = np.clip(np.rint(np.asarray(x, dtype=np.float32).astype(np.float64)), -7, 7).astype(np.int64)
    return (q & 0xF).astype(np.uint8)


def int4_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64) & 0xF
    return ((c ^ 8) - 8).astype(np.float64)


DYNAMIC_FORMATS = {
    "fp8": (448.0, 464.0, lambda y: e4m3_encode(y), e4m3_to_f64),
    "i8": (127.0, 127.5, lambda y: int8_encode(y), int8_to_f64),
    "i4": (7.0, 7.5, lambda y: int4_encode(y), int4_to_f64),
}


def append_dynamic(fmt, k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool,
                   k_scales, v_scales, P):
    """In place: token L-1 of each sequence into its page (fmt "fp8", "i8" or
    "i4"), with the page scale kept at amax / QMAX of the page's tokens (K and V
    each on their own); QMAX = 448 for fp8, 127 for int8, 7 for int4.

    For each b with L = seq_lens[b] >= 1, t = L - 1, page pg = block_tables[b, t//P]
    (a table index or page id out of range skips the sequence), slot j = t % P,
    and each kv head g, separately for K and V with x = the new row widened to
    fp32 and a = max |x|:
      j == 0 (first token of the page): s = a / QMAX, or 1 when a == 0;
      j > 0, s0 = the page's current scale: if a / s0 <= NOCLIP (the row's
        largest element rounds to the largest code or less, no clipping:
        464 for fp8, 127.5 for int8, 7.5 for int4) then s = s0;
        otherwise s = a / QMAX and every earlier slot j' < j is re-encoded:
        byte' = enc((dec(byte) * s0) / s);
      the new token: byte = enc(x / s); the page scale becomes s.
    Arithmetic is fp32 (each division and product rounded to nearest even);
    enc is the format's encoder, dec its exact value.
    """
    qmax, noclip, enc, dec = DYNAMIC_FORMATS[fmt]
    NP, Hkv = k_pool.shape[:2]
    D = pool_elems(k_pool, fmt) // P
    MP = np.asarray(block_tables).shape[1]
    koff, voff = _offsets(P, D, fmt)
    f32 = np.float32
    cmax, cnoclip = f32(qmax), f32(noclip)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        t = L - 1
        if t // P >= MP:
            continue
        pg = int(block_tables[b][t // P])
        if not 0 <= pg < NP:
            continue
        j = t % P
        for new, pool, scales, off in ((k_new, k_pool, k_scales, koff), (v_new, v_pool, v_scales, voff)):
            for g in range(Hkv):
                x = widen(np.asarray(new)[b, g], new_dtype).astype(np.float32)   # exact
                a = f32(np.abs(x).max())
                if j == 0:
                    s = f32(a / cmax) if a > 0 else f32(1)
                else:
                    s0 = f32(scales[pg, g])
                    if f32(a / s0) <= cnoclip:
                        s = s0
                    else:
                        s = f32(a / cmax)
                        idx = off[:j]                                          # [j, D]
                        real = dec(read_elems(pool, (pg, g, idx), fmt)).astype(np.float32) * s0
                        write_elems(pool, (pg, g, idx), enc(real.astype(np.float32) / s), fmt)
                write_elems(pool, (pg, g, off[j]), enc(x / s), fmt)
                scales[pg, g] = s


def append_fp8_dynamic(k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool,
                       k_scales, v_scales, P):
    """append_dynamic for an fp8 e4m3 cache (QMAX 448, no-clip bound 464)."""
    append_dynamic("fp8", k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool,
                   k_scales, v_scales, P)


def append_int4_dynamic(k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool,
                        k_scales, v_scales, P):
    """append_dynamic for a symmetric int4 cache (QMAX 7, no-clip bound 7.5)."""
    append_dynamic("i4", k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool,
                   k_scales, v_scales, P)


def append_int8_dynamic(k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool,
                        k_scales, v_scales, P):
    """append_dynamic for a symmetric int8 cache (QMAX 127, no-clip bound 127.5)."""
    append_dynamic("i8", k_new, v_new, new_dtype, block_tables, seq_lens, k_pool, v_pool,
                   k_scales, v_scales, P)


# ------------------------------------------------------ chunked prefill -------
#
# Source: the concept page's "key performance parameters" section: with paged
# attention the context is processed in parallel over many tokens at once (the
# compute that sets the first-token latency), beside the decode iterations of
# its "runtime execution model" section that read and update the same pages.
# Reading (the pages give no formula or interface): sequence b brings a chunk
# of C_b new tokens whose K/V rows are written into its pages first, so
# seq_lens[b] = L_b counts them; chunk token i sits at position p = L_b - C_b + i
# and attends to the cached tokens 0..p (causal).  q and the output hold the
# chunks back to back, rows cu_q[b] .. cu_q[b+1] for sequence b.  A position
# below zero (C_b > L_b) attends to nothing and gives zeros, as L = 0 does for
# decode.

def prefill(q, q_dtype, cu_q, k_pool, v_pool, kv_dtype, block_tables, seq_lens, Hq, P, scale,
            batches=None, k_scales=None, v_scales=None):
    """fp64 [T, Hq, D] outputs of causal chunked prefill over the paged cache.

    For the scaled caches (fp8, int8, int4) a stored element's value is its
    code times the (page, kv head) scale, as in decode."""
    cu = np.asarray(cu_q, dtype=np.int64)
    B = len(seq_lens)
    T = int(cu[-1])
    NP, Hkv = k_pool.shape[:2]
    D = pool_elems(k_pool, kv_dtype) // P
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qf = widen(q, q_dtype).reshape(T, Hq, D)
    for b in (range(B) if batches is None else batches):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        C, L = r1 - r0, int(seq_lens[b])
        if C <= 0 or L <= 0:
            continue
        pos = L - C + np.arange(C)                          # position of each chunk token
        allowed = np.arange(L)[None, :] <= pos[:, None]      # [C, L] causal mask
        live = pos >= 0
        k, v, pages = gather(k_pool, v_pool, kv_dtype, block_tables, seq_lens, P, b)
        kf, vf = widen(k, kv_dtype), widen(v, kv_dtype)
        if kv_dtype in SCALED:
            kf = kf * np.asarray(k_scales, np.float64)[pages].T[:, :, None]
            vf = vf * np.asarray(v_scales, np.float64)[pages].T[:, :, None]
        for g in range(Hkv):
            qg = qf[r0:r1, g * G:(g + 1) * G]                # [C, G, D]
            s = float(scale) * np.einsum("cgd,ld->cgl", qg, kf[g])
            s = np.where(allowed[:, None, :], s, -np.inf)
            m = np.where(live[:, None, None], s.max(axis=2, keepdims=True), 0.0)
            with np.errstate(invalid="ignore"):
                w = np.where(allowed[:, None, :], np.exp(s - m), 0.0)
            den = w.sum(axis=2, keepdims=True)
            o = np.einsum("cgl,ld->cgd", w, vf[g]) / np.where(live[:, None, None], den, 1.0)
            out[r0:r1, g * G:(g + 1) * G] = np.where(live[:, None, None], o, 0.0)
    return out


def append_chunk(k_new, v_new, kv_dtype, cu_new, block_tables, seq_lens, k_pool, v_pool, P):
    """In place: rows cu_new[b] .. cu_new[b+1] of k_new / v_new ([T, Hkv, D] stored
    elements; int4 rows packed, D/2 bytes) into positions L_b - C_b + i of
    sequence b.  A sequence whose chunk does not fit (C_b > L_b, or L_b beyond its
    page-table row) is skipped; a page id out of range raises."""
    cu = np.asarray(cu_new, dtype=np.int64)
    NP, Hkv = k_pool.shape[:2]
    D = pool_elems(k_pool, kv_dtype) // P
    MP = np.asarray(block_tables).shape[1]
    koff, voff = _offsets(P, D, kv_dtype)
    if kv_dtype == "i4":
        T = len(k_new)
        k_new = np.stack([np.asarray(k_new) & 0xF, np.asarray(k_new) >> 4], -1).reshape(T, Hkv, D)
        v_new = np.stack([np.asarray(v_new) & 0xF, np.asarray(v_new) >> 4], -1).reshape(T, Hkv, D)
    hh = np.arange(Hkv)[:, None]
    for b in range(len(seq_lens)):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        C, L = r1 - r0, int(seq_lens[b])
        if C <= 0 or C > L or L > MP * P:
            continue
        for i in range(C):
            t = L - C + i
            pg = int(block_tables[b][t // P])
            if not 0 <= pg < NP:
                raise IndexError("page id out of range")
            write_elems(k_pool, (pg, hh, koff[t % P][None, :]), k_new[r0 + i], kv_dtype)
            write_elems(v_pool, (pg, hh, voff[t % P][None, :]), v_new[r0 + i], kv_dtype)


# ------------------------------------------------ device page allocation ------
#
# Source: the concept page's "key mechanisms" section takes pages from a shared
# pool as a sequence grows, and its "runtime execution model" section has
# finished requests return their pages for reuse.  Reading (the pages give no
# data structure): the free pages form a stack (free_pages[0 .. count - 1],
# top at count - 1).  alloc: in sequence order, every sequence whose last token
# L_b - 1 opens a page (L_b >= 1, (L_b - 1) % P == 0, within its table row)
# and whose entry for that page is empty (negative) takes the top page into
# block_tables[b][(L_b - 1) / P]; once the stack is empty the remaining
# requests keep their -1.  (A sequence that did not grow this step already
# holds its page and takes none.)  release: in sequence order, every
# marked sequence pushes the ids in the first ceil(L_b / P) entries of its row
# (ids in [0, num_pages) only) and sets those entries to -1; pushes beyond the
# stack's capacity are dropped.

def alloc_pages(seq_lens, block_tables, free_pages, count, P):
    """In place on block_tables and free_pages; returns the new count."""
    MP = block_tables.shape[1]
    for b, L in enumerate(np.asarray(seq_lens)):
        L = int(L)
        if L < 1 or (L - 1) % P != 0 or (L - 1) // P >= MP or block_tables[b, (L - 1) // P] >= 0:
            continue
        if count > 0:
            count -= 1
            block_tables[b, (L - 1) // P] = free_pages[count]
    return count


def release_pages(release, seq_lens, block_tables, free_pages, count, capacity, num_pages, P):
    """In place; returns the new count."""
    MP = block_tables.shape[1]
    for b, r in enumerate(np.asarray(release)):
        if not r:
            continue
        L = int(seq_lens[b])
        n = min(max(-(-L // P), 0), MP)
        for i in range(n):
            pg = int(block_tables[b, i])
            if 0 <= pg < num_pages:
                if count < capacity:
                    free_pages[count] = pg
                    count += 1
            block_tables[b, i] = -1
    return count
