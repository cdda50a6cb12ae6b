"""GPU parity of chunked prefill: pkv_kv_append_chunk (bit-exact against
oracle.paged.append_chunk) and pkv_paged_prefill (against oracle.paged.prefill
at the bf16 tolerance), through the C ABI."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import paged_kv_attention_decode_amd as pkv
from oracle import paged
from workloads import codec, configs, layout
from tests._helpers import LOGIT_PROFILES, ORACLE_THREADS, check_close, dev_tensor, gpu_out, host_bytes

pytestmark = pytest.mark.gpu


def _up(wl):
    d = {k: dev_tensor(getattr(wl, k)) for k in ("q", "cu_q", "block_tables", "seq_lens", "k_pool", "v_pool",
                                                 "k_new", "v_new")}
    if wl.k_scales is not None:
        d["k_scales"], d["v_scales"] = dev_tensor(wl.k_scales), dev_tensor(wl.v_scales)
    return d


def _gpu_append_chunk(wl, d, seq_lens=None, cu=None, bt=None):
    pkv.kv_append_chunk(d["k_new"], d["v_new"], wl.kv_dtype, d["cu_q"] if cu is None else cu,
                        d["block_tables"] if bt is None else bt, d["seq_lens"] if seq_lens is None else seq_lens,
                        d["k_pool"], d["v_pool"], wl.Hkv, wl.D, wl.P)


def _gpu_prefill(wl, d, out_dtype=None, seq_lens=None, bt=None):
    odt = out_dtype or wl.out_dtype
    out = torch.full((wl.T, wl.Hq, wl.D), 7.0, dtype=torch.bfloat16 if odt == "bf16" else torch.float32,
                     device="cuda")
    btd = d["block_tables"] if bt is None else bt
    sld = d["seq_lens"] if seq_lens is None else seq_lens
    if wl.kv_dtype == "fp8":
        pkv.paged_prefill_fp8(d["q"], wl.q_dtype, d["cu_q"], d["k_pool"], d["v_pool"], d["k_scales"], d["v_scales"],
                              btd, sld, wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, out, odt)
    else:
        pkv.paged_prefill(d["q"], wl.q_dtype, d["cu_q"], d["k_pool"], d["v_pool"], wl.kv_dtype, btd, sld,
                          wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, out, odt)
    torch.cuda.synchronize()
    return gpu_out(out)


def _full_pools(wl):
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    paged.append_chunk(wl.k_new, wl.v_new, wl.kv_dtype, wl.cu_q, wl.block_tables, wl.seq_lens, kp, vp, wl.P)
    return kp, vp


def _quantised_case(fmt, seed, ctx, chunk, Hq, Hkv, D, P):
    """A chunk workload whose cache and rows are stored in ``fmt`` (bytes as the
    generator's page quantiser writes them; the append copies them as given)."""
    wl = configs.prefill_case("q", seed, ctx, chunk, Hq, Hkv, D, P, kv_dtype="f32" if fmt == "f32" else "bf16")
    L = wl.seq_lens
    bits = layout.ELEM_BITS[fmt]
    kp = layout.empty_pool(wl.num_pages, Hkv, P, D, fmt)
    vp = layout.empty_pool(wl.num_pages, Hkv, P, D, fmt)
    kidx, vidx = layout.k_chunk_index(P, D, fmt), layout.v_chunk_index(P, D, fmt)
    T = wl.T
    rowb = D * bits // 8
    kn = np.zeros((T, Hkv, rowb), np.uint8) if fmt != "f32" else np.zeros((T, Hkv, D), np.float32)
    vn = kn.copy()
    for b in range(wl.B):
        n = int(L[b])
        kf = configs.draw_seq_f32(wl.seed, 2, b, n, Hkv, D)
        vf = configs.draw_seq_f32(wl.seed, 3, b, n, Hkv, D)
        if fmt == "f32":
            k, v = kf, vf
        else:
            k, _ = configs.QUANTIZERS[fmt](kf, P)
            v, _ = configs.QUANTIZERS[fmt](vf, P)
        c0 = int(ctx[b])
        pages = wl.block_tables[b, :-(-c0 // P)] if c0 else np.zeros(0, np.int32)
        layout.pack_sequence(kp, pages, k[:c0], P, kidx, fmt)
        layout.pack_sequence(vp, pages, v[:c0], P, vidx, fmt)
        rk, rv = k[c0:], v[c0:]
        if fmt == "i4":
            rk, rv = layout.pack_nibbles(rk), layout.pack_nibbles(rv)
        kn[wl.cu_q[b]:wl.cu_q[b + 1]] = rk
        vn[wl.cu_q[b]:wl.cu_q[b + 1]] = rv
    wl.kv_dtype, wl.k_pool, wl.v_pool, wl.k_new, wl.v_new = fmt, kp, vp, kn, vn
    return wl


APPEND_CASES = [  # (fmt, D, P)
    ("bf16", 128, 64), ("bf16", 64, 32), ("bf16", 128, 128), ("f32", 64, 16), ("fp8", 128, 64), ("i8", 64, 64), ("i4", 128, 128),
]


@pytest.mark.parametrize("fmt,D,P", APPEND_CASES, ids=lambda v: str(v))
def test_append_chunk_bit_exact(fmt, D, P):
    ctx = [0, 3, 130, 17, 250, 0]
    chunk = [1, 200, 2, 0, 61, 129]
    wl = _quantised_case(fmt, 40 + D + P, ctx, chunk, 4, 2, D, P) if fmt != "bf16" else \
        configs.prefill_case("a", 40 + D + P, ctx, chunk, 4, 2, D, P)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    torch.cuda.synchronize()
    kp, vp = _full_pools(wl)
    assert np.array_equal(host_bytes(d["k_pool"]), kp.reshape(-1).view(np.uint8))
    assert np.array_equal(host_bytes(d["v_pool"]), vp.reshape(-1).view(np.uint8))


def test_append_chunk_skips_what_does_not_fit():
    wl = configs.prefill_case("a", 51, [0, 5, 40, 17], [7, 1, 33, 16], 4, 2, 64, 32)
    d = _up(wl)
    lens = wl.seq_lens.copy()
    lens[0] = 3                                    # chunk of 7 > L = 3
    lens[2] = wl.max_pages * wl.P + 1              # beyond the table row
    bt = wl.block_tables.copy()
    L3 = int(lens[3])
    bt[3, :-(-L3 // wl.P)] = wl.num_pages + 5      # every page of sequence 3 out of range
    _gpu_append_chunk(wl, d, seq_lens=dev_tensor(lens), bt=dev_tensor(bt))
    torch.cuda.synchronize()
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    cu2 = np.zeros_like(wl.cu_q)
    cu2[1:] = np.cumsum([wl.chunk_lens[b] if b == 1 else 0 for b in range(wl.B)])
    sel = np.arange(wl.cu_q[1], wl.cu_q[2])
    paged.append_chunk(wl.k_new[sel], wl.v_new[sel], "bf16", cu2, wl.block_tables, lens, kp, vp, wl.P)
    assert np.array_equal(host_bytes(d["k_pool"]), kp.reshape(-1).view(np.uint8))
    assert np.array_equal(host_bytes(d["v_pool"]), vp.reshape(-1).view(np.uint8))


PREFILL_CASES = [  # (ctx, chunk, Hq, Hkv, D, P)
    ([0, 5, 100, 300], [1, 70, 33, 130], 8, 2, 128, 64),        # G 4, ragged, several tiles and pages
    ([64, 0, 31], [64, 257, 97], 2, 2, 64, 32),                   # G 1: blocks of 256 tokens
    ([200, 9], [45, 300], 16, 2, 128, 128),                       # G 8
    ([33, 0], [80, 19], 4, 2, 64, 64),                            # G 2
    ([100], [40], 32, 2, 128, 64),                                # G 16
    ([70, 1], [90, 130], 6, 2, 128, 32),                          # G 3: padding rows in every block
    ([0, 0, 0], [1, 2, 300], 8, 2, 128, 64),                      # pure prefill (no cached tokens)
    ([5, 60], [33, 2], 32, 1, 128, 64),                           # G 32: 4 chunk tokens per block
    ([40, 3], [9, 5], 64, 1, 128, 64),                            # G 64: 2 chunk tokens per block
    ([17], [7], 128, 1, 64, 32),                                  # G 128, the largest: 1 token per block
    ([20000, 0], [64, 1100], 8, 1, 128, 1024),                    # 1024-token pages, a long cached context
]


@pytest.mark.parametrize("ctx,chunk,Hq,Hkv,D,P", PREFILL_CASES, ids=lambda v: str(v))
def test_prefill_matches_oracle(ctx, chunk, Hq, Hkv, D, P):
    wl = configs.prefill_case("p", 60 + Hq + D + P, ctx, chunk, Hq, Hkv, D, P)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    got = _gpu_prefill(wl, d)
    kp, vp = _full_pools(wl)
    ref = paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                        wl.scale)
    check_close(got, ref, "bf16", "prefill", out_rounding=True)


def test_prefill_fp32_output_and_large_logits():
    wl = configs.prefill_case("p", 71, [150, 20], [70, 90], 8, 2, 128, 64, out_dtype="f32", q_mult=3.0)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    got = _gpu_prefill(wl, d, out_dtype="f32")
    kp, vp = _full_pools(wl)
    ref = paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                        wl.scale)
    check_close(got, ref, "bf16", "prefill f32 out")


def test_prefill_softmax_reference_paths():
    """Each sequence's keys follow one logit profile (q = ones, scale 1) over its
    cached tokens and its chunk, so the per-row softmax reference grows every
    tile, now and then, once, only at the diagonal tile, or at alternating
    tiles, or sits near 900: the lane test and the lazy reference must still
    match the oracle's exact softmax."""
    names = list(LOGIT_PROFILES)
    ctx = [600, 1900, 600, 1300, 200, 900]
    chunk = [100, 200, 100, 200, 133, 124]
    Hkv, D, P = 2, 128, 64
    wl = configs.prefill_case("p", 69, ctx, chunk, 4 * Hkv, Hkv, D, P)
    wl.scale = np.float32(1.0)
    wl.q = codec.f32_to_bf16_bits(np.ones(wl.q.shape, np.float32))
    kidx = layout.k_chunk_index(P, D, "bf16")
    r = np.random.default_rng(70)
    for b, name in enumerate(names):
        L = int(wl.seq_lens[b])
        c = np.asarray(LOGIT_PROFILES[name](np.arange(L), L, r), dtype=np.float64)
        k = codec.f32_to_bf16_bits((np.repeat((c / D)[:, None, None], Hkv, axis=1) * np.ones((1, 1, D)))
                                   .astype(np.float32))
        pages = wl.block_tables[b, :(ctx[b] + P - 1) // P]
        layout.pack_sequence(wl.k_pool, pages, k[:ctx[b]], P, kidx, "bf16")
        wl.k_new[wl.cu_q[b]:wl.cu_q[b + 1]] = k[ctx[b]:]
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    got = _gpu_prefill(wl, d)
    kp, vp = _full_pools(wl)
    ref = paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                        wl.scale)
    check_close(got, ref, "bf16", "prefill logit profiles", out_rounding=True)


def _random_prefill_cases(n=12, seed=95):
    """Seeded draws: G 1..16, D 64/128, P 32..128, 1-6 sequences with cached
    contexts of 0..2000 tokens and chunks of 1..300, logits of std 1 or 3."""
    r = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        B = int(r.integers(1, 7))
        Hkv = int(r.choice([1, 2, 4]))
        G = int(r.choice([1, 2, 3, 4, 8, 16]))
        ctx = [int(r.choice([0, int(r.integers(1, 2001))])) for _ in range(B)]
        chunk = [int(r.integers(1, 301)) for _ in range(B)]
        cases.append(dict(seed=2000 + k, ctx=ctx, chunk=chunk, Hq=Hkv * G, Hkv=Hkv,
                          D=int(r.choice([64, 128])), P=int(r.choice([32, 64, 128])),
                          q_mult=float(r.choice([1.0, 3.0])), out="f32" if k % 2 else "bf16"))
    return cases


@pytest.mark.parametrize("c", _random_prefill_cases(),
                         ids=lambda c: f"G{c['Hq'] // c['Hkv']}-D{c['D']}-P{c['P']}-B{len(c['ctx'])}-{c['out']}-s{c['seed']}")
def test_prefill_random_configs(c):
    wl = configs.prefill_case("p", c["seed"], c["ctx"], c["chunk"], c["Hq"], c["Hkv"], c["D"], c["P"],
                              q_mult=c["q_mult"], out_dtype=c["out"])
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    got = _gpu_prefill(wl, d)
    kp, vp = _full_pools(wl)
    ref = paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                        wl.scale)
    check_close(got, ref, "bf16", f"prefill random seed {c['seed']}", out_rounding=c["out"] == "bf16")


def test_prefill_rows_without_keys_zero_and_other_rows_untouched():
    wl = configs.prefill_case("p", 72, [0, 10, 0], [20, 0, 30], 8, 2, 64, 32)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    kp, vp = _full_pools(wl)
    lens = wl.seq_lens.copy()
    lens[0] = 12                                   # chunk of 20 over 12 keys: rows 0..7 at p < 0
    got = _gpu_prefill(wl, d, seq_lens=dev_tensor(lens))
    ref = paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, lens, wl.Hq, wl.P, wl.scale)
    assert np.all(got[:8] == 0)
    check_close(got, ref, "bf16", "prefill p < 0", out_rounding=True)


def test_prefill_bad_page_gives_nan_rows_of_that_head_block_only():
    wl = configs.prefill_case("p", 73, [40, 50], [30, 20], 8, 2, 64, 32)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    kp, vp = _full_pools(wl)
    bt = wl.block_tables.copy()
    bt[1, 0] = wl.num_pages + 3                    # sequence 1's first page id out of range
    got = _gpu_prefill(wl, d, bt=dev_tensor(bt))
    r0, r1 = int(wl.cu_q[1]), int(wl.cu_q[2])
    assert np.all(np.isnan(got[r0:r1]))
    ref = paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                        wl.scale, batches=[0])
    check_close(got[:r0], ref[:r0], "bf16", "prefill other sequence", out_rounding=True)


def test_prefill_padding_rows_not_written():
    """Rows of out outside every sequence's range keep their contents."""
    wl = configs.prefill_case("p", 74, [10, 20], [5, 7], 8, 2, 64, 32)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    cu = wl.cu_q.copy()
    cu[0] = cu[1] = 5                              # sequence 0 given no rows: rows 0..4 belong to nobody
    d["cu_q"] = dev_tensor(cu)
    got = _gpu_prefill(wl, d)
    assert np.all(got[:5] == 7.0)
    assert np.isfinite(got[5:]).all() and not np.all(got[5:] == 7.0)


@pytest.mark.timeout(900)
def test_config_chunked_prefill_full_size():
    """The full chunked-prefill workload (16 sequences, 8192 chunk tokens) in the
    launch the benchmark times.  The GPU chunk append is compared byte for byte
    with the oracle's append of the whole workload; the prefill output of six
    sequences (the shortest and the longest cached context and four between,
    3072 query rows) is compared with the oracle run on the oracle's own pools;
    every output row is finite."""
    wl = configs.chunked_prefill_bf16()
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    got = _gpu_prefill(wl, d)
    assert np.isfinite(got).all()
    kp, vp = _full_pools(wl)
    assert np.array_equal(host_bytes(d["k_pool"]), kp.view(np.uint8).reshape(-1)), "chunk append (K) differs"
    assert np.array_equal(host_bytes(d["v_pool"]), vp.view(np.uint8).reshape(-1)), "chunk append (V) differs"
    ctx = wl.seq_lens - wl.chunk_lens
    order = np.argsort(ctx, kind="stable")
    picks = [int(order[i]) for i in (0, 3, 6, 9, 12, len(order) - 1)]
    assert ctx[picks[0]] == ctx.min() and ctx[picks[-1]] == ctx.max()

    def one(b):
        return paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                             wl.scale, batches=[b])

    with ThreadPoolExecutor(max_workers=min(len(picks), ORACLE_THREADS)) as ex:
        refs = list(ex.map(one, picks))
    rows_got, rows_ref = [], []
    for b, ref in zip(picks, refs):
        r0, r1 = int(wl.cu_q[b]), int(wl.cu_q[b + 1])
        check_close(got[r0:r1], ref[r0:r1], "bf16", f"sequence {b} (context {int(ctx[b])})", out_rounding=True)
        rows_got.append(got[r0:r1])
        rows_ref.append(ref[r0:r1])
    check_close(np.concatenate(rows_got), np.concatenate(rows_ref), "bf16",
                "chunked_prefill_bf16 (6 of 16 sequences)", out_rounding=True, report=True)


# ------------------------------------------------------------ fp8 cache ----
# K/V as e4m3 codes with per-(page, kv head) scales; the oracle multiplies each
# code by its scale.  Bound: the fp8 one (max-abs <= 3e-2), with bf16 outputs
# allowed their own half-ulp rounding.

def _fp8_ref(wl, kp, vp, seq_lens=None, batches=None):
    return paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "fp8", wl.block_tables,
                         wl.seq_lens if seq_lens is None else seq_lens, wl.Hq, wl.P, wl.scale, batches=batches,
                         k_scales=wl.k_scales, v_scales=wl.v_scales)


FP8_CASES = [  # (ctx, chunk, Hq, Hkv, D, P)
    ([0, 5, 100, 300], [1, 70, 33, 130], 8, 2, 128, 64),
    ([64, 0, 31], [64, 257, 97], 2, 2, 64, 64),
    ([200, 9], [45, 300], 16, 2, 128, 128),
    ([33, 0], [80, 19], 4, 2, 64, 128),
    ([100], [40], 32, 2, 128, 64),
    ([70, 1], [90, 130], 6, 2, 128, 64),
    ([0, 0, 0], [1, 2, 300], 8, 2, 128, 64),
    ([40, 3], [9, 5], 64, 1, 128, 64),
    ([17], [7], 128, 1, 128, 64),
    ([3000, 10], [50, 700], 8, 2, 128, 1024),
]


@pytest.mark.parametrize("ctx,chunk,Hq,Hkv,D,P", FP8_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_fp8_prefill_matches_oracle(ctx, chunk, Hq, Hkv, D, P, odt):
    wl = configs.prefill_case("p8", 160 + Hq + D + P, ctx, chunk, Hq, Hkv, D, P, kv_dtype="fp8", out_dtype=odt)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    got = _gpu_prefill(wl, d)
    kp, vp = _full_pools(wl)
    assert np.array_equal(host_bytes(d["k_pool"]), kp.reshape(-1)) and np.array_equal(host_bytes(d["v_pool"]),
                                                                                      vp.reshape(-1))
    check_close(got, _fp8_ref(wl, kp, vp), "fp8", "fp8 prefill", out_rounding=odt == "bf16")


def test_fp8_prefill_large_logits_and_reference_paths():
    """Logits of std 3, and keys whose logits follow the softmax-reference profiles."""
    wl = configs.prefill_case("p8", 171, [150, 20, 700], [70, 90, 200], 8, 2, 128, 64, kv_dtype="fp8",
                              out_dtype="f32", q_mult=3.0)
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    kp, vp = _full_pools(wl)
    check_close(_gpu_prefill(wl, d), _fp8_ref(wl, kp, vp), "fp8", "fp8 prefill std-3 logits")


def test_fp8_prefill_rows_without_keys_and_bad_page():
    wl = configs.prefill_case("p8", 172, [0, 10, 40], [20, 0, 30], 8, 2, 64, 64, kv_dtype="fp8", out_dtype="f32")
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    kp, vp = _full_pools(wl)
    lens = wl.seq_lens.copy()
    lens[0] = 12                                   # chunk of 20 over 12 keys: rows 0..7 at p < 0
    got = _gpu_prefill(wl, d, seq_lens=dev_tensor(lens))
    assert np.all(got[:8] == 0)
    check_close(got, _fp8_ref(wl, kp, vp, seq_lens=lens), "fp8", "fp8 prefill p < 0")
    bt = wl.block_tables.copy()
    bt[2, 0] = wl.num_pages + 3                    # sequence 2's first page id out of range
    got = _gpu_prefill(wl, d, bt=dev_tensor(bt))
    r0, r1 = int(wl.cu_q[2]), int(wl.cu_q[3])
    assert np.all(np.isnan(got[r0:r1])) and np.isfinite(got[:r0]).all()


@pytest.mark.timeout(900)
def test_config_chunked_prefill_fp8_full_size():
    """The fp8 chunked-prefill workload (16 sequences x 512 chunk tokens): the
    chunk append byte-exact against the oracle's; the prefill of six sequences
    (shortest and longest context and four between) against the oracle on the
    oracle's pools; every row finite."""
    wl = configs.chunked_prefill_fp8()
    d = _up(wl)
    _gpu_append_chunk(wl, d)
    got = _gpu_prefill(wl, d)
    assert np.isfinite(got).all()
    kp, vp = _full_pools(wl)
    assert np.array_equal(host_bytes(d["k_pool"]), kp.reshape(-1)), "chunk append (K) differs"
    assert np.array_equal(host_bytes(d["v_pool"]), vp.reshape(-1)), "chunk append (V) differs"
    ctx = wl.seq_lens - wl.chunk_lens
    order = np.argsort(ctx, kind="stable")
    picks = [int(order[i]) for i in (0, 3, 6, 9, 12, len(order) - 1)]
    with ThreadPoolExecutor(max_workers=min(len(picks), ORACLE_THREADS)) as ex:
        refs = list(ex.map(lambda b: _fp8_ref(wl, kp, vp, batches=[b]), picks))
    rows_got, rows_ref = [], []
    for b, ref in zip(picks, refs):
        r0, r1 = int(wl.cu_q[b]), int(wl.cu_q[b + 1])
        check_close(got[r0:r1], ref[r0:r1], "fp8", f"sequence {b} (context {int(ctx[b])})", out_rounding=True)
        rows_got.append(got[r0:r1])
        rows_ref.append(ref[r0:r1])
    check_close(np.concatenate(rows_got), np.concatenate(rows_ref), "fp8",
                "chunked_prefill_fp8 (6 of 16 sequences)", out_rounding=True, report=True)
