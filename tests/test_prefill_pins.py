"""Pins of the chunked-prefill oracle (oracle.paged.prefill, append_chunk).

Each test ties the oracle to something other than itself: the decode oracle
(pinned on its own in test_oracle_pins), torch's scaled_dot_product_attention
on the logical rows the generator drew (not read back through the oracle's
gather), a scalar loop with math.exp, closed forms, and the single-token
append oracle.
"""
import math

import numpy as np
import pytest
import torch

from oracle import paged
from workloads import codec, configs, layout


def _full_pools(wl):
    """The wl pools after the chunk rows are appended (oracle append_chunk)."""
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    paged.append_chunk(wl.k_new, wl.v_new, wl.kv_dtype, wl.cu_q, wl.block_tables, wl.seq_lens, kp, vp, wl.P)
    return kp, vp


def _oracle(wl, kp, vp, **kw):
    return paged.prefill(wl.q, wl.q_dtype, wl.cu_q, kp, vp, wl.kv_dtype, wl.block_tables, wl.seq_lens,
                         wl.Hq, wl.P, wl.scale, **kw)


def _logical(wl, b):
    """Generator's logical K, V of sequence b as fp64 [L, Hkv, D] (from the draws)."""
    L = int(wl.seq_lens[b])
    k = configs.draw_seq_f32(wl.seed, 2, b, L, wl.Hkv, wl.D)
    v = configs.draw_seq_f32(wl.seed, 3, b, L, wl.Hkv, wl.D)
    if wl.kv_dtype == "bf16":
        k = codec.bf16_bits_to_f32(codec.f32_to_bf16_bits(k))
        v = codec.bf16_bits_to_f32(codec.f32_to_bf16_bits(v))
    return k.astype(np.float64), v.astype(np.float64)


def _q64(wl):
    if wl.q_dtype == "bf16":
        return codec.bf16_bits_to_f32(wl.q).astype(np.float64)
    return wl.q.astype(np.float64)


RAGGED = dict(ctx_lens=[0, 5, 40, 17], chunk_lens=[7, 1, 33, 16], Hq=4, Hkv=2, D=16, P=32)


def test_append_chunk_equals_token_by_token_append_and_full_pack():
    wl = configs.prefill_case("t", 11, **RAGGED)
    kp, vp = _full_pools(wl)
    # token by token with the single-token append oracle
    kq, vq = wl.k_pool.copy(), wl.v_pool.copy()
    C = wl.chunk_lens
    for i in range(int(C.max())):
        rows = np.minimum(wl.cu_q[:-1] + i, wl.T - 1)
        lens = np.where(i < C, wl.seq_lens - C + i + 1, 0).astype(np.int32)
        paged.append(wl.k_new[rows], wl.v_new[rows], wl.kv_dtype, wl.block_tables, lens, kq, vq, wl.P)
    assert np.array_equal(kp.view(np.uint8), kq.view(np.uint8))
    assert np.array_equal(vp.view(np.uint8), vq.view(np.uint8))
    # the generator packing all L tokens directly
    kidx, vidx = layout.k_chunk_index(wl.P, wl.D, "bf16"), layout.v_chunk_index(wl.P, wl.D, "bf16")
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        k, v, _, _ = configs.seq_tokens(wl.seed, b, L, wl.Hkv, wl.D, "bf16", wl.P)
        pages = wl.block_tables[b, :-(-L // wl.P)]
        kk, vv = kp.copy(), vp.copy()
        layout.pack_sequence(kk, pages, k, wl.P, kidx, "bf16")
        layout.pack_sequence(vv, pages, v, wl.P, vidx, "bf16")
        assert np.array_equal(kk.view(np.uint8), kp.view(np.uint8)), b
        assert np.array_equal(vv.view(np.uint8), vp.view(np.uint8)), b


def test_append_chunk_skips_what_does_not_fit():
    wl = configs.prefill_case("t", 12, **RAGGED)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    lens = wl.seq_lens.copy()
    lens[0] = 3                                     # chunk of 7 > L = 3
    lens[2] = wl.max_pages * wl.P + 1               # beyond the table row
    cu = wl.cu_q
    keep = [1, 3]
    paged.append_chunk(wl.k_new, wl.v_new, "bf16", cu, wl.block_tables, lens, kp, vp, wl.P)
    ref_k, ref_v = wl.k_pool.copy(), wl.v_pool.copy()
    cu2 = np.zeros_like(cu)
    sel = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in keep])
    cu2[1:] = np.cumsum([wl.chunk_lens[b] if b in keep else 0 for b in range(wl.B)])
    paged.append_chunk(wl.k_new[sel], wl.v_new[sel], "bf16", cu2, wl.block_tables, lens, ref_k, ref_v, wl.P)
    assert np.array_equal(kp.view(np.uint8), ref_k.view(np.uint8))
    assert np.array_equal(vp.view(np.uint8), ref_v.view(np.uint8))


def test_chunks_of_one_equal_decode():
    wl = configs.prefill_case("t", 13, ctx_lens=[0, 9, 31, 64, 100], chunk_lens=[1] * 5, Hq=8, Hkv=2, D=32, P=32)
    kp, vp = _full_pools(wl)
    pre = _oracle(wl, kp, vp)
    dec = paged.decode(wl.q, wl.q_dtype, kp, vp, "bf16", wl.block_tables, wl.seq_lens, wl.Hq, wl.P, wl.scale)
    np.testing.assert_allclose(pre, dec, rtol=0, atol=1e-13)


def test_each_row_equals_decode_over_its_prefix():
    wl = configs.prefill_case("t", 14, **RAGGED)
    kp, vp = _full_pools(wl)
    pre = _oracle(wl, kp, vp)
    for b in range(wl.B):
        L, C = int(wl.seq_lens[b]), int(wl.chunk_lens[b])
        for i in range(C):
            r = int(wl.cu_q[b]) + i
            dec = paged.decode(wl.q[r:r + 1], wl.q_dtype, kp, vp, "bf16", wl.block_tables[b:b + 1],
                               np.array([L - C + i + 1], np.int32), wl.Hq, wl.P, wl.scale)
            np.testing.assert_allclose(pre[r], dec[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (16, 2)])
def test_matches_torch_sdpa_on_logical_rows(Hq, Hkv):
    wl = configs.prefill_case("t", 15, ctx_lens=[0, 23, 70], chunk_lens=[19, 5, 26], Hq=Hq, Hkv=Hkv, D=16, P=32)
    kp, vp = _full_pools(wl)
    pre = _oracle(wl, kp, vp)
    qf = _q64(wl)
    G = Hq // Hkv
    for b in range(wl.B):
        L, C = int(wl.seq_lens[b]), int(wl.chunk_lens[b])
        k, v = _logical(wl, b)
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)   # [Hq, L, D]
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(qf[wl.cu_q[b]:wl.cu_q[b + 1]]).permute(1, 0, 2)  # [Hq, C, D]
        mask = torch.arange(L)[None, :] <= (L - C + torch.arange(C))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                               scale=float(wl.scale))
        np.testing.assert_allclose(pre[wl.cu_q[b]:wl.cu_q[b + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_scalar_loop_tiny():
    wl = configs.prefill_case("t", 16, ctx_lens=[2, 0], chunk_lens=[3, 4], Hq=2, Hkv=1, D=4, P=16,
                              kv_dtype="f32")
    kp, vp = _full_pools(wl)
    pre = _oracle(wl, kp, vp)
    q = wl.q.astype(np.float64)
    for b in range(wl.B):
        k, v = _logical(wl, b)
        L, C = int(wl.seq_lens[b]), int(wl.chunk_lens[b])
        for i in range(C):
            p = L - C + i
            for h in range(wl.Hq):
                qr = q[wl.cu_q[b] + i, h]
                s = [float(wl.scale) * sum(qr[d] * k[t, 0, d] for d in range(wl.D)) for t in range(p + 1)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                o = [sum(w[t] * v[t, 0, d] for t in range(p + 1)) / sum(w) for d in range(wl.D)]
                np.testing.assert_allclose(pre[wl.cu_q[b] + i, h], o, rtol=0, atol=1e-14)


def test_identical_keys_give_causal_running_mean():
    wl = configs.prefill_case("t", 17, ctx_lens=[5], chunk_lens=[9], Hq=2, Hkv=1, D=8, P=16, kv_dtype="f32")
    kp, vp = _full_pools(wl)
    koff = layout.k_chunk_index(wl.P, wl.D, "f32")
    pg = wl.block_tables[0, 0]
    kp[pg, 0, koff[:14]] = kp[pg, 0, koff[0]]        # every key equal to token 0's
    pre = _oracle(wl, kp, vp)
    _, v = _logical(wl, 0)
    for i in range(9):
        p = 5 + i
        np.testing.assert_allclose(pre[i, 0], v[:p + 1, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_rows_without_keys_are_zero_and_empty_chunks_skip():
    wl = configs.prefill_case("t", 18, ctx_lens=[0, 4], chunk_lens=[6, 0], Hq=2, Hkv=1, D=8, P=32)
    kp, vp = _full_pools(wl)
    lens = wl.seq_lens.copy()
    lens[0] = 3                                      # chunk of 6 over L = 3: rows 0..2 at p < 0
    pre = paged.prefill(wl.q, "bf16", wl.cu_q, kp, vp, "bf16", wl.block_tables, lens, 2, wl.P, wl.scale)
    assert np.all(pre[:3] == 0)
    dec = paged.decode(wl.q[3:4], "bf16", kp, vp, "bf16", wl.block_tables[:1], np.array([1], np.int32), 2,
                       wl.P, wl.scale)
    np.testing.assert_allclose(pre[3], dec[0], rtol=0, atol=1e-13)
    assert pre.shape[0] == 6


def test_prefill_workload_shape_and_flops():
    wl = configs.prefill_case("t", 19, ctx_lens=[0, 3], chunk_lens=[4, 2], Hq=4, Hkv=2, D=8, P=32)
    # pairs: seq 0 rows see 1..4 keys (10), seq 1 rows see 4, 5 keys (9)
    assert wl.attended() == 19
    assert wl.flops() == 4 * 19 * 4 * 8
    assert wl.T == 6 and list(wl.cu_q) == [0, 4, 6]


# ------------------------------------------------------- fp8 cache prefill ----
# The cache holds e4m3 codes with per-(page, kv head) scales; a stored value is
# code x scale.  Pins: torch SDPA on the rows the generator drew and quantised
# (decoded here by torch's float8_e4m3fn, not through the oracle), chunks of
# one token against the decode oracle, every row against the decode oracle over
# its prefix, and the chunk append against the generator's packing of all L
# tokens.

FP8_CASE = dict(ctx_lens=[0, 23, 70, 130], chunk_lens=[19, 5, 66, 1], D=32, P=64)


def _fp8_full_pools(wl):
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    paged.append_chunk(wl.k_new, wl.v_new, "fp8", wl.cu_q, wl.block_tables, wl.seq_lens, kp, vp, wl.P)
    return kp, vp


def _fp8_oracle(wl, kp, vp, **kw):
    return paged.prefill(wl.q, wl.q_dtype, wl.cu_q, kp, vp, "fp8", wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                         wl.scale, k_scales=wl.k_scales, v_scales=wl.v_scales, **kw)


def _torch_dequant(codes, scales, P):
    """[L, Hkv, D] e4m3 codes times each token's logical-page scale, by torch."""
    x = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.repeat(scales.astype(np.float64), P, axis=0)[:codes.shape[0]])   # [L, Hkv]
    return x * s[:, :, None]


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (16, 2)])
def test_fp8_prefill_matches_torch_sdpa_on_dequantised_rows(Hq, Hkv):
    wl = configs.prefill_case("t", 21, Hq=Hq, Hkv=Hkv, kv_dtype="fp8", **FP8_CASE)
    kp, vp = _fp8_full_pools(wl)
    pre = _fp8_oracle(wl, kp, vp)
    qf = _q64(wl)
    G = Hq // Hkv
    for b in range(wl.B):
        L, C = int(wl.seq_lens[b]), int(wl.chunk_lens[b])
        kc, vc, ks, vs = configs.seq_tokens(wl.seed, b, L, wl.Hkv, wl.D, "fp8", wl.P)
        k = _torch_dequant(kc, ks, wl.P).permute(1, 0, 2).repeat_interleave(G, dim=0)     # [Hq, L, D]
        v = _torch_dequant(vc, vs, wl.P).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(qf[wl.cu_q[b]:wl.cu_q[b + 1]]).permute(1, 0, 2)
        mask = torch.arange(L)[None, :] <= (L - C + torch.arange(C))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, attn_mask=mask, scale=float(wl.scale))
        np.testing.assert_allclose(pre[wl.cu_q[b]:wl.cu_q[b + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_fp8_chunks_of_one_equal_decode():
    wl = configs.prefill_case("t", 22, ctx_lens=[0, 9, 63, 64, 100], chunk_lens=[1] * 5, Hq=8, Hkv=2, D=32, P=64,
                              kv_dtype="fp8")
    kp, vp = _fp8_full_pools(wl)
    pre = _fp8_oracle(wl, kp, vp)
    dec = paged.decode(wl.q, wl.q_dtype, kp, vp, "fp8", wl.block_tables, wl.seq_lens, wl.Hq, wl.P, wl.scale,
                       wl.k_scales, wl.v_scales)
    np.testing.assert_allclose(pre, dec, rtol=0, atol=1e-13)


def test_fp8_each_row_equals_decode_over_its_prefix():
    wl = configs.prefill_case("t", 23, Hq=4, Hkv=2, kv_dtype="fp8", **FP8_CASE)
    kp, vp = _fp8_full_pools(wl)
    pre = _fp8_oracle(wl, kp, vp)
    for b in range(wl.B):
        L, C = int(wl.seq_lens[b]), int(wl.chunk_lens[b])
        for i in range(C):
            r = int(wl.cu_q[b]) + i
            dec = paged.decode(wl.q[r:r + 1], wl.q_dtype, kp, vp, "fp8", wl.block_tables[b:b + 1],
                               np.array([L - C + i + 1], np.int32), wl.Hq, wl.P, wl.scale, wl.k_scales, wl.v_scales)
            np.testing.assert_allclose(pre[r], dec[0], rtol=0, atol=1e-13)


def test_fp8_chunk_append_gives_the_generators_full_packing():
    wl = configs.prefill_case("t", 24, Hq=4, Hkv=2, kv_dtype="fp8", **FP8_CASE)
    kp, vp = _fp8_full_pools(wl)
    kidx, vidx = layout.k_chunk_index(wl.P, wl.D, "fp8"), layout.v_chunk_index(wl.P, wl.D, "fp8")
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        k, v, ks, vs = configs.seq_tokens(wl.seed, b, L, wl.Hkv, wl.D, "fp8", wl.P)
        pages = wl.block_tables[b, :-(-L // wl.P)]
        kk, vv = kp.copy(), vp.copy()
        layout.pack_sequence(kk, pages, k, wl.P, kidx, "fp8")
        layout.pack_sequence(vv, pages, v, wl.P, vidx, "fp8")
        assert np.array_equal(kk, kp) and np.array_equal(vv, vp), b
        assert np.array_equal(wl.k_scales[pages], ks) and np.array_equal(wl.v_scales[pages], vs), b
