"""Pins for the CPU oracle, independent of the oracle itself.

* brute force: torch's scaled_dot_product_attention (fp64, a library routine)
  on the contiguous logical K/V that the generator drew, decoded by torch;
* closed forms: one token gives its value; identical keys or scale 0 give the
  mean of the values; a dominant key gives its value;
* invariants: outputs lie in the per-dimension value range; permuting physical
  pages while rewriting the page table changes nothing; poison in unused slots
  changes nothing; grouped-query attention equals multi-head attention with
  repeated kv heads;
* split-KV: merging per-partition (output, log-sum-exp) equals the unsplit result;
* the C and numpy oracles agree; the append and gather oracles reproduce the
  generator's pool placement byte for byte.
"""
import math

import numpy as np
import pytest
import torch

from oracle import c_oracle, paged
from workloads import codec, configs, layout


def _torch_widen(x, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float64)
    if dtype == "bf16":
        return torch.from_numpy(np.asarray(x, np.uint16).view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    if dtype == "i8":
        return torch.from_numpy(np.asarray(x, np.uint8).copy()).view(torch.int8).to(torch.float64)
    if dtype == "i4":   # nibble codes: shift the sign bit of the 4-bit code up to bit 7
        return (torch.from_numpy((np.asarray(x, np.uint8) << 4).copy()).view(torch.int8) >> 4).to(torch.float64)
    return torch.from_numpy(np.asarray(x, np.uint8).copy()).view(torch.float8_e4m3fn).to(torch.float64)


def _sdpa_reference(wl):
    """Brute force: regenerate each sequence's logical K/V and run torch SDPA in fp64."""
    B, Hq, Hkv, D, P = wl.B, wl.Hq, wl.Hkv, wl.D, wl.P
    out = np.zeros((B, Hq, D))
    qf = _torch_widen(wl.q, wl.q_dtype).reshape(B, Hq, D)
    for b in range(B):
        L = int(wl.seq_lens[b])
        if L == 0:
            continue
        k, v, ks, vs = configs.seq_tokens(wl.seed, b, L, Hkv, D, wl.kv_dtype, P)
        kt, vt = _torch_widen(k, wl.kv_dtype), _torch_widen(v, wl.kv_dtype)      # [L, Hkv, D]
        if wl.kv_dtype in ("fp8", "i8", "i4"):
            kt = kt * torch.from_numpy(np.repeat(ks, P, 0)[:L]).to(torch.float64)[:, :, None]
            vt = vt * torch.from_numpy(np.repeat(vs, P, 0)[:L]).to(torch.float64)[:, :, None]
        G = Hq // Hkv
        kt = kt.permute(1, 0, 2).repeat_interleave(G, 0)                           # [Hq, L, D]
        vt = vt.permute(1, 0, 2).repeat_interleave(G, 0)
        o = torch.nn.functional.scaled_dot_product_attention(
            qf[b][:, None, :], kt, vt, scale=float(wl.scale))
        out[b] = o[:, 0, :].numpy()
    return out


def _oracles(wl, **kw):
    a = paged.decode(wl.q, wl.q_dtype, wl.k_pool, wl.v_pool, wl.kv_dtype, wl.block_tables,
                     wl.seq_lens, wl.Hq, wl.P, wl.scale, wl.k_scales, wl.v_scales, **kw)
    b = c_oracle.decode(wl.q, wl.q_dtype, wl.k_pool, wl.v_pool, wl.kv_dtype, wl.block_tables,
                        wl.seq_lens, wl.Hq, wl.P, wl.scale, wl.k_scales, wl.v_scales)
    return a, b


SMALL = [
    dict(seed=11, lens=[1, 5, 16, 17, 40], Hq=4, Hkv=2, D=16, P=16, kv_dtype="f32"),
    dict(seed=12, lens=[3, 32, 33, 70], Hq=8, Hkv=2, D=32, P=32, kv_dtype="bf16"),
    dict(seed=13, lens=[1, 63, 64, 65, 130], Hq=4, Hkv=1, D=32, P=64, kv_dtype="fp8"),
    dict(seed=14, lens=[0, 7, 129], Hq=6, Hkv=3, D=16, P=128, kv_dtype="bf16"),
    dict(seed=15, lens=[2, 64, 65, 200], Hq=8, Hkv=2, D=32, P=64, kv_dtype="i8"),
    dict(seed=16, lens=[1, 128, 129, 300], Hq=8, Hkv=2, D=128, P=128, kv_dtype="i4"),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: f"{s['kv_dtype']}-P{s['P']}")
def test_brute_force_sdpa(spec):
    wl = configs.custom(**spec)
    ref = _sdpa_reference(wl)
    a, b = _oracles(wl)
    assert np.abs(a - ref).max() < 1e-12
    assert np.abs(b - ref).max() < 1e-12


def test_brute_force_tiny_fp32_config():
    wl = configs.tiny_fp32()
    ref = _sdpa_reference(wl)
    a, b = _oracles(wl)
    assert np.abs(a - ref).max() < 1e-12 and np.abs(b - ref).max() < 1e-12


def _pool_from_logical(k_log, v_log, P, kv_dtype, seed=0, extra_pages=3):
    """Build pools/tables from explicit logical arrays: list of [L, Hkv, D] per sequence."""
    rng = np.random.default_rng(seed)
    Hkv, D = k_log[0].shape[1], k_log[0].shape[2]
    L = np.array([k.shape[0] for k in k_log], np.int32)
    need = configs.pages_needed(L, P)
    NP = int(need.sum()) + extra_pages
    bt = configs.place_permuted(rng, L, P, NP, int(max(need.max(), 1)))
    kp = layout.empty_pool(NP, Hkv, P, D, kv_dtype)
    vp = layout.empty_pool(NP, Hkv, P, D, kv_dtype)
    ki, vi = layout.k_chunk_index(P, D, kv_dtype), layout.v_chunk_index(P, D, kv_dtype)
    for b in range(len(k_log)):
        layout.pack_sequence(kp, bt[b, :need[b]], k_log[b], P, ki, kv_dtype)
        layout.pack_sequence(vp, bt[b, :need[b]], v_log[b], P, vi, kv_dtype)
    return kp, vp, bt, L


def _run_both(q, kp, vp, bt, L, Hq, P, scale, dt="f32", qdt="f32"):
    a = paged.decode(q, qdt, kp, vp, dt, bt, L, Hq, P, scale)
    b = c_oracle.decode(q, qdt, kp, vp, dt, bt, L, Hq, P, scale)
    return a, b


def test_single_token_gives_value():
    rng = np.random.default_rng(3)
    k = [rng.standard_normal((1, 2, 16)).astype(np.float32) for _ in range(3)]
    v = [rng.standard_normal((1, 2, 16)).astype(np.float32) for _ in range(3)]
    kp, vp, bt, L = _pool_from_logical(k, v, 16, "f32")
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    for out in _run_both(q, kp, vp, bt, L, 4, 16, 0.25):
        for b in range(3):
            for h in range(4):
                assert np.array_equal(out[b, h], v[b][0, h // 2].astype(np.float64))


def test_identical_keys_and_zero_scale_give_mean():
    rng = np.random.default_rng(4)
    Ls = [5, 33, 100]
    row = rng.standard_normal((1, 2, 16)).astype(np.float32)
    k = [np.repeat(row, n, 0) for n in Ls]
    v = [rng.standard_normal((n, 2, 16)).astype(np.float32) for n in Ls]
    kp, vp, bt, L = _pool_from_logical(k, v, 16, "f32")
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    for scale in (0.3, 0.0):
        for out in _run_both(q, kp, vp, bt, L, 4, 16, scale):
            for b in range(3):
                mean = v[b].astype(np.float64).mean(axis=0)      # [Hkv, D]
                assert np.abs(out[b] - np.repeat(mean, 2, 0)).max() < 1e-14
    # scale 0 with arbitrary keys is also the mean
    k2 = [rng.standard_normal((n, 2, 16)).astype(np.float32) for n in Ls]
    kp, vp, bt, L = _pool_from_logical(k2, v, 16, "f32")
    for out in _run_both(q, kp, vp, bt, L, 4, 16, 0.0):
        for b in range(3):
            assert np.abs(out[b] - np.repeat(v[b].astype(np.float64).mean(0), 2, 0)).max() < 1e-14


def test_dominant_key_gives_its_value():
    rng = np.random.default_rng(5)
    n, D = 50, 16
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = (rng.standard_normal((n, 1, D)) * 0.01).astype(np.float32)
    k[17, 0] = q[0, 0] * 10.0          # logit gap ~ 10*|q|^2 >> 40
    v = rng.standard_normal((n, 1, D)).astype(np.float32)
    kp, vp, bt, L = _pool_from_logical([k], [v], 16, "f32")
    for out in _run_both(q, kp, vp, bt, L, 1, 16, 1.0):
        assert np.abs(out[0, 0] - v[17, 0]).max() < 1e-12


@pytest.mark.parametrize("spec", SMALL[:3], ids=lambda s: s["kv_dtype"])
def test_output_within_value_range(spec):
    wl = configs.custom(**spec)
    a, _ = _oracles(wl)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        if L == 0:
            continue
        _, v, _, vs = configs.seq_tokens(wl.seed, b, L, wl.Hkv, wl.D, wl.kv_dtype, wl.P)
        vf = _torch_widen(v, wl.kv_dtype).numpy()
        if wl.kv_dtype in configs.SCALED:
            vf = vf * np.repeat(vs, wl.P, 0)[:L][:, :, None]
        for h in range(wl.Hq):
            g = h // wl.G
            lo, hi = vf[:, g].min(0), vf[:, g].max(0)
            assert np.all(a[b, h] >= lo - 1e-12) and np.all(a[b, h] <= hi + 1e-12)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s["kv_dtype"])
def test_page_permutation_invariance(spec):
    wl = configs.custom(**spec)
    a0, b0 = _oracles(wl)
    perm = np.random.default_rng(99).permutation(wl.num_pages)      # new position of each page
    inv = np.empty_like(perm)
    inv[perm] = np.arange(wl.num_pages)
    kp = wl.k_pool[inv]
    vp = wl.v_pool[inv]
    bt = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    ks = None if wl.k_scales is None else wl.k_scales[inv]
    vs = None if wl.v_scales is None else wl.v_scales[inv]
    a1 = paged.decode(wl.q, wl.q_dtype, kp, vp, wl.kv_dtype, bt, wl.seq_lens, wl.Hq, wl.P, wl.scale, ks, vs)
    b1 = c_oracle.decode(wl.q, wl.q_dtype, kp, vp, wl.kv_dtype, bt, wl.seq_lens, wl.Hq, wl.P, wl.scale, ks, vs)
    assert np.array_equal(a0, a1) and np.array_equal(b0, b1)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s["kv_dtype"])
def test_poison_invariance(spec):
    wl = configs.custom(**spec)
    a0, b0 = _oracles(wl)
    # overwrite every slot that holds no valid token with different garbage
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    if wl.kv_dtype == "i4":               # work on the nibble codes, repack below
        kp, vp = layout.unpack_nibbles(kp), layout.unpack_nibbles(vp)
    valid_k = np.zeros(kp.shape, bool)
    valid_v = np.zeros(vp.shape, bool)
    ki, vi = layout.k_chunk_index(wl.P, wl.D, wl.kv_dtype), layout.v_chunk_index(wl.P, wl.D, wl.kv_dtype)
    for b in range(wl.B):
        for t in range(int(wl.seq_lens[b])):
            pg = wl.block_tables[b, t // wl.P]
            valid_k[pg, :, ki[t % wl.P]] = True
            valid_v[pg, :, vi[t % wl.P]] = True
    junk = np.random.default_rng(7).integers(0, 255, kp.shape).astype(kp.dtype)
    if wl.kv_dtype == "i4":
        junk &= 0xF
    kp[~valid_k] = junk[~valid_k]
    vp[~valid_v] = junk[~valid_v]
    if wl.kv_dtype == "i4":
        kp, vp = layout.pack_nibbles(kp), layout.pack_nibbles(vp)
    a1 = paged.decode(wl.q, wl.q_dtype, kp, vp, wl.kv_dtype, wl.block_tables, wl.seq_lens, wl.Hq, wl.P, wl.scale, wl.k_scales, wl.v_scales)
    b1 = c_oracle.decode(wl.q, wl.q_dtype, kp, vp, wl.kv_dtype, wl.block_tables, wl.seq_lens, wl.Hq, wl.P, wl.scale, wl.k_scales, wl.v_scales)
    assert np.array_equal(a0, a1) and np.array_equal(b0, b1)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(8)
    Ls, Hkv, G, D, P = [9, 40], 2, 4, 32, 32
    k = [codec.f32_to_bf16_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32)) for n in Ls]
    v = [codec.f32_to_bf16_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32)) for n in Ls]
    q = codec.f32_to_bf16_bits(rng.standard_normal((2, Hkv * G, D)).astype(np.float32))
    kp, vp, bt, L = _pool_from_logical(k, v, P, "bf16")
    gqa = _run_both(q, kp, vp, bt, L, Hkv * G, P, 0.2, "bf16", "bf16")
    kr = [np.repeat(x, G, axis=1) for x in k]
    vr = [np.repeat(x, G, axis=1) for x in v]
    kp2, vp2, bt2, L2 = _pool_from_logical(kr, vr, P, "bf16", seed=1)
    mha = _run_both(q, kp2, vp2, bt2, L2, Hkv * G, P, 0.2, "bf16", "bf16")
    # the C oracle runs the same scalar loop per row: bitwise; numpy's blocked matmul
    # may sum in another order when the group shape changes: within 1e-13
    assert np.array_equal(gqa[1], mha[1])
    assert np.abs(gqa[0] - mha[0]).max() < 1e-13


@pytest.mark.parametrize("part", [1, 16, 512])
def test_split_merge_equals_unsplit(part):
    rng = np.random.default_rng(9)
    L, G, D = 1500, 4, 32
    q = rng.standard_normal((G, D)) * 3
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    full = paged.decode_row_group(q, k, v, 1 / math.sqrt(D))
    o, lse = paged.partition_partials(q, k, v, 1 / math.sqrt(D), part)
    assert np.abs(paged.merge_partials(o, lse) - full).max() < 1e-12


@pytest.mark.parametrize("name", ["tiny_fp32", "llama3_8b_bf16", "inflight_bf16", "long_splitkv_bf16",
                                  "fp8_kv", "inflight_fp8", "int8_kv", "inflight_int8", "int4_kv",
                                  "inflight_int4"])
def test_c_and_numpy_oracles_agree(name):
    small = {"llama3_8b_bf16": dict(B=6), "inflight_bf16": dict(B=6, n_steps=2, max_len=3000),
             "long_splitkv_bf16": dict(B=2, L=3000), "fp8_kv": dict(B=4),
             "inflight_fp8": dict(B=6, n_steps=2, max_len=3000), "int8_kv": dict(B=4),
             "inflight_int8": dict(B=6, n_steps=2, max_len=3000), "int4_kv": dict(B=4),
             "inflight_int4": dict(B=6, n_steps=2, max_len=3000)}
    wl = configs.CONFIGS[name](**small.get(name, {}))
    a, b = _oracles(wl)
    assert np.abs(a - b).max() < 1e-12


def _row(x, kv_dtype):
    """A token row in the ABI's stored form (int4: packed two per byte)."""
    return layout.pack_nibbles(x) if kv_dtype == "i4" else x


@pytest.mark.parametrize("kv_dtype,P", [("f32", 16), ("bf16", 32), ("bf16", 64), ("fp8", 64), ("fp8", 128),
                                        ("i8", 64), ("i4", 128), ("i4", 256)])
def test_append_reproduces_packed_pool(kv_dtype, P):
    """Appending tokens one at a time (both oracles) rebuilds the generator's pool bytes."""
    wl = configs.custom(seed=21, lens=[1, P - 1, P, P + 1, 2 * P + 3], Hq=4, Hkv=2, D=32, P=P,
                        kv_dtype=kv_dtype)
    for impl in (paged.append, c_oracle.append):
        kp = layout.empty_pool(wl.num_pages, wl.Hkv, P, wl.D, kv_dtype)
        vp = layout.empty_pool(wl.num_pages, wl.Hkv, P, wl.D, kv_dtype)
        toks = [configs.seq_tokens(wl.seed, b, int(wl.seq_lens[b]), wl.Hkv, wl.D, kv_dtype, P)
                for b in range(wl.B)]
        for t in range(int(wl.seq_lens.max())):
            lens = np.where(wl.seq_lens > t, t + 1, 0).astype(np.int32)   # sequences still growing
            rl = wl.D // 2 if kv_dtype == "i4" else wl.D
            kn = np.zeros((wl.B, wl.Hkv, rl), kp.dtype)
            vn = np.zeros((wl.B, wl.Hkv, rl), kp.dtype)
            for b in range(wl.B):
                if lens[b]:
                    kn[b], vn[b] = _row(toks[b][0][t], kv_dtype), _row(toks[b][1][t], kv_dtype)
            impl(kn, vn, kv_dtype, wl.block_tables, lens, kp, vp, P)
        assert np.array_equal(kp.view(np.uint8), wl.k_pool.view(np.uint8))
        assert np.array_equal(vp.view(np.uint8), wl.v_pool.view(np.uint8))


@pytest.mark.parametrize("kv_dtype,P", [("f32", 16), ("bf16", 64), ("fp8", 64), ("i8", 64), ("i4", 128)])
def test_gather_returns_logical_tokens(kv_dtype, P):
    wl = configs.custom(seed=22, lens=[2, P, 3 * P - 1], Hq=2, Hkv=2, D=32, P=P, kv_dtype=kv_dtype)
    ko, vo = c_oracle.gather(wl.k_pool, wl.v_pool, kv_dtype, wl.block_tables, wl.seq_lens, P, 0)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        k, v, _, _ = configs.seq_tokens(wl.seed, b, L, wl.Hkv, wl.D, kv_dtype, P)
        k, v = _row(k, kv_dtype), _row(v, kv_dtype)
        assert np.array_equal(ko[b, :, :L].view(np.uint8), k.transpose(1, 0, 2).copy().view(np.uint8))
        assert np.array_equal(vo[b, :, :L].view(np.uint8), v.transpose(1, 0, 2).copy().view(np.uint8))
        kn, vn, _ = paged.gather(wl.k_pool, wl.v_pool, kv_dtype, wl.block_tables, wl.seq_lens, P, b)
        assert np.array_equal(_row(kn, kv_dtype).view(np.uint8), ko[b, :, :L].view(np.uint8))
        assert np.array_equal(_row(vn, kv_dtype).view(np.uint8), vo[b, :, :L].view(np.uint8))


def test_layout_offsets_are_permutations():
    for dt, P in [("f32", 16), ("bf16", 32), ("bf16", 128), ("fp8", 64), ("i4", 128)]:
        for D in (64, 128):
            for idx in (layout.k_chunk_index(P, D, dt), layout.v_chunk_index(P, D, dt)):
                assert np.array_equal(np.sort(idx.ravel()), np.arange(P * D))
