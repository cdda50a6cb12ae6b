"""Pins of the oracle's fp8 and int8 encoders and of its dynamic-scale appends.

The encoder is checked against torch's float8_e4m3fn conversion (round to
nearest even; torch turns values past 464 into NaN, so the saturation rule is
pinned on its own) and against the generator's independent frexp/rint encoder.
The append is checked against closed forms: the first token of a page sets
scale = amax / 448 and puts its largest element on +-448; appends that fit
leave earlier bytes alone; a scale that exactly doubles halves every earlier
normal value (code - 8); and writing a page token by token, when its first
token holds the page's amax, reproduces the generator's one-shot per-page
quantisation byte for byte.
"""
import numpy as np
import pytest
import torch

from oracle import paged
from workloads import codec, configs, layout

F32 = np.float32


def all_bf16_as_f32():
    return (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def test_encode_matches_torch_on_every_bf16_value_in_range():
    x = all_bf16_as_f32()
    m = np.isfinite(x) & (np.abs(x) <= 464)
    ref = torch.from_numpy(x[m]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(paged.e4m3_encode(x[m]), ref)


def test_encode_ties_go_to_the_even_code_and_neighbours_to_the_nearer():
    pos = paged.E4M3_TABLE[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)          # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    lo_code = np.arange(126)
    want_tie = np.where(lo_code % 2 == 0, lo_code, lo_code + 1)
    for sgn in (1, -1):
        got = paged.e4m3_encode(sgn * mids)
        assert np.array_equal(got & 0x7F, want_tie)
        below = np.nextafter(sgn * mids, F32(0))
        above = np.nextafter(sgn * mids, F32(sgn * np.inf))
        assert np.array_equal(paged.e4m3_encode(below) & 0x7F, lo_code)
        assert np.array_equal(paged.e4m3_encode(above) & 0x7F, lo_code + 1)
        ref = torch.from_numpy(np.concatenate([sgn * mids, below, above])).to(torch.float8_e4m3fn)
        assert np.array_equal(paged.e4m3_encode(np.concatenate([sgn * mids, below, above])),
                              ref.view(torch.uint8).numpy())


def test_encode_saturation_and_specials():
    big = np.array([448, 448.5, 463.9, 464, 465, 1e4, 3e38, np.inf], dtype=np.float32)
    assert np.all(paged.e4m3_encode(big) == 0x7E)
    assert np.all(paged.e4m3_encode(-big) == 0xFE)
    assert paged.e4m3_encode(np.array([0.0], F32))[0] == 0x00
    assert paged.e4m3_encode(np.array([-0.0], F32))[0] == 0x80
    assert paged.e4m3_encode(np.array([np.nan], F32))[0] == 0x7F
    # smallest subnormal 2**-9: half of it is a tie with zero -> 0 (even)
    assert paged.e4m3_encode(np.array([2.0 ** -10], F32))[0] == 0x00
    assert paged.e4m3_encode(np.array([1.5 * 2.0 ** -10], F32))[0] == 0x01


def test_encode_agrees_with_the_generator_encoder_everywhere():
    x = all_bf16_as_f32()
    f = np.isfinite(x)
    assert np.array_equal(paged.e4m3_encode(x[f]), codec.e4m3_encode(x[f]))


def test_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = paged.e4m3_to_f64(codes).astype(np.float32)
    vals[codes == 0x80] = -0.0
    assert np.array_equal(paged.e4m3_encode(vals), codes)


# ---------------------------------------------------------------- append ----

def empty_fp8(NP, Hkv, P, D):
    k = np.full((NP, Hkv, P * D), 0x7F, dtype=np.uint8)          # NaN poison
    return k, k.copy(), np.full((NP, Hkv), np.nan, F32), np.full((NP, Hkv), np.nan, F32)


def one_token(rng, Hkv, D, scale=1.0):
    return (rng.standard_normal((1, Hkv, D)) * scale).astype(F32)


def stored_row(pool, P, D, pg, g, j, which):
    koff, voff = paged._offsets(P, D, "fp8")
    return pool[pg, g, (koff if which == "k" else voff)[j]]


@pytest.mark.parametrize("D,P", [(64, 64), (128, 128)])
def test_first_token_sets_scale_and_hits_448(D, P):
    rng = np.random.default_rng(0)
    Hkv = 2
    kp, vp, ks, vs = empty_fp8(4, Hkv, P, D)
    x, y = one_token(rng, Hkv, D, 3.0), one_token(rng, Hkv, D, 0.01)
    bt = np.array([[2, 3]], dtype=np.int32)
    paged.append_fp8_dynamic(x, y, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
    for new, pool, sc, w in ((x, kp, ks, "k"), (y, vp, vs, "v")):
        for g in range(Hkv):
            a = F32(np.abs(new[0, g]).max())
            assert sc[2, g] == F32(a / F32(448))
            row = stored_row(pool, P, D, 2, g, 0, w)
            i = int(np.argmax(np.abs(new[0, g])))
            assert row[i] in (0x7E, 0xFE)
            back = paged.e4m3_to_f64(row) * float(sc[2, g])
            # within half a step of e4m3 at each value's magnitude (2**-4 relative,
            # or half the subnormal step)
            err = np.abs(back - new[0, g].astype(np.float64))
            bound = np.maximum(np.abs(new[0, g]) * 2.0 ** -4, 2.0 ** -10 * float(sc[2, g])) * (1 + 1e-6)
            assert np.all(err <= bound)
    assert np.all(kp[[0, 1, 3]] == 0x7F) and np.all(np.isnan(ks[[0, 1, 3]]))


def test_an_append_that_fits_leaves_earlier_bytes_and_scale_alone():
    rng = np.random.default_rng(1)
    Hkv, D, P = 1, 128, 64
    kp, vp, ks, vs = empty_fp8(2, Hkv, P, D)
    bt = np.array([[1]], dtype=np.int32)
    first = one_token(rng, Hkv, D, 4.0)
    paged.append_fp8_dynamic(first, first, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
    before_k, before_v, s_k = kp.copy(), vp.copy(), ks.copy()
    second = one_token(rng, Hkv, D, 0.5)
    paged.append_fp8_dynamic(second, second, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
    assert np.array_equal(ks, s_k, equal_nan=True)
    koff, voff = paged._offsets(P, D, "fp8")
    assert np.array_equal(kp[1, 0, koff[0]], before_k[1, 0, koff[0]])
    assert np.array_equal(vp[1, 0, voff[0]], before_v[1, 0, voff[0]])
    assert np.array_equal(kp[1, 0, koff[1]], paged.e4m3_encode(second[0, 0] / ks[1, 0]))


def test_scale_doubling_halves_every_earlier_value():
    """First token amax 56 -> scale 1/8 exactly; second token amax 112 -> 1/4: each
    earlier normal code with exponent field >= 2 drops by 8 (one binade);
    exponent field 1 becomes the subnormal (8 + m) / 2, ties to even."""
    Hkv, D, P = 1, 64, 64
    kp, vp, ks, vs = empty_fp8(1, Hkv, P, D)
    bt = np.array([[0]], dtype=np.int32)
    # every finite positive and negative code times 1/8, then the amax element 56
    codes = np.array([c for c in range(1, 127)] + [c | 0x80 for c in range(1, 127)], dtype=np.uint8)
    rows = (paged.e4m3_to_f64(codes) / 8).astype(F32)
    firsts = []
    for r0 in range(0, len(rows), D - 1):
        chunk = rows[r0:r0 + D - 1]
        firsts.append(np.concatenate([chunk, np.full(D - 1 - len(chunk), 0, F32), [F32(56)]]))
    for tok in firsts:
        kp[:], vp[:], ks[:], vs[:] = empty_fp8(1, Hkv, P, D)
        x = tok.reshape(1, 1, D)
        paged.append_fp8_dynamic(x, x, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
        assert ks[0, 0] == F32(0.125)
        old = stored_row(kp, P, D, 0, 0, 0, "k").copy()
        grow = np.zeros((1, 1, D), F32)
        grow[0, 0, 0] = 112
        paged.append_fp8_dynamic(grow, grow, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
        assert ks[0, 0] == F32(0.25)
        new = stored_row(kp, P, D, 0, 0, 0, "k")
        e = (old >> 3) & 0xF
        m = old & 7
        sign = old & 0x80
        hi = e >= 2
        assert np.array_equal(new[hi], old[hi] - 8)
        one = (e == 1)
        k = 8 + m[one].astype(np.int64)
        # (8+m)/2: exact for even m; for odd m a tie between two integers -> even
        want = np.where(k % 2 == 0, k // 2, np.where((k // 2) % 2 == 0, k // 2, k // 2 + 1))
        assert np.array_equal(new[one] & 0x7F, want.astype(np.uint8))
        assert np.array_equal(new[one] & 0x80, sign[one])
        assert np.array_equal(stored_row(vp, P, D, 0, 0, 0, "v")[hi], old[hi] - 8)


def test_token_by_token_equals_one_shot_when_the_first_token_holds_the_amax():
    rng = np.random.default_rng(2)
    Hkv, D, P = 2, 128, 64
    for L in (1, 17, 64):
        x = rng.standard_normal((L, Hkv, D)).astype(F32)
        y = rng.standard_normal((L, Hkv, D)).astype(F32)
        x[0, :, 5] = 9.0                                          # page amax on token 0
        y[0, :, 77] = -7.5
        kb, ksc = configs.quantize_fp8_pages(x, P)
        vb, vsc = configs.quantize_fp8_pages(y, P)
        kp, vp, ks, vs = empty_fp8(3, Hkv, P, D)
        bt = np.array([[1]], dtype=np.int32)
        for t in range(L):
            paged.append_fp8_dynamic(x[t:t + 1], y[t:t + 1], "f32", bt, np.array([t + 1], np.int32),
                                     kp, vp, ks, vs, P)
        assert ks[1, 0] == ksc[0, 0] and vs[1, 1] == vsc[0, 1]
        kidx, vidx = layout.k_chunk_index(P, D, "fp8"), layout.v_chunk_index(P, D, "fp8")
        for g in range(Hkv):
            assert np.array_equal(kp[1, g, kidx[:L]], kb[:, g])
            assert np.array_equal(vp[1, g, vidx[:L]], vb[:, g])


def test_bf16_input_is_widened_exactly():
    rng = np.random.default_rng(3)
    Hkv, D, P = 1, 64, 64
    xf = rng.standard_normal((1, Hkv, D)).astype(F32)
    bits = codec.f32_to_bf16_bits(xf)
    kp, vp, ks, vs = empty_fp8(1, Hkv, P, D)
    kq, vq, kqs, vqs = empty_fp8(1, Hkv, P, D)
    bt = np.array([[0]], dtype=np.int32)
    paged.append_fp8_dynamic(bits, bits, "bf16", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
    widened = codec.bf16_bits_to_f32(bits)
    paged.append_fp8_dynamic(widened, widened, "f32", bt, np.array([1], np.int32), kq, vq, kqs, vqs, P)
    assert np.array_equal(kp, kq) and np.array_equal(ks, kqs)


def test_skipped_sequences_change_nothing():
    rng = np.random.default_rng(4)
    Hkv, D, P = 1, 64, 64
    kp, vp, ks, vs = empty_fp8(2, Hkv, P, D)
    x = rng.standard_normal((3, Hkv, D)).astype(F32)
    bt = np.array([[0], [5], [-1]], dtype=np.int32)                # ok, bad id, bad id
    lens = np.array([0, 1, 1], np.int32)                            # empty, bad page, bad page
    paged.append_fp8_dynamic(x, x, "f32", bt, lens, kp, vp, ks, vs, P)
    assert np.all(kp == 0x7F) and np.all(np.isnan(ks))
    lens = np.array([65, 0, 0], np.int32)                           # past the table width
    paged.append_fp8_dynamic(x, x, "f32", bt, lens, kp, vp, ks, vs, P)
    assert np.all(kp == 0x7F)


def test_k_and_v_scales_move_independently():
    rng = np.random.default_rng(5)
    Hkv, D, P = 1, 64, 64
    kp, vp, ks, vs = empty_fp8(1, Hkv, P, D)
    bt = np.array([[0]], dtype=np.int32)
    x = rng.standard_normal((1, Hkv, D)).astype(F32)
    paged.append_fp8_dynamic(x, x, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
    k0 = kp.copy()
    ks0 = ks.copy()
    small, big = (x * 0.5).astype(F32), (x * 8).astype(F32)
    paged.append_fp8_dynamic(small, big, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
    assert np.array_equal(ks, ks0, equal_nan=True) and vs[0, 0] > ks[0, 0]
    koff, _ = paged._offsets(P, D, "fp8")
    assert np.array_equal(kp[0, 0, koff[0]], k0[0, 0, koff[0]])


def test_no_clip_threshold_keeps_the_scale_up_to_464():
    """A row whose largest element lands in (448, 464] under the page scale still
    rounds to +-448 without clipping: the scale stays; just above 464 it grows."""
    Hkv, D, P = 1, 64, 64
    bt = np.array([[0]], dtype=np.int32)
    for ratio, grows in ((448.0, False), (456.0, False), (464.0, False), (464.0 * (1 + 2 ** -20), True),
                         (470.0, True)):
        kp, vp, ks, vs = empty_fp8(1, Hkv, P, D)
        first = np.zeros((1, 1, D), F32)
        first[0, 0, 0] = 56.0                                     # scale exactly 1/8
        paged.append_fp8_dynamic(first, first, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
        second = np.zeros((1, 1, D), F32)
        second[0, 0, 1] = F32(ratio / 8)
        paged.append_fp8_dynamic(second, second, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
        assert (ks[0, 0] != F32(0.125)) == grows, ratio
        if not grows:
            assert stored_row(kp, P, D, 0, 0, 1, "k")[1] == 0x7E
            assert stored_row(kp, P, D, 0, 0, 0, "k")[0] == 0x7E       # untouched


def test_repeating_the_row_that_set_the_scale_never_regrows_it():
    """a / fp32(a / 448) can round just above 448; the no-clip rule keeps the scale."""
    rng = np.random.default_rng(9)
    Hkv, D, P = 1, 64, 64
    bt = np.array([[0]], dtype=np.int32)
    for _ in range(50):
        kp, vp, ks, vs = empty_fp8(1, Hkv, P, D)
        x = (rng.standard_normal((1, 1, D)) * 3).astype(F32)
        paged.append_fp8_dynamic(x, x, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
        s1 = ks[0, 0]
        paged.append_fp8_dynamic(x, x, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
        assert ks[0, 0] == s1


# ------------------------------------------------------------------ int8 ----

def test_int8_encode_matches_torch_round_and_clamp():
    x = all_bf16_as_f32()
    m = np.isfinite(x) & (np.abs(x) < 1e4)
    ties = (np.arange(-130, 130) + 0.5).astype(F32)
    y = np.concatenate([x[m], ties, np.nextafter(ties, F32(np.inf)), np.nextafter(ties, F32(-np.inf))])
    ref = torch.clamp(torch.round(torch.from_numpy(y)), -127, 127).to(torch.int8).numpy().view(np.uint8)
    assert np.array_equal(paged.int8_encode(y), ref)
    assert np.array_equal(paged.int8_encode(y), codec.int8_encode(y))


def test_int8_first_token_sets_scale_and_hits_127():
    rng = np.random.default_rng(20)
    Hkv, D, P = 2, 128, 64
    kp, vp, ks, vs = empty_fp8(2, Hkv, P, D)
    x = one_token(rng, Hkv, D, 2.0)
    bt = np.array([[1]], dtype=np.int32)
    paged.append_int8_dynamic(x, x, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
    for g in range(Hkv):
        a = F32(np.abs(x[0, g]).max())
        assert ks[1, g] == F32(a / F32(127))
        row = stored_row(kp, P, D, 1, g, 0, "k").view(np.int8)
        assert abs(int(row[int(np.argmax(np.abs(x[0, g])))])) == 127
        back = row.astype(np.float64) * float(ks[1, g])
        assert np.all(np.abs(back - x[0, g]) <= 0.5 * float(ks[1, g]) * (1 + 1e-6))


def test_int8_token_by_token_equals_one_shot():
    rng = np.random.default_rng(21)
    Hkv, D, P = 2, 64, 64
    L = 2 * P - 3
    x = rng.standard_normal((L, Hkv, D)).astype(F32)
    for p0 in range(0, L, P):
        x[p0, :, 7] = -9.0
    kb, ksc = configs.quantize_int8_pages(x, P)
    kp, vp, ks, vs = empty_fp8(3, Hkv, P, D)
    bt = np.array([[2, 0]], dtype=np.int32)
    for t in range(L):
        paged.append_int8_dynamic(x[t:t + 1], x[t:t + 1], "f32", bt, np.array([t + 1], np.int32),
                                  kp, vp, ks, vs, P)
    kidx = layout.k_chunk_index(P, D, "i8")
    for i, pg in enumerate((2, 0)):
        n = min(P, L - i * P)
        for g in range(Hkv):
            assert np.array_equal(kp[pg, g, kidx[:n]], kb[i * P:i * P + n, g])
        assert np.array_equal(ks[pg], ksc[i])


def test_int8_no_clip_bound_and_doubling():
    """Scale 1/2 from a first token of amax 63.5; a row reaching 127.5 * s keeps it
    (its top element rounds to 128 and clamps to 127, half a step); above, the
    scale grows; doubling the scale halves each code, ties to even."""
    Hkv, D, P = 1, 64, 64
    bt = np.array([[0]], dtype=np.int32)
    for top, grows in ((63.75, False), (63.75 * (1 + 2 ** -20), True)):
        kp, vp, ks, vs = empty_fp8(1, Hkv, P, D)
        first = np.zeros((1, 1, D), F32)
        first[0, 0, :] = (np.arange(D) - 31).astype(F32) / 2           # codes -62 .. 64 ... and 63.5 max
        first[0, 0, 0] = F32(63.5)
        paged.append_int8_dynamic(first, first, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
        assert ks[0, 0] == F32(0.5)
        old = stored_row(kp, P, D, 0, 0, 0, "k").view(np.int8).astype(np.int64)
        second = np.zeros((1, 1, D), F32)
        second[0, 0, 3] = F32(top)
        paged.append_int8_dynamic(second, second, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
        assert (ks[0, 0] != F32(0.5)) == grows
        new = stored_row(kp, P, D, 0, 0, 0, "k").view(np.int8).astype(np.int64)
        if not grows:
            assert np.array_equal(new, old)
            assert stored_row(kp, P, D, 0, 0, 1, "k").view(np.int8)[3] == 127
    kp, vp, ks, vs = empty_fp8(1, Hkv, P, D)
    first = np.zeros((1, 1, D), F32)
    first[0, 0, :] = (np.arange(D) - 32).astype(F32) / 2
    first[0, 0, 0] = F32(63.5)
    paged.append_int8_dynamic(first, first, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
    old = stored_row(kp, P, D, 0, 0, 0, "k").view(np.int8).astype(np.int64)
    second = np.zeros((1, 1, D), F32)
    second[0, 0, 5] = F32(127.0)                                      # scale 1 = twice 1/2
    paged.append_int8_dynamic(second, second, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
    assert ks[0, 0] == F32(1.0)
    new = stored_row(kp, P, D, 0, 0, 0, "k").view(np.int8).astype(np.int64)
    half = old / 2
    want = np.where(half == np.floor(half), half, np.where(np.floor(half) % 2 == 0, np.floor(half),
                                                             np.floor(half) + 1))
    assert np.array_equal(new, want.astype(np.int64))


# ------------------------------------------------------------------ int4 ----

def test_int4_encode_matches_torch_round_and_clamp():
    x = all_bf16_as_f32()
    m = np.isfinite(x) & (np.abs(x) < 100)
    ties = (np.arange(-10, 10) + 0.5).astype(F32)
    y = np.concatenate([x[m], ties, np.nextafter(ties, F32(np.inf)), np.nextafter(ties, F32(-np.inf))])
    ref = torch.clamp(torch.round(torch.from_numpy(y)), -7, 7).to(torch.int8).numpy().view(np.uint8) & 0xF
    assert np.array_equal(paged.int4_encode(y), ref)
    assert np.array_equal(paged.int4_encode(y), codec.int4_encode(y))
    assert np.array_equal(paged.int4_to_f64(np.arange(16)), np.array([0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5,
                                                                        -4, -3, -2, -1], np.float64))


def empty_i4(NP, Hkv, P, D):
    k = layout.empty_pool(NP, Hkv, P, D, "i4")
    return k, k.copy(), np.full((NP, Hkv), np.nan, F32), np.full((NP, Hkv), np.nan, F32)


def i4_row(pool, P, D, pg, g, j, which):
    koff, voff = paged._offsets(P, D, "i4")
    off = (koff if which == "k" else voff)[j]
    return paged.int4_to_f64(paged.read_elems(pool, (pg, g, off), "i4")).astype(np.int64)


def test_int4_first_token_and_token_by_token_equals_one_shot():
    rng = np.random.default_rng(30)
    Hkv, D, P = 2, 128, 128
    L = 2 * P - 9
    x = rng.standard_normal((L, Hkv, D)).astype(F32)
    for p0 in range(0, L, P):
        x[p0, :, 11] = 5.0
    kb, ksc = configs.quantize_int4_pages(x, P)
    kp, vp, ks, vs = empty_i4(3, Hkv, P, D)
    bt = np.array([[1, 2]], dtype=np.int32)
    for t in range(L):
        paged.append_int4_dynamic(x[t:t + 1], x[t:t + 1], "f32", bt, np.array([t + 1], np.int32),
                                  kp, vp, ks, vs, P)
        if t == 0:
            assert ks[1, 0] == F32(F32(5.0) / F32(7))
            assert i4_row(kp, P, D, 1, 0, 0, "k")[11] == 7
    kidx = layout.k_chunk_index(P, D, "i4")
    for i, pg in enumerate((1, 2)):
        n = min(P, L - i * P)
        for g in range(Hkv):
            got = paged.read_elems(kp, (pg, g, kidx[:n]), "i4")
            assert np.array_equal(got, kb[i * P:i * P + n, g])
        assert np.array_equal(ks[pg], ksc[i])


def test_int4_no_clip_bound_and_doubling():
    Hkv, D, P = 1, 128, 128
    bt = np.array([[0]], dtype=np.int32)
    for top, grows in ((7.5 * 0.5, False), (7.5 * 0.5 * (1 + 2 ** -20), True)):
        kp, vp, ks, vs = empty_i4(1, Hkv, P, D)
        first = np.zeros((1, 1, D), F32)
        first[0, 0, :15] = (np.arange(15) - 7).astype(F32) / 2      # codes -7 .. 7 at scale 1/2
        first[0, 0, 20] = F32(3.5)
        paged.append_int4_dynamic(first, first, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
        assert ks[0, 0] == F32(0.5)
        old = i4_row(kp, P, D, 0, 0, 0, "k")
        second = np.zeros((1, 1, D), F32)
        second[0, 0, 3] = F32(top)
        paged.append_int4_dynamic(second, second, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
        assert (ks[0, 0] != F32(0.5)) == grows
        if not grows:
            assert np.array_equal(i4_row(kp, P, D, 0, 0, 0, "k"), old)
            assert i4_row(kp, P, D, 0, 0, 1, "k")[3] == 7
    kp, vp, ks, vs = empty_i4(1, Hkv, P, D)
    first = np.zeros((1, 1, D), F32)
    first[0, 0, :15] = (np.arange(15) - 7).astype(F32) / 2
    first[0, 0, 20] = F32(3.5)
    paged.append_int4_dynamic(first, first, "f32", bt, np.array([1], np.int32), kp, vp, ks, vs, P)
    old = i4_row(kp, P, D, 0, 0, 0, "k")
    second = np.zeros((1, 1, D), F32)
    second[0, 0, 5] = F32(7.0)                                       # scale 1 = twice 1/2
    paged.append_int4_dynamic(second, second, "f32", bt, np.array([2], np.int32), kp, vp, ks, vs, P)
    assert ks[0, 0] == F32(1.0)
    half = old / 2
    want = np.where(half == np.floor(half), half, np.where(np.floor(half) % 2 == 0, np.floor(half),
                                                             np.floor(half) + 1))
    assert np.array_equal(i4_row(kp, P, D, 0, 0, 0, "k"), want.astype(np.int64))
    assert np.array_equal(i4_row(vp, P, D, 0, 0, 0, "v"), want.astype(np.int64))
