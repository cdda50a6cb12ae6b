"""Pins for the format decoders (oracle) and encoders (input generators).

Each side is checked against torch's own bf16 / float8_e4m3fn conversions, a
library routine independent of both, exhaustively over every code where the
code space is small.
"""
import numpy as np
import pytest
import torch

from oracle import paged
from workloads import codec


def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_numpy_exhaustive():
    ref = _torch_e4m3_values()
    got = paged.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_decode_c_exhaustive(c_oracle):
    ref = _torch_e4m3_values()
    got = np.array([c_oracle.lib().orc_e4m3_to_f64(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_named_codes():
    # Fixed points of the OCP e4m3 definition: max normal, min normal, min subnormal, one, NaN.
    t = paged.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x38] == 1.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and t[0x00] == 0.0


def test_bf16_decode_exhaustive(c_oracle):
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = paged.bf16_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    sample = codes[::97]
    got_c = np.array([c_oracle.lib().orc_bf16_to_f64(int(c)) for c in sample])
    ok = ~np.isnan(ref[::97])
    assert np.array_equal(ref[::97][ok], got_c[ok])


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(20_000) * 1e-38).astype(np.float32),          # subnormals
        np.array([np.inf, -np.inf, 0.0, -0.0, 3.4e38, -3.4e38], np.float32),
    ])
    # exact ties: bf16 value + half an ulp, with even and odd bf16 mantissas
    base = rng.integers(0, 0x7F00, 5000).astype(np.uint32) << np.uint32(16)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codec.f32_to_bf16_bits(x)
    assert np.array_equal(ref, got)
    nan = codec.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert nan[0] & 0x7FFF == 0x7FC0


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(1)
    vals = paged.E4M3_TABLE[:0x7F].copy()                      # non-negative finite codes
    mids = (vals[:-1] + vals[1:]) / 2                           # exact ties
    x = np.concatenate([rng.standard_normal(100_000) * 100, rng.standard_normal(20_000) * 1e-2,
                        vals, mids, -mids, [448.0, -448.0, 0.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codec.e4m3_encode(x)
    # torch maps -0.0 and 0.0 to the sign-preserving zero codes, as does the encoder
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    got = codec.e4m3_encode(np.array([449.0, 1e6, -500.0, np.inf], np.float32))
    assert list(got) == [0x7E, 0x7E, 0xFE, 0x7E]
