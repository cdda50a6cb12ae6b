"""Host-side checks of the C ABI: the library loads, exports every symbol that
include/pkv.h declares, and rejects bad arguments before touching a device."""
import os
import re

import pytest

import paged_kv_attention_decode_amd as pkv
from paged_kv_attention_decode_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")
# Fake non-NULL "device pointers": 16-byte aligned host values that validation
# must reject arguments around without ever dereferencing.
F = 0x1000


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    syms = declared_symbols()
    for name in ("pkv_kv_append", "pkv_paged_attn_decode", "pkv_paged_attn_decode_fp8",
                 "pkv_decode_workspace_bytes", "pkv_debug_gather", "pkv_debug_read_probe"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    L = pkv.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert set(declared_symbols()) == set(_native.SIGNATURES)


def test_version_and_strerror():
    assert pkv.version() == 100
    L = pkv.lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.pkv_strerror(code)
    assert L.pkv_strerror(-99) == b"unknown error code"


def _append(**over):
    a = dict(k=F, v=F, dt=1, bt=F, mp=4, sl=F, b=2, kp=F, vp=F, np_=8, hkv=2, d=128, p=64)
    a.update(over)
    L = pkv.lib()
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return L.pkv_kv_append(vp(a["k"]), vp(a["v"]), a["dt"], vp(a["bt"]), a["mp"], vp(a["sl"]), a["b"],
                           vp(a["kp"]), vp(a["vp"]), a["np_"], a["hkv"], a["d"], a["p"], None)


@pytest.mark.parametrize("over,code", [
    (dict(k=0), -1), (dict(bt=0), -1), (dict(d=96), -2), (dict(p=48), -2), (dict(p=2048), -2),
    (dict(dt=7), -3), (dict(hkv=0), -2), (dict(mp=0), -2), (dict(b=-1), -2),
    (dict(dt=2, p=32), -2), (dict(dt=0, p=16, k=0), -1),
    (dict(k=F + 8), -6), (dict(vp=F + 2), -6),
])
def test_append_rejects_bad_arguments(over, code):
    # Pointers are fake non-NULL host values: validation must fail before any use.
    assert _append(**over) == code
    assert pkv.lib().pkv_last_error()


def test_batch_zero_is_a_noop_without_device():
    assert _append(b=0, k=0, v=0) == 0


def _decode(fn="pkv_paged_attn_decode", **over):
    a = dict(q=F, qdt=1, kp=F, vp=F, kvdt=1, bt=F, mp=4, sl=F, b=2, np_=8, hq=8, hkv=2, d=128, p=64,
             scale=0.1, pt=0, out=F, odt=1, ws=F, wsb=1 << 30)
    a.update(over)
    L = pkv.lib()
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    if fn == "pkv_paged_attn_decode":
        return L.pkv_paged_attn_decode(vp(a["q"]), a["qdt"], vp(a["kp"]), vp(a["vp"]), a["kvdt"], vp(a["bt"]),
                                       a["mp"], vp(a["sl"]), a["b"], a["np_"], a["hq"], a["hkv"], a["d"], a["p"],
                                       a["scale"], a["pt"], vp(a["out"]), a["odt"], vp(a["ws"]), a["wsb"], None)
    return L.pkv_paged_attn_decode_fp8(vp(a["q"]), a["qdt"], vp(a["kp"]), vp(a["vp"]), vp(a.get("ks", 1)),
                                       vp(a.get("vs", 1)), vp(a["bt"]), a["mp"], vp(a["sl"]), a["b"], a["np_"],
                                       a["hq"], a["hkv"], a["d"], a["p"], a["scale"], a["pt"], vp(a["out"]),
                                       a["odt"], vp(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=0), -1), (dict(out=0), -1), (dict(ws=0), -1), (dict(kvdt=2), -3),
    (dict(qdt=0), -3), (dict(kvdt=0, qdt=0, p=16, odt=1), -3), (dict(hq=9), -2), (dict(hq=64, hkv=2), -2),
    (dict(d=80), -2), (dict(p=40), -2), (dict(pt=48), -2), (dict(pt=-32), -2), (dict(np_=0), -2),
    (dict(q=F + 4), -6), (dict(kp=F + 8), -6), (dict(out=F + 2), -6), (dict(ws=F + 1), -6),
])
def test_decode_rejects_bad_arguments(over, code):
    assert _decode(**over) == code


@pytest.mark.parametrize("over,code", [(dict(ks=0), -1), (dict(vs=0), -1), (dict(qdt=0), -3),
                                       (dict(p=32), -2), (dict(pt=96), -2)])
def test_decode_fp8_rejects_bad_arguments(over, code):
    assert _decode("pkv_paged_attn_decode_fp8", **over) == code


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(_native.NativeLibraryMissing):
        _native.lib()


def _step(**over):
    a = dict(q=F, qdt=1, kn=F, vn=F, kp=F, vp=F, kvdt=1, ks=0, vs=0, bt=F, mp=4, sl=F, b=2, np_=8, hq=8,
             hkv=2, d=128, p=64, scale=0.1, pt=0, out=F, odt=1, ws=F, wsb=1 << 30)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_decode_step(vp(a["q"]), a["qdt"], vp(a["kn"]), vp(a["vn"]), vp(a["kp"]), vp(a["vp"]),
                                     a["kvdt"], vp(a["ks"]), vp(a["vs"]), vp(a["bt"]), a["mp"], vp(a["sl"]),
                                     a["b"], a["np_"], a["hq"], a["hkv"], a["d"], a["p"], a["scale"], a["pt"],
                                     vp(a["out"]), a["odt"], vp(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("over,code", [(dict(kn=0), -1), (dict(vn=0), -1), (dict(kvdt=2, p=64), -1),
                                       (dict(kvdt=2, p=32, ks=1, vs=1), -2), (dict(d=32), -2),
                                       (dict(qdt=0), -3), (dict(hq=7), -2), (dict(kn=F + 8), -6),
                                       (dict(vn=F + 4), -6)])
def test_step_rejects_bad_arguments(over, code):
    assert _step(**over) == code


def _append_fp8(**over):
    a = dict(k=F, v=F, ndt=1, bt=F, mp=4, sl=F, b=2, kp=F, vp=F, ks=F, vs=F, np_=8, hkv=2, d=128, p=64)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_kv_append_fp8(vp(a["k"]), vp(a["v"]), a["ndt"], vp(a["bt"]), a["mp"], vp(a["sl"]),
                                       a["b"], vp(a["kp"]), vp(a["vp"]), vp(a["ks"]), vp(a["vs"]), a["np_"],
                                       a["hkv"], a["d"], a["p"], None)


@pytest.mark.parametrize("over,code", [
    (dict(ks=0), -1), (dict(vs=0), -1), (dict(k=0), -1), (dict(ndt=2), -3), (dict(ndt=7), -3),
    (dict(p=32), -2), (dict(d=96), -2), (dict(hkv=0), -2), (dict(kp=F + 4), -6), (dict(v=F + 2), -6),
])
def test_append_fp8_rejects_bad_arguments(over, code):
    assert _append_fp8(**over) == code


def test_append_fp8_batch_zero_is_a_noop():
    assert _append_fp8(b=0, k=0, v=0, ks=0, vs=0) == 0


def _append_chunk(**over):
    a = dict(k=F, v=F, dt=1, cu=F, tot=100, bt=F, mp=4, sl=F, b=2, kp=F, vp=F, np_=8, hkv=2, d=128, p=64)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_kv_append_chunk(vp(a["k"]), vp(a["v"]), a["dt"], vp(a["cu"]), a["tot"], vp(a["bt"]),
                                         a["mp"], vp(a["sl"]), a["b"], vp(a["kp"]), vp(a["vp"]), a["np_"],
                                         a["hkv"], a["d"], a["p"], None)


@pytest.mark.parametrize("over,code", [
    (dict(cu=0), -1), (dict(k=0), -1), (dict(tot=-1), -2), (dict(d=96), -2), (dict(p=48), -2),
    (dict(dt=9), -3), (dict(k=F + 4), -6),
])
def test_append_chunk_rejects_bad_arguments(over, code):
    assert _append_chunk(**over) == code
    assert pkv.lib().pkv_last_error()


def test_append_chunk_empty_is_a_noop():
    assert _append_chunk(b=0, k=0, v=0, cu=0) == 0
    assert _append_chunk(tot=0, k=0, v=0) == 0


def _prefill(**over):
    a = dict(q=F, qdt=1, cu=F, tot=100, kp=F, vp=F, kvdt=1, bt=F, mp=4, sl=F, b=2, np_=8, hq=8, hkv=2, d=128,
             p=64, scale=0.1, out=F, odt=1)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_paged_prefill(vp(a["q"]), a["qdt"], vp(a["cu"]), a["tot"], vp(a["kp"]), vp(a["vp"]),
                                       a["kvdt"], vp(a["bt"]), a["mp"], vp(a["sl"]), a["b"], a["np_"], a["hq"],
                                       a["hkv"], a["d"], a["p"], a["scale"], vp(a["out"]), a["odt"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=0), -1), (dict(cu=0), -1), (dict(out=0), -1), (dict(tot=-1), -2), (dict(hq=7), -2),
    (dict(hq=1024, hkv=2), -2), (dict(d=96), -2), (dict(kvdt=0, p=16), -3), (dict(kvdt=2), -3),
    (dict(qdt=0), -3), (dict(odt=2), -3), (dict(q=F + 2), -6), (dict(out=F + 8), -6),
])
def test_prefill_rejects_bad_arguments(over, code):
    assert _prefill(**over) == code
    assert pkv.lib().pkv_last_error()


def test_prefill_empty_is_a_noop():
    assert _prefill(b=0, q=0, out=0, cu=0) == 0
    assert _prefill(tot=0, q=0, out=0) == 0


def _alloc(**over):
    a = dict(sl=F, b=2, bt=F, mp=4, p=64, fp=F, fc=F, cap=16)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_alloc_pages(vp(a["sl"]), a["b"], vp(a["bt"]), a["mp"], a["p"], vp(a["fp"]), vp(a["fc"]),
                                     a["cap"], None)


@pytest.mark.parametrize("over,code", [
    (dict(fp=0), -1), (dict(fc=0), -1), (dict(sl=0), -1), (dict(b=-1), -2), (dict(mp=0), -2), (dict(p=0), -2),
    (dict(cap=0), -2),
])
def test_alloc_pages_rejects_bad_arguments(over, code):
    assert _alloc(**over) == code


def test_release_pages_rejects_bad_arguments():
    L = pkv.lib()
    assert L.pkv_release_pages(None, F, 2, F, 4, 64, 8, F, F, 16, None) == -1
    assert L.pkv_release_pages(F, F, 2, F, 4, 64, 0, F, F, 16, None) == -2
    assert _alloc(b=0, sl=0, bt=0) == 0


def test_read_probe_argument_errors():
    """Rejected before any GPU call: NULL pointers, a size not a multiple of 16,
    a misaligned buffer; zero bytes is a no-op."""
    L = pkv.lib()
    assert L.pkv_debug_read_probe(None, 16, F, None) == -1
    assert L.pkv_debug_read_probe(F, 16, None, None) == -1
    assert L.pkv_debug_read_probe(F, 17, F, None) == -2
    assert L.pkv_debug_read_probe(F + 4, 16, F, None) == -6
    assert L.pkv_debug_read_probe(None, 0, None, None) == 0


def _step_noalloc(**over):
    a = dict(q=F, qdt=1, kn=F, vn=F, kp=F, vp=F, kvdt=1, ks=0, vs=0, bt=F, mp=4, sl=F, b=2, np_=8, hq=8,
             hkv=2, d=128, p=64, scale=0.1, pt=0, out=F, odt=1)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_decode_step_noalloc(vp(a["q"]), a["qdt"], vp(a["kn"]), vp(a["vn"]), vp(a["kp"]),
                                             vp(a["vp"]), a["kvdt"], vp(a["ks"]), vp(a["vs"]), vp(a["bt"]),
                                             a["mp"], vp(a["sl"]), a["b"], a["np_"], a["hq"], a["hkv"], a["d"],
                                             a["p"], a["scale"], a["pt"], vp(a["out"]), a["odt"], None)


@pytest.mark.parametrize("over,code", [(dict(kn=0), -1), (dict(q=0), -1), (dict(kvdt=2, p=64), -1),
                                       (dict(kvdt=2, p=32, ks=1, vs=1), -2), (dict(d=32), -2),
                                       (dict(qdt=0), -3), (dict(hq=7), -2), (dict(kn=F + 8), -6),
                                       (dict(out=F + 4), -6), (dict(odt=7), -3)])
def test_step_noalloc_rejects_bad_arguments(over, code):
    """The allocation-free step validates like decode_step, before it looks up
    its static scratch (so no device is needed to reach these errors)."""
    assert _step_noalloc(**over) == code


def test_step_noalloc_batch_zero_is_a_noop_without_device():
    assert _step_noalloc(b=0, q=0, kn=0, vn=0, kp=0, vp=0, bt=0, sl=0, out=0) == 0


def _step_quant(**over):
    a = dict(q=F, qdt=1, kn=F, vn=F, ndt=1, kp=F, vp=F, kvdt=2, ks=F, vs=F, bt=F, mp=4, sl=F, b=2, np_=8, hq=8,
             hkv=2, d=128, p=64, scale=0.1, pt=0, out=F, odt=1, ws=F, wsb=1 << 30)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_decode_step_quant(vp(a["q"]), a["qdt"], vp(a["kn"]), vp(a["vn"]), a["ndt"], vp(a["kp"]),
                                           vp(a["vp"]), a["kvdt"], vp(a["ks"]), vp(a["vs"]), vp(a["bt"]), a["mp"],
                                           vp(a["sl"]), a["b"], a["np_"], a["hq"], a["hkv"], a["d"], a["p"],
                                           a["scale"], a["pt"], vp(a["out"]), a["odt"], vp(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("over,code", [(dict(kvdt=1), -3), (dict(kvdt=0), -3), (dict(ndt=2), -3), (dict(ndt=7), -3),
                                       (dict(kn=0), -1), (dict(ks=0), -1), (dict(vs=0), -1), (dict(p=32), -2),
                                       (dict(kvdt=4, p=64), -2), (dict(kvdt=4, p=128, d=64), -2),
                                       (dict(kn=F + 8), -6), (dict(hq=7), -2), (dict(qdt=0), -3)])
def test_step_quant_rejects_bad_arguments(over, code):
    assert _step_quant(**over) == code


def test_step_quant_batch_zero_is_a_noop_without_device():
    assert _step_quant(b=0, q=0, kn=0, vn=0, kp=0, vp=0, ks=0, vs=0, bt=0, sl=0, out=0, ws=0) == 0


def _prefill_fp8(**over):
    a = dict(q=F, qdt=1, cu=F, tot=100, kp=F, vp=F, ks=F, vs=F, bt=F, mp=4, sl=F, b=2, np_=8, hq=8, hkv=2, d=128,
             p=64, scale=0.1, out=F, odt=1)
    a.update(over)
    vp = lambda x: None if x in (0, None) else x  # noqa: E731
    return pkv.lib().pkv_paged_prefill_fp8(vp(a["q"]), a["qdt"], vp(a["cu"]), a["tot"], vp(a["kp"]), vp(a["vp"]),
                                           vp(a["ks"]), vp(a["vs"]), vp(a["bt"]), a["mp"], vp(a["sl"]), a["b"],
                                           a["np_"], a["hq"], a["hkv"], a["d"], a["p"], a["scale"], vp(a["out"]),
                                           a["odt"], None)


@pytest.mark.parametrize("over,code", [
    (dict(ks=0), -1), (dict(vs=0), -1), (dict(q=0), -1), (dict(tot=-1), -2), (dict(p=32), -2), (dict(d=96), -2),
    (dict(hq=7), -2), (dict(qdt=0), -3), (dict(odt=2), -3), (dict(kp=F + 4), -6),
])
def test_prefill_fp8_rejects_bad_arguments(over, code):
    assert _prefill_fp8(**over) == code
    assert pkv.lib().pkv_last_error()


def test_prefill_fp8_empty_is_a_noop():
    assert _prefill_fp8(b=0, q=0, cu=0, kp=0, vp=0, ks=0, vs=0, bt=0, sl=0, out=0) == 0
    assert _prefill_fp8(tot=0, q=0, out=0) == 0


def test_prefill_rejects_an_fp8_cache_and_names_the_fp8_entry():
    assert _prefill(kvdt=2) == -3
    assert b"pkv_paged_prefill_fp8" in pkv.lib().pkv_last_error()
