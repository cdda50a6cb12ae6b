"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

Appends and gathers must match byte for byte; attention outputs must satisfy
max-abs <= 1e-2 and mean-abs <= 1e-3 (fp32 / bf16 cache) or max-abs <= 3e-2
(fp8 e4m3 cache), element by element, on the same seeded bytes.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_decode_amd as pkv
from oracle import c_oracle, paged
from workloads import codec, configs, layout

from tests._helpers import LOGIT_PROFILES, PARITY_LOG, DeviceWorkload, check_close, dev_tensor, gpu_out, host_bytes, oracle_decode

pytestmark = pytest.mark.gpu


def _decode_vs_oracle(wl, what, partition_tokens=None, out_rounding=False, report=False):
    dw = DeviceWorkload(wl)
    out = dw.decode(partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    ref = oracle_decode(wl)
    return check_close(gpu_out(out), ref, wl.kv_dtype, what,
                       out_rounding=out_rounding and wl.out_dtype == "bf16", report=report)


# ------------------------------------------------------------------ formats ----

def test_fp8_codes_exhaustive_through_decode():
    """Single-token sequences return their value row: all 256 e4m3 codes, scale 1."""
    D, P = 128, 64
    codes = np.arange(256, dtype=np.uint8).reshape(2, 1, 1, D)      # [B, L=1, Hkv=1, D]
    kp = layout.empty_pool(4, 1, P, D, "fp8")
    vp = layout.empty_pool(4, 1, P, D, "fp8")
    bt = np.array([[2], [0]], np.int32)
    for b in range(2):
        layout.pack_sequence(kp, bt[b], np.zeros((1, 1, D), np.uint8), P, layout.k_chunk_index(P, D, "fp8"), "fp8")
        layout.pack_sequence(vp, bt[b], codes[b, :1], P, layout.v_chunk_index(P, D, "fp8"), "fp8")
    ones = np.ones((4, 1), np.float32)
    q = codec.f32_to_bf16_bits(np.ones((2, 1, D), np.float32))
    out = torch.empty((2, 1, D), dtype=torch.float32, device="cuda")
    ws = torch.zeros(pkv.decode_workspace_bytes(2, 1, 1, D), dtype=torch.uint8, device="cuda")
    pkv.paged_attn_decode_fp8(dev_tensor(q), "bf16", dev_tensor(kp), dev_tensor(vp), dev_tensor(ones),
                              dev_tensor(ones), dev_tensor(bt), dev_tensor(np.array([1, 1], np.int32)),
                              1, 1, D, P, 0.1, out, "f32", ws)
    got = out.cpu().numpy().astype(np.float64).reshape(256)
    ref = paged.E4M3_TABLE
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_int8_codes_exhaustive_through_decode():
    """Single-token sequences return their value row: all 256 int8 codes, scale 1
    (-128 included, though the quantiser never writes it)."""
    D, P = 128, 64
    codes = np.arange(256, dtype=np.uint8).reshape(2, 1, 1, D)
    kp = layout.empty_pool(4, 1, P, D, "i8")
    vp = layout.empty_pool(4, 1, P, D, "i8")
    bt = np.array([[1], [3]], np.int32)
    for b in range(2):
        layout.pack_sequence(kp, bt[b], np.zeros((1, 1, D), np.uint8), P, layout.k_chunk_index(P, D, "i8"), "i8")
        layout.pack_sequence(vp, bt[b], codes[b, :1], P, layout.v_chunk_index(P, D, "i8"), "i8")
    ones = np.ones((4, 1), np.float32)
    q = codec.f32_to_bf16_bits(np.ones((2, 1, D), np.float32))
    out = torch.empty((2, 1, D), dtype=torch.float32, device="cuda")
    ws = torch.zeros(pkv.decode_workspace_bytes(2, 1, 1, D), dtype=torch.uint8, device="cuda")
    pkv.paged_attn_decode_int8(dev_tensor(q), "bf16", dev_tensor(kp), dev_tensor(vp), dev_tensor(ones),
                               dev_tensor(ones), dev_tensor(bt), dev_tensor(np.array([1, 1], np.int32)),
                               1, 1, D, P, 0.1, out, "f32", ws)
    got = out.cpu().numpy().astype(np.float64).reshape(256)
    assert np.array_equal(got, np.arange(256, dtype=np.uint8).view(np.int8).astype(np.float64))


def test_int4_codes_exhaustive_through_decode():
    """Single-token sequences return their value row: all 16 int4 codes (each
    dim of the row holds code d % 16), scale 1: exact values -8 .. 7."""
    D, P = 128, 128
    codes = (np.arange(D) % 16).astype(np.uint8).reshape(1, 1, D)
    kp = layout.empty_pool(3, 1, P, D, "i4")
    vp = layout.empty_pool(3, 1, P, D, "i4")
    bt = np.array([[2]], np.int32)
    layout.pack_sequence(kp, bt[0], np.zeros((1, 1, D), np.uint8), P, layout.k_chunk_index(P, D, "i4"), "i4")
    layout.pack_sequence(vp, bt[0], codes, P, layout.v_chunk_index(P, D, "i4"), "i4")
    ones = np.ones((3, 1), np.float32)
    q = codec.f32_to_bf16_bits(np.ones((1, 1, D), np.float32))
    out = torch.empty((1, 1, D), dtype=torch.float32, device="cuda")
    ws = torch.zeros(pkv.decode_workspace_bytes(1, 1, 1, D), dtype=torch.uint8, device="cuda")
    pkv.paged_attn_decode_int4(dev_tensor(q), "bf16", dev_tensor(kp), dev_tensor(vp), dev_tensor(ones),
                               dev_tensor(ones), dev_tensor(bt), dev_tensor(np.array([1], np.int32)),
                               1, 1, D, P, 0.1, out, "f32", ws)
    got = out.cpu().numpy().astype(np.float64).reshape(D)
    assert np.array_equal(got, ((codes.reshape(D).astype(np.int64) ^ 8) - 8).astype(np.float64))


# ------------------------------------------------------------- append/gather ----

APPEND_CASES = [("f32", 16, 64), ("bf16", 32, 128), ("bf16", 64, 128), ("bf16", 128, 64),
                ("fp8", 64, 128), ("fp8", 128, 64), ("i8", 64, 128), ("i4", 128, 128), ("i4", 256, 128)]


@pytest.mark.parametrize("kv_dtype,P,D", APPEND_CASES)
def test_append_bit_exact(kv_dtype, P, D):
    lens0 = [0, 1, P - 2, P - 1, P, 2 * P - 1, 3 * P + 5]
    wl = configs.custom(seed=31, lens=[x + 2 for x in lens0], Hq=8, Hkv=4, D=D, P=P, kv_dtype=kv_dtype)
    # start from the pool holding lens0 tokens: re-pack with the shorter lengths
    ref_k = layout.empty_pool(wl.num_pages, wl.Hkv, P, D, kv_dtype)
    ref_v = layout.empty_pool(wl.num_pages, wl.Hkv, P, D, kv_dtype)
    ki, vi = layout.k_chunk_index(P, D, kv_dtype), layout.v_chunk_index(P, D, kv_dtype)
    for b, n in enumerate(lens0):
        k, v, _, _ = configs.seq_tokens(wl.seed, b, n, wl.Hkv, D, kv_dtype, P)
        pages = wl.block_tables[b, :int(configs.pages_needed(np.array([n]), P)[0])]
        layout.pack_sequence(ref_k, pages, k, P, ki, kv_dtype)
        layout.pack_sequence(ref_v, pages, v, P, vi, kv_dtype)
    dk, dv = dev_tensor(ref_k), dev_tensor(ref_v)
    bt = dev_tensor(wl.block_tables)
    rng = np.random.default_rng(5)
    for step in range(2):
        lens = np.array([x + step + 1 for x in lens0], np.int32)
        lens[0] = 0 if step == 0 else lens[0]        # a sequence that does not append this step
        row_bytes = D * layout.ELEM_BITS[kv_dtype] // 8
        kn = rng.integers(0, 255, (wl.B, wl.Hkv, row_bytes), dtype=np.uint8)
        vn = rng.integers(0, 255, (wl.B, wl.Hkv, row_bytes), dtype=np.uint8)
        kn = kn.view(layout.NP_DTYPE[kv_dtype])
        vn = vn.view(layout.NP_DTYPE[kv_dtype])
        pkv.kv_append(dev_tensor(kn), dev_tensor(vn), kv_dtype, bt, dev_tensor(lens), dk, dv, wl.Hkv, D, P)
        c_oracle.append(kn, vn, kv_dtype, wl.block_tables, lens, ref_k, ref_v, P)
        torch.cuda.synchronize()
        assert np.array_equal(host_bytes(dk), ref_k.view(np.uint8).reshape(-1))
        assert np.array_equal(host_bytes(dv), ref_v.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("kv_dtype,P,D", APPEND_CASES)
def test_gather_bit_exact(kv_dtype, P, D):
    wl = configs.custom(seed=32, lens=[1, P, P + 1, 3 * P - 1, 0], Hq=4, Hkv=2, D=D, P=P, kv_dtype=kv_dtype)
    dw = DeviceWorkload(wl)
    fill = 0x88 if kv_dtype == "i4" else layout.POISON[kv_dtype]
    row = D // 2 if kv_dtype == "i4" else D              # int4 rows are packed
    ko = torch.empty((wl.B, wl.Hkv, wl.max_pages * P, row), dtype=dw.k_pool.dtype, device="cuda")
    vo = torch.empty_like(ko)
    ko.view(torch.uint8).fill_(0xAB)
    vo.view(torch.uint8).fill_(0xAB)
    pkv.debug_gather(dw.k_pool, dw.v_pool, kv_dtype, dw.bt, dw.sl, wl.Hkv, D, P, ko, vo)
    torch.cuda.synchronize()
    rk, rv = c_oracle.gather(wl.k_pool, wl.v_pool, kv_dtype, wl.block_tables, wl.seq_lens, P, fill)
    gk = ko.cpu().view(torch.uint8).numpy().reshape(wl.B, wl.Hkv, wl.max_pages * P, -1)
    gv = vo.cpu().view(torch.uint8).numpy().reshape(wl.B, wl.Hkv, wl.max_pages * P, -1)
    rk8 = rk.view(np.uint8).reshape(gk.shape)
    rv8 = rv.view(np.uint8).reshape(gv.shape)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        assert np.array_equal(gk[b, :, :L], rk8[b, :, :L])
        assert np.array_equal(gv[b, :, :L], rv8[b, :, :L])
        assert (gk[b, :, L:] == 0xAB).all() and (gv[b, :, L:] == 0xAB).all()


# ------------------------------------------------------------ decode: edges ----

def _gappy_lens(n, seed):
    """n lengths of 1..199 tokens, about a third of them zero, with a run of
    empty sequences across sequence 256 and an empty last one: a wave's range
    then passes over empty sequences on its way to the next one with tokens,
    both among the first 256 sequences and past them."""
    r = np.random.default_rng(seed)
    lens = [int(x) for x in r.integers(1, 200, n)]
    for i in range(n):
        if r.random() < 0.3:
            lens[i] = 0
    for i in range(250, 262):
        lens[i] = 0
    lens[-1] = 0
    return lens


EDGE = [
    dict(seed=41, lens=[1, 15, 16, 17, 100], Hq=4, Hkv=4, D=64, P=16, kv_dtype="f32"),
    dict(seed=42, lens=[3, 33, 250], Hq=8, Hkv=4, D=128, P=32, kv_dtype="f32"),
    dict(seed=43, lens=[1, 31, 32, 33, 63, 64, 65, 511, 512, 513], Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16"),
    dict(seed=44, lens=[2, 40, 300], Hq=4, Hkv=4, D=64, P=32, kv_dtype="bf16"),
    dict(seed=45, lens=[7, 129, 1000], Hq=32, Hkv=2, D=128, P=128, kv_dtype="bf16"),
    dict(seed=46, lens=[255, 256, 257, 2000], Hq=16, Hkv=8, D=128, P=256, kv_dtype="bf16"),
    dict(seed=47, lens=[5, 77, 900], Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16", out_dtype="f32"),
    dict(seed=48, lens=[511, 512, 513, 1025, 3000], Hq=64, Hkv=8, D=128, P=128, kv_dtype="bf16",
         partition_tokens=512, q_mult=3.0),
    dict(seed=49, lens=[0, 5, 0, 700, 0], Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16"),
    dict(seed=50, lens=[1, 63, 64, 65, 1000], Hq=32, Hkv=8, D=128, P=64, kv_dtype="fp8"),
    dict(seed=51, lens=[64, 200, 1300], Hq=16, Hkv=4, D=64, P=128, kv_dtype="fp8", out_dtype="f32"),
    dict(seed=52, lens=[20000], Hq=8, Hkv=1, D=128, P=64, kv_dtype="bf16", q_mult=3.0),
    dict(seed=53, lens=[1, 2, 3, 4, 5] * 400, Hq=8, Hkv=2, D=64, P=32, kv_dtype="bf16"),
    dict(seed=54, lens=[100, 4097], Hq=12, Hkv=4, D=128, P=64, kv_dtype="fp8", partition_tokens=128),
    dict(seed=57, lens=[1, 2, 3, 4, 5] * 400, Hq=8, Hkv=2, D=64, P=32, kv_dtype="bf16", out_dtype="f32"),
    dict(seed=58, lens=[1, 63, 64, 65, 1000], Hq=32, Hkv=8, D=128, P=64, kv_dtype="i8"),
    dict(seed=59, lens=[64, 200, 1300], Hq=16, Hkv=4, D=64, P=128, kv_dtype="i8", out_dtype="f32"),
    dict(seed=60, lens=[0, 100, 4097], Hq=12, Hkv=4, D=128, P=64, kv_dtype="i8", partition_tokens=128),
    dict(seed=61, lens=[1, 127, 128, 129, 1000], Hq=32, Hkv=8, D=128, P=128, kv_dtype="i4"),
    dict(seed=62, lens=[64, 300, 1300], Hq=16, Hkv=4, D=128, P=256, kv_dtype="i4", out_dtype="f32"),
    dict(seed=63, lens=[0, 100, 4097], Hq=64, Hkv=8, D=128, P=128, kv_dtype="i4", partition_tokens=512,
         q_mult=3.0),
    dict(seed=64, lens=_gappy_lens(600, 64), Hq=8, Hkv=2, D=64, P=32, kv_dtype="bf16"),
    dict(seed=65, lens=_gappy_lens(400, 65), Hq=32, Hkv=8, D=128, P=64, kv_dtype="fp8", out_dtype="f32"),
    # the largest pages the boundary accepts (1024 tokens) and 512
    dict(seed=90, lens=[1, 1023, 1024, 1025, 3000], Hq=32, Hkv=8, D=128, P=1024, kv_dtype="bf16"),
    dict(seed=91, lens=[100, 512, 513, 2049], Hq=16, Hkv=4, D=64, P=512, kv_dtype="bf16", out_dtype="f32"),
    dict(seed=92, lens=[64, 1024, 1500], Hq=32, Hkv=8, D=128, P=1024, kv_dtype="fp8"),
    dict(seed=93, lens=[128, 1025, 2048], Hq=16, Hkv=4, D=128, P=1024, kv_dtype="i4", out_dtype="f32"),
]


def _random_cases(n=24, seed=90):
    """Seeded draws over the decode's valid shapes: every cache type, G 1..16,
    D 64/128, the page sizes each type allows, ragged and empty lengths (also
    around page and V-block boundaries), range sizes, negative and large
    scales, both output types."""
    r = np.random.default_rng(seed)
    tb = {"f32": 16, "bf16": 32, "fp8": 64, "i8": 64, "i4": 128}
    pages = {"f32": [16, 32, 64], "bf16": [32, 64, 128, 256], "fp8": [64, 128], "i8": [64, 128], "i4": [128, 256]}
    cases = []
    for k in range(n):
        kv = ["f32", "bf16", "bf16", "fp8", "i8", "i4"][k % 6]
        D = 128 if kv == "i4" else int(r.choice([64, 128]))
        P = int(r.choice(pages[kv]))
        Hkv = int(r.choice([1, 2, 4, 8]))
        G = int(r.choice([1, 2, 3, 4, 5, 8, 12, 16]))
        B = int(r.integers(1, 25))
        lens = []
        for _ in range(B):
            u = r.random()
            if u < 0.08:
                lens.append(0)
            elif u < 0.25:
                lens.append(int(r.integers(1, 4)))
            elif u < 0.5:
                lens.append(max(1, int(r.integers(1, 12)) * P + int(r.integers(-1, 2))))
            else:
                lens.append(int(r.integers(1, 3001)))
        spec = dict(seed=1000 + k, lens=lens, Hq=Hkv * G, Hkv=Hkv, D=D, P=P, kv_dtype=kv,
                    partition_tokens=int(r.choice([0, 0, 1, 2, 4, 16])) * tb[kv],
                    scale=float(r.choice([-1.0, 1.0, 1.0, 1.0]) * r.uniform(0.02, 0.25)),
                    q_mult=float(r.choice([1.0, 3.0])))
        if kv != "f32" and r.random() < 0.4:
            spec["out_dtype"] = "f32"
        cases.append(spec)
    return cases


RANDOM_CASES = _random_cases()


@pytest.mark.parametrize("spec", RANDOM_CASES,
                         ids=lambda s: f"{s['kv_dtype']}-D{s['D']}-P{s['P']}-G{s['Hq'] // s['Hkv']}-B{len(s['lens'])}-s{s['seed']}")
def test_decode_random_configs(spec):
    wl = configs.custom(**spec)
    _decode_vs_oracle(wl, f"random seed {spec['seed']}", out_rounding=True)


@pytest.mark.parametrize("spec", EDGE, ids=lambda s: f"{s['kv_dtype']}-D{s['D']}-P{s['P']}-G{s['Hq'] // s['Hkv']}-s{s['seed']}")
def test_decode_edge_cases(spec):
    wl = configs.custom(**spec)
    # very short sequences give |out| up to ~4, where bf16 output rounding alone
    # reaches 1e-2: allow the output format's half-ulp on top of the bound here
    _decode_vs_oracle(wl, f"seed {spec['seed']}", out_rounding=True)


def test_decode_all_empty_sequences():
    wl = configs.custom(seed=55, lens=[0, 0, 0], Hq=8, Hkv=2, D=128, P=64, kv_dtype="bf16")
    dw = DeviceWorkload(wl)
    dw.out.fill_(7.0)
    out = dw.decode()
    torch.cuda.synchronize()
    assert (gpu_out(out) == 0).all()


def test_decode_batch_zero_is_noop():
    wl = configs.custom(seed=56, lens=[3], Hq=8, Hkv=2, D=128, P=64, kv_dtype="bf16")
    dw = DeviceWorkload(wl)
    dw.out.fill_(7.0)
    pkv.lib().pkv_paged_attn_decode  # symbol present
    rc = pkv.lib().pkv_paged_attn_decode(None, 1, None, None, 1, None, 1, None, 0, 1, 8, 2, 128, 64,
                                         0.1, 0, None, 1, None, 0, None)
    assert rc == 0


# ------------------------------------------------------- decode: invariants ----

def test_decode_deterministic_and_page_permutation_invariant():
    wl = configs.custom(seed=61, lens=[300, 1, 2000, 64], Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16")
    dw = DeviceWorkload(wl)
    a = gpu_out(dw.decode()).copy()
    b = gpu_out(dw.decode()).copy()
    assert np.array_equal(a, b)
    perm = np.random.default_rng(3).permutation(wl.num_pages)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(wl.num_pages)
    wl.k_pool, wl.v_pool = wl.k_pool[inv].copy(), wl.v_pool[inv].copy()
    wl.block_tables = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    c = gpu_out(DeviceWorkload(wl).decode())
    assert np.array_equal(a, c)


def test_decode_poison_invariant():
    wl = configs.custom(seed=62, lens=[33, 65, 100], Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16")
    a = gpu_out(DeviceWorkload(wl).decode()).copy()
    # unused pages and the unused tail slots all hold NaN poison already; make it +-inf / junk
    valid = np.zeros(wl.k_pool.shape, bool)
    ki = layout.k_chunk_index(wl.P, wl.D, "bf16")
    vi = layout.v_chunk_index(wl.P, wl.D, "bf16")
    valid_v = np.zeros(wl.v_pool.shape, bool)
    for b in range(wl.B):
        for t in range(int(wl.seq_lens[b])):
            pg = wl.block_tables[b, t // wl.P]
            valid[pg, :, ki[t % wl.P]] = True
            valid_v[pg, :, vi[t % wl.P]] = True
    wl.k_pool = np.where(valid, wl.k_pool, np.uint16(0x7F80))     # +inf
    wl.v_pool = np.where(valid_v, wl.v_pool, np.uint16(0xFF80))   # -inf
    b2 = gpu_out(DeviceWorkload(wl).decode())
    assert np.array_equal(a, b2)


def test_partition_choice_within_tolerance():
    wl = configs.custom(seed=63, lens=[5000, 1234], Hq=64, Hkv=8, D=128, P=128, kv_dtype="bf16", q_mult=3.0)
    ref = oracle_decode(wl)
    dw = DeviceWorkload(wl)
    for pt in (0, 128, 512, 4096):
        out = gpu_out(dw.decode(partition_tokens=pt))
        check_close(out, ref, "bf16", f"partition {pt}")


def test_workspace_reuse_across_calls():
    """One workspace (filled with junk first) serves successive calls of different
    lengths and range sizes; stale descriptors and partials from earlier calls
    must not leak into later ones."""
    big = configs.custom(seed=66, lens=[4096] * 4, Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16")
    dw = DeviceWorkload(big)
    dw.ws.fill_(0x5A)
    for lens, pt in (([3000, 17, 900, 4096], 0), ([100, 0, 2500, 1], 512), ([4096, 4096, 4096, 4096], 0),
                     ([0, 5, 0, 64], 0), ([4096, 1, 4095, 2], 4096), ([3000, 17, 900, 4096], 128)):
        sl = np.array(lens, np.int32)
        out = gpu_out(dw.decode(seq_lens=dev_tensor(sl), partition_tokens=pt))
        check_close(out, oracle_decode(big, seq_lens=sl), "bf16", f"lens {lens} partition {pt}")


def test_concurrent_streams_match_serial():
    """Calls on two streams at once, each with its own workspace, output and
    cache (a fused step on a bf16 cache on one, decodes of an fp8 cache on the
    other), give bit for bit what the same calls give one at a time on one
    stream."""
    wa = configs.custom(seed=81, lens=[1, 700, 2100, 64, 3000, 129], Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16")
    wb = configs.custom(seed=82, lens=[5000, 33, 1200], Hq=16, Hkv=4, D=128, P=64, kv_dtype="fp8")
    rng = np.random.default_rng(83)
    kn = codec.f32_to_bf16_bits(rng.standard_normal((wa.B, wa.Hkv, wa.D)).astype(np.float32))
    vn = codec.f32_to_bf16_bits(rng.standard_normal((wa.B, wa.Hkv, wa.D)).astype(np.float32))

    def run(sa, sb):
        da, db = DeviceWorkload(wa), DeviceWorkload(wb)
        kn_d, vn_d = dev_tensor(kn), dev_tensor(vn)
        torch.cuda.synchronize()
        for _ in range(4):
            with torch.cuda.stream(sa):
                da.step(kn_d, vn_d, da.sl)
            with torch.cuda.stream(sb):
                db.decode()
        torch.cuda.synchronize()
        return gpu_out(da.out), gpu_out(db.out), host_bytes(da.k_pool), host_bytes(da.v_pool)

    cur = torch.cuda.current_stream()
    serial = run(cur, cur)
    both = run(torch.cuda.Stream(), torch.cuda.Stream())
    for name, x, y in zip(("out a", "out b", "k pool a", "v pool a"), serial, both):
        assert np.array_equal(x, y), name
    check_close(serial[1], oracle_decode(wb), "fp8", "fp8 cache on its own stream")


@pytest.mark.parametrize("partition", [0, 512])
def test_softmax_reference_paths(partition):
    """Logit profiles that drive the softmax reference up every tile, now and then,
    once, or only in the last (masked) tile, plus logits near 900: the lazy
    reference must give the same output as the oracle's exact softmax."""
    names = list(LOGIT_PROFILES)
    lens = [700, 2100, 700, 1500, 333, 1024]
    D, P, Hkv, G = 128, 64, 2, 4
    wl = configs.custom(seed=67, lens=lens, Hq=Hkv * G, Hkv=Hkv, D=D, P=P, kv_dtype="bf16", scale=1.0,
                        partition_tokens=partition)
    wl.q = codec.f32_to_bf16_bits(np.ones(wl.q.shape, np.float32))
    kidx = layout.k_chunk_index(P, D, "bf16")
    r = np.random.default_rng(68)
    for b, name in enumerate(names):
        L = lens[b]
        t = np.arange(L)
        c = np.asarray(LOGIT_PROFILES[name](t, L, r), dtype=np.float64)
        k = np.repeat((c / D)[:, None, None], Hkv, axis=1) * np.ones((1, 1, D))
        pages = wl.block_tables[b, :(L + P - 1) // P]
        layout.pack_sequence(wl.k_pool, pages, codec.f32_to_bf16_bits(k.astype(np.float32)), P, kidx, "bf16")
    dw = DeviceWorkload(wl)
    out = gpu_out(dw.decode())
    check_close(out, oracle_decode(wl), "bf16", f"logit profiles, partition {partition}")


def test_bad_page_id_gives_nan_row():
    wl = configs.custom(seed=64, lens=[100, 100], Hq=8, Hkv=2, D=128, P=64, kv_dtype="bf16")
    wl.block_tables[1, 1] = wl.num_pages + 5          # out of range: row must be NaN, nothing faults
    dw = DeviceWorkload(wl)
    out = gpu_out(dw.decode())
    assert np.isnan(out[1]).all()
    ref = oracle_decode(wl, seq_lens=np.array([100, 0], np.int32))
    check_close(out[0:1], ref[0:1], "bf16", "good row beside a bad one")


def test_error_codes_on_device():
    wl = configs.custom(seed=65, lens=[10], Hq=8, Hkv=2, D=128, P=64, kv_dtype="bf16")
    dw = DeviceWorkload(wl)
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_decode(dw.q, "bf16", dw.k_pool, dw.v_pool, "bf16", dw.bt, dw.sl, 8, 2, 128, 64,
                              0.1, dw.out, "bf16", small)
    assert e.value.code == -4
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_decode(dw.q, "bf16", dw.k_pool, dw.v_pool, "fp8", dw.bt, dw.sl, 8, 2, 128, 64,
                              0.1, dw.out, "bf16", dw.ws)
    assert e.value.code == -3


# ------------------------------------------------- fused step (append+decode) ----

STEP_CASES = [
    dict(seed=71, lens=[1, 2, 31, 32, 33, 64, 65, 300], Hq=32, Hkv=8, D=128, P=64, kv_dtype="bf16"),
    dict(seed=72, lens=[1, 15, 16, 17, 50], Hq=8, Hkv=4, D=64, P=16, kv_dtype="f32"),
    dict(seed=73, lens=[1, 63, 64, 65, 129, 700], Hq=32, Hkv=8, D=128, P=64, kv_dtype="fp8"),
    dict(seed=74, lens=[0, 128, 129, 5000], Hq=64, Hkv=8, D=128, P=128, kv_dtype="bf16", partition_tokens=512),
    dict(seed=75, lens=[1, 2, 3, 4, 5] * 100, Hq=8, Hkv=2, D=64, P=32, kv_dtype="bf16", out_dtype="f32"),
    dict(seed=77, lens=[1, 63, 64, 65, 129, 700], Hq=32, Hkv=8, D=128, P=64, kv_dtype="i8"),
    dict(seed=78, lens=[1, 127, 128, 129, 257, 700], Hq=32, Hkv=8, D=128, P=128, kv_dtype="i4"),
    dict(seed=79, lens=_gappy_lens(300, 79), Hq=16, Hkv=4, D=128, P=64, kv_dtype="bf16"),
    dict(seed=80, lens=[1, 1023, 1024, 1025, 2500], Hq=32, Hkv=8, D=128, P=1024, kv_dtype="bf16"),
    dict(seed=83, lens=[1, 1023, 1024, 1025], Hq=32, Hkv=8, D=128, P=1024, kv_dtype="i8"),
]


@pytest.mark.parametrize("spec", STEP_CASES, ids=lambda s: f"{s['kv_dtype']}-P{s['P']}-s{s['seed']}")
def test_step_equals_append_then_decode(spec):
    """decode_step leaves the pools byte-identical to kv_append, and its output
    matches the oracle run on the appended pool."""
    wl = configs.custom(**spec)
    lens_now = wl.seq_lens.copy()
    lens_prev = np.maximum(lens_now - 1, 0)
    # the cache holds lens_prev tokens; token lens_now-1 arrives this step
    ki, vi = layout.k_chunk_index(wl.P, wl.D, wl.kv_dtype), layout.v_chunk_index(wl.P, wl.D, wl.kv_dtype)
    kp = layout.empty_pool(wl.num_pages, wl.Hkv, wl.P, wl.D, wl.kv_dtype)
    vp = layout.empty_pool(wl.num_pages, wl.Hkv, wl.P, wl.D, wl.kv_dtype)
    i4 = wl.kv_dtype == "i4"
    knew = np.zeros((wl.B, wl.Hkv, wl.D // 2 if i4 else wl.D), layout.NP_DTYPE[wl.kv_dtype])
    vnew = np.zeros_like(knew)
    for b in range(wl.B):
        n = int(lens_now[b])
        k, v, _, _ = configs.seq_tokens(wl.seed, b, n, wl.Hkv, wl.D, wl.kv_dtype, wl.P)
        pages = wl.block_tables[b, :int(configs.pages_needed(np.array([n]), wl.P)[0])]
        layout.pack_sequence(kp, pages, k[:int(lens_prev[b])], wl.P, ki, wl.kv_dtype)
        layout.pack_sequence(vp, pages, v[:int(lens_prev[b])], wl.P, vi, wl.kv_dtype)
        if n:
            knew[b] = layout.pack_nibbles(k[n - 1]) if i4 else k[n - 1]
            vnew[b] = layout.pack_nibbles(v[n - 1]) if i4 else v[n - 1]
    wl.k_pool, wl.v_pool = kp, vp
    dw = DeviceWorkload(wl)
    out = gpu_out(dw.step(dev_tensor(knew), dev_tensor(vnew), dw.sl))
    ref_k, ref_v = kp.copy(), vp.copy()
    c_oracle.append(knew, vnew, wl.kv_dtype, wl.block_tables, lens_now, ref_k, ref_v, wl.P)
    assert np.array_equal(host_bytes(dw.k_pool), ref_k.view(np.uint8).reshape(-1))
    assert np.array_equal(host_bytes(dw.v_pool), ref_v.view(np.uint8).reshape(-1))
    ref = oracle_decode(wl, ref_k, ref_v, lens_now)
    check_close(out, ref, wl.kv_dtype, f"step seed {spec['seed']}", out_rounding=wl.out_dtype == "bf16")


def _random_step_cases(n=12, seed=888):
    """The random decode shapes (every cache type, G 1-16, ragged and empty
    lengths, range sizes, both output types) as fused steps."""
    return [dict(spec, seed=5000 + i) for i, spec in enumerate(_random_cases(n=n, seed=seed))]


@pytest.mark.parametrize("spec", _random_step_cases(),
                         ids=lambda s: f"{s['kv_dtype']}-D{s['D']}-P{s['P']}-G{s['Hq'] // s['Hkv']}-s{s['seed']}")
def test_step_random_configs(spec):
    test_step_equals_append_then_decode(spec)


def test_step_bad_page_stores_nothing():
    wl = configs.custom(seed=76, lens=[70, 70], Hq=8, Hkv=2, D=128, P=64, kv_dtype="bf16")
    wl.block_tables[1, 1] = wl.num_pages + 3          # slot 69 of sequence 1 lies on a bad page
    dw = DeviceWorkload(wl)
    before = host_bytes(dw.k_pool).copy()
    kn = dev_tensor(np.full((2, 2, 128), 0x3F80, np.uint16))
    out = gpu_out(dw.step(kn, kn, dw.sl))
    after = host_bytes(dw.k_pool)
    assert np.isnan(out[1]).all() and np.isfinite(out[0]).all()
    # only sequence 0's slot 69 changed
    changed = np.nonzero(before != after)[0]
    pg = wl.block_tables[0, 1]
    lo, hi = pg * wl.Hkv * wl.P * wl.D * 2, (pg + 1) * wl.Hkv * wl.P * wl.D * 2
    assert changed.size > 0 and (changed >= lo).all() and (changed < hi).all()


# --------------------------------------------------------- the five configs ----
# Every output row of every workload is compared with the oracle; each
# comparison's max- and mean-abs error is listed at the end of the run.

def test_config_tiny_fp32():
    mx, mean = _decode_vs_oracle(configs.tiny_fp32(), "tiny_fp32", report=True)
    assert mx < 1e-5                       # fp32 data, fp32 MFMA: far inside the bound


def test_config_llama3_8b_bf16():
    _decode_vs_oracle(configs.llama3_8b_bf16(), "llama3_8b_bf16", report=True)


def test_config_fp8_kv():
    _decode_vs_oracle(configs.fp8_kv(), "fp8_kv", report=True)


def test_config_int8_kv():
    _decode_vs_oracle(configs.int8_kv(), "int8_kv", report=True)


def test_config_int4_kv():
    _decode_vs_oracle(configs.int4_kv(), "int4_kv", report=True)


def _pools_equal(dw, ref_k, ref_v):
    return (np.array_equal(host_bytes(dw.k_pool), ref_k.view(np.uint8).reshape(-1)) and
            np.array_equal(host_bytes(dw.v_pool), ref_v.view(np.uint8).reshape(-1)))


@pytest.mark.timeout(900)
def test_config_inflight_16_steps():
    """Each step: append one token per sequence on the GPU, then decode.  After
    every one of the 16 steps both pools equal the oracle's appends byte for
    byte and all 256 x 32 output rows are compared with the oracle."""
    wl = configs.inflight_bf16()
    dw = DeviceWorkload(wl)
    ref_k, ref_v = wl.k_pool.copy(), wl.v_pool.copy()
    worst = (0.0, 0.0)
    for s, st in enumerate(wl.steps):
        sl = dev_tensor(st.seq_lens)
        dw.append(dev_tensor(st.k_new), dev_tensor(st.v_new), sl)
        c_oracle.append(st.k_new, st.v_new, "bf16", wl.block_tables, st.seq_lens, ref_k, ref_v, wl.P)
        out = gpu_out(dw.decode(seq_lens=sl))
        assert _pools_equal(dw, ref_k, ref_v), f"step {s}: pools differ from the oracle append"
        mx, mean = check_close(out, oracle_decode(wl, ref_k, ref_v, st.seq_lens), "bf16", f"step {s}")
        worst = (max(worst[0], mx), max(worst[1], mean))
    PARITY_LOG.append(("inflight_bf16 append+decode, 16 steps (worst)", "bf16", wl.B * wl.Hq * wl.D * 16) + worst)


@pytest.mark.timeout(900)
def test_config_inflight_16_steps_fused():
    """The same 16 iterations through the fused decode_step entry point: pools
    byte-compared and every output row compared after every step."""
    wl = configs.inflight_bf16()
    dw = DeviceWorkload(wl)
    ref_k, ref_v = wl.k_pool.copy(), wl.v_pool.copy()
    worst = (0.0, 0.0)
    for s, st in enumerate(wl.steps):
        sl = dev_tensor(st.seq_lens)
        out = gpu_out(dw.step(dev_tensor(st.k_new), dev_tensor(st.v_new), sl))
        c_oracle.append(st.k_new, st.v_new, "bf16", wl.block_tables, st.seq_lens, ref_k, ref_v, wl.P)
        assert _pools_equal(dw, ref_k, ref_v), f"fused step {s}: pools differ from the oracle append"
        mx, mean = check_close(out, oracle_decode(wl, ref_k, ref_v, st.seq_lens), "bf16", f"fused step {s}")
        worst = (max(worst[0], mx), max(worst[1], mean))
    PARITY_LOG.append(("inflight_bf16 fused decode_step, 16 steps (worst)", "bf16", wl.B * wl.Hq * wl.D * 16) + worst)


def test_config_long_splitkv_reduced():
    """Same shape family as the long-context workload at B=2, L=16384: full comparison."""
    _decode_vs_oracle(configs.long_splitkv_bf16(B=2, L=16384), "long_splitkv B=2 L=16384")


@pytest.mark.timeout(900)
def test_config_long_splitkv_full():
    """B=8 x 131072 tokens, 512-token partitions (16 per wave, 16 contributors
    merged per (sequence, kv head)): all 512 output rows against the oracle."""
    _decode_vs_oracle(configs.long_splitkv_bf16(), "long_splitkv_bf16", report=True)
