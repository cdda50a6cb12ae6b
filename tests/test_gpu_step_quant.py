"""GPU parity of the quantising decode step (pkv_decode_step_quant): bf16 /
fp32 rows quantised on write into an fp8, int8 or int4 cache with dynamic
per-(page, kv head) scales, fused into the decode of that cache.

After every step the pools and the scales must equal the oracle's quantising
append (oracle.paged.append_dynamic) bit for bit, and the output must match
the oracle's decode of the appended cache (fp8: max-abs <= 3e-2; int8, int4:
the bf16 bounds).  Sequences whose pages run past the table or onto a bad
page id must give NaN rows and leave the pools alone.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_decode_amd as pkv
from oracle import c_oracle, paged
from workloads import configs
from tests._helpers import PARITY_LOG, DeviceWorkload, check_close, dev_tensor, gpu_out, host_bytes
from tests.test_gpu_quant import _compare, _rows, empty_pools

pytestmark = pytest.mark.gpu

F32 = np.float32
CASES = [  # (fmt, D, P, new_dtype, G, steps)
    ("fp8", 128, 128, "bf16", 4, 140), ("fp8", 64, 64, "f32", 2, 75), ("fp8", 128, 64, "bf16", 8, 80),
    ("i8", 128, 128, "bf16", 4, 140), ("i8", 64, 128, "f32", 1, 135), ("i8", 128, 64, "bf16", 16, 70),
    ("i4", 128, 128, "bf16", 4, 140), ("i4", 128, 256, "f32", 3, 270),
    ("fp8", 128, 256, "bf16", 4, 270),
]


def _step(fmt, q, x, y, new_dtype, kp_d, vp_d, ks_d, vs_d, bt_d, sl_d, Hq, Hkv, D, P, scale, out, ws, pt=0):
    pkv.decode_step_quant(q, "bf16", x, y, new_dtype, kp_d, vp_d, fmt, ks_d, vs_d, bt_d, sl_d, Hq, Hkv, D, P,
                          scale, out, "f32", ws, partition_tokens=pt)


def _good_rows(bt, lens, P, NP):
    """Sequences whose every page id is valid (decodable by the oracle)."""
    MP = bt.shape[1]
    ok = []
    for b, L in enumerate(lens):
        if L <= 0 or L > MP * P:
            continue
        n = -(-int(L) // P)
        if np.all((bt[b, :n] >= 0) & (bt[b, :n] < NP)):
            ok.append(b)
    return ok


@pytest.mark.parametrize("fmt,D,P,new_dtype,G,steps", CASES, ids=lambda v: str(v))
def test_step_quant_every_step(fmt, D, P, new_dtype, G, steps):
    rng = np.random.default_rng(300 + D + P + G)
    B, Hkv, MP = 7, 2, 2
    Hq = G * Hkv
    NP = B * MP + 3
    perm = rng.permutation(NP).astype(np.int32)
    bt = perm[:B * MP].reshape(B, MP).copy()
    bt[5, 1] = -1                       # sequence 5 runs onto a missing page after P tokens
    bt[6, 1] = NP + 7                   # sequence 6 onto a page id out of range
    start = np.array([0, 0, 3, 10, P - 2, 1, 2])    # step at which each sequence starts
    kp, vp, ks, vs = empty_pools(fmt, NP, Hkv, P, D)
    kp_d, vp_d, ks_d, vs_d = (dev_tensor(a) for a in (kp, vp, ks, vs))
    bt_d = dev_tensor(bt)
    from workloads import codec
    qf = rng.standard_normal((B, Hq, D)).astype(F32)
    q = codec.f32_to_bf16_bits(qf)
    q_d = dev_tensor(q)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = torch.zeros(pkv.decode_workspace_bytes(B, Hq, Hkv, D), dtype=torch.uint8, device="cuda")
    scale = F32(1.0 / np.sqrt(D))
    worst = (0.0, 0.0)
    holed = set()                        # sequences whose skipped append left an unwritten slot
    vmax = np.zeros(B)                   # largest |v| appended to each sequence
    for s in range(steps):
        lens = np.where(s >= start, s - start + 1, 0).astype(np.int32)
        if s % 17 == 5:
            if lens[4] >= 1:
                holed.add(4)
            lens[4] = MP * P + 1         # a call past the end of the table: skipped, NaN row
        x, y = _rows(rng, B, Hkv, D, new_dtype), _rows(rng, B, Hkv, D, new_dtype)
        pt = 0 if s % 3 else 4 * {"fp8": 64, "i8": 64, "i4": 128}[fmt]     # every third step: wider ranges
        _step(fmt, q_d, dev_tensor(x), dev_tensor(y), new_dtype, kp_d, vp_d, ks_d, vs_d, bt_d, dev_tensor(lens),
              Hq, Hkv, D, P, scale, out, ws, pt)
        paged.append_dynamic(fmt, x, y, new_dtype, bt, lens, kp, vp, ks, vs, P)
        yf = codec.bf16_bits_to_f32(y) if new_dtype == "bf16" else y
        vmax = np.maximum(vmax, np.where((lens >= 1) & (lens <= MP * P), np.abs(yf).reshape(B, -1).max(1), 0))
        torch.cuda.synchronize()
        _compare(kp_d, vp_d, ks_d, vs_d, kp, vp, ks, vs, f"step {s}")
        got = gpu_out(out)
        good = [b for b in _good_rows(bt, lens, P, NP) if b not in holed]
        for b in range(B):
            if b in holed and lens[b] <= MP * P:
                continue                 # reads the unwritten slot: no defined result
            if lens[b] <= 0:
                assert np.all(got[b] == 0), f"step {s}: empty sequence {b} not zero"
            elif b not in good:
                assert np.isnan(got[b]).all(), f"step {s}: sequence {b} on a bad page not NaN"
        if good:
            ref = c_oracle.decode(q, "bf16", kp, vp, fmt, bt, np.where(np.isin(np.arange(B), good), lens, 0),
                                  Hq, P, scale, ks, vs)
            # The bounds are stated for N(0,1) values, which stay below 4 in
            # magnitude; these rows reach 16x that, and the decode's rounding
            # errors (weights rounded to 11-16 bits) grow with |v|: compare in
            # units of max(1, max|v| / 4) per sequence.
            u = np.maximum(1.0, vmax[good] / 4.0)[:, None, None]
            mx, mean = check_close(got[good] / u, ref[good] / u, fmt, f"step {s}")
            worst = (max(worst[0], mx), max(worst[1], mean))
    assert worst[0] > 0.0


def test_step_quant_errors():
    x = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    sl = torch.ones(2, dtype=torch.int32, device="cuda")
    pool = torch.zeros((4, 2, 64 * 128), dtype=torch.uint8, device="cuda")
    sc = torch.ones((4, 2), dtype=torch.float32, device="cuda")
    out = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(pkv.decode_workspace_bytes(2, 8, 2, 128), dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError) as e:          # not a quantised cache
        pkv.decode_step_quant(q, "bf16", x, x, "bf16", pool, pool, "bf16", sc, sc, bt, sl, 8, 2, 128, 64, 0.1,
                              out, "f32", ws)
    assert e.value.code == -3
    with pytest.raises(pkv.PkvError) as e:          # rows already quantised
        pkv.decode_step_quant(q, "bf16", x, x, "fp8", pool, pool, "fp8", sc, sc, bt, sl, 8, 2, 128, 64, 0.1,
                              out, "f32", ws)
    assert e.value.code == -3
    with pytest.raises(pkv.PkvError) as e:          # page size not a multiple of the fp8 V block
        pkv.decode_step_quant(q, "bf16", x, x, "bf16", pool, pool, "fp8", sc, sc, bt, sl, 8, 2, 128, 32, 0.1,
                              out, "f32", ws)
    assert e.value.code == -2


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fmt", ["fp8", "i8", "i4"])
def test_config_inflight_quant_fused_full(fmt):
    """The in-flight batch with a quantised cache through the fused quantising
    step: 16 steps; scales bit-exact after every step and the pools after every
    step; every output row against the oracle after every step."""
    gen = {"fp8": configs.inflight_fp8, "i8": configs.inflight_int8, "i4": configs.inflight_int4}[fmt]
    wl = gen()
    dw = DeviceWorkload(wl)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    ks, vs = wl.k_scales.copy(), wl.v_scales.copy()
    worst = (0.0, 0.0)
    for s, st in enumerate(wl.steps):
        sl = dev_tensor(st.seq_lens)
        pkv.decode_step_quant(dw.q, wl.q_dtype, dev_tensor(st.k_new), dev_tensor(st.v_new), "bf16", dw.k_pool,
                              dw.v_pool, fmt, dw.ks, dw.vs, dw.bt, sl, wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, dw.out,
                              wl.out_dtype, dw.ws)
        paged.append_dynamic(fmt, st.k_new, st.v_new, "bf16", wl.block_tables, st.seq_lens, kp, vp, ks, vs, wl.P)
        torch.cuda.synchronize()
        _compare(dw.k_pool, dw.v_pool, dw.ks, dw.vs, kp, vp, ks, vs, f"fused step {s}")
        ref = c_oracle.decode(wl.q, wl.q_dtype, kp, vp, fmt, wl.block_tables, st.seq_lens, wl.Hq, wl.P, wl.scale,
                              ks, vs, nthreads=16)
        mx, mean = check_close(gpu_out(dw.out), ref, fmt, f"fused step {s}")
        worst = (max(worst[0], mx), max(worst[1], mean))
    PARITY_LOG.append((f"inflight_{fmt} fused quantising step, 16 steps (worst)", fmt,
                       wl.B * wl.Hq * wl.D * len(wl.steps)) + worst)
