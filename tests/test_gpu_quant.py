"""GPU parity of the one-byte appends with dynamic page scales
(pkv_kv_append_fp8, pkv_kv_append_int8).

Every case runs the HIP kernel through the C ABI and the oracle
(oracle.paged.append_dynamic) on the same inputs, step after step, and
requires the pools and the scales to be equal bit for bit after every step;
decode over the resulting cache is then checked against the oracle's decode
within the fp8 tolerance.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_decode_amd as pkv
from oracle import paged
from workloads import codec, configs, layout
from tests._helpers import PARITY_LOG, DeviceWorkload, check_close, dev_tensor, gpu_out, host_bytes, oracle_decode

pytestmark = pytest.mark.gpu

F32 = np.float32
FMTS = ["fp8", "i8", "i4"]
APPEND_FN = {"fp8": "kv_append_fp8", "i8": "kv_append_int8", "i4": "kv_append_int4"}


def gpu_append(fmt, *args):
    getattr(pkv, APPEND_FN[fmt])(*args)


def empty_pools(fmt, NP, Hkv, P, D):
    kp = layout.empty_pool(NP, Hkv, P, D, fmt)
    return kp, kp.copy(), np.full((NP, Hkv), np.nan, F32), np.full((NP, Hkv), np.nan, F32)


def _rows(rng, B, Hkv, D, new_dtype):
    """New rows whose magnitude jumps around, so that scales are set, kept and
    grown at every slot position; some rows are zero, some tiny, some -0."""
    x = rng.standard_normal((B, Hkv, D)).astype(F32)
    f = rng.choice(np.array([1, 1, 1, 0.5, 2, 4, 16, 1e-3, 0], F32), size=(B, Hkv, 1))
    x = (x * f).astype(F32)
    neg0 = rng.random((B, Hkv, D)) < 0.02
    x[neg0] = -0.0
    if new_dtype == "bf16":
        return codec.f32_to_bf16_bits(x)
    return x


def _compare(kp_dev, vp_dev, ks_dev, vs_dev, kp, vp, ks, vs, what):
    assert np.array_equal(host_bytes(kp_dev), kp.reshape(-1).view(np.uint8)), f"{what}: K bytes"
    assert np.array_equal(host_bytes(vp_dev), vp.reshape(-1).view(np.uint8)), f"{what}: V bytes"
    assert np.array_equal(host_bytes(ks_dev), ks.reshape(-1).view(np.uint8)), f"{what}: K scales"
    assert np.array_equal(host_bytes(vs_dev), vs.reshape(-1).view(np.uint8)), f"{what}: V scales"


CASES = [  # (fmt, D, P, new_dtype, steps)
    (fmt, D, P, nd, st) for fmt in ("fp8", "i8")
    for (D, P, nd, st) in ((128, 128, "bf16", 140), (64, 64, "f32", 75), (128, 64, "bf16", 80),
                           (64, 128, "bf16", 135))
] + [("i4", 128, 128, "bf16", 140), ("i4", 128, 256, "f32", 270),
      # long pages: a re-encode takes more than one round of loads (K past 128
      # or 256 slots, V past 1024 groups)
      ("fp8", 128, 256, "bf16", 270), ("i8", 64, 512, "f32", 530)]


@pytest.mark.parametrize("fmt,D,P,new_dtype,steps", CASES, ids=lambda v: str(v))
def test_append_bit_exact_every_step(fmt, D, P, new_dtype, steps):
    rng = np.random.default_rng(100 + D + P)
    B, Hkv, MP = 7, 2, 2
    NP = B * MP + 3
    perm = rng.permutation(NP).astype(np.int32)
    bt = perm[:B * MP].reshape(B, MP).copy()
    bt[5, 1] = -1                       # sequence 5 runs onto a missing page after P tokens
    bt[6, 1] = NP + 7                   # sequence 6 onto a page id out of range
    start = np.array([0, 0, 3, 10, P - 2, 1, 2])    # step at which each sequence starts
    kp, vp, ks, vs = empty_pools(fmt, NP, Hkv, P, D)
    kp_d, vp_d, ks_d, vs_d = (dev_tensor(a) for a in (kp, vp, ks, vs))
    bt_d = dev_tensor(bt)
    for s in range(steps):
        lens = np.where(s >= start, s - start + 1, 0).astype(np.int32)
        if s % 17 == 5:
            lens[4] = MP * P + 1         # a call past the end of the table: skipped
        x, y = _rows(rng, B, Hkv, D, new_dtype), _rows(rng, B, Hkv, D, new_dtype)
        gpu_append(fmt, dev_tensor(x), dev_tensor(y), new_dtype, bt_d, dev_tensor(lens), kp_d, vp_d,
                   ks_d, vs_d, Hkv, D, P)
        paged.append_dynamic(fmt, x, y, new_dtype, bt, lens, kp, vp, ks, vs, P)
        torch.cuda.synchronize()
        _compare(kp_d, vp_d, ks_d, vs_d, kp, vp, ks, vs, f"step {s}")


@pytest.mark.parametrize("fmt,P", [(f, 128) for f in FMTS] + [("fp8", 256)])
def test_append_grows_at_every_slot(fmt, P):
    """One sequence, each new token larger than the last: the scale grows on every
    append, so every slot position re-encodes all earlier ones."""
    rng = np.random.default_rng(7)
    B, Hkv, D = 1, 1, 128
    bt = np.array([[2]], np.int32)
    kp, vp, ks, vs = empty_pools(fmt, 3, Hkv, P, D)
    kp_d, vp_d, ks_d, vs_d = (dev_tensor(a) for a in (kp, vp, ks, vs))
    for t in range(P):
        x = (rng.standard_normal((1, 1, D)) * 1.05 ** t).astype(F32)
        x[0, 0, t % D] = 10 * 1.05 ** t                    # a new maximum every time
        y = (-x).astype(F32)
        lens = np.array([t + 1], np.int32)
        gpu_append(fmt, dev_tensor(x), dev_tensor(y), "f32", dev_tensor(bt), dev_tensor(lens), kp_d, vp_d,
                   ks_d, vs_d, Hkv, D, P)
        paged.append_dynamic(fmt, x, y, "f32", bt, lens, kp, vp, ks, vs, P)
    torch.cuda.synchronize()
    _compare(kp_d, vp_d, ks_d, vs_d, kp, vp, ks, vs, "growing")


@pytest.mark.parametrize("fmt", FMTS)
def test_append_matches_one_shot_generator_pages(fmt):
    """Token-by-token GPU appends with the page amax on each page's first token
    reproduce the generator's one-shot per-page quantisation."""
    rng = np.random.default_rng(8)
    Hkv, D, P = 2, 128, 64 if fmt != "i4" else 128
    L = 3 * P - 5
    xk = rng.standard_normal((L, Hkv, D)).astype(F32)
    xv = rng.standard_normal((L, Hkv, D)).astype(F32)
    for p0 in range(0, L, P):
        xk[p0, :, 3] = 12.0
        xv[p0, :, 9] = -11.0
    kb, ksc = configs.QUANTIZERS[fmt](xk, P)
    vb, vsc = configs.QUANTIZERS[fmt](xv, P)
    pages = np.array([4, 0, 2], np.int32)
    NP = 5
    kp_d, vp_d, ks_d, vs_d = (dev_tensor(a) for a in empty_pools(fmt, NP, Hkv, P, D))
    bt_d = dev_tensor(pages.reshape(1, -1))
    for t in range(L):
        gpu_append(fmt, dev_tensor(xk[t:t + 1]), dev_tensor(xv[t:t + 1]), "f32", bt_d,
                   dev_tensor(np.array([t + 1], np.int32)), kp_d, vp_d, ks_d, vs_d, Hkv, D, P)
    torch.cuda.synchronize()
    kidx, vidx = layout.k_chunk_index(P, D, fmt), layout.v_chunk_index(P, D, fmt)
    kp = kp_d.cpu().numpy()
    vp = vp_d.cpu().numpy()
    for i, pg in enumerate(pages):
        n = min(P, L - i * P)
        for g in range(Hkv):
            assert np.array_equal(paged.read_elems(kp, (pg, g, kidx[:n]), fmt), kb[i * P:i * P + n, g])
            assert np.array_equal(paged.read_elems(vp, (pg, g, vidx[:n]), fmt), vb[i * P:i * P + n, g])
    assert np.array_equal(ks_d.cpu().numpy()[pages], ksc)
    assert np.array_equal(vs_d.cpu().numpy()[pages], vsc)


def test_append_quant_errors():
    x = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    sl = torch.ones(2, dtype=torch.int32, device="cuda")
    pool = torch.zeros((4, 2, 64 * 128), dtype=torch.uint8, device="cuda")
    sc = torch.ones((4, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.kv_append_fp8(x, x, "fp8", bt, sl, pool, pool.clone(), sc, sc.clone(), 2, 128, 64)
    assert e.value.code == -3
    with pytest.raises(pkv.PkvError) as e:
        pkv.kv_append_fp8(x, x, "bf16", bt, sl, pool, pool.clone(), sc, sc.clone(), 2, 128, 32)
    assert e.value.code == -2
    with pytest.raises(pkv.PkvError) as e:
        pkv.kv_append_int8(x, x, "i8", bt, sl, pool, pool.clone(), sc, sc.clone(), 2, 128, 64)
    assert e.value.code == -3


def _inflight_quant_run(fmt, B, n_steps, max_len, decode_every, pools_every=True, report=None):
    gen = {"fp8": configs.inflight_fp8, "i8": configs.inflight_int8, "i4": configs.inflight_int4}[fmt]
    wl = gen(B=B, n_steps=n_steps, max_len=max_len)
    dw = DeviceWorkload(wl)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    ks, vs = wl.k_scales.copy(), wl.v_scales.copy()
    worst = (0.0, 0.0)
    for s, st in enumerate(wl.steps):
        sl = dev_tensor(st.seq_lens)
        gpu_append(fmt, dev_tensor(st.k_new), dev_tensor(st.v_new), "bf16", dw.bt, sl, dw.k_pool,
                   dw.v_pool, dw.ks, dw.vs, wl.Hkv, wl.D, wl.P)
        paged.append_dynamic(fmt, st.k_new, st.v_new, "bf16", wl.block_tables, st.seq_lens, kp, vp, ks, vs,
                             wl.P)
        torch.cuda.synchronize()
        if pools_every or s == n_steps - 1:
            _compare(dw.k_pool, dw.v_pool, dw.ks, dw.vs, kp, vp, ks, vs, f"step {s}")
        else:       # scales every step; the pools (a wrong byte persists) at the end
            assert np.array_equal(host_bytes(dw.ks), ks.reshape(-1).view(np.uint8)), f"step {s}: K scales"
            assert np.array_equal(host_bytes(dw.vs), vs.reshape(-1).view(np.uint8)), f"step {s}: V scales"
        if decode_every or s == n_steps - 1:
            out = gpu_out(dw.decode(seq_lens=sl))
            wl_now = configs.Workload(**{**wl.__dict__, "k_scales": ks, "v_scales": vs})
            mx, mean = check_close(out, oracle_decode(wl_now, kp, vp, st.seq_lens), fmt, f"decode after step {s}")
            worst = (max(worst[0], mx), max(worst[1], mean))
    if report:
        PARITY_LOG.append((report, fmt, wl.B * wl.Hq * wl.D * n_steps) + worst)


@pytest.mark.parametrize("fmt", FMTS)
def test_config_inflight_quant_reduced_every_step(fmt):
    _inflight_quant_run(fmt, B=16, n_steps=16, max_len=4000, decode_every=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fmt", FMTS)
def test_config_inflight_quant_full(fmt):
    """The in-flight batch with a quantised cache: 16 quantise-on-write steps;
    scales bit-exact after every step, pools after the last one; every output
    row decoded after every step against the oracle."""
    _inflight_quant_run(fmt, B=256, n_steps=16, max_len=32768, decode_every=True, pools_every=False,
                        report=f"inflight_{fmt} append+decode, 16 steps (worst)")
