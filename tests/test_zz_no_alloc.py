"""GPU check of pkv_decode_step_noalloc, the step entry point that takes its
workspace from the library's static per-device scratch array instead of a
caller buffer: through the C ABI, two calls in a row (the second on a smaller
batch, so it runs over what the first left in the array), each equal bit for
bit to pkv_decode_step on the same inputs (output and pools) and within the
parity bounds of the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_attention_decode_amd as pkv
from oracle import c_oracle
from workloads import configs, layout
from tests._helpers import DeviceWorkload, check_close, dev_tensor, gpu_out, host_bytes, oracle_decode

pytestmark = pytest.mark.gpu


def _step_inputs(spec):
    """A workload whose cache holds L_b - 1 tokens and whose step brings token
    L_b - 1 (stored bytes, as decode_step takes them)."""
    wl = configs.custom(**spec)
    lens_now = wl.seq_lens.copy()
    lens_prev = np.maximum(lens_now - 1, 0)
    ki, vi = layout.k_chunk_index(wl.P, wl.D, wl.kv_dtype), layout.v_chunk_index(wl.P, wl.D, wl.kv_dtype)
    kp = layout.empty_pool(wl.num_pages, wl.Hkv, wl.P, wl.D, wl.kv_dtype)
    vp = layout.empty_pool(wl.num_pages, wl.Hkv, wl.P, wl.D, wl.kv_dtype)
    knew = np.zeros((wl.B, wl.Hkv, wl.D), layout.NP_DTYPE[wl.kv_dtype])
    vnew = np.zeros_like(knew)
    for b in range(wl.B):
        n = int(lens_now[b])
        k, v, _, _ = configs.seq_tokens(wl.seed, b, n, wl.Hkv, wl.D, wl.kv_dtype, wl.P)
        pages = wl.block_tables[b, :int(configs.pages_needed(np.array([n]), wl.P)[0])]
        layout.pack_sequence(kp, pages, k[:int(lens_prev[b])], wl.P, ki, wl.kv_dtype)
        layout.pack_sequence(vp, pages, v[:int(lens_prev[b])], wl.P, vi, wl.kv_dtype)
        if n:
            knew[b], vnew[b] = k[n - 1], v[n - 1]
    wl.k_pool, wl.v_pool = kp, vp
    return wl, knew, vnew


def _noalloc(dw, kn, vn):
    wl = dw.wl
    out = torch.full_like(dw.out, 7.0)
    pkv.decode_step_noalloc(dw.q, wl.q_dtype, kn, vn, dw.k_pool, dw.v_pool, wl.kv_dtype, dw.bt, dw.sl, wl.Hq,
                            wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype, k_scales=dw.ks, v_scales=dw.vs,
                            partition_tokens=wl.partition_tokens)
    return out


# Call 1: a Llama-3-8B-shaped batch split over many waves; call 2: a smaller
# batch of another shape (G 2, D 64), so its partial slots and descriptors sit
# at other offsets of the array than call 1's.
CALLS = {
    "bf16": [dict(seed=901, lens=list(np.random.default_rng(901).integers(1, 4097, 64)), Hq=32, Hkv=8, D=128,
                  P=64, kv_dtype="bf16"),
             dict(seed=902, lens=[1, 7, 300, 2500, 33], Hq=8, Hkv=4, D=64, P=32, kv_dtype="bf16")],
    "fp8": [dict(seed=903, lens=list(np.random.default_rng(903).integers(1, 8193, 128)), Hq=32, Hkv=8, D=128,
                 P=64, kv_dtype="fp8"),
            dict(seed=904, lens=[5, 64, 65, 1000], Hq=32, Hkv=8, D=128, P=64, kv_dtype="fp8")],
}


@pytest.mark.parametrize("kind", sorted(CALLS))
def test_noalloc_step_equals_decode_step(kind):
    for i, spec in enumerate(CALLS[kind]):
        wl, knew, vnew = _step_inputs(spec)
        a, b = DeviceWorkload(wl), DeviceWorkload(wl)        # two copies of the cache
        kn, vn = dev_tensor(knew), dev_tensor(vnew)
        ref_out = a.step(kn, vn, a.sl)
        got_out = _noalloc(b, kn, vn)
        torch.cuda.synchronize()
        what = f"{kind} call {i + 1} (B={wl.B})"
        assert torch.equal(got_out.view(torch.uint8), ref_out.view(torch.uint8)), f"{what}: output differs"
        assert np.array_equal(host_bytes(b.k_pool), host_bytes(a.k_pool)), f"{what}: K pool differs"
        assert np.array_equal(host_bytes(b.v_pool), host_bytes(a.v_pool)), f"{what}: V pool differs"
        ref_k, ref_v = wl.k_pool.copy(), wl.v_pool.copy()
        c_oracle.append(knew, vnew, wl.kv_dtype, wl.block_tables, wl.seq_lens, ref_k, ref_v, wl.P)
        assert np.array_equal(host_bytes(b.k_pool), ref_k.view(np.uint8).reshape(-1)), f"{what}: K append"
        assert np.array_equal(host_bytes(b.v_pool), ref_v.view(np.uint8).reshape(-1)), f"{what}: V append"
        check_close(gpu_out(got_out), oracle_decode(wl, ref_k, ref_v, wl.seq_lens), wl.kv_dtype, what)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A shape whose workspace exceeds the 40 MiB array fails before any launch
    (fake pointers: nothing is dereferenced)."""
    F = 0x1000
    L = pkv.lib()
    B, Hq, Hkv, D = 65536, 128, 8, 128
    assert pkv.decode_workspace_bytes(B, Hq, Hkv, D) > 40 << 20
    rc = L.pkv_decode_step_noalloc(F, 1, F, F, F, F, 1, None, None, F, 4, F, B, 8, Hq, Hkv, D, 64,
                                   ctypes.c_float(0.1), 0, F, 1, None)
    assert rc == -4, rc
    assert b"static scratch" in L.pkv_last_error()
