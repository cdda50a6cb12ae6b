"""The allocation-free decode step under HIP graph capture: one
pkv_decode_step_noalloc call captured into a graph (torch.cuda.CUDAGraph) and
replayed several times, with eager library and torch work and
synchronisations between the replays; every replay's output and pools must
equal an eager call's bit for bit.  The step clears nothing with memset and
allocates nothing, so the captured graph holds only its two kernels."""
import numpy as np
import pytest
import torch

import paged_kv_attention_decode_amd as pkv
from tests._helpers import DeviceWorkload, dev_tensor, host_bytes
from tests.test_zz_no_alloc import _step_inputs

pytestmark = pytest.mark.gpu


def _noalloc_into(dw, kn, vn, out):
    wl = dw.wl
    pkv.decode_step_noalloc(dw.q, wl.q_dtype, kn, vn, dw.k_pool, dw.v_pool, wl.kv_dtype, dw.bt, dw.sl, wl.Hq,
                            wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype, k_scales=dw.ks, v_scales=dw.vs,
                            partition_tokens=wl.partition_tokens)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_noalloc_step_replays_from_a_hip_graph(kv_dtype):
    rng = np.random.default_rng(905)
    spec = dict(seed=905, lens=list(rng.integers(1, 3000, 48)), Hq=32, Hkv=8, D=128, P=64, kv_dtype=kv_dtype)
    wl, knew, vnew = _step_inputs(spec)
    kn, vn = dev_tensor(knew), dev_tensor(vnew)
    a, b, c = DeviceWorkload(wl), DeviceWorkload(wl), DeviceWorkload(wl)   # three copies of the cache
    ref = torch.empty_like(a.out)
    _noalloc_into(a, kn, vn, ref)          # eager; the first call also sets up the static scratch
    torch.cuda.synchronize()
    ref_out = ref.view(torch.uint8).clone()
    ref_k, ref_v = host_bytes(a.k_pool), host_bytes(a.v_pool)

    out = torch.empty_like(b.out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc_into(b, kn, vn, out)
    for r in range(3):
        # eager work between replays: poison the output, run the step with a
        # caller workspace on the third copy, synchronise
        out.fill_(7.0)
        c.step(kn, vn, c.sl)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), ref_out), f"replay {r}: output differs from the eager call"
        assert np.array_equal(host_bytes(b.k_pool), ref_k), f"replay {r}: K pool differs"
        assert np.array_equal(host_bytes(b.v_pool), ref_v), f"replay {r}: V pool differs"
    assert torch.equal(c.out.view(torch.uint8), ref_out)   # the eager workspace call agrees too
