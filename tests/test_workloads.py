"""Host-side checks of the seeded workload generators and page placement."""
import numpy as np
import pytest

from workloads import configs, layout


def _live_pages(wl, lens):
    pages = []
    for b in range(wl.B):
        n = int(configs.pages_needed(np.array([lens[b]]), wl.P)[0])
        pages.extend(wl.block_tables[b, :n].tolist())
    return pages


@pytest.mark.parametrize("name,kw", [("tiny_fp32", {}), ("llama3_8b_bf16", dict(B=8)),
                                     ("inflight_bf16", dict(B=16, n_steps=16, max_len=4000)),
                                     ("long_splitkv_bf16", dict(B=2, L=2048)), ("fp8_kv", dict(B=4)),
                                     ("inflight_fp8", dict(B=16, n_steps=16, max_len=4000))])
def test_deterministic_and_valid(name, kw):
    a = configs.CONFIGS[name](**kw)
    b = configs.CONFIGS[name](**kw)
    assert np.array_equal(a.k_pool.view(np.uint8), b.k_pool.view(np.uint8))
    assert np.array_equal(a.block_tables, b.block_tables)
    final = a.steps[-1].seq_lens if a.steps else a.seq_lens
    live = _live_pages(a, final)
    assert len(live) == len(set(live)), "a page is shared by two live sequences"
    assert all(0 <= p < a.num_pages for p in live)
    assert final.max() <= a.max_pages * a.P
    assert a.k_pool.shape == (a.num_pages, a.Hkv, a.P * a.D)


def test_tiny_config_matches_its_description():
    wl = configs.tiny_fp32()
    assert list(wl.seq_lens) == [1, 17, 64, 130]
    assert (wl.Hq, wl.Hkv, wl.D, wl.P, wl.num_pages) == (8, 8, 64, 16, 64)
    assert wl.scale == np.float32(0.125)
    perm = np.random.default_rng(1).permutation(64)
    assert list(wl.block_tables[3, :9]) == list(perm[7:16])


def test_inflight_steps_allocate_fresh_pages():
    wl = configs.inflight_bf16(B=32, n_steps=16, max_len=4000)
    L0 = wl.seq_lens
    for s, st in enumerate(wl.steps):
        assert np.array_equal(st.seq_lens, L0 + s + 1)
    # sequences whose length crosses a page boundary got a page id beyond their start pages
    for b in range(wl.B):
        n0 = int(configs.pages_needed(np.array([L0[b]]), wl.P)[0])
        n1 = int(configs.pages_needed(np.array([L0[b] + 16]), wl.P)[0])
        assert (wl.block_tables[b, :n1] >= 0).all() and (wl.block_tables[b, n1:] == -1).all()
        assert n1 - n0 in (0, 1)


def test_fp8_scales_are_amax_over_448():
    wl = configs.fp8_kv(B=3)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        kf = configs.draw_seq_f32(wl.seed, 2, b, L, wl.Hkv, wl.D)
        p = 1
        pg = wl.block_tables[b, p]
        amax = np.abs(kf[p * wl.P:(p + 1) * wl.P, 0]).max()
        assert wl.k_scales[pg, 0] == np.float32(amax / np.float32(448.0))
