"""Pins of the device page-allocation oracle (oracle.paged.alloc_pages,
release_pages): closed cases written out by hand, a conservation invariant
(pages are neither created nor lost), and agreement with the in-flight
workload generator's own host-side allocation rule (a step takes a fresh page
when a sequence's last page is full)."""
import numpy as np

from oracle import paged
from workloads import configs


def test_alloc_closed_case():
    P = 4
    lens = np.array([1, 2, 5, 0, 9, 13, 4], np.int32)      # openers: 1 (page 0), 5 (1), 9 (2), 13 (3)
    bt = np.full((7, 3), -1, np.int32)
    fp = np.array([10, 11, 12, 13, 14], np.int32)
    n = paged.alloc_pages(lens, bt, fp, 5, P)
    # sequence order takes the stack top first: b0 <- 14, b2 <- 13, b4 <- 12; b5 (page 3) is past MP = 3
    assert n == 2
    assert bt[0, 0] == 14 and bt[2, 1] == 13 and bt[4, 2] == 12
    assert (bt[[1, 3, 5, 6]] == -1).all()


def test_alloc_leaves_held_pages():
    """A sequence whose opening page is already in its table (it did not grow
    this step) takes no page."""
    bt = np.array([[5, -1], [6, 8]], np.int32)
    n = paged.alloc_pages(np.array([9, 9], np.int32), bt, np.array([1, 2], np.int32), 2, 8)
    assert n == 1 and bt.tolist() == [[5, 2], [6, 8]]


def test_alloc_runs_dry():
    bt = np.full((4, 2), -1, np.int32)
    n = paged.alloc_pages(np.array([1, 1, 1, 1], np.int32), bt, np.array([7], np.int32), 1, 16)
    assert n == 0 and list(bt[:, 0]) == [7, -1, -1, -1]


def test_release_closed_case_and_capacity():
    P = 4
    bt = np.array([[3, 4, -1], [5, -1, -1], [6, 7, 8], [9, 99, -1]], np.int32)
    lens = np.array([5, 4, 12, 6], np.int32)
    fp = np.zeros(6, np.int32)
    n = paged.release_pages(np.array([1, 0, 1, 1]), lens, bt, fp, 1, 6, 50, P)
    # pushes in order: 3, 4 (b0), 6, 7, 8 (b2), then b3's 9 would exceed capacity 6; 99 is no page id
    assert n == 6 and list(fp[1:6]) == [3, 4, 6, 7, 8]
    assert (bt[[0, 2, 3]][:, :2] == -1).all() and bt[1, 0] == 5


def test_alloc_release_conserve_pages():
    rng = np.random.default_rng(5)
    P, MP, NP, B = 8, 6, 40, 12
    bt = np.full((B, MP), -1, np.int32)
    fp = np.zeros(NP, np.int32)
    fp[:] = rng.permutation(NP)
    count = NP
    lens = np.zeros(B, np.int32)
    for step in range(60):
        lens = lens + (rng.random(B) < 0.8)
        count = paged.alloc_pages(lens, bt, fp, count, P)
        done = (lens > 20) & (rng.random(B) < 0.3)
        count = paged.release_pages(done, lens, bt, fp, count, NP, NP, P)
        lens[done] = 0
        held = bt[bt >= 0]
        assert len(set(held.tolist())) == len(held)                     # no page held twice
        assert sorted(held.tolist() + fp[:count].tolist()) == list(range(NP))   # none created or lost
    assert (bt < 0).any()                                                # the stack did run dry


def test_alloc_matches_generator_step_rule():
    """The in-flight generator gives a sequence a fresh page exactly when its new
    token opens one; the oracle requests a page for exactly those sequences."""
    wl = configs.inflight_bf16(B=16, n_steps=4, max_len=3000)
    prev = wl.block_tables.copy()
    for st in wl.steps:
        L = st.seq_lens
        opener = (L >= 1) & ((L - 1) % wl.P == 0)
        bt = prev.copy()
        for b in np.nonzero(opener)[0]:
            bt[b, (L[b] - 1) // wl.P] = -1
        fp = np.array([1000 + i for i in range(64)], np.int32)
        n = paged.alloc_pages(L, bt, fp, 64, wl.P)
        assert 64 - n == int(opener.sum())
        assert np.array_equal(bt >= 0, prev >= 0)
