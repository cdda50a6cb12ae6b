"""GPU parity of device page allocation (pkv_alloc_pages, pkv_release_pages)
against oracle.paged.alloc_pages / release_pages: tables, stacks and counts
equal after every call."""
import numpy as np
import pytest
import torch

import paged_kv_attention_decode_amd as pkv
from oracle import paged
from tests._helpers import dev_tensor

pytestmark = pytest.mark.gpu


def _state(bt, fp, n):
    return dev_tensor(bt), dev_tensor(fp), dev_tensor(np.array([n], np.int32))


def _check(dbt, dfp, dfc, bt, fp, n, what):
    torch.cuda.synchronize()
    assert np.array_equal(dbt.cpu().numpy(), bt), f"{what}: block tables"
    assert np.array_equal(dfp.cpu().numpy(), fp), f"{what}: free stack"
    assert int(dfc.cpu().numpy()[0]) == n, f"{what}: free count"


@pytest.mark.parametrize("B", [1, 63, 64, 65, 300])
def test_alloc_release_steps_match_oracle(B):
    rng = np.random.default_rng(B)
    P, MP = 16, 8
    NP = 2 * B + 3                                  # runs dry at times
    bt = np.full((B, MP), -1, np.int32)
    fp = rng.permutation(NP).astype(np.int32)
    n = NP
    lens = np.zeros(B, np.int32)
    dbt, dfp, dfc = _state(bt, fp, n)
    for step in range(3 * P + 5):
        lens = (lens + (rng.random(B) < 0.85)).astype(np.int32)
        dsl = dev_tensor(lens)
        pkv.alloc_pages(dsl, dbt, P, dfp, dfc)
        n = paged.alloc_pages(lens, bt, fp, n, P)
        _check(dbt, dfp, dfc, bt, fp, n, f"alloc step {step}")
        done = ((lens > P) & (rng.random(B) < 0.02)).astype(np.int32)
        pkv.release_pages(dev_tensor(done), dsl, dbt, P, NP, dfp, dfc)
        n = paged.release_pages(done, lens, bt, fp, n, NP, NP, P)
        _check(dbt, dfp, dfc, bt, fp, n, f"release step {step}")
        lens[done != 0] = 0


def test_release_capacity_and_foreign_ids():
    P, MP = 4, 3
    bt = np.array([[3, 4, -1], [5, -1, -1], [6, 7, 8], [9, 99, -1]], np.int32)
    lens = np.array([5, 4, 12, 6], np.int32)
    fp = np.zeros(6, np.int32)
    dbt, dfp, dfc = _state(bt, fp, 1)
    rel = np.array([1, 0, 1, 1], np.int32)
    pkv.release_pages(dev_tensor(rel), dev_tensor(lens), dbt, P, 50, dfp, dfc)
    n = paged.release_pages(rel, lens, bt, fp, 1, 6, 50, P)
    _check(dbt, dfp, dfc, bt, fp, n, "release")


def test_alloc_clamps_a_corrupt_count():
    """A count beyond the stack's capacity is clamped (no read outside it)."""
    bt = np.full((3, 2), -1, np.int32)
    fp = np.array([7, 8, 9], np.int32)
    dbt, dfp, dfc = _state(bt, fp, 1000)
    pkv.alloc_pages(dev_tensor(np.array([1, 1, 1], np.int32)), dbt, 16, dfp, dfc)
    n = paged.alloc_pages(np.array([1, 1, 1], np.int32), bt, fp, 3, 16)
    _check(dbt, dfp, dfc, bt, fp, n, "clamped")
