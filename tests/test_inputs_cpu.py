"""The seeded input generator is deterministic: the bytes of every tensor of
the five workloads hash to pinned values (a change of seed, recipe, draw
order or rounding shows up here), and two draws are identical. The
generator holds none of the method's arithmetic; it feeds the oracle and the
GPU path the same values."""
import hashlib

import pytest
import torch

import flce_inputs as fi

# sha256 (first 16 hex digits) of the raw bytes of h, W and labels
PINNED = {
    1: ("f6aa5711c925ede5", "484fc895135aba91", "55292b19ca09b847"),
    2: ("51aaee4f1e08f48c", "a7dc184e8f6d1951", "1443c3947a020752"),
    3: ("2b1e705ce057f631", "eca476c9edbd6738", "1d66b14ba2246d6d"),
    4: ("833a02646992adc0", "b62694760ed8b186", "5b2f6379897da4a7"),
    5: ("33bcb13bc9ade74e", "e19330bba589e725", "2b8c8529799e33f2"),
}


def _digest(x: torch.Tensor) -> str:
    b = x.contiguous().view(torch.uint8) if x.dtype != torch.int64 else \
        x.contiguous().view(torch.uint8)
    return hashlib.sha256(memoryview(b.numpy())).hexdigest()[:16]


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_workload_bytes_pinned(k):
    w = fi.make_workload(k)
    assert (_digest(w.h), _digest(w.W), _digest(w.labels)) == PINNED[k]
    assert int((w.labels != w.ignore_index).sum()) == w.expected_valid


def test_two_draws_identical():
    a = fi.make_custom(300, 72, 900, dtype=torch.bfloat16, seed=5, labels="zipf")
    b = fi.make_custom(300, 72, 900, dtype=torch.bfloat16, seed=5, labels="zipf")
    for x, y in ((a.h, b.h), (a.W, b.W), (a.labels, b.labels)):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int64 else x,
                           y.view(torch.uint8) if y.dtype != torch.int64 else y)
    c = fi.make_custom(300, 72, 900, dtype=torch.bfloat16, seed=6, labels="zipf")
    assert not torch.equal(a.h.view(torch.uint8), c.h.view(torch.uint8))
