"""The no-allocation forward (flce_forward_noalloc, the library's fixed
per-GPU scratch instead of a caller workspace), called through the C-ABI,
against flce_forward on the same inputs: loss, count, lse and status
bit-identical, on two calls in a row with the second one smaller (the
scratch keeps the first call's bytes), on the current and on a second
stream, and a problem larger than the scratch refused before any launch."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_linear_amd._lib as L
    L.load()
    yield


def _inputs(w):
    dev = gu.device()
    return (w.h.reshape(-1, w.H).to(dev), w.W.to(dev), w.labels.reshape(-1).to(dev))


def _both(w, stream=None):
    """(flce_forward results, flce_forward_noalloc results) on w's inputs."""
    import lm_head_linear_amd as m
    h, W, y = _inputs(w)
    dev = h.device
    kw = dict(ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction,
              num_label_tokens=w.num_label_tokens)
    out = []
    for fn in ("ref", "noalloc"):
        loss = torch.full((), float("nan"), dtype=torch.float32, device=dev)
        nt = torch.full((), -1, dtype=torch.int64, device=dev)
        lse = torch.full((h.shape[0],), float("nan"), dtype=torch.float32, device=dev)
        st = torch.full((), -1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        if fn == "ref":
            m.flce_forward(h, W, y, loss=loss, num_tokens=nt, lse_out=lse, status=st, **kw)
        else:
            before = torch.cuda.memory_allocated(dev)
            s = stream or torch.cuda.current_stream(dev)
            with torch.cuda.stream(s):
                m.flce_forward_noalloc(h, W, y, loss=loss, num_tokens=nt, lse_out=lse,
                                       status=st, **kw)
            assert torch.cuda.memory_allocated(dev) == before     # nothing allocated
            s.synchronize()
        torch.cuda.synchronize()
        out.append((loss, nt, lse, st))
    return out


def _same_bits(a, b):
    (la, na, sa, ta), (lb, nb, sb, tb) = a, b
    assert la.view(torch.int32).item() == lb.view(torch.int32).item()
    assert na.item() == nb.item() and ta.item() == tb.item() == 0
    assert torch.equal(sa.view(torch.int32), sb.view(torch.int32))


def test_noalloc_matches_forward_two_calls_second_smaller():
    big = fi.make_custom(2300, 1024, 50000, dtype=torch.bfloat16, seed=41, softcap=30.0,
                         reduction="mean")
    small = fi.make_custom(300, 136, 1000, dtype=torch.bfloat16, seed=42, ignore_frac=0.3)
    a, b = _both(big)
    _same_bits(a, b)
    a, b = _both(small)
    _same_bits(a, b)
    # and the oracle agrees with the small one
    r = gu.run_oracle(small)
    gu.assert_loss(b[0].item(), r.loss64)
    assert b[1].item() == r.num_tokens


def test_noalloc_full_large_vocab_then_tiny_fp32_on_a_second_stream():
    w = fi.make_workload(3)
    a, b = _both(w)
    _same_bits(a, b)
    assert b[1].item() == 0
    tiny = fi.make_workload(1)
    side = torch.cuda.Stream()
    a, b = _both(tiny, stream=side)
    _same_bits(a, b)


def test_noalloc_refuses_a_problem_beyond_the_scratch():
    import lm_head_linear_amd as m
    from lm_head_linear_amd import _lib
    N, H, V = 16384, 64, 1 << 20          # forward partials alone: 512 MiB
    assert m.flce_forward_workspace_size(N, H, V, torch.bfloat16) > _lib.NOALLOC_SCRATCH_BYTES
    dev = gu.device()
    h = torch.zeros(N, H, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(V, H, dtype=torch.bfloat16, device=dev)
    y = torch.zeros(N, dtype=torch.int64, device=dev)
    loss = torch.full((), 5.0, device=dev)
    nt = torch.full((), 9, dtype=torch.int64, device=dev)
    with pytest.raises(m.FlceError) as e:
        m.flce_forward_noalloc(h, W, y, loss=loss, num_tokens=nt)
    assert e.value.code == _lib.ERR_SCRATCH
    torch.cuda.synchronize()
    assert loss.item() == 5.0 and nt.item() == 9        # nothing launched
    del h, W, y
    torch.cuda.empty_cache()
    # a valid call right after still works
    w = fi.make_custom(64, 64, 300, dtype=torch.bfloat16, seed=43)
    a, b = _both(w)
    _same_bits(a, b)
