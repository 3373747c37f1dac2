"""The whole step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the library allocates nothing, never synchronises the host and clears memory
with kernels only, so a caller can capture a call. Each replay, with eager work
and synchronisations between the replays, must give exactly the eager
result (the path is deterministic)."""
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


@pytest.mark.parametrize("mode", ["step", "nr", "forward", "f32grad", "logits", "odd_h"])
def test_graph_replays_match_eager(mode, monkeypatch):
    import lm_head_linear_amd as m
    monkeypatch.setenv("FLCE_VCHUNK", "512")          # several backward chunks
    dev = gu.device()
    # odd_h: the step at a hidden size that is not a multiple of 8 (padded
    # copies and the copy-out kernels in the graph too)
    w = fi.make_custom(700, 133 if mode == "odd_h" else 136, 1500, dtype=torch.bfloat16,
                       seed=300, softcap=30.0)
    h = w.h.reshape(-1, w.H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    N, H, V = w.N, w.H, w.V
    gdt = torch.float32 if mode == "f32grad" else torch.bfloat16
    dH = torch.empty(N, H, dtype=gdt, device=dev)
    dW = torch.empty(V, H, dtype=gdt, device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    nt = torch.empty((), dtype=torch.int64, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    if mode == "nr":
        ws = torch.empty(m.flce_workspace_size_nr(N, H, V, W.dtype, 256), dtype=torch.uint8, device=dev)
    elif mode in ("forward", "logits"):
        ws = torch.empty(m.flce_forward_workspace_size(N, H, V, W.dtype), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(m.flce_workspace_size(N, H, V, W.dtype, gdt), dtype=torch.uint8, device=dev)

    lg = torch.empty(N, V, dtype=torch.bfloat16, device=dev)
    fwd_only = mode in ("forward", "logits")

    def call():
        if mode == "logits":
            m.flce_forward_logits(h, W, y, softcap=w.softcap, workspace=ws, loss=loss,
                                  num_tokens=nt, lse_out=lse, logits=lg)
        elif mode == "forward":
            m.flce_forward(h, W, y, softcap=w.softcap, workspace=ws, loss=loss, num_tokens=nt,
                           lse_out=lse)
        else:
            m.flce_forward_backward(h, W, y, softcap=w.softcap, dH=dH, dW=dW, workspace=ws,
                                    loss=loss, num_tokens=nt, lse_out=lse, grad_dtype=gdt,
                                    recompute=mode != "nr", token_chunk=256)

    def snapshot():
        out = [loss.clone(), nt.clone(), lse.clone()]
        if not fwd_only:
            out += [dH.clone(), dW.clone()]
        if mode == "logits":
            out.append(lg.clone())
        return out

    call()
    torch.cuda.synchronize()
    ref = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm up on the capture stream
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        # overwrite the outputs and run unrelated eager work between replays
        for t in [loss, lse] + ([dH, dW] if not fwd_only else []) + ([lg] if mode == "logits" else []):
            t.fill_(float("nan"))
        nt.fill_(-1)
        junk = torch.randn(1024, 1024, device=dev) @ torch.randn(1024, 1024, device=dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, ref):          # bit for bit (NaN-free by construction)
            assert torch.equal(a.reshape(-1).view(torch.uint8), b.reshape(-1).view(torch.uint8)), (mode, rep)
        del junk
