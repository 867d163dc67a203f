"""Stream-ordered execution through the C ABI: concurrent calls and graph replay.

The library launches only on the caller's stream, never synchronises with the
host and keeps all state in the caller's workspace, so

* two problems on two streams with distinct workspaces, their calls
  interleaved on the host, both give the oracle's results;
* the whole forward + backward can be captured into a HIP graph and replayed:
  every replay, with eager work and synchronisations between replays, gives
  bit for bit the eager result (same kernels, same tile order, so the same
  floating-point sums).
"""
import numpy as np
import pytest
import torch

from oracle import lce_oracle as O
from vocab_projection_amd import binding as B
from vocab_projection_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def make(w):
    hid, wt, t = S.hidden(w), S.weight(w), S.targets(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    h = torch.from_numpy(hid).to(DEV).to(dt).contiguous()
    W = torch.from_numpy(wt).to(DEV).to(dt).contiguous()
    tt = torch.from_numpy(t).to(DEV)
    p = B.make_problem(h, W, ignore_index=S.IGNORE_INDEX, reduction=w.reduction, strip=w.strip)
    bufs = dict(
        ws=B.workspace(p, DEV),
        go=torch.full((1,), w.grad_out, dtype=torch.float32, device=DEV),
        loss=torch.empty(1, dtype=torch.float32, device=DEV),
        lse=torch.empty(h.shape[0], dtype=torch.float32, device=DEV),
        dh=torch.empty(h.shape, dtype=torch.float32, device=DEV),
        dw=torch.empty(W.shape, dtype=torch.float32, device=DEV),
    )
    return (hid, wt, t), (h, W, tt), p, bufs


def step(p, h, W, tt, b):
    B.lce_forward(p, h, W, tt, b["loss"], b["lse"], None, b["ws"])
    B.lce_backward(p, h, W, tt, b["lse"], b["go"], b["dh"], b["dw"], b["ws"])


def check_against_oracle(w, host, b):
    hid, wt, t = host
    loss, lse, _ = O.forward(hid, wt, t, ignore_index=S.IGNORE_INDEX, reduction=w.reduction)
    dh, dw = O.backward(hid, wt, t, ignore_index=S.IGNORE_INDEX, reduction=w.reduction,
                        grad_out=w.grad_out)
    assert abs(b["loss"].item() - loss) <= 2e-3 * abs(loss)
    for got, ref in ((b["dh"], dh), (b["dw"], dw)):
        got = got.cpu().numpy().astype(np.float64)
        assert np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref)


def test_two_streams_distinct_workspaces():
    w1 = S.small("bf16_stream_a", 1500, 192, 2300, 1024, ignore_frac=0.1)
    w2 = S.small("bf16_stream_b", 700, 96, 3100, 512, reduction="sum", grad_out=0.5, seed=11)
    host1, (h1, W1, t1), p1, b1 = make(w1)
    host2, (h2, W2, t2), p2, b2 = make(w2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    torch.cuda.synchronize()
    for _ in range(2):  # interleave the host calls of the two problems
        B.lce_forward(p1, h1, W1, t1, b1["loss"], b1["lse"], None, b1["ws"], s1)
        B.lce_forward(p2, h2, W2, t2, b2["loss"], b2["lse"], None, b2["ws"], s2)
        B.lce_backward(p1, h1, W1, t1, b1["lse"], b1["go"], b1["dh"], b1["dw"], b1["ws"], s1)
        B.lce_backward(p2, h2, W2, t2, b2["lse"], b2["go"], b2["dh"], b2["dw"], b2["ws"], s2)
    torch.cuda.synchronize()
    check_against_oracle(w1, host1, b1)
    check_against_oracle(w2, host2, b2)


def test_graph_capture_and_replay():
    w = S.small("bf16_graph", 1300, 160, 2500, 1024, ignore_frac=0.05)
    host, (h, W, tt), p, b = make(w)
    step(p, h, W, tt, b)
    torch.cuda.synchronize()
    eager = {k: b[k].clone() for k in ("loss", "lse", "dh", "dw")}
    check_against_oracle(w, host, b)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(p, h, W, tt, b)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in ("loss", "lse", "dh", "dw"):
            b[k].fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("loss", "lse", "dh", "dw"):
            assert torch.equal(b[k], eager[k]), (rep, k)
