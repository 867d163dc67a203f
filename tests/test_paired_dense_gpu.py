"""Paired test against dense cross-entropy, the implementation the strip fold
replaces.

The first page ("Running 128K-Sequence MoE RL ...", section 8, primitives and
their paired test) validates a primitive by running the new and the replaced
implementation side by side and comparing loss, gradients, peak memory and
time.  Here the replaced implementation is PyTorch's dense path on the same
GPU: full float32 logits h.W^T, cross_entropy, autograd.  On the 4096-token,
151936-vocabulary bf16 workload both fit.  The strip path must agree with it
within the bf16 tolerances (loss 2e-3 relative, gradients 1e-2 relative
Frobenius), its peak extra memory must stay at one strip plus the outputs,
and the dense path must hold at least the full logits.  Times are printed,
not asserted.
"""
import sys
import time

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from vocab_projection_amd import binding as B
from vocab_projection_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def rel_fro(got, ref):
    return (torch.linalg.vector_norm((got - ref).double()) /
            torch.linalg.vector_norm(ref.double())).item()


def timed(fn, reps=3):
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def test_paired_with_dense_cross_entropy():
    w = S.WORKLOADS["bf16_n4k_h2k_v152k"]
    hid, wt, t = S.hidden(w, threads=16), S.weight(w, threads=16), S.targets(w)
    h = torch.from_numpy(hid).to(DEV).to(torch.bfloat16).contiguous()
    W = torch.from_numpy(wt).to(DEV).to(torch.bfloat16).contiguous()
    tt = torch.from_numpy(t).to(DEV)
    n, v = w.n_tokens, w.vocab

    # strip path through the C ABI
    p = B.make_problem(h, W, ignore_index=S.IGNORE_INDEX, reduction=w.reduction, strip=w.strip)
    go = torch.ones(1, dtype=torch.float32, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    lse = torch.empty(n, dtype=torch.float32, device=DEV)
    dh = torch.empty(h.shape, dtype=torch.float32, device=DEV)
    dw = torch.empty(W.shape, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws = B.workspace(p, DEV)

    def strip_step():
        B.lce_forward(p, h, W, tt, loss, lse, None, ws)
        B.lce_backward(p, h, W, tt, lse, go, dh, dw, ws)

    ms_strip = timed(strip_step)
    peak_strip = torch.cuda.max_memory_allocated() - base
    ws_bytes = B.lce_workspace_bytes(p)
    del ws

    # dense path: float32 logits, cross_entropy, autograd
    h32 = h.float().requires_grad_(True)
    W32 = W.float().requires_grad_(True)
    t64 = tt.long()
    out = {}

    def dense_step():
        h32.grad = None
        W32.grad = None
        logits = h32 @ W32.t()
        l = F.cross_entropy(logits, t64, ignore_index=S.IGNORE_INDEX, reduction="mean")
        l.backward()
        out["loss"] = l.detach()

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_d = torch.cuda.memory_allocated()
    ms_dense = timed(dense_step)
    peak_dense = torch.cuda.max_memory_allocated() - base_d

    lo, ld = loss.item(), out["loss"].item()
    e_h = rel_fro(dh, h32.grad)
    e_w = rel_fro(dw, W32.grad)
    flop = 8.0 * n * w.hidden * v
    say(f"paired c1: loss strip {lo:.6f} dense {ld:.6f}; dH rel {e_h:.2e}; dW rel {e_w:.2e}")
    say(f"paired c1: strip {ms_strip:.2f} ms ({flop / ms_strip / 1e9:.0f} TFLOP/s), peak extra "
        f"{peak_strip / 1e9:.3f} GB; dense {ms_dense:.2f} ms ({flop / ms_dense / 1e9:.0f} TFLOP/s), "
        f"peak extra {peak_dense / 1e9:.3f} GB; fp32 logits {n * v * 4 / 1e9:.3f} GB")
    assert abs(lo - ld) <= 2e-3 * abs(ld)
    assert e_h <= 1e-2 and e_w <= 1e-2
    outputs = 4 * (n * (1 + w.hidden) + v * w.hidden) + 4
    assert peak_strip <= ws_bytes + outputs + (64 << 20)
    assert peak_dense >= n * v * 4
    assert np.isfinite(lo)
