"""lce_backward_static (the backward with the library's static per-GPU
workspace) against lce_backward with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller problem of the other element type,
so the second call runs on whatever the first left in the static array: both
must give the same bits as lce_backward (the same kernels on the same inputs),
and those must match the oracle within the stated tolerances.  A problem whose
workspace exceeds the array is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

from oracle import lce_oracle as O
from vocab_projection_amd import binding as B
from vocab_projection_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    S.small("static_bf16", 3000, 256, 20000, 4096, ignore_frac=0.1),
    S.small("static_f32_smaller", 700, 132, 3001, 1024, "f32", weight_std=0.2, ignore_frac=0.05),
]


def _inputs(w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    hid, wt, t = S.hidden(w), S.weight(w), S.targets(w)
    return (hid, wt, t, torch.from_numpy(hid).to(DEV).to(dt).contiguous(),
            torch.from_numpy(wt).to(DEV).to(dt).contiguous(), torch.from_numpy(t).to(DEV))


def test_static_workspace_backward_matches_lce_backward():
    for w in CASES:
        hid, wt, t, h, W, tt = _inputs(w)
        p = B.make_problem(h, W, ignore_index=S.IGNORE_INDEX, reduction=w.reduction, strip=w.strip)
        assert B.lce_workspace_bytes(p) <= B.LCE_STATIC_SCRATCH_BYTES
        ws = B.workspace(p, DEV)
        loss = torch.empty(1, dtype=torch.float32, device=DEV)
        lse = torch.empty(w.n_tokens, dtype=torch.float32, device=DEV)
        go = torch.tensor([w.grad_out], dtype=torch.float32, device=DEV)
        B.lce_forward(p, h, W, tt, loss, lse, None, ws)
        dh_ref = torch.empty(h.shape, dtype=torch.float32, device=DEV)
        dw_ref = torch.empty(W.shape, dtype=torch.float32, device=DEV)
        B.lce_backward(p, h, W, tt, lse, go, dh_ref, dw_ref, ws)
        dh = torch.full(h.shape, float("nan"), dtype=torch.float32, device=DEV)
        dw = torch.full(W.shape, float("nan"), dtype=torch.float32, device=DEV)
        B.lce_backward_static(p, h, W, tt, lse, go, dh, dw)
        torch.cuda.synchronize()
        assert torch.equal(dh, dh_ref), w.name
        assert torch.equal(dw, dw_ref), w.name
        ref_dh, ref_dw = O.backward(hid, wt, t, ignore_index=S.IGNORE_INDEX,
                                    reduction=w.reduction, grad_out=w.grad_out)
        for got, ref in ((dh, ref_dh), (dw, ref_dw)):
            g = got.cpu().numpy().astype(np.float64)
            if w.dtype == "f32":
                assert np.abs(g - ref).max() <= 1e-4 * np.abs(ref).max(), w.name
            else:
                assert np.linalg.norm(g - ref) <= 1e-2 * np.linalg.norm(ref), w.name
        print(f"{w.name}: static-workspace backward equals lce_backward bit for bit", flush=True)


def test_static_workspace_refuses_oversized_problem():
    # 20000 tokens x a strip of 8192 bf16 = 328 MB > the 256 MiB array: refused
    # on the host, before anything is enqueued (the pointers are never touched)
    p = B.problem(20000, 64, 10000, torch.bfloat16, strip=8192)
    assert B.lce_workspace_bytes(p) > B.LCE_STATIC_SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.float32, device=DEV)
    with pytest.raises(B.LceError, match="LCE_ERR_WORKSPACE"):
        B.lce_backward_static(p, fake, fake, fake, fake, fake, fake, fake)
