"""The backward without a strip buffer (lce_backward_fused) against the oracle.

Both forms - one sweep with fixed-order partial copies, and two sweeps with
row ownership - are checked element by element against the oracle's full
backward (float32: max|diff|/max|ref| <= 1e-4 over the tensor and row by
row; bf16: relative Frobenius <= 1e-2), run twice for bit-identical results,
and compared with the strip path (lce_backward) on the same inputs.  Cases
cover ragged token and vocabulary tails (including tails shorter than the
tile engine's three-stage ring, which go one output tile per call), more
token tiles than blocks (two sweeps with no partial copies), and the
4096-token, H = 512, V = 32768 shape the strip path is timed against.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import lce_oracle as O
from vocab_projection_amd import binding as B
from vocab_projection_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    S.small("fused_bf16_ragged", 1000, 200, 3001, 1024, ignore_frac=0.1),
    S.small("fused_f32_ragged", 300, 132, 777, 256, "f32", weight_std=0.2, ignore_frac=0.05),
    # tails of 5 tokens and 40 vocabulary rows: K shorter than the ring
    S.small("fused_bf16_short_tails", 517, 64, 2600, 512, reduction="sum", grad_out=0.37,
            target_law="zipf"),
    # 260 token tiles and 274 vocabulary tiles: two sweeps own whole rows
    S.small("fused_bf16_many_tiles", 66560, 64, 70000, 8192, ignore_frac=0.05),
    S.small("fused_bf16_n4k_h512_v32k", 4096, 512, 32768, 8192, weight_std=0.02,
            ignore_frac=0.1),
]


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def check(w, got, ref, what):
    got = got.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), what
    if w.dtype == "f32":
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err <= 1e-4, (what, err)
        scale = np.abs(ref).max(axis=1)
        diff = np.abs(got - ref).max(axis=1)
        assert not np.any(diff[scale == 0] != 0), what
        rows = float((diff[scale > 0] / scale[scale > 0]).max())
        assert rows <= 1e-4, (what, "row by row", rows)
    else:
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= 1e-2, (what, err)
    return err


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_fused_backward_matches_oracle(w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    hid, wt, t = S.hidden(w), S.weight(w), S.targets(w)
    h = torch.from_numpy(hid).to(DEV).to(dt).contiguous()
    W = torch.from_numpy(wt).to(DEV).to(dt).contiguous()
    tt = torch.from_numpy(t).to(DEV)
    p = B.make_problem(h, W, ignore_index=S.IGNORE_INDEX, reduction=w.reduction, strip=w.strip)
    ws = B.workspace(p, DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    lse = torch.empty(w.n_tokens, dtype=torch.float32, device=DEV)
    go = torch.tensor([w.grad_out], dtype=torch.float32, device=DEV)
    B.lce_forward(p, h, W, tt, loss, lse, None, ws)
    dh_s = torch.empty(h.shape, dtype=torch.float32, device=DEV)
    dw_s = torch.empty(W.shape, dtype=torch.float32, device=DEV)
    B.lce_backward(p, h, W, tt, lse, go, dh_s, dw_s, ws)
    ref_dh, ref_dw = O.backward(hid, wt, t, ignore_index=S.IGNORE_INDEX, reduction=w.reduction,
                                grad_out=w.grad_out)
    for name, mode in B.FUSED_MODES.items():
        fws = torch.full((B.lce_backward_fused_workspace_bytes(p, mode),), 255, dtype=torch.uint8,
                         device=DEV)
        outs = []
        for _ in range(2):
            dh = torch.full(h.shape, float("nan"), dtype=torch.float32, device=DEV)
            dw = torch.full(W.shape, float("nan"), dtype=torch.float32, device=DEV)
            B.lce_backward_fused(p, h, W, tt, lse, go, dh, dw, mode, fws)
            outs.append((dh, dw))
        torch.cuda.synchronize()
        (dh, dw), (dh2, dw2) = outs
        assert torch.equal(dh, dh2) and torch.equal(dw, dw2), (w.name, name, "not deterministic")
        e1 = check(w, dh, ref_dh, f"{name} dH")
        e2 = check(w, dw, ref_dw, f"{name} dW")
        # against the strip path on the same inputs
        tol = 1e-5 if w.dtype == "f32" else 2e-3
        for a, b in ((dh, dh_s), (dw, dw_s)):
            assert (a - b).norm().item() <= tol * b.norm().item(), (w.name, name)
        say(f"{w.name} {name}: dH err {e1:.2e}, dW err {e2:.2e}, workspace "
            f"{fws.numel() / 1e6:.1f} MB (strip path {ws.numel() / 1e6:.1f} MB)")
        del fws
