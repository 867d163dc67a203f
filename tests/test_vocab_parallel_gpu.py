"""Vocabulary-parallel cross-entropy on one GPU: shards of the vocabulary, one batch.

The second page (section 5) contrasts Ring-DTP with a vocabulary-parallel
reduction that keeps the whole batch on every device; the first page's
full-logits formula counts the logits of one such vocab_partition.  Here P
devices are emulated on one GPU: device r holds the whole batch and the
vocabulary rows of shard r, folds them (in strips) into its own running state
in its own workspace, and exports that state (lce_forward_state).  The
states are then merged token by token (lce_forward_merge_state) into one
workspace, in two different orders, as an all-gather or a ring would, and
finalised.  The backward pass needs the merged lse on every device: each
runs lce_backward_begin and lce_backward_fold over its own shard only, and
the devices' d_hidden are summed (the all-reduce); d_weight rows stay with
their shard.  Checked against the oracle for the whole vocabulary at the
other parity tests' tolerances, and the two merge orders against each other.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import lce_oracle as O
from vocab_projection_amd import binding as B
from vocab_projection_amd import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    # dtype, N, H, V, shard boundaries, strip width within a shard, reduction
    "bf16_p4": ("bf16", 700, 128, 5000, [0, 1200, 2500, 3700, 5000], 1024, "mean"),
    "f32_p3": ("f32", 333, 68, 1000, [0, 257, 700, 1000], 256, "sum"),
    # a shard whose tokens' targets all lie elsewhere, and one shard per 256-row tile
    "bf16_p8_zipf": ("bf16", 1500, 64, 2048, [256 * i for i in range(9)], 256, "mean"),
}


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def strips(v0, v1, vs):
    return [(a, min(vs, v1 - a)) for a in range(v0, v1, vs)]


def check(dtype, got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), what
    if dtype == "f32":
        err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert err <= 1e-4, (what, err)
    else:
        err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err <= 1e-2, (what, err)
    return err


@pytest.mark.parametrize("case", list(CASES))
def test_vocab_parallel_state_merge(case):
    dtype, N, H, V, bounds, vs, reduction = CASES[case]
    P = len(bounds) - 1
    say(f"vocab-parallel {case}: P={P} N={N} H={H} V={V} shards {np.diff(bounds).tolist()}")
    law = "zipf" if "zipf" in case else "uniform"
    w = S.small(case, N, H, V, vs, dtype, weight_std=0.1, ignore_frac=0.1, target_law=law,
                reduction=reduction, grad_out=0.5)
    hid, wt, tg = S.hidden(w), S.weight(w), S.targets(w)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    h = torch.from_numpy(hid).to(DEV).to(dt).contiguous()
    W = torch.from_numpy(wt).to(DEV).to(dt).contiguous()
    t = torch.from_numpy(tg).to(DEV)
    p = B.make_problem(h, W, ignore_index=S.IGNORE_INDEX, reduction=reduction, strip=vs)

    # forward: every device folds its own shard and exports its state
    ws = [B.workspace(p, DEV) for _ in range(P)]
    states = []
    for r in range(P):
        B.lce_forward_begin(p, ws[r])
        for v0, vl in strips(bounds[r], bounds[r + 1], vs):
            B.lce_forward_fold(p, h, W[v0:v0 + vl], v0, vl, t, ws[r])
        st = torch.empty(3 * N, dtype=torch.float32, device=DEV)
        B.lce_forward_state(p, st, ws[r])
        states.append(st)

    results = []
    for home, order in ((0, list(range(1, P))), (P - 1, list(range(P - 2, -1, -1)))):
        # a fresh copy of the home device's state, then the others in `order`
        acc = B.workspace(p, DEV)
        B.lce_forward_begin(p, acc)
        B.lce_forward_merge_state(p, states[home], acc)
        for r in order:
            B.lce_forward_merge_state(p, states[r], acc)
        loss = torch.empty(1, dtype=torch.float32, device=DEV)
        lse = torch.empty(N, dtype=torch.float32, device=DEV)
        row_loss = torch.empty(N, dtype=torch.float32, device=DEV)
        B.lce_forward_end(p, t, loss, lse, row_loss, acc)
        results.append((loss, lse, row_loss))
    torch.cuda.synchronize()

    ref_loss, ref_lse, ref_row = O.forward(hid, wt, tg, ignore_index=S.IGNORE_INDEX,
                                           reduction=reduction)
    tol = 1e-5 if dtype == "f32" else 2e-3
    for loss, lse, row_loss in results:
        assert abs(loss.item() - ref_loss) <= tol * abs(ref_loss), (loss.item(), ref_loss)
        got = lse.cpu().numpy().astype(np.float64)
        assert (np.abs(got - ref_lse) / (1.0 + np.abs(ref_lse))).max() <= 2e-5
        np.testing.assert_allclose(row_loss.cpu().numpy(), ref_row, rtol=1e-4, atol=1e-3)
    (l0, s0, _), (l1, s1, _) = results
    assert abs(l0.item() - l1.item()) <= 1e-6 * abs(l0.item())
    np.testing.assert_allclose(s0.cpu().numpy(), s1.cpu().numpy(), rtol=1e-6, atol=1e-6)

    # backward: every device its own shard, with the merged lse; d_hidden summed
    lse = results[0][1]
    go = torch.tensor([w.grad_out], dtype=torch.float32, device=DEV)
    dh_sum = torch.zeros((N, H), dtype=torch.float32, device=DEV)
    dw = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)
    for r in range(P):
        dh_r = torch.empty((N, H), dtype=torch.float32, device=DEV)
        B.lce_backward_begin(p, t, go, ws[r])
        for k, (v0, vl) in enumerate(strips(bounds[r], bounds[r + 1], vs)):
            B.lce_backward_fold(p, h, W[v0:v0 + vl], v0, vl, t, lse, dh_r, k > 0,
                                dw[v0:v0 + vl], ws[r])
        dh_sum += dh_r
    torch.cuda.synchronize()
    ref_dh, ref_dw = O.backward(hid, wt, tg, ignore_index=S.IGNORE_INDEX, reduction=reduction,
                                grad_out=w.grad_out)
    e_dh = check(dtype, dh_sum.cpu().numpy(), ref_dh, "dH")
    e_dw = check(dtype, dw.cpu().numpy(), ref_dw, "dW")
    say(f"  loss {results[0][0].item():.6f} vs {ref_loss:.6f}; dH err {e_dh:.1e}; dW err {e_dw:.1e}")
