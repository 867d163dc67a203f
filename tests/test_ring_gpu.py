"""Ring-DTP's schedule on one GPU: distinct batches meet every vocabulary shard.

The second page's Ring-DTP (section 3.2, appendix C) gives each of P ranks its
own token batch and one vocabulary shard.  Over P steps every batch meets
every shard once (rank r meets shard (r + t) mod P at step t) and folds the
meeting into its own running per-token state; the backward pass replays the
meetings, so a batch's d_hidden accumulates over the shards it meets and a
shard's d_weight over the batches it meets.  Here the P ranks run on one GPU,
step by step, each with its own workspace, state, lse and d_hidden; the
transfers between ranks are what is left out.

Each meeting is one strip-level call (lce_forward_fold / lce_backward_fold;
odd ranks run the backward meeting as two step calls, so that d_weight is
formed by its own GEMM launch rather than the launch it can share with
d_hidden); a shard's weight gradient is written by its first meeting and
added to by the later ones (LCE_ACC_DWEIGHT).  Checked against the oracle:
every batch's loss, lse and d_hidden equal those of that batch alone against
the whole weight, and every shard's d_weight equals the sum over the batches
of their weight gradients, the gradient of the sum of the P losses.  Tolerances as in the
other parity tests: f32 |dloss|/loss <= 1e-5 and max|diff|/max|ref| <= 1e-4,
bf16 |dloss|/loss <= 2e-3 and ||diff||_F/||ref||_F <= 1e-2.
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
    # dtype, H, V, shard boundaries, batch sizes (ragged; ranks differ in size)
    "bf16_p4": ("bf16", 128, 3001, [0, 800, 1500, 2300, 3001], [300, 517, 64, 1000]),
    "f32_p3": ("f32", 68, 1000, [0, 400, 700, 1000], [256, 130, 77]),
    # eight ranks, as on one node
    "bf16_p8": ("bf16", 256, 8 * 1037, [1037 * i for i in range(9)],
                [1000 + 257 * r for r in range(8)]),
}


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def check(dtype, got, ref, what, loss=False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), what
    if loss:
        tol = 1e-5 if dtype == "f32" else 2e-3
        assert abs(got - ref) <= tol * abs(ref), (what, float(got), float(ref))
        return abs(got - ref) / abs(ref)
    if dtype == "f32":
        # max|diff| / max|ref| over the tensor, and the same row by row
        err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert err <= 1e-4, (what, err)
        g2, r2 = np.atleast_2d(got), np.atleast_2d(ref)
        scale = np.abs(r2).max(axis=1)
        diff = np.abs(g2 - r2).max(axis=1)
        assert not np.any(diff[scale == 0] != 0), (what, "zero row")
        if np.any(scale > 0):
            err_rows = float((diff[scale > 0] / scale[scale > 0]).max())
            assert err_rows <= 1e-4, (what, "row by row", err_rows)
    else:
        err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err <= 1e-2, (what, err)
    return err


@pytest.mark.parametrize("case", list(CASES))
def test_ring_schedule_on_one_gpu(case):
    dtype, H, V, bounds, sizes = CASES[case]
    P = len(sizes)
    shards = [(bounds[s], bounds[s + 1] - bounds[s]) for s in range(P)]
    vs = max(w for _, w in shards)
    say(f"ring {case}: P={P} H={H} V={V} shards {[w for _, w in shards]} batches {sizes}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    wgen = S.small(f"{case}_weight", 1, H, V, vs, dtype, weight_std=0.1, seed=900)
    wt = S.weight(wgen)
    batches = [S.small(f"{case}_batch{r}", n, H, V, vs, dtype, weight_std=0.1,
                       ignore_frac=0.1, seed=901 + r) for r, n in enumerate(sizes)]
    hid = [S.hidden(b) for b in batches]
    tgt = [S.targets(b) for b in batches]

    W = torch.from_numpy(wt).to(DEV).to(dt).contiguous()
    ranks = []
    for r in range(P):
        h = torch.from_numpy(hid[r]).to(DEV).to(dt).contiguous()
        p = B.make_problem(h, W, ignore_index=S.IGNORE_INDEX, reduction="mean", strip=vs)
        ranks.append(dict(
            h=h, t=torch.from_numpy(tgt[r]).to(DEV), p=p, ws=B.workspace(p, DEV),
            loss=torch.empty(1, dtype=torch.float32, device=DEV),
            lse=torch.empty(sizes[r], dtype=torch.float32, device=DEV),
            dh=torch.empty(h.shape, dtype=torch.float32, device=DEV),
            go=torch.ones(1, dtype=torch.float32, device=DEV)))
    # Poison d_weight: the first meeting of every shard must overwrite it.
    dw = torch.full((V, H), float("nan"), dtype=torch.float32, device=DEV)

    for k in ranks:
        B.lce_forward_begin(k["p"], k["ws"])
    for step in range(P):
        for r, k in enumerate(ranks):
            v0, vl = shards[(r + step) % P]
            B.lce_forward_fold(k["p"], k["h"], W[v0:v0 + vl], v0, vl, k["t"], k["ws"])
    for k in ranks:
        B.lce_forward_end(k["p"], k["t"], k["loss"], k["lse"], None, k["ws"])
        B.lce_backward_begin(k["p"], k["t"], k["go"], k["ws"])
    for step in range(P):
        for r, k in enumerate(ranks):
            v0, vl = shards[(r + step) % P]
            args = (k["p"], k["h"], W[v0:v0 + vl], v0, vl, k["t"], k["lse"], k["dh"], step > 0,
                    dw[v0:v0 + vl], k["ws"])
            if r % 2 == 0:
                B.lce_backward_fold(*args, accumulate_dw=step > 0)
            else:
                B.lce_backward_fold_steps(*args, B.LCE_STEP_GRAD | B.LCE_STEP_DHIDDEN,
                                          accumulate_dw=step > 0)
                B.lce_backward_fold_steps(*args, B.LCE_STEP_DWEIGHT, accumulate_dw=step > 0)
    torch.cuda.synchronize()

    ref_dw = np.zeros((V, H))
    for r, k in enumerate(ranks):
        loss, lse, _ = O.forward(hid[r], wt, tgt[r], ignore_index=S.IGNORE_INDEX, reduction="mean")
        dh, dwr = O.backward(hid[r], wt, tgt[r], ignore_index=S.IGNORE_INDEX, reduction="mean")
        ref_dw += dwr
        e_loss = check(dtype, k["loss"].item(), loss, f"loss of batch {r}", loss=True)
        got_lse = k["lse"].cpu().numpy().astype(np.float64)
        assert (np.abs(got_lse - lse) / (1.0 + np.abs(lse))).max() <= 2e-5, r
        e_dh = check(dtype, k["dh"].cpu().numpy(), dh, f"dH of batch {r}")
        say(f"  batch {r}: loss err {e_loss:.1e}, dH err {e_dh:.1e}")
    got_dw = dw.cpu().numpy()
    for s, (v0, vl) in enumerate(shards):
        e = check(dtype, got_dw[v0:v0 + vl], ref_dw[v0:v0 + vl], f"dW of shard {s}")
        say(f"  shard {s}: dW err {e:.1e}")
