"""Write the oracle's forward results for the large workloads to tests/golden/.

Calls only the CPU oracle (``oracle/``) and the seeded input generator.  The
GPU parity tests at full size compare sampled gradient rows against the
oracle; a row of dW needs every token's log-sum-exp, which is a full
forward pass over N x V logits in float64 (tens of minutes on a host CPU), so
it is computed once here and stored with a fingerprint of the inputs it was
computed from.

Usage:  python tests/golden/make_golden.py [workload ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import lce_oracle as O  # noqa: E402
from vocab_projection_amd import synthetic as S  # noqa: E402

LARGE = [n for n in S.WORKLOAD_ORDER if n != "tiny_f32"]


def fingerprint(w: S.Workload, hid: np.ndarray | None = None, wt: np.ndarray | None = None):
    """A few generated values that identify the inputs (rows 0 and last of h and W)."""
    rows_h = np.array([0, w.n_tokens - 1])
    rows_w = np.array([0, w.vocab - 1])
    h = hid[rows_h] if hid is not None else S.hidden(w, rows=rows_h)
    ww = wt[rows_w] if wt is not None else S.weight(w, rows=rows_w)
    t = S.targets(w)
    return np.concatenate([h[:, :8].ravel(), ww[:, :8].ravel()]).astype(np.float64), \
        np.array([int(t.astype(np.int64).sum()), int((t == S.IGNORE_INDEX).sum())])


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"{name}.npz")


def make(name: str) -> None:
    w = S.WORKLOADS[name]
    t0 = time.time()
    hid = S.hidden(w)
    wt = S.weight(w)
    t = S.targets(w)
    print(f"{name}: inputs in {time.time() - t0:.1f}s", flush=True)
    t0 = time.time()
    loss, lse, row_loss = O.forward(hid, wt, t, ignore_index=S.IGNORE_INDEX,
                                    reduction=w.reduction, row_chunk=256)
    print(f"{name}: oracle forward in {time.time() - t0:.1f}s loss={loss!r}", flush=True)
    fv, ft = fingerprint(w, hid, wt)
    np.savez_compressed(golden_path(name), loss=np.float64(loss), lse=lse, fp_values=fv,
                        fp_targets=ft)


if __name__ == "__main__":
    for n in sys.argv[1:] or LARGE:
        make(n)
