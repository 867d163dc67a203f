"""CPU oracle for the linear cross-entropy: loss = CE(h . W^T, targets).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the tests, the package smoke check and the CPU
baseline leg of the benchmark do.  It shares no code with the GPU path.

What it computes, and from where
--------------------------------
The method on the pages ("Linear CE" in *Running 128K-Sequence MoE RL on 32
H100s*, section "Linear CE: Avoiding Materialization of Full Logits"; Ring-DTP
in *Flattening Every Memory Peak in Long-Context Mixture-of-Experts Training*,
sections 2 and 3.2 and appendix C) changes only the order of computation of
softmax cross-entropy over the vocabulary projection: an exact operator must
return the forward values and the gradients of the implementation it
replaces (section 2 of the second page).  The oracle is therefore that
replaced implementation written out: it materialises every logit of a row in
float64, takes a textbook two-pass log-sum-exp, and forms the gradients of
softmax minus one-hot.  It folds nothing and keeps no running state; rows are
processed in independent chunks only to bound host memory, which the
definition permits because the loss is a sum of per-row terms.

Readings where the pages are silent (each also listed in the design notes):
  * no bias, logit scale, softcap, label smoothing or z-loss;
  * a row whose target equals ``ignore_index`` contributes 0 to the loss, is
    left out of the mean's denominator and gets zero gradient;
  * mean reduction divides by the number of non-ignored rows (0/0 = NaN when
    every row is ignored; the gradients are then 0);
  * a non-ignored target outside [0, V) is a caller error (raises here);
  * grad_out is the upstream gradient of the reduced scalar loss.

All arithmetic is float64 on the float32 (or bf16-valued) inputs.
Every function is pinned by the CPU tests (brute force against an independent
library evaluation, finite differences and closed forms); none is unpinned.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


def logits(hidden: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """z[i, v] = sum_k h[i, k] * W[v, k]: the full logits of the given rows."""
    return _f64(hidden) @ _f64(weight).T


def _check_targets(targets: np.ndarray, vocab: int, ignore_index: int) -> np.ndarray:
    t = np.asarray(targets, dtype=np.int64)
    valid = t != ignore_index
    bad = valid & ((t < 0) | (t >= vocab))
    if bad.any():
        raise ValueError(f"target out of range at rows {np.nonzero(bad)[0][:8].tolist()}")
    return valid


def row_terms(hidden_rows: np.ndarray, weight: np.ndarray, targets_rows: np.ndarray,
              ignore_index: int):
    """Per-row log-sum-exp, target logit and loss term of the given rows.

    lse_i = m_i + log(sum_v exp(z_iv - m_i)) with m_i = max_v z_iv (two passes
    over the materialised row); loss_i = lse_i - z_{i, t_i}, or 0 for an ignored
    row.  Returns (lse, z_target, row_loss, valid).
    """
    z = logits(hidden_rows, weight)
    valid = _check_targets(targets_rows, weight.shape[0], ignore_index)
    m = z.max(axis=1)
    s = np.exp(z - m[:, None]).sum(axis=1)
    lse = m + np.log(s)
    idx = np.where(valid, np.asarray(targets_rows, dtype=np.int64), 0)
    z_target = np.where(valid, z[np.arange(z.shape[0]), idx], np.nan)
    row_loss = np.where(valid, lse - np.where(valid, z_target, 0.0), 0.0)
    return lse, z_target, row_loss, valid


def reduce_loss(row_loss: np.ndarray, valid: np.ndarray, reduction: str) -> float:
    """Sum of the row terms, divided by the number of valid rows for "mean"."""
    total = float(np.sum(row_loss, dtype=F64))
    if reduction == "sum":
        return total
    if reduction == "mean":
        n_valid = int(np.count_nonzero(valid))
        return total / n_valid if n_valid else float("nan")
    raise ValueError(f"unknown reduction {reduction!r}")


def forward(hidden: np.ndarray, weight: np.ndarray, targets: np.ndarray, *,
            ignore_index: int = -100, reduction: str = "mean", row_chunk: int = 512):
    """Loss, per-row lse and per-row loss over every row of ``hidden``.

    Returns (loss, lse[N], row_loss[N]).
    """
    n = hidden.shape[0]
    w64 = _f64(weight)  # converted once, not per chunk
    lse = np.empty(n, dtype=F64)
    row_loss = np.empty(n, dtype=F64)
    valid = np.empty(n, dtype=bool)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        a, _, c, d = row_terms(hidden[r0:r1], w64, targets[r0:r1], ignore_index)
        lse[r0:r1], row_loss[r0:r1], valid[r0:r1] = a, c, d
    return reduce_loss(row_loss, valid, reduction), lse, row_loss


def grad_scale(targets: np.ndarray, *, ignore_index: int, reduction: str,
               grad_out: float) -> np.ndarray:
    """d loss / d row_loss_i: grad_out (sum) or grad_out / n_valid (mean); 0 if ignored."""
    valid = np.asarray(targets) != ignore_index
    if reduction == "sum":
        g = float(grad_out)
    elif reduction == "mean":
        n_valid = int(np.count_nonzero(valid))
        g = float(grad_out) / n_valid if n_valid else 0.0
    else:
        raise ValueError(f"unknown reduction {reduction!r}")
    return np.where(valid, g, 0.0).astype(F64)


def logit_grad(z: np.ndarray, lse: np.ndarray, targets_rows: np.ndarray,
               scale_rows: np.ndarray) -> np.ndarray:
    """G[i, v] = d loss / d z_iv = scale_i * (softmax_iv - [v == t_i]).

    Ignored rows have scale 0 and so a zero row of G.
    """
    p = np.exp(z - _f64(lse)[:, None])
    g = _f64(scale_rows)[:, None] * p
    t = np.asarray(targets_rows, dtype=np.int64)
    rows = np.nonzero((t >= 0) & (t < z.shape[1]))[0]
    g[rows, t[rows]] -= _f64(scale_rows)[rows]
    return g


def backward(hidden: np.ndarray, weight: np.ndarray, targets: np.ndarray, *,
             ignore_index: int = -100, reduction: str = "mean", grad_out: float = 1.0,
             row_chunk: int = 512):
    """Gradients (dH [N,H], dW [V,H]) of the reduced loss times grad_out.

    dH = G . W and dW = G^T . h, with G from ``logit_grad`` over the full logits.
    """
    n = hidden.shape[0]
    _check_targets(targets, weight.shape[0], ignore_index)
    scale = grad_scale(targets, ignore_index=ignore_index, reduction=reduction,
                       grad_out=grad_out)
    w64 = _f64(weight)
    d_hidden = np.empty((n, hidden.shape[1]), dtype=F64)
    d_weight = np.zeros(weight.shape, dtype=F64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        h64 = _f64(hidden[r0:r1])
        z = h64 @ w64.T
        m = z.max(axis=1)
        lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        g = logit_grad(z, lse, targets[r0:r1], scale[r0:r1])
        d_hidden[r0:r1] = g @ w64
        d_weight += g.T @ h64
    return d_hidden, d_weight


def hidden_grad_rows(hidden_rows: np.ndarray, weight: np.ndarray, targets_rows: np.ndarray,
                     scale_rows: np.ndarray) -> np.ndarray:
    """dH for the given rows only (each row of dH needs only its own logits)."""
    z = logits(hidden_rows, weight)
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return logit_grad(z, lse, targets_rows, scale_rows) @ _f64(weight)


def weight_grad_rows(hidden: np.ndarray, weight_rows: np.ndarray, vocab_ids: np.ndarray,
                     targets: np.ndarray, lse: np.ndarray, scale: np.ndarray,
                     row_chunk: int = 8192) -> np.ndarray:
    """dW for the given vocabulary rows: dW_v = sum_i G[i, v] * h_i.

    Needs every row's lse (from ``forward`` of this oracle) and the per-row
    scale from ``grad_scale``.  Only the logits of the requested columns are formed.
    """
    ids = np.asarray(vocab_ids, dtype=np.int64)
    w64 = _f64(weight_rows)
    out = np.zeros((ids.size, hidden.shape[1]), dtype=F64)
    t_all = np.asarray(targets, dtype=np.int64)
    for r0 in range(0, hidden.shape[0], row_chunk):
        r1 = min(hidden.shape[0], r0 + row_chunk)
        h64 = _f64(hidden[r0:r1])
        z = h64 @ w64.T  # [rows, len(ids)]
        p = np.exp(z - _f64(lse[r0:r1])[:, None])
        sc = _f64(scale[r0:r1])
        g = sc[:, None] * p
        onehot = t_all[r0:r1, None] == ids[None, :]
        g -= np.where(onehot, sc[:, None], 0.0)
        out += g.T @ h64
    return out


def logits_bytes(local_tokens: int, vocab_partition: int, bytes_per_element: int = 4) -> int:
    """Bytes of fully materialised logits: local_tokens * vocab_partition * element size.

    The memory estimate of the Linear CE section of the first page (the
    formula before Figure 5), which the strip fold avoids.
    """
    return int(local_tokens) * int(vocab_partition) * int(bytes_per_element)
