"""Strip-wise linear cross-entropy for AMD MI355X (gfx950).

loss = CE(h . W^T, targets) and its gradients, computed by hand-written HIP
kernels in liblce.so without holding the N x V logits.  The library is loaded
on first use; building it is ``python -m vocab_projection_amd.build``.
"""
from .binding import (  # noqa: F401
    LceError,
    LinearCrossEntropy,
    backward,
    forward,
    lce_backward,
    lce_backward_begin,
    lce_backward_fold,
    lce_forward,
    lce_forward_begin,
    lce_forward_end,
    lce_forward_fold,
    lce_pick_strip,
    lce_workspace_bytes,
    make_problem,
    problem,
    workspace,
)
