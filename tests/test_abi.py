"""The C ABI of liblce.so on the host (CPU only, nothing is launched).

Checks that the library loads, exports every function include/lce.h declares,
and rejects bad arguments before enqueuing anything.  Also checks the
strip-width policy and the workspace size formula.
"""
import ctypes
import os
import re

import pytest
import torch

from vocab_projection_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lce_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("liblce.so is not built (python -m vocab_projection_amd.build)")
    return B.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 19
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(B.EXPORTS)


def test_status_strings(lib):
    for code, name in enumerate(["LCE_OK", "LCE_ERR_INVALID_VALUE", "LCE_ERR_UNSUPPORTED",
                                 "LCE_ERR_WORKSPACE", "LCE_ERR_LAUNCH"]):
        assert lib.lce_status_string(code).decode() == name


def P(n=64, h=64, v=1000, dtype=torch.bfloat16, **kw):
    return B.problem(n, h, v, dtype, **kw)


def test_workspace_formula(lib):
    """One strip of round_up(N, 16) x round_up(Vs, 256) elements plus a 256-byte
    header (the strip buffer keeps whole 16-token bands)."""
    p = P(131072, 2048, 151936, strip=8192)
    assert B.lce_workspace_bytes(p) == 256 + 131072 * 8192 * 2
    p = P(256, 128, 1024, torch.float32, strip=256)
    assert B.lce_workspace_bytes(p) == 256 + 256 * 256 * 4
    p = P(100, 64, 1000, strip=300)  # 256-column tiles, 16-token bands
    assert B.lce_workspace_bytes(p) == 256 + 112 * 512 * 2
    p = P(1, 8, 1, strip=1)  # one token: one band of one tile
    assert B.lce_workspace_bytes(p) == 256 + 16 * 256 * 2
    # three tokens, a million vocabulary rows: the forward's partials and state
    # still fit in the one-band strip region
    p = P(3, 8, 1 << 20, strip=256)
    assert B.lce_workspace_bytes(p) == 256 + 16 * 256 * 2


def test_pick_strip_policy(lib):
    n = 131072
    p = P(n, 2048, 151936)
    fixed = 256
    vs = B.lce_pick_strip(p, fixed + n * 2 * 8192)
    assert vs == 8192
    assert B.lce_pick_strip(p, fixed + n * 2 * 8192 - 1) == 8192 - 256
    assert B.lce_pick_strip(p, 0) == -1           # not even one tile fits
    assert B.lce_pick_strip(p, 256 + n * 2 * 256) == 256
    assert B.lce_pick_strip(p, 1 << 50) == 151936  # ceiling: the whole vocabulary
    for budget in (1 << 28, 1 << 30, 3 << 30):
        vs = B.lce_pick_strip(p, budget)
        p2 = P(n, 2048, 151936, strip=vs)
        assert B.lce_workspace_bytes(p2) <= budget
        assert vs % 256 == 0
    bad = P(0, 64, 10)
    assert B.lce_pick_strip(bad, 1 << 20) == -1


def test_problem_validation(lib):
    assert lib.lce_workspace_bytes(ctypes.byref(P(0))) == 0
    assert lib.lce_workspace_bytes(ctypes.byref(P(v=0))) == 0
    assert lib.lce_workspace_bytes(ctypes.byref(P(strip=1001))) == 0
    p = P()
    p.dtype = 7
    assert lib.lce_workspace_bytes(ctypes.byref(p)) == 0
    p = P()
    p.reduction = 5
    assert lib.lce_workspace_bytes(ctypes.byref(p)) == 0
    assert lib.lce_workspace_bytes(ctypes.byref(P(h=12))) == 0          # bf16 needs H % 8 == 0
    assert lib.lce_workspace_bytes(ctypes.byref(P(h=12, dtype=torch.float32))) > 0
    # tile offsets stay below 2^31: H <= 2^20, strip <= 2^21
    assert lib.lce_workspace_bytes(ctypes.byref(P(n=4, h=1 << 20, v=300))) > 0
    assert lib.lce_workspace_bytes(ctypes.byref(P(n=4, h=(1 << 20) + 8, v=300))) == 0
    assert lib.lce_workspace_bytes(ctypes.byref(P(n=4, h=8, v=1 << 23, strip=1 << 21))) > 0
    assert lib.lce_workspace_bytes(ctypes.byref(P(n=4, h=8, v=1 << 23, strip=(1 << 21) + 1))) == 0
    assert B.lce_pick_strip(P(n=1, h=8, v=1 << 24), 1 << 50) == 1 << 21


def _call_fwd(lib, p, ws_bytes, ptrs):
    return lib.lce_forward(ctypes.byref(p), *ptrs[:6], ptrs[6], ws_bytes, None)


def test_errors_are_returned_before_any_launch(lib):
    p = P()
    need = B.lce_workspace_bytes(p)
    fake = 0x10000  # aligned, never dereferenced: every call below fails its checks first
    ok = [fake] * 7
    assert _call_fwd(lib, p, need - 1, ok) == 3                      # workspace too small
    assert _call_fwd(lib, p, need, [fake, None] + [fake] * 5) == 1  # null weight
    assert _call_fwd(lib, p, need, [fake + 2] + [fake] * 6) == 1     # misaligned hidden
    assert _call_fwd(lib, p, need, [fake] * 6 + [None]) == 3         # null workspace
    assert _call_fwd(lib, P(h=12), need, ok) == 2                    # unsupported H
    assert _call_fwd(lib, P(n=-1), need, ok) == 1
    assert lib.lce_forward_fold(ctypes.byref(p), fake, fake, 990, 20, fake, fake, need, None) == 1
    assert lib.lce_forward_fold(ctypes.byref(p), fake, fake, 0, 0, fake, fake, need, None) == 1
    p.strip = 256
    need = B.lce_workspace_bytes(p)
    wide = B.lce_forward_fold_max(p)   # the forward's partials capacity, here the whole V
    assert wide == 1000
    p.vocab = 1 << 20
    wide = B.lce_forward_fold_max(p)
    assert wide >= 256 and wide % 128 == 0
    assert lib.lce_forward_fold(ctypes.byref(p), fake, fake, 0, wide + 1, fake, fake, need,
                                None) == 1
    assert lib.lce_backward_fold(ctypes.byref(p), fake, fake, 0, 257, fake, fake, fake, 0, fake,
                                 fake, need, None) == 1
    p.vocab = 1000
    assert lib.lce_backward_fold(ctypes.byref(p), fake, fake, 0, 10, fake, None, fake, 0, fake,
                                 fake, need, None) == 1
    assert lib.lce_forward_state(ctypes.byref(p), None, fake, need, None) == 1
    assert lib.lce_forward_merge_state(ctypes.byref(p), None, fake, need, None) == 1
    assert lib.lce_forward_state(ctypes.byref(p), fake, fake, need - 1, None) == 3
    assert lib.lce_forward_merge_state(ctypes.byref(P(n=0)), fake, fake, need, None) == 1
    # accumulate is a bit set of LCE_ACC_DHIDDEN (1) and LCE_ACC_DWEIGHT (2); any other bit fails
    for bad_bits in (4, 5, -1):
        assert lib.lce_backward_fold(ctypes.byref(p), fake, fake, 0, 10, fake, fake, fake,
                                     bad_bits, fake, fake, need, None) == 1
    assert lib.lce_backward(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, need,
                            None) == 1


def test_pick_strip_counts_the_whole_workspace(lib):
    """For a handful of tokens the forward's partials and running state, not
    the gradient strip, set the workspace; the picked width must still fit."""
    for n, v, budget in ((1, 1 << 20, 64 << 10), (3, 300000, 40 << 10), (17, 5000, 1 << 16)):
        p = P(n, 64, v)
        vs = B.lce_pick_strip(p, budget)
        assert vs > 0
        assert B.lce_workspace_bytes(P(n, 64, v, strip=vs)) <= budget
        wider = min(vs + 256, v)
        if wider > vs:
            assert B.lce_workspace_bytes(P(n, 64, v, strip=wider)) > budget
    # strip = 0 with nothing fitting the default budget still plans one tile
    big = P(1 << 31, 8, 1000)
    assert B.lce_workspace_bytes(big) == 256 + (1 << 31) * 256 * 2


def test_fused_backward_workspace_plan(lib):
    """The strip-free backward's workspace: header + one 256 x 256 G tile per
    block + fp32 partial copies.  Two sweeps at 131072 tokens and 151936 rows
    need no partial copies (both dimensions have more tiles than the 256
    blocks); one sweep needs copies of d_hidden and d_weight that grow with H."""
    p = P(131072, 2048, 151936, strip=8192)
    two = B.lce_backward_fused_workspace_bytes(p, B.LCE_FUSED_TWO_SWEEPS)
    assert two == 256 + 256 * 256 * 256 * 2
    one = B.lce_backward_fused_workspace_bytes(p, B.LCE_FUSED_ONE_SWEEP)
    assert one > 10 * B.lce_workspace_bytes(p)
    small = P(4096, 512, 32768, strip=8192)
    for mode in (B.LCE_FUSED_ONE_SWEEP, B.LCE_FUSED_TWO_SWEEPS):
        n = B.lce_backward_fused_workspace_bytes(small, mode)
        assert n > 256 and (n - 256) % 256 == 0
    assert lib.lce_backward_fused_workspace_bytes(ctypes.byref(p), 3) == 0
    fake = 0x10000
    assert lib.lce_backward_fused(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, 1,
                                  fake, one - 1, None) == 3
