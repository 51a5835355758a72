"""The no-allocation LM head (w4a16_lmhead_argmax_noalloc) against the
workspace entry point it shares its kernels with (w4a16_lmhead_argmax).

Both are called through the C ABI (the ctypes binding) on the same seeded
inputs; the argmax indices and the fp32 logits must be bitwise equal.  Two
calls in a row on the library's one scratch array, the second with a smaller
problem, so a stale key left by the first call would show in the second.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import decode_w4a16_affine_amd as w4
import synthetic
from parity import DevWeights, dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.lib()
    yield
    torch.cuda.synchronize()


def run_both(w, x_bits, logits_dtype):
    dw = DevWeights(w)
    x = dev_bf16(x_bits)
    M, N = x.shape[0], w.qw.shape[0]
    ws = torch.empty(max(1, w4.w4a16_lmhead_argmax_workspace_bytes(M, N, w.K)), dtype=torch.uint8, device="cuda")
    ref_am = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    got_am = torch.full((M,), -9, dtype=torch.int32, device="cuda")
    ref_lg = got_lg = None
    if logits_dtype is not None:
        ref_lg = torch.full((M, N), 3.0, dtype=logits_dtype, device="cuda")
        got_lg = torch.full((M, N), -5.0, dtype=logits_dtype, device="cuda")
    w4.w4a16_lmhead_argmax(x, dw.qw, dw.s, dw.b, ref_lg, ref_am, ws)
    w4.w4a16_lmhead_argmax_noalloc(x, dw.qw, dw.s, dw.b, got_lg, got_am)
    torch.cuda.synchronize()
    assert torch.equal(got_am, ref_am), (got_am.tolist(), ref_am.tolist())
    if logits_dtype is not None:
        iv = torch.int32 if logits_dtype == torch.float32 else torch.int16
        assert torch.equal(got_lg.view(iv), ref_lg.view(iv))
    return got_am.cpu().numpy()


def test_noalloc_equals_workspace_entry_point_twice_smaller_second():
    cases = [
        # (M, N, K, logits dtype, bias): the vocabulary head at M = 3, then smaller problems
        (3, 262144, 2560, torch.float32, "exact"),
        (1, 70000, 2560, torch.bfloat16, "noise"),
        (2, 5000, 512, None, "noise"),
    ]
    for i, (M, N, K, dt, bias) in enumerate(cases):
        say(f"no-alloc LM head call {i}: M={M} N={N} K={K} logits={dt}")
        w = synthetic.quantized_weights(N, K, seed=0, tag=(N, 5), bias=bias)
        x = synthetic.activations(M, K, seed=0, tag=(N, 5))
        am = run_both(w, x, dt)
        assert np.all((am >= 0) & (am < N))


def test_noalloc_rejects_problems_beyond_its_scratch():
    # more per-block keys than the built-in scratch holds: refused before any
    # launch, with the scratch status (the shapes are valid; only their size
    # is beyond the array)
    M, K = 8, 64
    N = w4.MAX_N
    need = w4.w4a16_lmhead_argmax_workspace_bytes(M, N, K)
    assert need > w4.NOALLOC_SCRATCH_BYTES
    A16 = 0x10000
    st = w4.lib().w4a16_lmhead_argmax_noalloc(A16, A16, A16, A16, None, 0, A16, M, N, K, 64, None)
    assert st == 7, st
