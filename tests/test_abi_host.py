"""C-ABI checks that need no GPU: the library loads, exports every function
include/w4a16.h declares, and rejects bad arguments before touching HIP.

Pointers used here are fake, non-dereferenced addresses: each call must fail
validation, so nothing is ever launched.
"""
import ctypes
import os
import re

import pytest

import decode_w4a16_affine_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP, ESCRATCH = range(8)
A16 = 0x10000          # 16-byte aligned fake address
A4 = 0x20004           # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_binding_constants_match_header():
    text = open(HEADER).read()
    for name, value in (("W4A16_MAX_M", w4.MAX_M), ("W4A16_MAX_PREFILL_M", w4.MAX_PREFILL_M),
                        ("W4A16_MAX_GROUP", w4.MAX_GROUP)):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == value, name
    for name, value in (("W4A16_MAX_N", w4.MAX_N), ("W4A16_MAX_K", w4.MAX_K)):
        m = re.search(rf"#define {name} \(1 << (\d+)\)", text)
        assert m and 1 << int(m.group(1)) == value, name


@pytest.fixture(scope="module")
def L():
    return w4.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(w4.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_every_declared_probe_symbol_is_exported():
    # the measurement library (include/w4a16_probe.h) the benchmark and the
    # conversion test load
    from decode_w4a16_affine_amd import profiling
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "w4a16_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(w4a16_probe_[a-z0-9_]+)\s*\(", text)))
    assert set(names) == set(profiling.PROBE_EXPORTS)
    P = profiling.probe_lib()
    for n in names:
        assert hasattr(P, n), n
    # invalid arguments are refused before any launch
    assert P.w4a16_probe_bf16_round_check(None, A16, None) != 0
    assert P.w4a16_probe_bf16_round_check(A4, A16, None) != 0
    assert P.w4a16_probe_stream_read(None, 16, A16, 0, 1, None) != 0
    assert P.w4a16_probe_stream_read(A16, 15, A16, 0, 1, None) != 0


def test_abi_version_and_status_strings(L):
    assert w4.w4a16_abi_version() == 2
    seen = set()
    for s in range(8):
        txt = w4.w4a16_status_str(s)
        assert txt and txt not in seen
        seen.add(txt)
    assert w4.w4a16_status_str(99) == "unknown status"


def mm(L, x=A16, qw=A16, s=A16, b=A16, y=A16, out=0, M=1, N=256, K=512, group=64):
    return L.w4a16_matmul(x, qw, s, b, y, out, M, N, K, group, None)


def test_matmul_rejects_bad_arguments(L):
    assert mm(L, group=32) == EUNSUP
    assert mm(L, group=256) == EUNSUP
    assert mm(L, group=128, K=192) == ESHAPE          # K must be a multiple of the group
    assert mm(L, out=2) == EUNSUP
    assert mm(L, M=9) == EUNSUP
    assert mm(L, M=-1) == ESHAPE
    assert mm(L, N=-5) == ESHAPE
    for K in (0, 32, 100, 576 + 8, -64):
        assert mm(L, K=K) == ESHAPE, K
    assert mm(L, x=None) == ENULL
    assert mm(L, qw=None) == ENULL
    assert mm(L, s=None) == ENULL
    assert mm(L, b=None) == ENULL
    assert mm(L, y=None) == ENULL
    assert mm(L, qw=A4) == EALIGN            # packed codes need 16-byte loads
    assert mm(L, x=A16 + 2) == EALIGN
    assert mm(L, x=A4) == EALIGN              # activations are read 16 bytes at a time
    assert mm(L, s=A16 + 1) == EALIGN
    assert mm(L, y=A16 + 2, out=1) == EALIGN  # fp32 output needs 4 bytes


def test_sizes_that_would_overflow_block_counts_are_rejected(L):
    # block counts are (N + rows per block - 1) / rows per block in int, and a
    # wave's byte offsets are 32-bit: N and K beyond the header's limits fail
    # validation before any launch
    big = 2 ** 31 - 1
    assert mm(L, N=big) == ESHAPE
    assert mm(L, N=w4.MAX_N + 1) == ESHAPE
    assert mm(L, N=w4.MAX_N, x=None) == ENULL       # the limit itself passes the size check
    assert mm(L, K=w4.MAX_K + 64) == ESHAPE
    assert mm(L, K=w4.MAX_K, x=None) == ENULL
    assert L.w4a16_lmhead_argmax(A16, A16, A16, A16, None, 0, A16, A16, 1 << 20, 1, big, 512, 64, None) == ESHAPE
    assert L.w4a16_lmhead_argmax_workspace_bytes(1, big, 512, 64) == 0
    assert L.w4a16_matmul_prefill(A16, A16, A16, A16, A16, 0, 100, big, 512, 64, None) == ESHAPE
    assert L.w4a16_matmul_id(A16, 0, A16, A16, A16, A16, A16, 0, 1, 8, 64, big, 512, 64, None) == ESHAPE
    assert L.w4a16_matmul_geglu(A16, A16, A16, A16, A16, 0, 1, 2 ** 29 + 1, 512, 64, None) == ESHAPE
    assert L.w4a16_dequant(A16, A16, A16, None, 0, A16, big, 512, 64, None) == ESHAPE
    assert L.w4a16_gather_rows(A16, A16, A16, A16, 4, A16, big, 512, 64, None) == ESHAPE
    arr = (w4.Matrix * 1)()
    arr[0] = w4.Matrix(A16, A16, A16, A16, big)
    assert L.w4a16_matmul_grouped(A16, arr, 1, 0, 1, 512, 64, None) == ESHAPE


def test_prefill_rejects_bad_arguments(L):
    def pf(x=A16, qw=A16, y=A16, out=0, M=100, N=256, K=512, group=64):
        return L.w4a16_matmul_prefill(x, qw, A16, A16, y, out, M, N, K, group, None)
    assert pf(M=-1) == ESHAPE
    assert pf(M=65537) == EUNSUP
    assert pf(group=32) == EUNSUP
    assert pf(K=100) == ESHAPE
    assert pf(x=A4) == EALIGN
    assert pf(qw=None) == ENULL
    assert pf(out=7) == EUNSUP
    assert pf(x=None, qw=None, y=None, M=0) == OK
    assert pf(x=None, qw=None, y=None, N=0) == OK


def test_geglu_rejects_bad_arguments(L):
    def gg(x=A16, qw=A16, s=A16, h=A16, out=0, M=1, I=3000, K=512, group=64):
        return L.w4a16_matmul_geglu(x, qw, s, s, h, out, M, I, K, group, None)
    assert gg(M=9) == EUNSUP
    assert gg(M=-1) == ESHAPE
    assert gg(I=-1) == ESHAPE
    assert gg(I=1 << 30) == ESHAPE           # 2I overflows
    assert gg(group=32) == EUNSUP
    assert gg(K=100) == ESHAPE
    assert gg(out=3) == EUNSUP
    assert gg(x=None) == ENULL
    assert gg(h=None) == ENULL
    assert gg(qw=A4) == EALIGN
    assert gg(h=A16 + 2, out=1) == EALIGN
    for I in (1, 2048):                       # the K-split form: the same checks
        assert gg(I=I, x=None) == ENULL
        assert gg(I=I, qw=A4) == EALIGN
    assert gg(x=None, qw=None, s=None, h=None, M=0) == OK
    assert gg(x=None, qw=None, s=None, h=None, I=0) == OK


def test_matmul_empty_problems_launch_nothing(L):
    # empty problems succeed even with NULL pointers: nothing is read or written
    assert mm(L, x=None, qw=None, s=None, b=None, y=None, M=0) == OK
    assert mm(L, x=None, qw=None, s=None, b=None, y=None, N=0) == OK


def test_matmul_id_rejects_bad_arguments(L):
    def mid(ids=A16, M=1, top_k=8, E=64, N=64, K=128, group=64, stride=0, out=0):
        return L.w4a16_matmul_id(A16, stride, A16, A16, A16, ids, A16, out, M, top_k, E, N, K, group, None)

    assert mid(group=16) == EUNSUP
    assert mid(M=9) == EUNSUP
    assert mid(top_k=0) == ESHAPE
    assert mid(top_k=65) == ESHAPE
    assert mid(E=0) == ESHAPE
    assert mid(K=96) == ESHAPE
    assert mid(ids=None) == ENULL
    assert mid(ids=A16 + 2) == EALIGN
    assert mid(M=0, ids=None) == OK
    # the per-slot row stride: 0 (shared rows) or >= K and a multiple of 8
    assert mid(stride=128, ids=None) == ENULL
    assert mid(stride=136, ids=None) == ENULL
    for bad in (-128, 8, 120, 130, 2 ** 41):
        assert mid(stride=bad) == ESHAPE, bad


def test_grouped_rejects_bad_arguments(L):
    arr = (w4.Matrix * 3)()
    for i in range(3):
        arr[i] = w4.Matrix(A16, A16, A16, A16, 64)

    def gr(count=3, M=1, K=128, group=64, out=0, x=A16):
        return L.w4a16_matmul_grouped(x, arr, count, out, M, K, group, None)

    assert gr(count=9) == ESHAPE
    assert gr(count=-1) == ESHAPE
    assert gr(K=100) == ESHAPE
    assert gr(group=32) == EUNSUP
    assert gr(M=9) == EUNSUP
    assert gr(x=None) == ENULL
    assert gr(x=A16 + 8) == EALIGN
    arr[1] = w4.Matrix(A4, A16, A16, A16, 64)
    assert gr() == EALIGN
    arr[1] = w4.Matrix(A16, None, A16, A16, 64)
    assert gr() == ENULL
    arr[1] = w4.Matrix(A16, A16, A16, A16, -2)
    assert gr() == ESHAPE
    assert L.w4a16_matmul_grouped(A16, None, 2, 0, 1, 128, 64, None) == ENULL
    arr[1] = w4.Matrix(A16, A16, A16, A16, 64)
    assert gr(count=0) == OK
    assert gr(M=0) == OK


def test_lmhead_workspace_rules(L):
    ws = L.w4a16_lmhead_argmax_workspace_bytes
    assert ws(1, 262144, 2560, 64) > 0
    assert ws(3, 262144, 2560, 64) >= ws(1, 262144, 2560, 64)
    assert ws(1, 262144, 2560, 32) == 0
    assert ws(1, 1000, 2560, 128) == ws(1, 1000, 2560, 64) > 0
    assert ws(1, 262144, 100, 64) == 0
    assert ws(0, 262144, 2560, 64) == 0
    need = ws(1, 1000, 512, 64)

    def lm(wsp=A16, nbytes=need, am=A16, logits=None, M=1, N=1000, K=512, group=64, out=0):
        return L.w4a16_lmhead_argmax(A16, A16, A16, A16, logits, out, am, wsp, nbytes, M, N, K, group, None)

    assert lm(nbytes=need - 1) == EWS
    assert lm(wsp=None) == EWS
    assert lm(wsp=A16 + 4) == EALIGN
    assert lm(am=None) == ENULL
    assert lm(am=A16 + 2) == EALIGN
    assert lm(logits=A16 + 2, out=1) == EALIGN
    assert lm(group=256) == EUNSUP


def test_lmhead_noalloc_validation(L):
    # the same checks as the workspace entry point, and a size limit instead of
    # the workspace: problems needing more keys than the built-in scratch are
    # refused before anything touches HIP
    def na(x=A16, qw=A16, am=A16, logits=None, M=1, N=1000, K=512, group=64, out=0):
        return L.w4a16_lmhead_argmax_noalloc(x, qw, A16, A16, logits, out, am, M, N, K, group, None)

    assert na(group=32) == EUNSUP
    assert na(M=9) == EUNSUP
    assert na(N=2 ** 31 - 1) == ESHAPE
    assert na(K=100) == ESHAPE
    assert na(x=None) == ENULL
    assert na(am=None) == ENULL
    assert na(qw=A4) == EALIGN
    assert na(am=A16 + 2) == EALIGN
    assert na(logits=A16 + 2, out=1) == EALIGN
    assert na(x=None, M=0) == OK
    big = w4.MAX_N
    assert L.w4a16_lmhead_argmax_workspace_bytes(8, big, 64, 64) > w4.NOALLOC_SCRATCH_BYTES
    assert na(M=8, N=big, K=64) == ESCRATCH
    # the 262144-row vocabulary fits the scratch at every M
    for M in range(1, 9):
        assert 0 < L.w4a16_lmhead_argmax_workspace_bytes(M, 262144, 2560, 64) <= w4.NOALLOC_SCRATCH_BYTES, M


def test_dequant_gather_and_pack_reject_bad_arguments(L):
    dq = L.w4a16_dequant
    assert dq(A16, A16, A16, None, 0, A16, 16, 128, 32, None) == EUNSUP
    assert dq(A16, A16, A16, None, 0, A16, 16, 100, 64, None) == ESHAPE
    assert dq(A16, A16, A16, A16, -1, A16, 16, 128, 64, None) == ESHAPE
    assert dq(A16, A16, A16, None, 0, A16 + 4, 16, 128, 64, None) == EALIGN
    assert dq(None, A16, A16, None, 0, A16, 16, 128, 64, None) == ENULL
    assert dq(None, None, None, A16, 0, None, 16, 128, 64, None) == OK      # zero rows requested
    gr = L.w4a16_gather_rows
    assert gr(A16, A16, A16, A16, 4, A16, 16, 128, 32, None) == EUNSUP
    assert gr(A16, A16, A16, A16, 4, A16, 16, 100, 64, None) == ESHAPE
    assert gr(A16, A16, A16, A16, -1, A16, 16, 128, 64, None) == ESHAPE
    assert gr(A4 + 2, A16, A16, A16, 4, A16, 16, 128, 64, None) == EALIGN
    assert gr(A16, A16, A16, A16, 4, A16 + 4, 16, 128, 64, None) == EALIGN
    assert gr(A16, A16, A16, None, 4, A16, 16, 128, 64, None) == ENULL
    assert gr(None, None, None, None, 0, None, 16, 128, 64, None) == OK       # zero rows requested
    pk = L.w4a16_pack
    assert pk(A16, A16, 4, 12, None) == ESHAPE
    assert pk(None, A16, 4, 16, None) == ENULL
    assert pk(A16, A16 + 2, 4, 16, None) == EALIGN
    assert pk(None, None, 0, 16, None) == OK


def test_python_binding_rejects_host_tensors():
    import torch

    x = torch.zeros((1, 64), dtype=torch.bfloat16)
    qw = torch.zeros((4, 8), dtype=torch.int32)
    s = torch.zeros((4, 1), dtype=torch.bfloat16)
    y = torch.zeros((1, 4), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w4.w4a16_matmul(x, qw, s, s, y)
    with pytest.raises(TypeError):
        w4.w4a16_matmul(x.float(), qw, s, s, y)


def test_python_binding_checks_shapes_before_the_library():
    # mis-shaped or mistyped tensors raise before any pointer reaches the
    # library (CPU tensors: a call that got through would fail on the device
    # check instead, with a different message)
    import torch

    bf, i32 = torch.bfloat16, torch.int32
    x = torch.zeros((2, 128), dtype=bf)
    qw = torch.zeros((4, 16), dtype=i32)
    s = torch.zeros((4, 2), dtype=bf)
    y = torch.zeros((2, 4), dtype=bf)

    def raises(fn, *a, match, **k):
        with pytest.raises(ValueError, match=match):
            fn(*a, **k)

    raises(w4.w4a16_matmul, x, qw[:, :8], s, s, y, match="qw must have shape")
    raises(w4.w4a16_matmul, x, qw, s[:, :1], s, y, match="scales must have shape")
    raises(w4.w4a16_matmul, x, qw, s, s[:3], y, match="biases must have shape")
    raises(w4.w4a16_matmul, x, qw, s, s, y[:, :3], match="y must have shape")
    raises(w4.w4a16_matmul, x, qw, s, s, y, group=128, match="scales must have shape")
    raises(w4.w4a16_matmul, x[0], qw, s, s, y, match="x must be 2-D")
    raises(w4.w4a16_matmul, x, qw, s, s, y, match="on the GPU")           # shapes fine: device check
    raises(w4.w4a16_matmul_prefill, x, qw, s, s, y[:1], match="y must have shape")
    raises(w4.w4a16_matmul_geglu, x, qw, s, s, torch.zeros((2, 4), dtype=bf), match="h must have shape")
    raises(w4.w4a16_matmul_geglu, x, qw[:3], s[:3], s[:3], torch.zeros((2, 1), dtype=bf), match="even number")
    raises(w4.w4a16_matmul_grouped, x, [(qw, s, s, y), (qw, s, s, y[:, :2])], match=r"mats\[1\].y")
    # routed: expert stack, ids and the per-slot activation layout
    E, top_k = 3, 2
    eq = torch.zeros((E, 4, 16), dtype=i32)
    es = torch.zeros((E, 4, 2), dtype=bf)
    ids = torch.zeros((2, top_k), dtype=i32)
    yr = torch.zeros((2, top_k, 4), dtype=bf)
    raises(w4.w4a16_matmul_id, x, eq[:, :, :8], es, es, ids, yr, match="qw must have shape")
    raises(w4.w4a16_matmul_id, x, eq, es[:2], es, ids, yr, match="scales must have shape")
    raises(w4.w4a16_matmul_id, x, eq, es, es, ids, yr[:, :1], match="y must have shape")
    raises(w4.w4a16_matmul_id, x[:1], eq, es, es, ids, yr, match="x must have shape")
    raises(w4.w4a16_matmul_id, torch.zeros((2, 3, 128), dtype=bf), eq, es, es, ids, yr, match="x must have shape")
    raises(w4.w4a16_matmul_id, torch.zeros((2, top_k, 256), dtype=bf)[:, :, ::2], eq, es, es, ids, yr,
           match="unit stride")
    raises(w4.w4a16_matmul_id, x, eq, es, es, ids[0], yr, match="ids must be 2-D")
    with pytest.raises(TypeError):
        w4.w4a16_matmul_id(x, eq, es, es, ids.long(), yr)
    # LM head, dequant, gather, pack
    am = torch.zeros((2,), dtype=i32)
    ws = torch.zeros((64,), dtype=torch.uint8)
    raises(w4.w4a16_lmhead_argmax, x, qw, s, s, None, am[:1], ws, match="argmax must have shape")
    raises(w4.w4a16_lmhead_argmax, x, qw, s, s, y[:, :2], am, ws, match="logits must have shape")
    with pytest.raises(TypeError):
        w4.w4a16_lmhead_argmax(x, qw, s, s, None, am, ws.float())
    out = torch.zeros((4, 128), dtype=torch.float32)
    raises(w4.w4a16_dequant, qw, s, s, out[:3], match="out must have shape")
    raises(w4.w4a16_dequant, qw, s, s, out[:2], rows=torch.zeros((3,), dtype=i32), match="out must have shape")
    with pytest.raises(TypeError):
        w4.w4a16_dequant(qw, s, s, out[:2], rows=torch.zeros((2,), dtype=torch.int64))
    raises(w4.w4a16_gather_rows, qw, s, s, torch.zeros((2,), dtype=i32), torch.zeros((2, 64), dtype=bf),
           match="out must have shape")
    raises(w4.w4a16_pack, torch.zeros((4, 128), dtype=torch.uint8), qw[:, :8], match="qw must have shape")
    raises(w4.w4a16_pack, torch.zeros((4, 12), dtype=torch.uint8), qw, match="multiple of 8")
