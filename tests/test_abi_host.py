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

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP = range(7)
A16 = 0x10000          # 16-byte aligned fake address
A4 = 0x20004           # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_binding_constants_match_header():
    text = open(HEADER).read()
    for name, value in (("W4A16_MAX_M", w4.MAX_M), ("W4A16_MAX_PREFILL_M", w4.MAX_PREFILL_M)):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == value, name


@pytest.fixture(scope="module")
def L():
    return w4.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(w4.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    assert w4.w4a16_abi_version() == 1
    seen = set()
    for s in range(7):
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
    def mid(ids=A16, M=1, top_k=8, E=64, N=64, K=128, group=64, x_per_slot=0, out=0):
        return L.w4a16_matmul_id(A16, x_per_slot, A16, A16, A16, ids, A16, out, M, top_k, E, N, K, group, None)

    assert mid(group=16) == EUNSUP
    assert mid(M=9) == EUNSUP
    assert mid(top_k=0) == ESHAPE
    assert mid(top_k=65) == ESHAPE
    assert mid(E=0) == ESHAPE
    assert mid(K=96) == ESHAPE
    assert mid(ids=None) == ENULL
    assert mid(ids=A16 + 2) == EALIGN
    assert mid(M=0, ids=None) == OK


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
