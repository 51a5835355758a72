"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every input is seeded and synthetic (module ``synthetic``); no expected value
comes from the GPU.  Each test prints the case it is about to run.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import decode_w4a16_affine_amd as w4
import synthetic
from parity import (DevWeights, check_argmax, check_bf16, check_f32, dev_bf16, dev_i32, dev_qw, host_bits,
                    host_f32, oracle_qmm, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.lib()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def run_mm(dw, x_bits, N, f32=False):
    x = dev_bf16(x_bits)
    y = torch.empty((x.shape[0], N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    w4.w4a16_matmul(x, dw.qw, dw.s, dw.b, y)
    torch.cuda.synchronize()
    return host_f32(y) if f32 else host_bits(y)


def full_check(orc, w, x_bits, y64, absy, what):
    dw = DevWeights(w)
    y32 = run_mm(dw, x_bits, w.qw.shape[0], f32=True)
    yb = run_mm(dw, x_bits, w.qw.shape[0], f32=False)
    rel = check_f32(y32, y64, absy, what)
    ex = check_bf16(orc, yb, y64, absy, w.K, what)
    say(f"  {what}: max |err|/sum|wx| = {rel:.2e}, bf16 exempt {ex}/{yb.size}")
    # bf16 output is the RNE of the fp32 output, bit for bit
    assert np.array_equal(yb, synthetic.bf16_bits(y32)), what
    return dw, y32, yb


# ---------------------------------------------------------------------------
# Layout and dequantization
# ---------------------------------------------------------------------------

def test_pack_matches_oracle(orc):
    for (N, K) in [(37, 264), (5, 8), (256, 512)]:
        say(f"pack N={N} K={K}")
        codes = synthetic.random_codes(N, K, seed=N)
        qw = w4.pack(torch.from_numpy(codes).cuda())
        torch.cuda.synchronize()
        got = qw.cpu().numpy().view(np.uint32)
        assert np.array_equal(got, orc.pack_rows(codes))


def crafted_scales(N, G, seed):
    """bf16 scale/bias patterns over a wide range: signs, zero, subnormal, |s| >= 2^100."""
    g = np.random.default_rng(seed)
    e_s = g.integers(90, 160, size=(N, G))
    e_b = g.integers(90, 160, size=(N, G))
    s = ((g.integers(0, 2, size=(N, G)) << 15) | (e_s << 7) | g.integers(0, 128, size=(N, G))).astype(np.uint16)
    b = ((g.integers(0, 2, size=(N, G)) << 15) | (e_b << 7) | g.integers(0, 128, size=(N, G))).astype(np.uint16)
    s[0, 0] = 0x0000
    s[0, 1 % G] = 0x8000
    s[1 % N, 0] = 0x0003                      # subnormal scale
    s[2 % N, 0] = 0x7180                      # 2^100: takes the plain path
    s[3 % N, 0] = 0xF1C0                      # -1.5 * 2^100
    b[3 % N, 0] = 0x0001
    return s, b


def test_dequant_bit_exact(orc):
    for (N, K, kind) in [(256, 512, "config"), (64, 2560, "crafted"), (9, 192, "crafted")]:
        say(f"dequant N={N} K={K} {kind}")
        w = synthetic.quantized_weights(N, K, seed=N + K)
        if kind == "crafted":
            w.scales, w.biases = crafted_scales(N, K // 64, seed=N)
        got = w4.dequant(dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases))
        torch.cuda.synchronize()
        ref = orc.dequant_rows(w.qw, w.scales, w.biases, K)
        assert np.array_equal(host_f32(got).view(np.uint32), ref.view(np.uint32))
    say("dequant row gather with an out-of-range row")
    w = synthetic.quantized_weights(40, 320, seed=5)
    rows = np.array([39, 0, 17, 40, -1, 17], dtype=np.int32)
    got = host_f32(w4.dequant(dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases), rows=dev_i32(rows)))
    ref = orc.dequant_rows(w.qw, w.scales, w.biases, 320, rows=[39, 0, 17, 17])
    assert np.array_equal(got[[0, 1, 2, 5]].view(np.uint32), ref.view(np.uint32))
    assert np.isnan(got[3]).all() and np.isnan(got[4]).all()


def test_gather_rows_bit_exact(orc):
    # embedding-style lookup: selected rows, repeats, any order, to bf16
    for (N, K, kind) in [(300, 2560, "config"), (64, 2560, "crafted"), (9, 192, "crafted"), (5000, 64, "config")]:
        say(f"gather rows N={N} K={K} {kind}")
        w = synthetic.quantized_weights(N, K, seed=N + K + 1)
        if kind == "crafted":
            w.scales, w.biases = crafted_scales(N, K // 64, seed=N + 1)
        rows = np.random.default_rng(N).integers(0, N, size=37).astype(np.int32)
        rows[:3] = [N - 1, 0, N - 1]
        got = host_bits(w4.gather_rows(dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases), dev_i32(rows)))
        torch.cuda.synchronize()
        ref = orc.f64_to_bf16(orc.dequant_rows(w.qw, w.scales, w.biases, K, rows=rows).astype(np.float64))
        assert np.array_equal(got, ref), (N, K, kind)
    say("gather rows: out-of-range rows give NaN rows, the others are untouched by them")
    w = synthetic.quantized_weights(40, 320, seed=6)
    rows = np.array([39, 40, -1, 0, 2147483647, 17], dtype=np.int32)
    got = host_bits(w4.gather_rows(dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases), dev_i32(rows)))
    ref = orc.f64_to_bf16(orc.dequant_rows(w.qw, w.scales, w.biases, 320, rows=[39, 0, 17]).astype(np.float64))
    assert np.array_equal(got[[0, 3, 5]], ref)
    assert (got[[1, 2, 4]] == 0x7FC0).all()


# ---------------------------------------------------------------------------
# Dense product: the five workloads and their edges
# ---------------------------------------------------------------------------

def test_tiny_config(orc):
    say("tiny qmv M=1 N=256 K=512 seed 0")
    w = synthetic.quantized_weights(256, 512, seed=0)
    x = synthetic.activations(1, 512, seed=0)
    y64, absy = orc.qmm(x, w.qw, w.scales, w.biases)
    full_check(orc, w, x, y64, absy, "tiny")


@pytest.mark.parametrize("name", ["q", "k", "gate_up", "down"])
def test_decode_projections_and_verify_batches(orc, name):
    N, K = synthetic.PROJECTIONS[name]
    tag = (list(synthetic.PROJECTIONS).index(name),)
    w = synthetic.quantized_weights(N, K, seed=0, tag=tag)
    x5 = synthetic.activations(5, K, seed=0, tag=tag)
    say(f"decode projection {name} N={N} K={K}: oracle")
    y64, absy = oracle_qmm(orc, x5, w)
    dw = None
    singles32, singlesb = [], []
    for m in range(5):
        say(f"  {name} M=1 row {m}")
        dw, y32, yb = full_check(orc, w, x5[m:m + 1], y64[m:m + 1], absy[m:m + 1], f"{name} M=1 row{m}")
        singles32.append(y32[0]); singlesb.append(yb[0])
    for M in synthetic.VERIFY_M:
        say(f"  {name} verify M={M}")
        _, y32, yb = full_check(orc, w, x5[:M], y64[:M], absy[:M], f"{name} M={M}")
        for m in range(M):   # batch invariance: bitwise equal to the 1-row call
            assert np.array_equal(y32[m].view(np.uint32), singles32[m].view(np.uint32)), (name, M, m)
            assert np.array_equal(yb[m], singlesb[m]), (name, M, m)


# (4200, 4672) and (4500, 7680): one row group per row, walked in several
# K-tiles (two full tiles and a ragged tail; three full tiles: the
# double-buffered walk); (16400, 576) and (16390, 2560): N >= 16384, where the
# rows per lane and the tile length change with M (16390 rows at two rows per
# lane: 512 blocks of 32 rows and a 6-row tail block); (1003, 6208): a K-split
# row whose blocks hold two row sets at M = 3, with a ragged last block, and
# whose one-chunk tiles are walked with the next tile in flight from M = 2;
# (1000, 4096) and (77, 8256): the same walk in the shorter K-split class;
# (2049, 5120) and (2600, 6208): K-split grids past one round over the CUs at
# two rows per lane, ending in one-row-per-lane blocks (a 1-row and a 4-row
# tail)
RAGGED = [(8, 64), (10, 192), (37, 576), (300, 2112), (4097, 640), (5000, 320), (4096, 2560), (61, 2560), (300, 5120),
          (2049, 5120), (4200, 4672), (4500, 7680), (16400, 576), (16390, 2560), (1003, 6208), (1000, 4096),
          (77, 8256), (2600, 6208)]


@pytest.mark.parametrize("N,K", RAGGED)
def test_every_M_ragged_shapes_batch_invariant(orc, N, K):
    w = synthetic.quantized_weights(N, K, seed=N * 7 + K)
    x = synthetic.activations(8, K, seed=N + K)
    say(f"ragged N={N} K={K}: oracle")
    y64, absy = oracle_qmm(orc, x, w)
    dw = DevWeights(w)
    ref32 = None
    for M in range(1, 9):
        say(f"  ragged N={N} K={K} M={M}")
        y32 = run_mm(dw, x[:M], N, f32=True)
        check_f32(y32, y64[:M], absy[:M], f"N={N} K={K} M={M}")
        yb = run_mm(dw, x[:M], N, f32=False)
        check_bf16(orc, yb, y64[:M], absy[:M], K, f"N={N} K={K} M={M}")
        if M == 1:
            ref32 = [run_mm(dw, x[m:m + 1], N, f32=True)[0] for m in range(8)]
        for m in range(M):
            assert np.array_equal(y32[m].view(np.uint32), ref32[m].view(np.uint32)), (N, K, M, m)


@pytest.mark.parametrize("M", [1, 5, 8])
def test_long_reduction_segments(orc, M):
    # K beyond one LDS segment for every M, with a ragged final segment
    N, K = 300, 16384 + 3 * 64
    w = synthetic.quantized_weights(N, K, seed=77)
    x = synthetic.activations(8, K, seed=78)
    rows = np.arange(0, N, 3, dtype=np.int32)
    say(f"long K={K} M={M}: oracle on {len(rows)} rows")
    y64, absy = oracle_qmm(orc, x[:M], w, rows=rows)
    dw = DevWeights(w)
    y32 = run_mm(dw, x[:M], N, f32=True)
    check_f32(y32[:, rows], y64, absy, f"long K M={M}")
    yb = run_mm(dw, x[:M], N)
    check_bf16(orc, yb[:, rows], y64, absy, K, f"long K M={M}")
    for m in range(M):
        y1 = run_mm(dw, x[m:m + 1], N, f32=True)
        assert np.array_equal(y1[0].view(np.uint32), y32[m].view(np.uint32)), m


_SQUARE = {}


def square_case(orc):
    """The 16384 x 16384 workload and the oracle's outputs for all of its rows
    at the eight activation rows (row m depends on x[m] alone, so the M = 1
    and 4 calls compare with the first rows)."""
    if not _SQUARE:
        N = K = 16384
        w = synthetic.quantized_weights(N, K, seed=0, tag=(16384,))
        x = synthetic.activations(8, K, seed=0, tag=(16384,))
        say(f"square 16384^2: oracle on all {N} rows, M=8 (16 threads)")
        y64, absy = oracle_qmm(orc, x, w, workers=16)
        _SQUARE.update(w=w, x=x, y64=y64, absy=absy, dw=DevWeights(w))
    return _SQUARE


@pytest.mark.parametrize("M", synthetic.SQUARE["M"])
def test_square_16384(orc, M):
    N = K = 16384
    c = square_case(orc)
    x, dw = c["x"], c["dw"]
    y64, absy = c["y64"][:M], c["absy"][:M]
    say(f"square 16384^2 M={M}: every output against the oracle")
    y32 = run_mm(dw, x[:M], N, f32=True)
    check_f32(y32, y64, absy, f"square M={M}")
    yb = run_mm(dw, x[:M], N)
    check_bf16(orc, yb, y64, absy, K, f"square M={M}")
    assert np.array_equal(yb, synthetic.bf16_bits(y32))
    if M > 1:
        for m in range(M):
            y1 = run_mm(dw, x[m:m + 1], N, f32=True)
            assert np.array_equal(y1[0].view(np.uint32), y32[m].view(np.uint32)), m


def test_closed_forms_on_gpu(orc):
    say("closed forms: identity-like weights copy x")
    N, K, M = 64, 128, 3
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[np.arange(N), np.arange(N)] = 1
    qw = orc.pack_rows(codes)
    ones = synthetic.bf16_bits(np.ones((N, K // 64), dtype=np.float32))
    zeros = np.zeros((N, K // 64), dtype=np.uint16)
    x = synthetic.activations(M, K, seed=31)
    y = w4.matmul(dev_bf16(x), dev_qw(qw), dev_bf16(ones), dev_bf16(zeros))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), x[:, :N])

    say("closed forms: zero activations give +0")
    w = synthetic.quantized_weights(300, 640, seed=32)
    yz = run_mm(DevWeights(w), np.zeros((4, 640), dtype=np.uint16), 300, f32=True)
    assert np.all(yz == 0) and not np.signbit(yz).any()

    say("closed forms: rows whose dequantized weights are all zero give exactly 0")
    w = synthetic.quantized_weights(5000, 512, seed=33, bias="exact")
    w.qw[::7] = 0x88888888                     # q = 8 with b = -8 s: w = 0 exactly
    x = synthetic.activations(2, 512, seed=33)
    y32 = run_mm(DevWeights(w), x, 5000, f32=True)
    assert np.all(y32[:, ::7] == 0)
    y64, absy = orc.qmm(x, w.qw, w.scales, w.biases, rows=np.arange(0, 5000, 7))
    assert np.all(y64 == 0) and np.all(absy == 0)

    say("closed forms: all codes equal")
    for c in (0, 9, 15):
        w = synthetic.quantized_weights(100, 1024, seed=34 + c)
        w.qw[:] = np.uint32(int(f"{c:x}" * 8, 16))
        x = synthetic.activations(2, 1024, seed=34)
        y64, absy = orc.qmm(x, w.qw, w.scales, w.biases)
        full_check(orc, w, x, y64, absy, f"codes={c}")


@pytest.mark.parametrize("K", [2560, 6208])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_grouped_equals_separate_calls(orc, M, K):
    # the q, k, v projections of a decode layer in one grouped call, plus a wide
    # matrix in another K-split class and an empty one; K = 6208 puts the narrow
    # ones in the long-row K-split class (two row sets per block from M = 2),
    # with row counts that leave partial blocks
    shapes = ([("q", 2560), ("k", 512), ("v", 512), ("wide", 5000), ("empty", 0)] if K == 2560 else
              [("q", 2568), ("k", 300), ("v", 13), ("wide", 4100), ("empty", 0)])
    x = synthetic.activations(M, K, seed=51)
    xd = dev_bf16(x)
    mats, outs, ws = [], [], []
    for i, (name, N) in enumerate(shapes):
        w = synthetic.quantized_weights(max(N, 1), K, seed=51, tag=(i,))
        dw = DevWeights(w)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        mats.append((dw.qw[:N], dw.s[:N], dw.b[:N], y))
        outs.append(y)
        ws.append((w, dw))
    say(f"grouped q/k/v/wide/empty M={M} K={K}")
    w4.w4a16_matmul_grouped(xd, mats)
    torch.cuda.synchronize()
    for (name, N), y, (w, dw) in zip(shapes, outs, ws):
        if N == 0:
            continue
        ref = run_mm(dw, x, N, f32=True)
        assert np.array_equal(host_f32(y).view(np.uint32), ref.view(np.uint32)), name
        rows = np.arange(0, N, 7, dtype=np.int32)
        y64, absy = orc.qmm(x, w.qw, w.scales, w.biases, rows=rows)
        check_f32(host_f32(y)[:, rows], y64, absy, f"grouped {name} M={M} K={K}")


def test_deterministic_and_no_stray_writes(orc):
    N, K, M = 5000, 2560, 3
    say(f"determinism and guard bands N={N} K={K} M={M}")
    w = synthetic.quantized_weights(N, K, seed=41)
    dw = DevWeights(w)
    x = dev_bf16(synthetic.activations(M, K, seed=41))
    pad = 4096
    for dt, sentinel in ((torch.float32, 1234.5), (torch.bfloat16, -7.0)):
        buf = torch.full((M * N + 2 * pad,), sentinel, dtype=dt, device="cuda")
        y = buf[pad:pad + M * N].view(M, N)
        w4.w4a16_matmul(x, dw.qw, dw.s, dw.b, y)
        first = y.clone()
        w4.w4a16_matmul(x, dw.qw, dw.s, dw.b, y)
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           y.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
        assert bool((buf[:pad] == sentinel).all()) and bool((buf[pad + M * N:] == sentinel).all())


def test_empty_problems_write_nothing():
    say("empty problems")
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    qw = torch.zeros((16, 16), dtype=torch.int32, device="cuda")
    s = torch.zeros((16, 2), dtype=torch.bfloat16, device="cuda")
    y = torch.full((0, 16), 3.0, dtype=torch.bfloat16, device="cuda")
    w4.w4a16_matmul(x, qw, s, s, y)
    x1 = torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda")
    y1 = torch.full((1, 0), 3.0, dtype=torch.bfloat16, device="cuda")
    w4.w4a16_matmul(x1, qw[:0], s[:0], s[:0], y1)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# LM head with fused argmax
# ---------------------------------------------------------------------------

def test_lmhead_argmax_config(orc):
    N, K = synthetic.LM_HEAD["N"], synthetic.LM_HEAD["K"]
    w = synthetic.quantized_weights(N, K, seed=0, tag=(262144,), bias="exact")
    x3 = synthetic.activations(3, K, seed=0, tag=(262144,))
    say(f"lm head N={N} K={K}: oracle (all rows, M=3)")
    y64, absy = oracle_qmm(orc, x3, w, workers=16)
    dw = DevWeights(w)
    for M in synthetic.LM_HEAD["M"]:
        say(f"  lm head M={M}")
        xd = dev_bf16(x3[:M])
        am, logits = w4.lmhead_argmax(xd, dw.qw, dw.s, dw.b, out_dtype=torch.float32)
        am2, none = w4.lmhead_argmax(xd, dw.qw, dw.s, dw.b, want_logits=False)
        amb, lb = w4.lmhead_argmax(xd, dw.qw, dw.s, dw.b, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        am = am.cpu().numpy()
        assert none is None and np.array_equal(am, am2.cpu().numpy()) and np.array_equal(am, amb.cpu().numpy())
        y32 = host_f32(logits)
        check_f32(y32, y64[:M], absy[:M], f"lm head logits M={M}")
        check_bf16(orc, host_bits(lb), y64[:M], absy[:M], K, f"lm head bf16 M={M}")
        # the argmax is that of the fp32 logits, lowest index on ties
        for m in range(M):
            assert am[m] == int(np.flatnonzero(y32[m] == y32[m].max())[0])
        n = check_argmax(orc, am, y64[:M], absy[:M], f"lm head M={M}")
        say(f"  lm head M={M}: argmax {am.tolist()}, checked {n}/{M} rows")
        # the seeded workload leaves row 0's top-2 gap above the bounds, so the
        # oracle comparison (iv) binds on at least that row
        assert n >= 1, f"lm head M={M}: no row with a top-2 gap above the bounds"
        # logits equal the dense product bit for bit
        ym = torch.empty((M, N), dtype=torch.float32, device="cuda")
        w4.w4a16_matmul(xd, dw.qw, dw.s, dw.b, ym)
        torch.cuda.synchronize()
        assert np.array_equal(host_f32(ym).view(np.uint32), y32.view(np.uint32))


def test_lmhead_planted_maximum_and_ties_at_vocabulary_size(orc):
    # the 262144 x 2560 head (the vocabulary-head schedule) with one planted
    # maximum per activation row, each with an identical later copy: the copy
    # ties bit for bit, and the lower index must win, wherever the two rows
    # fall (same row group, next block, the far end of the vocabulary)
    N, K = synthetic.LM_HEAD["N"], synthetic.LM_HEAD["K"]
    w = synthetic.quantized_weights(N, K, seed=0, tag=(262144,), bias="exact")
    x3 = synthetic.activations(3, K, seed=0, tag=(262144,))
    xv = synthetic.bf16_values(x3)
    star = [131071, 7, 200000]
    dups = [N - 1, 8, 200000 + 37]
    for m, (st, du) in enumerate(zip(star, dups)):
        row = orc.pack_rows(np.where(xv[m] > 0, 15, 0).astype(np.uint8)[None, :])[0]
        for n in (st, du):
            w.qw[n] = row
            w.scales[n] = w.scales[st]
            w.biases[n] = w.biases[st]
    say(f"lm head planted maxima {star} with later copies {dups}: oracle (all rows, M=3)")
    y64, absy = oracle_qmm(orc, x3, w, workers=16)
    for m in range(3):
        best, gap = orc.argmax(y64[m])
        assert best == star[m] and y64[m, dups[m]] == y64[m, star[m]], (m, best)
        assert gap == 0.0                      # the copy ties exactly in the oracle too
        rest = np.delete(y64[m], [star[m], dups[m]])
        assert y64[m, star[m]] - rest.max() > 1e-3 * (absy[m, star[m]] + absy[m].max())
    dw = DevWeights(w)
    for M in synthetic.LM_HEAD["M"]:
        say(f"  planted lm head M={M}")
        am, logits = w4.lmhead_argmax(dev_bf16(x3[:M]), dw.qw, dw.s, dw.b, out_dtype=torch.float32)
        torch.cuda.synchronize()
        y = host_f32(logits)
        for m in range(M):
            assert int(am[m]) == star[m], (M, m, int(am[m]))
            assert y[m, star[m]] == y[m, dups[m]]
        check_f32(y, y64[:M], absy[:M], f"planted lm head M={M}")


@pytest.mark.parametrize("N", [1, 100, 5000, 70000])
def test_lmhead_ties_and_planted_maximum(orc, N):
    K = 512
    say(f"lm head ties N={N}")
    w = synthetic.quantized_weights(N, K, seed=N, bias="exact")
    x = synthetic.activations(2, K, seed=N)
    xv = synthetic.bf16_values(x)
    codes = orc.unpack_rows(w.qw, K)
    star = N // 3
    codes[star] = np.where(xv[0] > 0, 15, 0)
    qw = orc.pack_rows(codes)
    dup = [n for n in (N - 1, star + 1) if n != star and n < N]
    for d in dup:                                   # later duplicates must lose the tie
        qw[d] = qw[star]; w.scales[d] = w.scales[star]; w.biases[d] = w.biases[star]
    am, logits = w4.lmhead_argmax(dev_bf16(x), dev_qw(qw), dev_bf16(w.scales), dev_bf16(w.biases),
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(am[0]) == star
    y = host_f32(logits)
    assert int(am[1]) == int(np.flatnonzero(y[1] == y[1].max())[0])


# K-split LM heads (N <= 4096) at every M, including the wide five-way split
# whose rows go four per lane from M = 6 and a ragged last block, and four-way
# splits whose rows span several one-chunk tiles (with and without a ragged one).
@pytest.mark.parametrize("N,K", [(3001, 2560), (700, 5120), (2500, 1024), (1200, 6208), (900, 4096)])
def test_lmhead_k_split_every_M(orc, N, K):
    w = synthetic.quantized_weights(N, K, seed=N + K, tag=(5,), bias="exact")
    x = synthetic.activations(8, K, seed=N + K, tag=(5,))
    say(f"lm head K-split N={N} K={K}: oracle (all rows, M=8)")
    y64, absy = oracle_qmm(orc, x, w)
    dw = DevWeights(w)
    for M in range(1, 9):
        say(f"  lm head N={N} K={K} M={M}")
        xd = dev_bf16(x[:M])
        am, logits = w4.lmhead_argmax(xd, dw.qw, dw.s, dw.b, out_dtype=torch.float32)
        ym = torch.empty((M, N), dtype=torch.float32, device="cuda")
        w4.w4a16_matmul(xd, dw.qw, dw.s, dw.b, ym)
        torch.cuda.synchronize()
        y32, am = host_f32(logits), am.cpu().numpy()
        check_f32(y32, y64[:M], absy[:M], f"lm head N={N} K={K} M={M}")
        assert np.array_equal(host_f32(ym).view(np.uint32), y32.view(np.uint32))
        for m in range(M):
            assert am[m] == int(np.flatnonzero(y32[m] == y32[m].max())[0]), (N, K, M, m)


# ---------------------------------------------------------------------------
# Routed (expert-gathered) product
# ---------------------------------------------------------------------------

def routed_inputs(E, N, K, M, top_k, seed):
    w = synthetic.quantized_weights(N, K, seed=seed, lead=(E,))
    x = synthetic.activations(M, K, seed=seed)
    ids = synthetic.expert_ids(M, top_k, E, seed=seed)
    return w, x, ids


def run_id(dw_stack, x_bits, ids, N, f32=True):
    """x_bits [M, K]: a token's slots share its row; [M, top_k, K]: one row per slot."""
    y = w4.matmul_id(dev_bf16(x_bits), dw_stack[0], dw_stack[1], dw_stack[2], dev_i32(ids),
                     out_dtype=torch.float32 if f32 else torch.bfloat16)
    torch.cuda.synchronize()
    return host_f32(y) if f32 else host_bits(y)


def test_routed_moe_config(orc):
    E, N, K, top_k = synthetic.MOE["E"], synthetic.MOE["N"], synthetic.MOE["K"], synthetic.MOE["top_k"]
    w, x, ids = routed_inputs(E, N, K, 8, top_k, seed=0)
    say(f"moe E={E} N={N} K={K} top_k={top_k}: oracle M=8")
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(8) as ex:
        res = list(ex.map(lambda m: orc.qmm_id(x[m:m + 1], w.qw, w.scales, w.biases, ids[m:m + 1]), range(8)))
    y64 = np.concatenate([r[0] for r in res])
    absy = np.concatenate([r[1] for r in res])
    stack = (dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases))
    say(f"  moe M=8 ids unique experts {len(np.unique(ids))}")
    y8 = run_id(stack, x, ids, N)
    check_f32(y8, y64, absy, "moe M=8")
    yb8 = run_id(stack, x, ids, N, f32=False)
    check_bf16(orc, yb8, y64, absy, K, "moe M=8")
    for m in range(8):
        say(f"  moe M=1 token {m}")
        y1 = run_id(stack, x[m:m + 1], ids[m:m + 1], N)
        assert np.array_equal(y1[0].view(np.uint32), y8[m].view(np.uint32)), m      # batch invariance
    # every slot equals the dense product on its expert, bit for bit
    for m, j in [(0, 0), (3, 5), (7, 7)]:
        e = int(ids[m, j])
        yd = torch.empty((1, N), dtype=torch.float32, device="cuda")
        w4.w4a16_matmul(dev_bf16(x[m:m + 1]), stack[0][e], stack[1][e], stack[2][e], yd)
        torch.cuda.synchronize()
        assert np.array_equal(host_f32(yd)[0].view(np.uint32), y8[m, j].view(np.uint32))


@pytest.mark.parametrize("E,N,K", [(3, 4100, 4288), (2, 600, 6208)])
def test_routed_long_rows(orc, E, N, K):
    # experts tall enough for one row group per row and K spanning two full
    # K-tiles plus a ragged tail; short experts with a four-way K-split whose
    # rows span three one-chunk tiles plus a ragged tail
    M, top_k = 3, 2
    w, x, _ = routed_inputs(E, N, K, M, top_k, seed=21)
    stack = (dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases))
    ids = np.array([[0, 2], [1, 0], [2, 1]] if E == 3 else [[0, 1], [1, 0], [0, 1]], dtype=np.int32)
    say(f"routed long rows E={E} N={N} K={K} M={M}: oracle")
    y64, absy = orc.qmm_id(x, w.qw, w.scales, w.biases, ids)
    y = run_id(stack, x, ids, N)
    check_f32(y, y64, absy, "routed long rows")
    for m in range(M):
        say(f"  routed long rows token {m}")
        y1 = run_id(stack, x[m:m + 1], ids[m:m + 1], N)
        check_f32(y1, y64[m:m + 1], absy[m:m + 1], f"routed long rows M=1 token {m}")
        assert np.array_equal(y1[0].view(np.uint32), y[m].view(np.uint32)), m


def test_routed_variants(orc):
    E, N, K, M, top_k = 6, 700, 576, 5, 3
    w, x, _ = routed_inputs(E, N, K, M, top_k, seed=9)
    stack = (dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases))
    ids = np.array([[0, 1, 2], [2, 2, 5], [5, 0, 1], [3, 3, 3], [1, 4, 0]], dtype=np.int32)  # shared + duplicate ids
    say("routed: shared and duplicate ids")
    y64, absy = orc.qmm_id(x, w.qw, w.scales, w.biases, ids)
    y = run_id(stack, x, ids, N)
    check_f32(y, y64, absy, "routed dup")
    say("routed: one input row per slot")
    xs = synthetic.activations(M * top_k, K, seed=10).reshape(M, top_k, K)
    y64s, abss = orc.qmm_id(xs, w.qw, w.scales, w.biases, ids, x_per_slot=True)
    ys = run_id(stack, xs, ids, N)
    check_f32(ys, y64s, abss, "routed per-slot")
    check_bf16(orc, run_id(stack, xs, ids, N, f32=False), y64s, abss, K, "routed per-slot bf16")
    say("routed: per-slot rows at a padded stride (K + 40) read the same values")
    pad = torch.full((M, top_k, K + 40), float("nan"), dtype=torch.bfloat16, device="cuda")
    pad[:, :, :K] = dev_bf16(xs)
    yp = torch.empty((M, top_k, N), dtype=torch.float32, device="cuda")
    w4.w4a16_matmul_id(pad[:, :, :K], stack[0], stack[1], stack[2], dev_i32(ids), yp)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(yp).view(np.uint32), ys.view(np.uint32))
    say("routed: out-of-range id fills its slot with NaN")
    bad = ids.copy()
    bad[1, 1] = E
    bad[4, 0] = -3
    yb = run_id(stack, x, bad, N)
    assert np.isnan(yb[1, 1]).all() and np.isnan(yb[4, 0]).all()
    keep = np.ones((M, top_k), dtype=bool)
    keep[1, 1] = keep[4, 0] = False
    assert np.array_equal(yb[keep].view(np.uint32), y[keep].view(np.uint32))


# ---------------------------------------------------------------------------
# Group size 128 (the tiny-llm page's group): same kernels, scales and biases
# per 128 codes
# ---------------------------------------------------------------------------

def run_mm_g(dw, x_bits, N, group, f32=False):
    x = dev_bf16(x_bits)
    y = torch.empty((x.shape[0], N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    w4.w4a16_matmul(x, dw.qw, dw.s, dw.b, y, group=group)
    torch.cuda.synchronize()
    return host_f32(y) if f32 else host_bits(y)


# one case per schedule class: tiny, one-chunk K-split, long-row K-split (two
# row sets from M = 2), one row group per row, several K-tiles (double
# buffered at M = 1), N >= 16384 with K % 2560 == 0
G128 = [(8, 128), (300, 2560), (3001, 2560), (1003, 6272), (2300, 6272), (4097, 768), (4200, 5120), (16400, 2560)]


@pytest.mark.parametrize("N,K", G128)
def test_group128_every_M_batch_invariant(orc, N, K):
    w = synthetic.quantized_weights(N, K, group=128, seed=N + K)
    x = synthetic.activations(8, K, seed=N + K + 1)
    say(f"group 128 N={N} K={K}: oracle")
    y64, absy = oracle_qmm(orc, x, w)
    dw = DevWeights(w)
    ref32 = [run_mm_g(dw, x[m:m + 1], N, 128, f32=True)[0] for m in range(8)]
    for M in range(1, 9):
        say(f"  group 128 N={N} K={K} M={M}")
        y32 = run_mm_g(dw, x[:M], N, 128, f32=True)
        check_f32(y32, y64[:M], absy[:M], f"G=128 N={N} K={K} M={M}")
        yb = run_mm_g(dw, x[:M], N, 128)
        check_bf16(orc, yb, y64[:M], absy[:M], K, f"G=128 N={N} K={K} M={M}")
        assert np.array_equal(yb, synthetic.bf16_bits(y32))
        for m in range(M):
            assert np.array_equal(y32[m].view(np.uint32), ref32[m].view(np.uint32)), (N, K, M, m)


def test_group128_routed_lmhead_dequant_gather(orc):
    say("group 128: routed product")
    E, N, K, M, top_k = 4, 700, 1024, 3, 2
    w = synthetic.quantized_weights(N, K, group=128, seed=31, lead=(E,))
    x = synthetic.activations(M, K, seed=31)
    ids = np.array([[0, 3], [3, 1], [2, 2]], dtype=np.int32)
    y64, absy = orc.qmm_id(x, w.qw, w.scales, w.biases, ids, group=128)
    y = w4.matmul_id(dev_bf16(x), dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases), dev_i32(ids),
                     out_dtype=torch.float32, group=128)
    torch.cuda.synchronize()
    check_f32(host_f32(y), y64, absy, "G=128 routed")

    say("group 128: LM head with argmax")
    N, K, M = 5000, 2560, 3
    w = synthetic.quantized_weights(N, K, group=128, seed=32, bias="exact")
    x = synthetic.activations(M, K, seed=32)
    y64, absy = oracle_qmm(orc, x, w)
    am, logits = w4.lmhead_argmax(dev_bf16(x), dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases),
                                  out_dtype=torch.float32, group=128)
    torch.cuda.synchronize()
    check_f32(host_f32(logits), y64, absy, "G=128 LM head")
    assert check_argmax(orc, am.cpu().numpy(), y64, absy, "G=128 LM head") >= 1   # rows whose top-2 gap exceeds the bound

    say("group 128: dequant and row gather")
    w = synthetic.quantized_weights(50, 640, group=128, seed=33)
    ref = orc.dequant_rows(w.qw, w.scales, w.biases, 640, group=128)
    got = w4.dequant(dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases), group=128)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(got).view(np.uint32), ref.view(np.uint32))
    rows = np.array([49, 0, 7, 7, 50], dtype=np.int32)
    g = host_bits(w4.gather_rows(dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases), dev_i32(rows), group=128))
    assert np.array_equal(g[:4], orc.f64_to_bf16(ref[[49, 0, 7, 7]].astype(np.float64)))
    assert (g[4] == 0x7FC0).all()


# ---------------------------------------------------------------------------
# Prefill-shaped product (M > 8) on the matrix cores
# ---------------------------------------------------------------------------

def run_prefill(dw, x_bits, N, group=64, f32=False):
    x = dev_bf16(x_bits)
    y = torch.empty((x.shape[0], N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    w4.w4a16_matmul_prefill(x, dw.qw, dw.s, dw.b, y, group=group)
    torch.cuda.synchronize()
    return host_f32(y) if f32 else host_bits(y)


# ragged M, N and K, both group sizes, tiles and tails in every dimension.  Up
# to 16 rows (M = 1, 9 below) run the decode kernels on chunks of eight.  The
# LDS-tiled form runs where M > 64 and there are >= 96 tiles of 128 x 128, or
# M > 40 and 160..255 of 64 x 128: with >= 256 128-row tiles one group of waves per tile
# (300 x 12837, 520 x 16390, 256 x 32768 whose grid is permuted across the
# XCDs, and 100 x 32768 with one partial row tile); with 96..255 of them and
# not 160..255 64-row tiles, two groups splitting K (100 x 20480, and
# 100 x 24576 at G = 128); with 160..255 64-row tiles, 64-row tiles and two
# groups (257 x 4097, 520 x 2560, 300 x 4000 at G = 128, 200 x 8000 with an
# odd number of K steps, 100 x 12500 with one partial row tile, and
# 48 x 20480 and 60 x 24000 at G = 128 with a single partial row tile); the other
# shapes run the per-wave form, which walks K in blocks of 128 codes
# (300 x 3000 at G = 128 and 100 x 9000: 120 and 142 64-row tiles):
# 64 x 32 tiles (31 x 9000, 40 x 9000 and 20 x 2560 <- 10240: long K walks),
# 32 x 16 tiles (33 x 300, 100 x 1000, 70 x 513, 64 x 128, 20 x 2560), 32 x 32
# tiles (90 x 2600, 48 x 3000, ragged in both), 64 x 32 tiles without a
# K-split (40 x 40000, over 1024 tiles), and a last block of 64 codes
# (K = 64, 1344, 320).
PREFILL = [(9, 40, 128, 64), (33, 300, 640, 64), (100, 1000, 2560, 64), (257, 4097, 1024, 64), (64, 128, 64, 64),
           (70, 513, 1280, 128), (1, 77, 256, 128), (520, 2560, 2560, 64), (300, 12837, 640, 128),
           (520, 16390, 512, 64), (256, 32768, 256, 64), (300, 3000, 640, 128), (200, 8000, 704, 64),
           (40, 9000, 640, 64), (100, 32768, 256, 128), (31, 9000, 2560, 64), (20, 2560, 10240, 64),
           (90, 2600, 1024, 128), (100, 9000, 640, 64), (48, 3000, 1344, 64), (40, 40000, 320, 64),
           (300, 4000, 640, 128), (100, 12500, 640, 64), (100, 20480, 640, 64), (100, 24576, 256, 128),
           (48, 20480, 2560, 64), (60, 24000, 640, 128)]


@pytest.mark.parametrize("M,N,K,G", PREFILL)
def test_prefill_matches_oracle(orc, M, N, K, G):
    w = synthetic.quantized_weights(N, K, group=G, seed=M + N + K)
    x = synthetic.activations(M, K, seed=M * 3 + K)
    rows = np.arange(0, N, max(1, N // 300), dtype=np.int32)
    say(f"prefill M={M} N={N} K={K} G={G}: oracle on {len(rows)} rows")
    y64, absy = oracle_qmm(orc, x, w, rows=rows)
    dw = DevWeights(w)
    y32 = run_prefill(dw, x, N, G, f32=True)
    rel = check_f32(y32[:, rows], y64, absy, f"prefill M={M} N={N} K={K}")
    yb = run_prefill(dw, x, N, G)
    ex = check_bf16(orc, yb[:, rows], y64, absy, K, f"prefill M={M} N={N} K={K}")
    say(f"  max |err|/sum|wx| = {rel:.2e}, bf16 exempt {ex}")
    assert np.array_equal(yb, synthetic.bf16_bits(y32))
    assert np.array_equal(run_prefill(dw, x, N, G, f32=True).view(np.uint32), y32.view(np.uint32))   # deterministic


def test_prefill_maximum_rows(orc):
    # the largest accepted M (65536 rows: 512 row tiles of one weight tile)
    M, N, K = w4.MAX_PREFILL_M, 130, 64
    w = synthetic.quantized_weights(N, K, seed=65)
    x = synthetic.activations(M, K, seed=65)
    say(f"prefill M={M} N={N} K={K}")
    # the oracle takes at most 4096 activation rows per call; rows are independent
    parts = [oracle_qmm(orc, x[i:i + 4096], w) for i in range(0, M, 4096)]
    y64 = np.concatenate([p[0] for p in parts], axis=0)
    absy = np.concatenate([p[1] for p in parts], axis=0)
    dw = DevWeights(w)
    y32 = run_prefill(dw, x, N, f32=True)
    check_f32(y32, y64, absy, f"prefill M={M}")
    assert np.array_equal(run_prefill(dw, x, N), synthetic.bf16_bits(y32))


@pytest.mark.parametrize("M,N,K", [(20, 64, 2560), (200, 32768, 256), (150, 8192, 640)])
def test_prefill_crafted_scales(orc, M, N, K):
    # signs, zero, subnormal and |s| >= 2^100 scales (the plain dequant path),
    # in the per-wave (M = 20), LDS-tiled (M = 200) and 64-row tiled (M = 150,
    # 192 tiles) forms
    w = synthetic.quantized_weights(N, K, seed=41)
    w.scales, w.biases = crafted_scales(N, K // 64, seed=41)
    x = synthetic.activations(M, K, seed=41)
    # the first rows hold the zero, subnormal and huge scales
    rows = np.union1d(np.arange(8), np.arange(0, N, max(1, N // 400))).astype(np.int32)
    say(f"prefill crafted scales M={M} N={N} K={K}")
    y64, absy = oracle_qmm(orc, x, w, rows=rows)
    y32 = run_prefill(DevWeights(w), x, N, f32=True)
    check_f32(y32[:, rows], y64, absy, "prefill crafted")


@pytest.mark.parametrize("M,N,K", [(100, 1000, 640), (384, 4096, 2560), (1024, 4096, 1280)])
def test_prefill_zero_weight_rows_exact(orc, M, N, K):
    # rows stored as q = 8, b = -8 s hold w = 0 exactly, so their outputs are
    # exactly 0 in the per-wave (M = 100), 64-row tiled (192 tiles) and tiled
    # (256 tiles) forms; the other rows stay within the bound
    w = synthetic.quantized_weights(N, K, seed=N + 5, bias="exact")
    zero = np.arange(3, N, 7)
    w.qw[zero] = 0x88888888
    x = synthetic.activations(M, K, seed=M + 5)
    say(f"prefill zero rows M={M} N={N} K={K}")
    y32 = run_prefill(DevWeights(w), x, N, f32=True)
    assert np.all(y32[:, zero] == 0), int(np.count_nonzero(y32[:, zero]))
    rows = np.arange(0, N, max(1, N // 200), dtype=np.int32)
    y64, absy = oracle_qmm(orc, x, w, rows=rows)
    assert np.all(y64[:, np.isin(rows, zero)] == 0)
    check_f32(y32[:, rows], y64, absy, "prefill zero rows")


@pytest.mark.parametrize("M,N,K", [(20, 64, 2560), (384, 4096, 2560), (1024, 4096, 1280)])
def test_prefill_cancelling_rows_within_the_documented_bounds(orc, M, N, K):
    # rows whose every code is 15 with b = -15 s (s a power of two, so b is
    # exact in bf16) dequantize to w = 0 exactly: the oracle gives 0 with a
    # bound of 0.  The per-wave form (M = 20) splits each w into bf16 parts and
    # returns exactly 0.  The LDS-tiled forms (64-row and 128-row tiles) use the
    # rearranged sums s * sum(x (q - 8)) + (b + 8 s) * sum(x), whose rounding is
    # bounded on sum |s x (q - 8)| + |(b + 8 s) x| instead (the documented
    # bound of w4a16_matmul_prefill): their residue must stay within 1e-3 of
    # that sum.  The other rows keep the usual bound.
    w = synthetic.quantized_weights(N, K, seed=N + 9, bias="exact")
    cancel = np.arange(1, N, 5)
    w.qw[cancel] = 0xFFFFFFFF
    s_pow2 = synthetic.bf16_bits(np.float32(2.0 ** 10))
    b_neg = synthetic.bf16_bits(np.float32(-15.0 * 2.0 ** 10))
    w.scales[cancel] = s_pow2
    w.biases[cancel] = b_neg
    x = synthetic.activations(M, K, seed=M + 9)
    t128, t64 = -(-M // 128) * -(-N // 128), -(-M // 64) * -(-N // 128)
    tiled = (M > 64 and t128 >= 96) or (M > 40 and t128 < 256 and 160 <= t64 < 256)   # the entry point's choice of form
    say(f"prefill cancelling rows M={M} N={N} K={K} ({'tiled' if tiled else 'per-wave'} form)")
    y32 = run_prefill(DevWeights(w), x, N, f32=True)
    y64, absy = oracle_qmm(orc, x, w, rows=cancel.astype(np.int32))
    assert np.all(y64 == 0) and np.all(absy == 0)
    got = y32[:, cancel].astype(np.float64)
    assert np.all(np.isfinite(got))
    if not tiled:
        assert np.all(got == 0), int(np.count_nonzero(got))
    else:
        # sum_k |s x (q - 8)| + |(b + 8 s) x| with q = 15, s = 2^10, b + 8 s = -7 * 2^10
        xs = np.abs(synthetic.bf16_values(x).astype(np.float64)).sum(axis=1)
        weak = (2.0 ** 10 * 7 + 7 * 2.0 ** 10) * xs
        assert np.all(np.abs(got) <= 1e-3 * weak[:, None]), float(np.max(np.abs(got) / weak[:, None]))
        say(f"  largest residue / weak bound sum: {float(np.max(np.abs(got) / weak[:, None])):.2e}")
    others = np.setdiff1d(np.arange(0, N, max(1, N // 150)), cancel).astype(np.int32)
    y64o, abso = oracle_qmm(orc, x, w, rows=others)
    check_f32(y32[:, others], y64o, abso, "prefill cancelling, other rows")


@pytest.mark.parametrize("M,N,K", [(13, 2560, 10240), (16, 20480, 2560), (9, 5000, 640)])
def test_prefill_small_M_is_the_decode_path(orc, M, N, K):
    # up to 16 rows the prefill entry runs the decode kernels on chunks of at
    # most eight rows: bitwise the w4a16_matmul results on those chunks
    w = synthetic.quantized_weights(N, K, seed=M + N, tag=(3,))
    x = synthetic.activations(M, K, seed=M + K, tag=(3,))
    say(f"prefill small M={M} N={N} K={K}")
    dw = DevWeights(w)
    y = run_prefill(dw, x, N, f32=True)
    chunks = np.concatenate([run_mm(dw, x[m0:m0 + 8], N, f32=True) for m0 in range(0, M, 8)])
    assert np.array_equal(y.view(np.uint32), chunks.view(np.uint32))
    rows = np.arange(0, N, max(1, N // 200), dtype=np.int32)
    y64, absy = oracle_qmm(orc, x, w, rows=rows)
    check_f32(y[:, rows], y64, absy, f"prefill small M={M}")
