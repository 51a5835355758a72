"""The decode kernels' dequantized weights, read out through their own outputs.

An activation row that is 1.0 at column k and 0 elsewhere turns every output
of a product into one weight: y[n] = 1 * w[n, k] plus sums of exact zeros, so
the fp32 output is the value the kernel held in registers for w[n, k], bit for
bit up to the sign of a zero.  Reading every column this way checks that the
hot kernels themselves (dense K-split and row-streaming schedules at every M,
the LM head, the routed product) dequantize each weight exactly as the
oracle's fp32 fma(scale, q, bias) of tiny-llm's "Reconstruct a Stored Group",
not only the separate dequant kernel.  Calls cycle through M = 1..8 one-hot
rows, so every activation-row count's schedule takes part.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import decode_w4a16_affine_amd as w4
import synthetic
from parity import dev_bf16, dev_i32, dev_qw, host_f32, say

pytestmark = pytest.mark.gpu

ONE = 0x3F80    # bf16 bits of 1.0


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.lib()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def one_hot_calls(cols):
    """Split the columns into calls of 1, 2, ..., 8, 1, 2, ... one-hot rows."""
    i = j = 0
    while j < len(cols):
        M = min(1 + i % 8, len(cols) - j)
        yield cols[j:j + M]
        j += M
        i += 1


def one_hot(ks, K):
    x = np.zeros((len(ks), K), dtype=np.uint16)
    x[np.arange(len(ks)), ks] = ONE
    return x


def read_columns(call, N, K, cols):
    """[N, len(cols)] fp32: call(x_bits) -> [M, N] fp32 host array."""
    out = np.empty((N, len(cols)), dtype=np.float32)
    j = 0
    for ks in one_hot_calls(np.asarray(cols)):
        out[:, j:j + len(ks)] = call(one_hot(ks, K)).T
        j += len(ks)
    return out


def assert_same_weights(got, ref, what):
    ok = got == ref                       # +0 and -0 compare equal
    if not ok.all():
        n, k = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} weights differ; first [{n}, {k}]: "
                             f"kernel {got[n, k]!r} oracle {ref[n, k]!r}")
    nz = ref != 0
    assert np.array_equal(got[nz].view(np.uint32), ref[nz].view(np.uint32)), what


def crafted(w, seed):
    """Scale/bias bits over a wide finite range, some groups past 2^100 (the plain dequant path)."""
    g = np.random.default_rng(seed)
    N, G = w.scales.shape
    sign = lambda: g.integers(0, 2, size=(N, G)) << 15
    s = (sign() | (g.integers(100, 150, size=(N, G)) << 7) | g.integers(0, 128, size=(N, G))).astype(np.uint16)
    b = (sign() | (g.integers(100, 150, size=(N, G)) << 7) | g.integers(0, 128, size=(N, G))).astype(np.uint16)
    big = g.random((N, G)) < 0.02
    s[big] = (s[big] & 0x807F) | (227 << 7)       # |s| in [2^100, 2^101)
    s[0, 0], b[0, 0] = 0x8000, 0x8000             # -0 * q + -0: a group of weights equal to -0
    s[min(2, N - 1), 0], b[min(2, N - 1), 0] = 0x0000, 0x0000   # and one of +0
    s[min(1, N - 1), 0] = 0x0005                  # subnormal scale
    w.scales, w.biases = s, b
    return w


# (N, K, group, scales): K-split 5 narrow and wide (four rows per lane from
# M = 6), K-split 4 with long and short rows, row streaming for K % 2560 = 0
# below and above N = 16384 (the fused gate+up shape), other K above 16384.
DENSE = [(600, 2560, 64, "crafted"), (2600, 2560, 64, "config"), (300, 10240, 64, "crafted"),
         (1000, 1024, 128, "config"), (5000, 2560, 64, "crafted"), (20480, 2560, 64, "config"),
         (16400, 576, 64, "crafted"), (16384, 640, 128, "crafted")]


@pytest.mark.parametrize("N,K,G,kind", DENSE)
def test_dense_kernels_hold_the_exact_weights(orc, N, K, G, kind):
    say(f"read-out dense N={N} K={K} G={G} {kind}")
    w = synthetic.quantized_weights(N, K, group=G, seed=N ^ K, tag=(17,))
    if kind == "crafted":
        w = crafted(w, N + K)
    qw, s, b = dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases)

    def call(x_bits):
        x = dev_bf16(x_bits)
        y = torch.empty((x.shape[0], N), dtype=torch.float32, device="cuda")
        w4.w4a16_matmul(x, qw, s, b, y, group=G)
        torch.cuda.synchronize()
        return host_f32(y)

    got = read_columns(call, N, K, np.arange(K))
    ref = orc.dequant_rows(w.qw, w.scales, w.biases, K, group=G)
    assert_same_weights(got, ref, f"dense N={N} K={K} G={G} {kind}")


def test_lmhead_kernel_holds_the_exact_weights(orc):
    # a vocabulary-sized head (its own schedule class), columns from every
    # lane position of a chunk, both halves of a word and the last group
    N, K = 131109, 2560
    say(f"read-out lm head N={N} K={K}")
    w = crafted(synthetic.quantized_weights(N, K, seed=3, tag=(17,)), 3)
    qw, s, b = dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases)
    cols = np.unique(np.concatenate([np.arange(0, 40), np.arange(K - 40, K), np.arange(5, K, 131)]))

    def call(x_bits):
        am, logits = w4.lmhead_argmax(dev_bf16(x_bits), qw, s, b, out_dtype=torch.float32)
        torch.cuda.synchronize()
        return host_f32(logits)

    got = read_columns(call, N, K, cols)
    for r0 in range(0, N, 16384):                 # the oracle in row slices (2.7 GB whole)
        rows = np.arange(r0, min(N, r0 + 16384), dtype=np.int32)
        ref = orc.dequant_rows(w.qw, w.scales, w.biases, K, rows=rows)[:, cols]
        assert_same_weights(got[rows], ref, f"lm head rows {r0}..")


@pytest.mark.parametrize("E,N,K", [(3, 700, 2048), (2, 300, 2560)])
def test_routed_kernel_holds_the_exact_weights(orc, E, N, K):
    # every token routes to every expert, in a rotated order per token, so one
    # call reads its tokens' columns out of the whole stack
    say(f"read-out routed E={E} N={N} K={K}")
    w = synthetic.quantized_weights(N, K, seed=E + N, tag=(17,), lead=(E,))
    qw, s, b = dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases)
    got = np.empty((E, N, K), dtype=np.float32)
    for ks in one_hot_calls(np.arange(K)):
        M = len(ks)
        ids = np.array([np.roll(np.arange(E), t) for t in range(M)], dtype=np.int32)
        y = w4.matmul_id(dev_bf16(one_hot(ks, K)), qw, s, b, dev_i32(ids), out_dtype=torch.float32)
        torch.cuda.synchronize()
        y = host_f32(y)                           # [M, E, N]
        for t in range(M):
            for j in range(E):
                got[ids[t, j], :, ks[t]] = y[t, j]
    for e in range(E):
        ref = orc.dequant_rows(w.qw[e], w.scales[e], w.biases[e], K)
        assert_same_weights(got[e], ref, f"routed expert {e}")
