"""GPU parity of the fused GeGLU product (w4a16_matmul_geglu) against the oracle.

h[m, j] = GELU(g) * u, where g and u are the products of gate row j and up row
I + j of a fused [2I, K] matrix and GELU(g) = g * Phi(g) (exact form).
Per-element bounds:
  * each fp32 sum: at most K/16 + 8 roundings of 2^-24 relative error on
    sum_k |w x| (a K/16-long fma chain per lane, the dequantization and the
    16-lane tree), doubled for margin: B = 2 (K/16 + 8) 2^-24 sum|wx|;
  * the activation: GELU' = Phi + g phi lies within [-0.13, 1.13], so
    |GELU(g32) u32 - GELU(g) u| <= 1.13 Bg (|u| + Bu) + |GELU(g)| Bu, and its
    fp32 evaluation adds at most 16 2^-24 |g u| + 8 2^-24 |h| (the sum
    1 + erf cancels for negative g, leaving an error of a few ulps of 1).
The bf16 output is the round-to-nearest-even of the fp32 output bit for bit,
and every row is bitwise that of the 1-row call.  A crafted case whose sums
are exact in fp32 checks the activation alone, with a bound tight enough to
reject the tanh form of GELU.  Inputs are the seeded synthetic workloads.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import decode_w4a16_affine_amd as w4
import synthetic
from parity import dev_bf16, dev_qw, host_bits, host_f32, oracle_qmm, say, ulp_distance

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.lib()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


class Fused:
    """A fused gate+up matrix on the device."""

    def __init__(self, w):
        self.w = w
        self.I = w.qw.shape[0] // 2
        self.qw, self.s, self.b = dev_qw(w.qw), dev_bf16(w.scales), dev_bf16(w.biases)

    def run(self, x_bits, f32):
        x = dev_bf16(x_bits)
        h = torch.empty((x.shape[0], self.I), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
        w4.w4a16_matmul_geglu(x, self.qw, self.s, self.b, h, group=self.w.group)
        torch.cuda.synchronize()
        return host_f32(h) if f32 else host_bits(h)


def oracle_geglu(orc, x_bits, w, cols):
    """The oracle's h, g, |g| scale, u, |u| scale on columns `cols`."""
    I = w.qw.shape[0] // 2
    g, ga = oracle_qmm(orc, x_bits, w, rows=cols)
    u, ua = oracle_qmm(orc, x_bits, w, rows=cols + I)
    return orc.geglu_values(g, u), g, ga, u, ua


def bound(orc, g, ga, u, ua, h, K):
    c = 2 * (K / 16 + 8) * U
    bg, bu = c * ga, c * ua
    gel = np.abs(orc.geglu_values(g, np.ones_like(g)))
    return (1.13 * bg * (np.abs(u) + bu) + gel * bu + 16 * U * (np.abs(g) + bg) * (np.abs(u) + bu)
            + 8 * U * np.abs(h))


def check(orc, fz, x_bits, cols, ref, what):
    """fp32 and bf16 h against the oracle's `ref` on columns `cols`; returns the fp32 h (all columns)."""
    K = fz.w.K
    M = x_bits.shape[0]
    h64, g, ga, u, ua = (a[:M] for a in ref)
    h32 = fz.run(x_bits, f32=True)
    hb = fz.run(x_bits, f32=False)
    lim = bound(orc, g, ga, u, ua, h64, K)
    err = np.abs(h32[:, cols].astype(np.float64) - h64)
    bad = ~(err <= lim)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} fp32 h outside the bound; first {i}: gpu {h32[:, cols][i]!r} "
                             f"oracle {h64[i]!r} bound {lim[i]!r} (g {g[i]!r} u {u[i]!r})")
    assert np.array_equal(hb, synthetic.bf16_bits(h32)), f"{what}: bf16 h is not the RNE of fp32 h"
    # bf16: within 1 ulp of RNE(h64) wherever the fp32 bound is below half a bf16 ulp
    near = ulp_distance(hb[:, cols], orc.f64_to_bf16(h64))
    judged = lim < 2.0 ** -9 * np.abs(h64)
    assert not ((near > 1) & judged).any(), f"{what}: bf16 h beyond 1 ulp"
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(lim > 0, err / lim, 0.0)
    say(f"  {what}: max err/bound = {float(r.max()):.3f}, bf16 judged {int(judged.sum())}/{judged.size}")
    return h32


# (I, K, group): the decode gate_up layer (2I = 20480, K = 2560); ragged I just
# above the K-split limit; N = 2I past 16384 with a short K; a vocabulary-sized
# fused matrix (2I >= 131072); group 128.  K-split form (2I <= 4096): five
# slices (K = 2560, 5120; 2I > 2048 takes four rows per lane from M = 6, also
# with a ragged last block), four (K = 1024, 640), four with K > 4096 (the
# class with two rows per lane from M = 3), and I below one block's rows.
CASES = [(10240, 2560, 64), (2049, 640, 64), (8195, 576, 64), (65600, 256, 64), (2100, 1280, 128),
         (3000, 5120, 128),
         (2048, 2560, 64), (1100, 2560, 64), (700, 5120, 128), (1000, 1024, 64), (37, 640, 128), (1500, 6144, 64),
         (1, 2560, 64), (5, 1024, 64)]


@pytest.mark.parametrize("I,K,G", CASES)
def test_geglu_matches_oracle_every_M(orc, I, K, G):
    w = synthetic.quantized_weights(2 * I, K, group=G, seed=I + K, tag=(9,))
    x = synthetic.activations(8, K, seed=I + K, tag=(9,))
    cols = np.arange(I, dtype=np.int32) if I <= 10240 else np.unique(
        np.concatenate([np.arange(64), np.arange(I - 64, I), np.arange(0, I, 97)])).astype(np.int32)
    say(f"geglu I={I} K={K} G={G}: oracle on {len(cols)} columns")
    ref = oracle_geglu(orc, x, w, cols)   # rows of x are independent: one call serves every M
    fz = Fused(w)
    singles = [fz.run(x[m:m + 1], f32=True)[0] for m in range(8)]
    for M in range(1, 9):
        say(f"geglu I={I} K={K} G={G} M={M}")
        h32 = check(orc, fz, x[:M], cols, ref, f"I={I} K={K} G={G} M={M}")
        for m in range(M):   # batch invariance
            assert np.array_equal(h32[m].view(np.uint32), singles[m].view(np.uint32)), (I, K, M, m)


def test_geglu_exact_sums_reject_tanh_form(orc):
    """Sums exact in fp32 (x in {+-1/2, +-1}, w multiples of 2^-6 below 1/2, K = 256):
    g and u carry no error, so h is off only by the activation's own fp32
    evaluation, and the bound sits far below the gap to the tanh form."""
    I, K, M = 2560, 256, 4
    gen = synthetic.rng(41, "x")
    x = synthetic.bf16_bits(gen.choice(np.array([-1.0, -0.5, 0.5, 1.0], dtype=np.float32), size=(M, K)))
    codes = synthetic.random_codes(2 * I, K, seed=41)
    s = synthetic.rng(41, "scales").choice(np.array([2.0 ** -6, 2.0 ** -5, 2.0 ** -4], dtype=np.float32),
                                           size=(2 * I, K // 64))
    w = synthetic.QWeights(orc.pack_rows(codes), synthetic.bf16_bits(s), synthetic.bf16_bits(-8 * s), 2 * I, K, 64)
    cols = np.arange(I, dtype=np.int32)
    h64, g, ga, u, ua = oracle_geglu(orc, x, w, cols)
    fz = Fused(w)
    say("geglu exact sums")
    h32 = fz.run(x, f32=True).astype(np.float64)
    lim = 16 * U * np.abs(g * u) + 8 * U * np.abs(h64)
    assert np.all(np.abs(h32 - h64) <= lim), float(np.max(np.abs(h32 - h64) - lim))
    # the bound's power: the tanh form of GELU falls outside it on these sums
    tanh_form = 0.5 * g * (1 + np.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3))) * u
    assert np.count_nonzero(np.abs(tanh_form - h64) > lim) > I // 4
    assert np.abs(g).max() > 4 and np.abs(u).max() > 4


def test_geglu_rejects_and_empty():
    say("geglu argument checks")
    K = 256
    x = torch.zeros((1, K), dtype=torch.bfloat16, device="cuda")
    I = 2100
    qw = torch.zeros((2 * I, K // 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((2 * I, K // 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w4.W4A16Error) as e:   # M > 8
        w4.w4a16_matmul_geglu(torch.zeros((9, K), dtype=torch.bfloat16, device="cuda"), qw, s, s,
                              torch.empty((9, I), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 3
    with pytest.raises(ValueError):           # odd row count
        w4.w4a16_matmul_geglu(x, qw[:-1], s[:-1], s[:-1], torch.empty((1, I), dtype=torch.bfloat16, device="cuda"))
    h0 = torch.full((0, I), 3.0, dtype=torch.bfloat16, device="cuda")
    w4.w4a16_matmul_geglu(torch.zeros((0, K), dtype=torch.bfloat16, device="cuda"), qw, s, s, h0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("I,K", [(2100, 640), (300, 1024)])
def test_geglu_crafted_scales(orc, I, K):
    # signs, zero, subnormal and |s| >= 2^100 scales and biases over a wide
    # exponent range (the plain dequantization path) in both forms
    from test_parity_gpu import crafted_scales
    w = synthetic.quantized_weights(2 * I, K, seed=43)
    w.scales, w.biases = crafted_scales(2 * I, K // 64, seed=43)
    # the up rows paired with the first gate rows (which hold the 2^100
    # scales) get ordinary scales and biases, so g * u stays finite in fp32
    w.scales[I:I + 8] = synthetic.bf16_bits(np.full((8, K // 64), 0.01, dtype=np.float32))
    w.biases[I:I + 8] = synthetic.bf16_bits(np.full((8, K // 64), -0.08, dtype=np.float32))
    x = synthetic.activations(3, K, seed=43)
    cols = np.arange(I, dtype=np.int32)
    say(f"geglu crafted scales I={I} K={K}")
    ref = oracle_geglu(orc, x, w, cols)
    check(orc, Fused(w), x, cols, ref, f"crafted I={I} K={K}")
