"""Pins for the CPU oracle: it is checked against what the pages and mathematics
fix, never against a re-typed copy of its own arithmetic.

Each test names the passage it pins.  A plausible slip anywhere in the oracle
(wrong nibble order, dropped bias, wrong group index, transposed operands,
double rounding, a sign error in the tie rule) fails at least one of them.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthetic
from exact import bf16_bits_of, bf16_fraction, to_bf16, to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def packed(orc, codes):
    return orc.pack_rows(np.asarray(codes, dtype=np.uint8))


def ones_bf16(shape, value=1.0):
    return synthetic.bf16_bits(np.full(shape, value, dtype=np.float32))


# ---------------------------------------------------------------------------
# Packing ("Packed Storage Layout": a in bits 0-3 ... h in bits 28-31)
# ---------------------------------------------------------------------------

def test_pack_reads_as_reversed_hex_digits(orc):
    # The page's formula puts code a in the lowest nibble, so the word printed
    # in hex lists the eight codes right to left.
    assert orc.pack8([1, 2, 3, 4, 5, 6, 7, 8]) == 0x87654321
    g = np.random.default_rng(1)
    for _ in range(200):
        c = g.integers(0, 16, size=8)
        w = orc.pack8(c)
        assert f"{w:08x}" == "".join("%x" % v for v in c[::-1])


def test_pack_unpack_exhaustive(orc):
    for pos in range(8):
        for code in range(16):
            c = np.zeros(8, dtype=np.uint8)
            c[pos] = code
            w = orc.pack8(c)
            assert w == code * 16 ** pos
            assert [orc.unpack(w, i) for i in range(8)] == list(c)


def test_pack_rows_roundtrip_and_row_layout(orc):
    codes = synthetic.random_codes(7, 192, seed=3)
    qw = orc.pack_rows(codes)
    assert qw.shape == (7, 24)
    assert np.array_equal(orc.unpack_rows(qw, 192), codes)
    # word j of row n holds codes k = 8j .. 8j+7 of that row
    for n in (0, 6):
        for j in (0, 5, 23):
            assert f"{int(qw[n, j]):08x}" == "".join("%x" % v for v in codes[n, 8 * j:8 * j + 8][::-1])


# ---------------------------------------------------------------------------
# bf16 conversions (BF16 everywhere: "Group-Wise Affine Quantization")
# ---------------------------------------------------------------------------

def test_bf16_widening_matches_torch_for_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_rounding_matches_torch_on_fp32_values(orc):
    g = np.random.default_rng(2)
    vals = [g.standard_normal(20000).astype(np.float32),
            (g.standard_normal(5000) * 1e-39).astype(np.float32),       # bf16 subnormals
            np.clip(g.standard_normal(5000) * 3e38, -3.4e38, 3.4e38).astype(np.float32),  # overflow edge
            np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-45], dtype=np.float32)]
    # exact ties between neighbouring bf16 values: low half = 0x8000
    tie_bits = (g.integers(0, 2**16, 5000).astype(np.uint32) << 16) | 0x8000
    tie_bits = tie_bits[((tie_bits >> 23) & 0xFF) != 0xFF]
    vals.append(tie_bits.view(np.float32))
    v = np.concatenate(vals)
    v = v[np.isfinite(v)]
    ours = orc.f64_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounding_is_single_rounding_from_fp64(orc):
    # Values a hair above a bf16 midpoint that fp32 cannot hold: a double
    # rounding through fp32 would land on the midpoint and round to even.
    g = np.random.default_rng(4)
    for _ in range(2000):
        e = int(g.integers(-120, 120))
        m = int(g.integers(128, 256))
        lo = Fraction(m, 128) * Fraction(2) ** e
        mid = lo + Fraction(1, 256) * Fraction(2) ** e
        for delta in (Fraction(1, 2 ** 40), -Fraction(1, 2 ** 40), Fraction(0)):
            v = mid + delta * Fraction(2) ** e
            fv = float(v)
            exact = to_bf16(Fraction(fv))
            assert int(orc.f64_to_bf16([fv])[0]) == bf16_bits_of(exact)


# ---------------------------------------------------------------------------
# Dequantization ("Reconstruct a Stored Group": w = q*s + b, signed scale)
# ---------------------------------------------------------------------------

def _golden_orientation():
    rows = []
    with open(os.path.join(GOLDEN, "orientation_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, s, b, q, approx = line.split()
                rows.append((name, float(s), float(b), int(q), float(approx)))
    return rows


def test_dequant_printed_orientation_example(orc):
    rows = _golden_orientation()
    assert len(rows) == 4
    got = {}
    for name, s, b, q, approx in rows:
        sb = int(synthetic.bf16_bits(np.float32([s]))[0])
        bb = int(synthetic.bf16_bits(np.float32([b]))[0])
        w = float(orc.dequant(sb, bb, q))
        # "about" the printed endpoint: within one bf16 rounding of the stored
        # scale (15 codes of 2^-12 each) plus the bias rounding
        assert abs(w - approx) < 0.01, (name, q, w, approx)
        got[(name, q)] = w
    # stored bias is the q=0 endpoint exactly when it is exact in bf16 (-0.5 is)
    assert got[("positive", 0)] == -0.5
    assert got[("positive", 15)] == 15 * 0.0869140625 - 0.5      # bf16(0.0867) = 0.0869140625
    # same range, opposite code order
    assert got[("positive", 0)] == pytest.approx(got[("negative", 15)], abs=0.005)
    assert got[("positive", 15)] == pytest.approx(got[("negative", 0)], abs=0.005)
    assert got[("negative", 0)] > got[("negative", 15)]


def test_dequant_is_one_fp32_rounding_of_the_exact_value(orc):
    g = np.random.default_rng(5)
    pats = []
    for _ in range(400):
        e_s = int(g.integers(100, 140))
        e_b = int(g.integers(100, 140))
        s = int(g.integers(0, 2)) << 15 | e_s << 7 | int(g.integers(0, 128))
        b = int(g.integers(0, 2)) << 15 | e_b << 7 | int(g.integers(0, 128))
        pats.append((s, b))
    pats += [(0, 0), (0x8000, 0x3F80), (0x3F80, 0), (0x0001, 0x0001), (0x8001, 0x7F7F),
             (0x0080, 0x8080), (0x3E00, 0xBF00)]
    for s, b in pats:
        for q in range(16):
            exact = bf16_fraction(s) * q + bf16_fraction(b)
            want = to_f32(exact)
            got = Fraction(float(orc.dequant(s, b, q)))
            assert got == want, (hex(s), hex(b), q)


@pytest.mark.parametrize("G", [64, 128])
def test_dequant_rows_brute_force(orc, G):
    wts = synthetic.quantized_weights(5, 256, group=G, seed=6)
    out = orc.dequant_rows(wts.qw, wts.scales, wts.biases, 256, group=G, rows=[4, 0, 2])
    codes = orc.unpack_rows(wts.qw, 256)
    for r, n in enumerate([4, 0, 2]):
        for k in range(0, 256, 7):
            g = k // G
            exact = bf16_fraction(int(wts.scales[n, g])) * int(codes[n, k]) + bf16_fraction(int(wts.biases[n, g]))
            assert Fraction(float(out[r, k])) == to_f32(exact)


# ---------------------------------------------------------------------------
# The product: closed forms ("Quantized Matrix Multiplication" equations)
# ---------------------------------------------------------------------------

def _scales_biases(N, K, seed, bias="noise", group=64):
    w = synthetic.quantized_weights(N, K, group=group, seed=seed, bias=bias)
    return w.scales, w.biases


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("c", [0, 1, 7, 8, 15])
def test_cf1_all_codes_equal(orc, c, G):
    # all codes = c: y = sum_g (s_g c + b_g) * sum_{k in g} x_k, groups of G codes
    N, K, M = 6, 384, 2
    codes = np.full((N, K), c, dtype=np.uint8)
    qw = packed(orc, codes)
    s, b = _scales_biases(N, K, seed=7, group=G)
    assert s.shape == (N, K // G)
    x = synthetic.activations(M, K, seed=7)
    y, _ = orc.qmm(x, qw, s, b, group=G)
    for m in range(M):
        xs = [bf16_fraction(int(v)) for v in x[m]]
        for n in range(N):
            want = Fraction(0)
            for g in range(K // G):
                wg = bf16_fraction(int(s[n, g])) * c + bf16_fraction(int(b[n, g]))
                assert to_f32(wg) == wg          # exact in fp32 for these values
                want += wg * sum(xs[G * g:G * g + G])
            assert abs(Fraction(y[m, n]) - want) <= Fraction(1, 2 ** 45) * (abs(want) + 1)


def test_cf2_identity_like_weights_copy_x(orc):
    # s = 1, b = 0, q[n,k] = [k == n]  ->  y[m,n] = x[m,n], bf16 output is x bitwise
    N, K, M = 64, 128, 3
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[np.arange(N), np.arange(N)] = 1
    qw = packed(orc, codes)
    s = ones_bf16((N, K // 64))
    b = np.zeros((N, K // 64), dtype=np.uint16)
    x = synthetic.activations(M, K, seed=8)
    y, a = orc.qmm(x, qw, s, b)
    assert np.array_equal(orc.f64_to_bf16(y), x[:, :N])
    assert np.array_equal(a, np.abs(y))


def test_cf3_ramp_codes(orc):
    # q[n,k] = (k + n) mod 16, s = 1/8, b = 1, x = 1: every 16 consecutive k
    # carry each code once, so y = K*(7.5/8 + 1) exactly for K a multiple of 16
    N, K = 20, 448
    k = np.arange(K)
    codes = np.stack([(k + n) % 16 for n in range(N)]).astype(np.uint8)
    qw = packed(orc, codes)
    s = ones_bf16((N, K // 64), 0.125)
    b = ones_bf16((N, K // 64), 1.0)
    x = ones_bf16((1, K))
    y, _ = orc.qmm(x, qw, s, b)
    assert np.all(y == K * (7.5 / 8 + 1))


def test_cf4_zero_scale_is_bias_only_and_zero_bias_is_scale_only(orc):
    N, K, M = 5, 256, 2
    wts = synthetic.quantized_weights(N, K, seed=9)
    x = synthetic.activations(M, K, seed=9)
    zeros = np.zeros_like(wts.scales)
    y_b, _ = orc.qmm(x, wts.qw, zeros, wts.biases)
    codes = orc.unpack_rows(wts.qw, K)
    for m in range(M):
        xs = [bf16_fraction(int(v)) for v in x[m]]
        for n in range(N):
            want = sum(bf16_fraction(int(wts.biases[n, g])) * sum(xs[64 * g:64 * g + 64]) for g in range(K // 64))
            assert abs(Fraction(y_b[m, n]) - want) <= Fraction(1, 2 ** 45) * (abs(want) + 1)
    y_s, _ = orc.qmm(x, wts.qw, wts.scales, zeros)
    for m in range(M):
        xs = [bf16_fraction(int(v)) for v in x[m]]
        for n in range(N):
            want = sum(bf16_fraction(int(wts.scales[n, g])) * sum(xs[k] * int(codes[n, k]) for k in range(64 * g, 64 * g + 64))
                       for g in range(K // 64))
            assert abs(Fraction(y_s[m, n]) - want) <= Fraction(1, 2 ** 45) * (abs(want) + 1)


def test_cf5_orientation_equivalence(orc):
    # (s, b, q) and (-s, b + 15 s, 15 - q) reconstruct the same weights; with s a
    # power of two and b a multiple of s every step is exact, so y is bitwise equal
    N, K, M = 9, 192, 2
    codes = synthetic.random_codes(N, K, seed=10)
    g = np.random.default_rng(10)
    s_val = 2.0 ** g.integers(-9, -4, size=(N, K // 64))
    b_val = s_val * g.integers(-12, 4, size=(N, K // 64))
    s = synthetic.bf16_bits(s_val.astype(np.float32))
    b = synthetic.bf16_bits(b_val.astype(np.float32))
    s2 = synthetic.bf16_bits((-s_val).astype(np.float32))
    b2 = synthetic.bf16_bits((b_val + 15 * s_val).astype(np.float32))
    x = synthetic.activations(M, K, seed=10)
    y1, _ = orc.qmm(x, packed(orc, codes), s, b)
    y2, _ = orc.qmm(x, packed(orc, (15 - codes).astype(np.uint8)), s2, b2)
    assert np.array_equal(y1, y2)


def test_cf6_zero_activations_give_positive_zero(orc):
    N, K = 4, 128
    wts = synthetic.quantized_weights(N, K, seed=11)
    x = np.zeros((2, K), dtype=np.uint16)
    y, a = orc.qmm(x, wts.qw, wts.scales, wts.biases)
    assert np.all(y == 0) and not np.any(np.signbit(y))
    assert np.all(orc.f64_to_bf16(y) == 0)
    assert np.all(a == 0)


def test_cf7_exact_bias_distribution_is_exact(orc):
    # b = -8 s exactly: w = s (q - 8) is exact, every x*w product is exact in fp64
    # and the sum is small enough to be exact, so y64 equals the rational sum
    N, K, M = 6, 256, 2
    wts = synthetic.quantized_weights(N, K, seed=12, bias="exact")
    x = synthetic.activations(M, K, seed=12)
    y, _ = orc.qmm(x, wts.qw, wts.scales, wts.biases)
    codes = orc.unpack_rows(wts.qw, K)
    for m in range(M):
        xs = [bf16_fraction(int(v)) for v in x[m]]
        for n in range(N):
            want = sum(xs[k] * bf16_fraction(int(wts.scales[n, k // 64])) * (int(codes[n, k]) - 8) for k in range(K))
            assert Fraction(y[m, n]) == want


def test_brute_force_against_exact_rationals(orc):
    for (M, N, K, G, seed) in [(1, 3, 64, 64, 20), (2, 16, 128, 64, 21), (3, 5, 192, 64, 22), (2, 7, 256, 128, 24),
                               (1, 4, 384, 128, 25)]:
        wts = synthetic.quantized_weights(N, K, group=G, seed=seed)
        x = synthetic.activations(M, K, seed=seed)
        y, a = orc.qmm(x, wts.qw, wts.scales, wts.biases, group=G)
        codes = orc.unpack_rows(wts.qw, K)
        for m in range(M):
            xs = [bf16_fraction(int(v)) for v in x[m]]
            for n in range(N):
                ws = [to_f32(bf16_fraction(int(wts.scales[n, k // G])) * int(codes[n, k])
                             + bf16_fraction(int(wts.biases[n, k // G]))) for k in range(K)]
                want = sum(xv * wv for xv, wv in zip(xs, ws))
                absw = sum(abs(xv * wv) for xv, wv in zip(xs, ws))
                assert abs(Fraction(y[m, n]) - want) <= Fraction(K, 2 ** 52) * absw
                assert abs(Fraction(a[m, n]) - absw) <= Fraction(K, 2 ** 52) * absw


def test_brute_force_wide_exponent_spread(orc):
    # scale and bias several binades apart: the dequantized weights carry ~24
    # significant bits, so x*w needs more than fp32 and the sums must be fp64
    M, N, K = 2, 6, 128
    g = np.random.default_rng(23)
    codes = synthetic.random_codes(N, K, seed=23)
    e_s = g.integers(100, 112, size=(N, K // 64))
    e_b = e_s + g.integers(8, 14, size=(N, K // 64))
    s = ((g.integers(0, 2, size=e_s.shape) << 15) | (e_s << 7) | g.integers(0, 128, size=e_s.shape)).astype(np.uint16)
    b = ((g.integers(0, 2, size=e_b.shape) << 15) | (e_b << 7) | g.integers(0, 128, size=e_b.shape)).astype(np.uint16)
    x = synthetic.activations(M, K, seed=23)
    y, a = orc.qmm(x, packed(orc, codes), s, b)
    for m in range(M):
        xs = [bf16_fraction(int(v)) for v in x[m]]
        for n in range(N):
            ws = [to_f32(bf16_fraction(int(s[n, k // 64])) * int(codes[n, k]) + bf16_fraction(int(b[n, k // 64])))
                  for k in range(K)]
            want = sum(xv * wv for xv, wv in zip(xs, ws))
            absw = sum(abs(xv * wv) for xv, wv in zip(xs, ws))
            assert abs(Fraction(y[m, n]) - want) <= Fraction(K, 2 ** 52) * absw


def test_rows_selection_and_permutation(orc):
    N, K, M = 12, 256, 2
    wts = synthetic.quantized_weights(N, K, seed=13)
    x = synthetic.activations(M, K, seed=13)
    y, _ = orc.qmm(x, wts.qw, wts.scales, wts.biases)
    perm = np.random.default_rng(13).permutation(N)
    yp, _ = orc.qmm(x, wts.qw[perm], wts.scales[perm], wts.biases[perm])
    assert np.array_equal(yp, y[:, perm])
    ys, _ = orc.qmm(x, wts.qw, wts.scales, wts.biases, rows=[11, 3, 3])
    assert np.array_equal(ys, y[:, [11, 3, 3]])


def test_linearity_in_x(orc):
    # doubling x is exact in bf16 and doubles every product and partial sum
    N, K = 8, 192
    wts = synthetic.quantized_weights(N, K, seed=14)
    x = synthetic.activations(2, K, seed=14)
    x2 = synthetic.bf16_bits(2 * synthetic.bf16_values(x))
    y1, _ = orc.qmm(x, wts.qw, wts.scales, wts.biases)
    y2, _ = orc.qmm(x2, wts.qw, wts.scales, wts.biases)
    assert np.array_equal(y2, 2 * y1)
    # rows of x are independent: row m of a 2-row call equals the 1-row call
    y0, _ = orc.qmm(x[1:], wts.qw, wts.scales, wts.biases)
    assert np.array_equal(y0[0], y1[1])


# ---------------------------------------------------------------------------
# Routed form (hy4 page kernel table: mul_mv_id)
# ---------------------------------------------------------------------------

def test_routed_reduces_to_plain_product(orc):
    E, N, K, M, top_k = 4, 10, 128, 3, 2
    wts = synthetic.quantized_weights(N, K, seed=15, lead=(E,))
    x = synthetic.activations(M, K, seed=15)
    ids = np.array([[2, 0], [2, 3], [1, 2]], dtype=np.int32)
    y, a = orc.qmm_id(x, wts.qw, wts.scales, wts.biases, ids)
    for m in range(M):
        for j in range(top_k):
            e = ids[m, j]
            ye, ae = orc.qmm(x[m:m + 1], wts.qw[e], wts.scales[e], wts.biases[e])
            assert np.array_equal(y[m, j], ye[0]) and np.array_equal(a[m, j], ae[0])
    # E = 1, every id 0: the plain product
    y1, _ = orc.qmm_id(x, wts.qw[:1], wts.scales[:1], wts.biases[:1], np.zeros((M, 1), dtype=np.int32))
    yp, _ = orc.qmm(x, wts.qw[0], wts.scales[0], wts.biases[0])
    assert np.array_equal(y1[:, 0, :], yp)
    # per-slot inputs
    xs = synthetic.activations(M * top_k, K, seed=16).reshape(M, top_k, K)
    ys, _ = orc.qmm_id(xs, wts.qw, wts.scales, wts.biases, ids, x_per_slot=True)
    for m in range(M):
        for j in range(top_k):
            e = ids[m, j]
            ye, _ = orc.qmm(xs[m, j][None], wts.qw[e], wts.scales[e], wts.biases[e])
            assert np.array_equal(ys[m, j], ye[0])
    with pytest.raises(ValueError):
        orc.qmm_id(x, wts.qw, wts.scales, wts.biases, np.full((M, top_k), E, dtype=np.int32))


# ---------------------------------------------------------------------------
# Argmax (Gemma-4 megakernel page: 4-bit LM head with in-kernel argmax;
# ties go to the lowest index)
# ---------------------------------------------------------------------------

def test_argmax_ties_and_gap(orc):
    assert orc.argmax([1.0, 3.0, 3.0, 2.0]) == (1, 0.0)
    assert orc.argmax([5.0]) == (0, float("inf"))
    assert orc.argmax([-1.0, -0.5, -2.0]) == (1, 0.5)
    assert orc.argmax([0.0, -0.0, 0.0])[0] == 0


def test_argmax_planted_row_and_duplicates(orc):
    N, K = 300, 256
    wts = synthetic.quantized_weights(N, K, seed=17, bias="exact")
    x = synthetic.activations(1, K, seed=17)
    xv = synthetic.bf16_values(x)[0]
    codes = orc.unpack_rows(wts.qw, K)
    star = 123
    codes[star] = np.where(xv > 0, 15, 0)          # maximises sum x (q - 8) s
    codes[200] = codes[star]
    qw = packed(orc, codes)
    s = wts.scales.copy()
    s[200] = s[star]
    b = wts.biases.copy()
    b[200] = b[star]
    y, a = orc.qmm(x, qw, s, b)
    best, gap = orc.argmax(y[0])
    assert best == star                              # duplicate at 200 loses the tie
    assert y[0, star] == y[0, 200] and gap == 0.0
    y2, _ = orc.qmm(x, np.delete(qw, 200, 0), np.delete(s, 200, 0), np.delete(b, 200, 0))
    best2, gap2 = orc.argmax(y2[0])
    assert best2 == star and gap2 > 1e-3 * 2 * a[0, star]


# ---------------------------------------------------------------------------
# GeGLU activation (Gemma-4 page: GeGLU MLP; GELU(g) = g * Phi(g), exact form)
# ---------------------------------------------------------------------------

# standard normal CDF values from published tables (15 significant digits)
PHI_TABLE = {0.5: 0.691462461274013, 1.0: 0.841344746068543, 2.0: 0.977249868051821,
             3.0: 0.998650101968370, -1.0: 0.158655253931457, -2.5: 0.00620966532577613}


def test_gelu_matches_tabulated_normal_cdf(orc):
    xs = np.array(sorted(PHI_TABLE), dtype=np.float64)
    got = orc.geglu_values(xs, 1.0)
    want = np.array([x * PHI_TABLE[x] for x in xs])
    assert np.all(np.abs(got - want) <= 1e-14 * np.maximum(1.0, np.abs(want)))
    assert orc.geglu_values(np.array([0.0]), 5.0)[0] == 0.0


def test_gelu_odd_part_is_the_identity(orc):
    # Phi(x) + Phi(-x) = 1, so GELU(x) - GELU(-x) = x for every x
    x = np.linspace(-8.0, 8.0, 1601)
    d = orc.geglu_values(x, 1.0) - orc.geglu_values(-x, 1.0)
    assert np.all(np.abs(d - x) <= 4e-16 * np.maximum(1.0, np.abs(x)))


def simpson_phi(x, n=20000):
    """Standard normal CDF by composite Simpson integration of the density from
    -12 (where the mass below is < 1e-32): independent of erf."""
    t = np.linspace(-12.0, x, n + 1)
    f = np.exp(-0.5 * t * t) / np.sqrt(2.0 * np.pi)
    h = (x + 12.0) / n
    return h / 3.0 * (f[0] + f[-1] + 4.0 * f[1:-1:2].sum() + 2.0 * f[2:-1:2].sum())


def test_gelu_against_integrated_normal_density(orc):
    xs = np.array([-5.0, -2.2, -0.7, -0.01, 0.3, 1.3, 2.9, 6.0])
    got = orc.geglu_values(xs, 1.0)
    want = np.array([x * simpson_phi(x) for x in xs])
    assert np.all(np.abs(got - want) <= 1e-11 * np.maximum(1.0, np.abs(xs)))


def test_geglu_gates_the_up_rows(orc):
    # fused [2I, K] matrix: gate rows of codes 9 and up rows of codes 3 with
    # s = 1/4, b = -2 (both exact), so gate = 0.25 * sum(x) and up = -1.25 * sum(x);
    # h = GELU(gate) * up, and swapping the halves changes h
    I, K, M = 3, 128, 2
    codes = np.concatenate([np.full((I, K), 9, dtype=np.uint8), np.full((I, K), 3, dtype=np.uint8)])
    qw = packed(orc, codes)
    s = ones_bf16((2 * I, K // 64), 0.25)
    b = ones_bf16((2 * I, K // 64), -2.0)
    x = synthetic.activations(M, K, seed=21)
    h, g, _, u, _ = orc.geglu(x, qw, s, b, I)
    sx = np.array([float(sum(bf16_fraction(int(v)) for v in x[m])) for m in range(M)])
    assert np.allclose(g, np.repeat((0.25 * sx)[:, None], I, axis=1), rtol=1e-15, atol=0)
    assert np.allclose(u, np.repeat((-1.25 * sx)[:, None], I, axis=1), rtol=1e-15, atol=0)
    for m in range(M):
        gm = 0.25 * sx[m]
        um = -1.25 * sx[m]
        want = gm * simpson_phi(gm) * um
        # the integration is accurate to ~1e-13 in Phi (absolute), so scale by |g u|
        assert np.all(np.abs(h[m] - want) <= 1e-11 * abs(gm * um))
    h2 = orc.geglu(x, qw, s, b, I, cols=[2, 0])[0]
    assert np.array_equal(h2, h[:, [2, 0]])
    swapped = orc.geglu_values(u, g)
    assert not np.allclose(swapped, h)
