"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test ties one oracle function to something other than itself: hand-derived
golden bytes, closed forms, brute force on tiny inputs, library routines for special
cases, or invariants.  Pages cited:
  [AT] aratech.ae BitNet b1.58 article: "Ternary weights {-1, 0, +1}", "BitLinear: the
       building block", and the information-content paragraph on log2(3) ~ 1.58 bits.
  [BH] bhfrc.com news 56965: section 1.1 (add / subtract / skip; ~10x vs fp16) and
       section 4.1 (2-bit code table).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from bitlinear_fwd_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load_json(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ exact rounding helper
def test_round_rational_ieee_cases():
    f = oracle.round_rational_to_f32
    assert f(1, 1) == np.float32(1.0)
    assert f(1, 3) == np.float32(1.0 / 3.0)
    # exactly half-way between 1 and 1+2^-23: ties to the even significand (1.0)
    assert f((1 << 24) + 1, 1 << 24) == np.float32(1.0)
    # half-way between 1+2^-23 (odd) and 1+2^-22 (even) -> 1+2^-22
    assert f((1 << 24) + 3, 1 << 24) == np.float32(1.0 + 2.0 ** -22)
    # just above half-way rounds up
    assert f((1 << 25) + 3, 1 << 25) == np.float32(1.0 + 2.0 ** -23)
    # subnormals: 2^-150 is half of the smallest step -> 0 (even); 3*2^-150 -> 2^-148
    assert f(1, 1 << 150) == np.float32(0.0)
    assert f(3, 1 << 150) == np.float32(2.0 ** -148)
    assert f(1, 1 << 149) == np.float32(2.0 ** -149)
    assert f(0, 7) == np.float32(0.0)


# ------------------------------------------------------------------ P2: gamma = mean|W|
def test_gamma_bruteforce_tiny_wide_range():
    rng = _rng(1)
    for trial in range(40):
        n = int(rng.integers(1, 40))
        w = (rng.standard_normal(n) * 10.0 ** rng.uniform(-40, 30, n)).astype(np.float32)
        if trial % 5 == 0:
            w[: n // 2] = np.float32(1e-45) * rng.integers(1, 100, n // 2)  # subnormals
        g = oracle.gamma_absmean(w)
        assert g == oracle.gamma_bruteforce(w)


def test_gamma_is_nearest_float_to_exact_mean():
    from fractions import Fraction
    rng = _rng(2)
    for _ in range(20):
        w = rng.standard_normal(33).astype(np.float32) * np.float32(0.02)
        g = oracle.gamma_absmean(w)
        mean = sum(Fraction(abs(float(v))) for v in w) / len(w)
        err = abs(Fraction(float(g)) - mean)
        for nb in (np.nextafter(g, np.float32(np.inf)), np.nextafter(g, np.float32(0))):
            assert err <= abs(Fraction(float(nb)) - mean)


def test_gamma_closed_forms():
    assert oracle.gamma_absmean(np.full((3, 5), -0.375, np.float32)) == np.float32(0.375)
    assert oracle.gamma_absmean(np.array([[1.0, -3.0]], np.float32)) == np.float32(2.0)
    assert oracle.gamma_absmean(np.zeros((4, 4), np.float32)) == np.float32(0.0)
    w = np.array([1.0, 2.0, 4.0], np.float32)  # 7/3
    assert oracle.gamma_absmean(w) == np.float32(7.0 / 3.0)


def test_gamma_matches_float64_library_mean():
    w = synth.latent_weights(256, 1024, seed=7).numpy()
    g = oracle.gamma_absmean(w)
    assert g == np.float32(np.mean(np.abs(w), dtype=np.float64))


def _is_nearest_f32(g, exact) -> bool:
    """g (fp32) is at least as close to the rational `exact` as both fp32 neighbours."""
    from fractions import Fraction
    g = np.float32(g)
    err = abs(Fraction(float(g)) - exact)
    return all(err <= abs(Fraction(float(nb)) - exact)
               for nb in (np.nextafter(g, np.float32(np.inf)), np.nextafter(g, np.float32(0))))


BIG = (1 << 24) + (1 << 20) + 7  # above 2^24 weights, as the 2048-token and 100B-class matrices


def test_gamma_above_2_24_weights_closed_forms():
    from fractions import Fraction
    # a constant tensor has mean |c| exactly, at any magnitude: subnormal, tiny, typical, the
    # largest binade (the sum then needs the top limbs of the accumulator)
    for c in (-0.375, 1.0e-40, -2.0 ** -126, 0.02, 3.0e38):
        w = np.full(BIG, c, np.float32)
        assert oracle.gamma_absmean(w) == np.abs(np.float32(c)), c
    # two values, the switch placed on either side of index 2^24: the exact mean is the
    # weighted rational, and gamma is the fp32 nearest to it
    for a, b, n1 in ((0.02, -0.03, (1 << 24) - 1), (1.0e-3, 7.0e-41, 1 << 24), (-5.0, 1.0e30, (1 << 24) + 1)):
        fa, fb = np.float32(a), np.float32(b)
        w = np.empty(BIG, np.float32)
        w[:n1], w[n1:] = fa, fb
        exact = (n1 * Fraction(abs(float(fa))) + (BIG - n1) * Fraction(abs(float(fb)))) / BIG
        assert _is_nearest_f32(oracle.gamma_absmean(w), exact), (a, b, n1)
    # 3 * 2^24 + 3 copies of 1.0 and of 2^-24 split 1:2: mean (1 + 2 * 2^-24) / 3 exactly
    n3 = 3 * ((1 << 24) + 1)
    w = np.full(n3, 2.0 ** -24, np.float32)
    w[: n3 // 3] = 1.0
    assert _is_nearest_f32(oracle.gamma_absmean(w), (1 + 2 * Fraction(1, 1 << 24)) / 3)


def test_gamma_large_tensor_exact_sum_matches_fsum():
    # 2^25 + 5 Gaussian latents with values planted across the exponent range (subnormals,
    # the smallest and largest binades, signs) scattered over the tensor and at the indices
    # around 2^24.  math.fsum gives the correctly rounded fp64 sum of the same values, an
    # independent routine: the exact integer sum must round to it.
    from fractions import Fraction
    n = (1 << 25) + 5
    w = synth.latent_weights(1, n, seed=19).numpy().ravel().copy()
    rng = _rng(8)
    planted = np.array([1.0e-45, -3.0e-42, 1.17549435e-38, -2.0 ** -126, 3.4e38, -1.0e38, 0.5, -1.5, 1e-20, 7.0,
                        2.0 ** 100, -2.0 ** -140], np.float32)
    where = np.concatenate([rng.integers(0, n, 4000), np.arange((1 << 24) - 6, (1 << 24) + 6)])
    w[where] = planted[np.arange(where.size) % planted.size]
    s = oracle.exact_abs_sum_scaled(w)
    ref = math.fsum(np.abs(w).astype(np.float64).tolist())
    assert float(Fraction(s, 1 << 149)) == ref
    # the Gaussian part alone, against the same routine
    w2 = synth.latent_weights(1, n, seed=20).numpy().ravel()
    s2 = oracle.exact_abs_sum_scaled(w2)
    assert float(Fraction(s2, 1 << 149)) == math.fsum(np.abs(w2).astype(np.float64).tolist())
    g2 = oracle.gamma_absmean(w2)
    assert _is_nearest_f32(g2, Fraction(s2, n << 149))
    # and gamma against the fp64 library mean: within half an fp32 ulp of fsum / n
    half_ulp = (float(np.nextafter(g2, np.float32(np.inf))) - float(g2)) / 2
    assert abs(float(g2) - math.fsum(np.abs(w2).astype(np.float64).tolist()) / n) <= half_ulp * (1 + 1e-9)


def test_gamma_rejects_non_finite():
    for bad in (np.inf, -np.inf, np.nan):
        w = np.ones(10, np.float32)
        w[7] = bad
        with pytest.raises(ValueError):
            oracle.gamma_absmean(w)


def test_gamma_gaussian_expectation():
    # E|W| = sigma * sqrt(2/pi) for W ~ N(0, sigma^2); std error sigma*sqrt(1-2/pi)/sqrt(n)
    w = synth.latent_weights(512, 2048, seed=11).numpy()
    g = float(oracle.gamma_absmean(w))
    sigma = synth.SIGMA_W
    mu = sigma * math.sqrt(2 / math.pi)
    se = sigma * math.sqrt(1 - 2 / math.pi) / math.sqrt(w.size)
    assert abs(g - mu) < 5 * se


# ------------------------------------------------------------------ P1/P3: ternary codes
def test_ternary_values_and_golden():
    for case in _load_json("quant_examples.json")["weights"]:
        w = np.array(case["W"], np.float32)
        g, q, _ = oracle.quantize_weights(w)
        assert g == np.float32(case["gamma"]), case
        assert q.tolist() == case["q"], case


def test_ternary_distribution_closed_form():
    # t = W / gamma ~ N(0, pi/2) for Gaussian W; q = 0 iff |t| <= 1/2:
    # P0 = erf(1 / (2 sqrt(pi))) = 0.3101, P(+1) = P(-1) = (1 - P0) / 2.
    w = synth.latent_weights(1024, 2048, seed=13).numpy()
    g, q, _ = oracle.quantize_weights(w)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    n = q.size
    p0 = math.erf(1 / (2 * math.sqrt(math.pi)))
    f0 = float(np.mean(q == 0))
    fp = float(np.mean(q == 1))
    fm = float(np.mean(q == -1))
    assert abs(f0 - p0) < 5 * math.sqrt(p0 * (1 - p0) / n)
    p1 = (1 - p0) / 2
    for f in (fp, fm):
        assert abs(f - p1) < 5 * math.sqrt(p1 * (1 - p1) / n)
    # entropy of the code distribution stays below log2(3) ~ 1.585 bits ([AT], [BH] 1.1)
    h = -sum(p * math.log2(p) for p in (f0, fp, fm))
    assert 1.57 < h <= math.log2(3)
    assert abs(math.log2(3) - 1.58496) < 1e-5


def test_ternarise_metamorphic():
    w = synth.latent_weights(64, 512, seed=17).numpy()
    g, q, _ = oracle.quantize_weights(w)
    g2, q2, _ = oracle.quantize_weights(-w)  # RNE is symmetric
    assert g2 == g and np.array_equal(q2, -q)
    for j in (-3, 5):  # exact power-of-two scaling leaves every code unchanged
        g3, q3, _ = oracle.quantize_weights(w * np.float32(2.0 ** j))
        assert g3 == g * np.float32(2.0 ** j) and np.array_equal(q3, q)


# ------------------------------------------------------------------ packing layout
def _golden_q(case):
    q = np.full((case["N"], case["K"]), case["fill"], np.int8)
    for n, k, v in case["set"]:
        q[n, k] = v
    return q


def test_pack_golden_bytes():
    for case in _load_json("pack_layout.json")["cases"]:
        p = oracle.pack(_golden_q(case))
        assert p.size == case["expect_size"], case["name"]
        if "expect_all_bytes" in case:
            assert np.all(p == case["expect_all_bytes"]), case["name"]
            continue
        seen = np.zeros(p.size, bool)
        for off, vals in case["expect_bytes"].items():
            off = int(off)
            assert p[off:off + 4].tolist() == vals, (case["name"], off)
            seen[off:off + 4] = True
        if "expect_other_bytes" in case:
            assert np.all(p[~seen] == case["expect_other_bytes"]), case["name"]


def test_pack_roundtrip_and_padding_codes():
    rng = _rng(3)
    for n, k in [(1, 1), (16, 256), (17, 300), (33, 513), (40, 1000)]:
        q = rng.integers(-1, 2, (n, k)).astype(np.int8)
        p = oracle.pack(q)
        assert p.size == oracle.n_pad(n) * oracle.k_pad(k) // 4
        assert np.array_equal(oracle.unpack(p, n, k), q)
        codes = oracle.unpack_codes(p, n, k)
        inner = codes[:n, :k]
        assert not np.any(inner == 3)  # no padding code inside the matrix
        assert np.all(codes[n:, :] == 3) and np.all(codes[:, k:] == 3)
        # code table: 00 -> 0, 01 -> +1, 10 -> -1 ([BH] 4.1)
        assert np.array_equal(inner == 0, q == 0)
        assert np.array_equal(inner == 1, q == 1)
        assert np.array_equal(inner == 2, q == -1)


def test_pack_rejects_non_ternary():
    with pytest.raises(ValueError):
        oracle.pack(np.array([[2]], np.int8))


def test_packed_size_closed_forms():
    # 100B-class matrix 28672 x 8192 at 2 bits/weight
    assert oracle.packed_bytes(28672, 8192) == 58_720_256
    assert oracle.packed_bytes(8192, 28672) == 58_720_256
    assert oracle.packed_bytes(6912, 2560) == 4_423_680
    assert oracle.packed_bytes(512, 256) == 32_768
    # 2e9 weights at 2 bits are 0.5 GB, inside [BH] 5.1's 0.4-0.6 GB for a 2B model;
    # at the log2(3) information bound they would be ~396 MB ([AT]: ~400 MB)
    assert 0.4e9 <= 2e9 * 2 / 8 <= 0.6e9
    assert abs(2e9 * math.log2(3) / 8 / 1e6 - 396.2) < 0.5
    # 1000 trits carry ~1585 bits ([AT]); fp16 -> ~1.58 bits is ~10x ([BH] 1.1)
    assert round(1000 * math.log2(3)) == 1585
    assert round(16 / math.log2(3)) == 10


# ------------------------------------------------------------------ P4: activation quant
def test_act_quant_golden():
    for case in _load_json("quant_examples.json")["acts"]:
        x = np.array([case["x"]], np.float32)
        xq, a = oracle.quant_acts(x)
        assert a[0] == np.float32(case["absmax"])
        assert xq[0, : x.shape[1]].tolist() == case["xq"], case
        assert np.all(xq[0, x.shape[1]:] == 0)


def test_act_quant_invariants():
    x = synth.activations(37, 700, seed=19, dtype=torch.float32, outlier_p=0.01, outlier_mult=20.0).numpy()
    x[5] = 0.0
    xq, a = oracle.quant_acts(x)
    assert xq.shape == (37, 768)
    assert np.all(np.abs(xq.astype(np.int32)) <= 127)
    assert np.all(xq[:, 700:] == 0)
    assert np.all(xq[5] == 0) and a[5] == 0
    for m in range(37):
        if m == 5:
            continue
        assert a[m] == np.max(np.abs(x[m]))
        j = int(np.argmax(np.abs(x[m])))
        assert abs(int(xq[m, j])) == 127 and np.sign(xq[m, j]) == np.sign(x[m, j])
        # quantisation error bound: |xq * a/127 - x| <= a/254 (+ fp32 slack)
        err = np.abs(xq[m, :700].astype(np.float64) * a[m] / 127 - x[m])
        assert np.all(err <= a[m] / 254 * (1 + 1e-5))
        # monotone in x within a row
        order = np.argsort(x[m], kind="stable")
        assert np.all(np.diff(xq[m, order].astype(np.int32)) >= 0)
    xq_neg, a_neg = oracle.quant_acts(-x)
    assert np.array_equal(xq_neg, -xq) and np.array_equal(a_neg, a)
    xq_s, _ = oracle.quant_acts(x * np.float32(8.0))
    assert np.array_equal(xq_s, xq)


def test_act_quant_exhaustive_bf16_rounding():
    # every finite bf16 value, quantised against a row maximum a: the code is the integer
    # nearest to the fp32 product x * fl32(127 / a), with ties going to the even integer
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(vals[finite].view(np.uint32), ref[finite].view(np.uint32))
    vals = vals[finite]
    for a in (np.float32(3.0), np.float32(1.0), np.float32(1e-3), np.float32(6.5e4)):
        row = vals[np.abs(vals) <= a]
        row = np.concatenate([row, [a]]).astype(np.float32)
        xq, amax = oracle.quant_acts(row[None, :])
        assert amax[0] == a
        s = np.float32(127.0) / a
        prod = (row * s).astype(np.float64)  # fp32 product, exact in float64
        code = xq[0, : row.size].astype(np.float64)
        diff = prod - code
        assert np.all(np.abs(diff) <= 0.5)
        tie = np.abs(diff) == 0.5
        assert np.all(code[tie] % 2 == 0)


# ------------------------------------------------------------------ SubLN + activation quant
# [AT] "BitLinear: the building block": a simplified LayerNorm right before the
# activation quantiser; read as RMS normalisation n = x * g / sqrt(mean(x^2) + eps).
def _subln(x, gain=None, eps=0.0):
    xq, sc32, sc64, ha = oracle.subln_quant_acts(np.asarray(x, np.float32), gain, eps)
    return xq, sc32, sc64, ha


def test_subln_closed_forms():
    k = 300
    # (3, 4): mean square 12.5; codes round(127 * 3/4) = round(95.25) = 95 and 127
    xq, _, sc, ha = _subln([[3.0, 4.0]])
    assert xq[0, :2].tolist() == [95, 127] and ha[0] == 4.0
    assert sc[0] == pytest.approx(4.0 / math.sqrt(12.5), rel=1e-15)
    # the gain scales the features but not the mean square: h = (3, 8)
    xq, _, sc, ha = _subln([[3.0, 4.0]], gain=[1.0, 2.0])
    assert xq[0, :2].tolist() == [48, 127] and ha[0] == 8.0  # round(47.625)
    assert sc[0] == pytest.approx(8.0 / math.sqrt(12.5), rel=1e-15)
    # constant row c: every normalised entry is c / |c|, so the scale is 1 (exactly
    # where c^2 sums without rounding in fp64)
    for c in (0.75, -3.0e-3, 1.0e4):
        xq, sc32, sc, _ = _subln([[c] * k])
        assert np.all(xq[0, :k] == 127 * int(np.sign(c))) and np.all(xq[0, k:] == 0)
        assert sc[0] == pytest.approx(1.0, rel=1e-13) and sc32[0] == 1.0
        assert c != 0.75 or sc[0] == 1.0
    # eps sits inside the square root, added to the mean square
    _, _, sc, _ = _subln([[0.75] * k], eps=0.25)
    assert sc[0] == pytest.approx(0.75 / math.sqrt(0.5625 + 0.25), rel=1e-15)
    # one non-zero feature v: mean square v^2 / K, so the scale is sqrt(K) at any v
    for kk, v in ((1000, -2.5), (777, 1.0e-20), (4096, 3.0e30)):
        row = np.zeros((1, kk), np.float32)
        row[0, 7] = v
        xq, _, sc, _ = _subln(row)
        assert xq[0, 7] == 127 * int(np.sign(v)) and np.count_nonzero(xq) == 1
        assert sc[0] == pytest.approx(math.sqrt(kk), rel=1e-15)
        _, _, sc, _ = _subln(row, gain=np.full(kk, 3.0, np.float32))  # h = fl32(3 v)
        assert sc[0] == pytest.approx(3.0 * math.sqrt(kk), rel=2.0 ** -24)
    # a zero row, or a zero gain, gives zero codes and a zero scale at any eps
    for eps in (0.0, 1e-5):
        xq, sc32, sc, _ = _subln(np.zeros((1, k), np.float32), eps=eps)
        assert not xq.any() and sc[0] == 0.0 and sc32[0] == 0.0
        xq, _, sc, _ = _subln(np.ones((1, k), np.float32), gain=np.zeros(k, np.float32), eps=eps)
        assert not xq.any() and sc[0] == 0.0


def test_subln_codes_reduce_to_the_plain_quantiser():
    x = synth.activations(9, 700, seed=23, dtype=torch.float32, outlier_p=0.01, outlier_mult=20.0).numpy()
    g = _rng(4).uniform(-2.0, 2.0, 700).astype(np.float32)
    # no gain: the codes and the absmax they were decided on are the plain quantiser's
    xq, _, _, ha = _subln(x, eps=1e-5)
    xq0, a0 = oracle.quant_acts(x)
    assert np.array_equal(xq, xq0) and np.array_equal(ha, a0)
    # a gain: the plain quantiser applied to the fp32 products x * g
    xq, _, _, ha = _subln(x, gain=g, eps=1e-5)
    xq1, a1 = oracle.quant_acts(x * g)
    assert np.array_equal(xq, xq1) and np.array_equal(ha, a1)


def test_subln_positive_scale_invariance():
    # with eps = 0 the normalisation removes any positive per-row factor: a power of two
    # scales x, x^2 and the square root exactly, so codes and scale are unchanged
    x = synth.activations(6, 513, seed=29, dtype=torch.float32).numpy()
    g = _rng(5).uniform(0.5, 1.5, 513).astype(np.float32)
    xq, sc32, sc, _ = _subln(x, gain=g)
    for f in (2.0 ** 7, 2.0 ** -9):
        xq2, sc32b, sc2, _ = _subln(x * np.float32(f), gain=g)
        assert np.array_equal(xq2, xq) and np.array_equal(sc2, sc) and np.array_equal(sc32b, sc32)
    xqn, _, scn, _ = _subln(-x, gain=g)
    assert np.array_equal(xqn, -xq) and np.array_equal(scn, sc)


def test_subln_matches_normalise_then_quantise():
    # normalise first in fp64, then quantise the normalised row: the same codes except at
    # near-ties (where fp32 rounding of x * g decides), and scale = max |n|
    m, k, eps = 12, 1000, 1e-5
    x = synth.activations(m, k, seed=31, dtype=torch.float32, outlier_p=0.005, outlier_mult=30.0).numpy()
    g = _rng(6).uniform(-1.5, 1.5, k).astype(np.float32)
    xq, _, sc, _ = _subln(x, gain=g, eps=eps)
    xd = x.astype(np.float64)
    eps32 = float(np.float32(eps))
    n = xd * g.astype(np.float64) / np.sqrt(np.mean(xd * xd, axis=1, keepdims=True) + eps32)
    amax = np.max(np.abs(n), axis=1)
    assert np.allclose(sc, amax, rtol=1e-7, atol=0)
    t = n * 127.0 / amax[:, None]
    lit = np.rint(t)
    # The oracle decides each code on r = fl32(fl32(x * g) * fl32(127 / max|fl32(x * g)|)):
    # four roundings of relative size <= 2^-24 each, on a value of magnitude <= 127.  So
    # |r - t| <= 127 * ((1 + 2^-24)^4 - 1) (plus the fp64 error of t, ~1e-13), and the two
    # codes can differ only where t lies that close to a half-integer.
    window = 127.0 * ((1.0 + 2.0 ** -24) ** 4 - 1.0) + 1e-12
    near_tie = np.abs(np.abs(t - np.trunc(t)) - 0.5) <= window
    agree = lit == xq[:, :k]
    assert np.all(agree | near_tie)
    assert np.all(np.abs(lit.astype(np.int64) - xq[:, :k]) <= 1)  # a near-tie moves a code by one step
    # the same on many rows: every disagreement sits inside that window
    x2 = synth.activations(256, 2048, seed=37, dtype=torch.float32, outlier_p=0.005, outlier_mult=30.0).numpy()
    g2 = _rng(7).uniform(-1.5, 1.5, 2048).astype(np.float32)
    xq2, _, sc2, _ = _subln(x2, gain=g2, eps=eps)
    xd2 = x2.astype(np.float64)
    n2 = xd2 * g2.astype(np.float64) / np.sqrt(np.mean(xd2 * xd2, axis=1, keepdims=True) + eps32)
    a2 = np.max(np.abs(n2), axis=1)
    assert np.allclose(sc2, a2, rtol=1e-7, atol=0)
    t2 = n2 * 127.0 / a2[:, None]
    off = np.rint(t2) != xq2[:, :2048]
    assert np.all(np.abs(np.abs(t2[off] - np.trunc(t2[off])) - 0.5) <= window)


# ------------------------------------------------------------------ squared-ReLU gating
# [AT] "BitLinear: the building block": squared ReLU in the feed-forward layers; read for a
# gate / up pair as h = relu(gate)^2 * up.
def test_gated_relu2_closed_forms():
    g = np.array([2.0, -1.0, 0.0, 0.5, -0.0, 3.0, 1e-3])
    u = np.array([3.0, 5.0, 7.0, -4.0, 2.0, 0.0, 1e6])
    h = oracle.gated_relu2(g, u)
    assert h.tolist() == [12.0, 0.0, 0.0, -1.0, 0.0, 0.0, pytest.approx(1.0, rel=1e-12)]
    assert not np.signbit(h[1])  # a negative gate: relu gives +0, times a positive up is +0


def test_gated_relu2_properties():
    rng = _rng(11)
    g, u = rng.normal(size=(5, 300)), rng.normal(size=(5, 300))
    h = oracle.gated_relu2(g, u)
    assert np.all(h[g <= 0] == 0)
    pos = g > 0
    # homogeneous of degree 2 in the gate and 1 in up (powers of two keep it exact)
    assert np.array_equal(oracle.gated_relu2(4.0 * g, u), 16.0 * h)
    assert np.array_equal(oracle.gated_relu2(g, -2.0 * u), -2.0 * h)
    # equals the square of the gate times up where the gate is positive
    assert np.allclose(h[pos], g[pos] ** 2 * u[pos], rtol=1e-15, atol=0)


def test_ffn_gate_up_matches_two_forwards():
    rng = _rng(12)
    k, n, m = 300, 40, 3
    qg, qu = (rng.integers(-1, 2, (n, k)).astype(np.int8) for _ in range(2))
    x = synth.activations(m, k, seed=41, dtype=torch.float32).numpy()
    xq, a = oracle.quant_acts(x)
    h = oracle.ffn_gate_up(qg, np.float32(0.02), qu, np.float32(0.03), xq, a, k)
    # with the gate equal to up and all-(+1) codes, h = relu(s)^3 for s = sum(xq) * gamma * a / 127
    ones = np.ones((1, k), np.int8)
    s = xq[:, :k].astype(np.int64).sum(axis=1) * float(np.float32(0.5)) * a.astype(np.float64) / 127
    h1 = oracle.ffn_gate_up(ones, np.float32(0.5), ones, np.float32(0.5), xq, a, k)[:, 0]
    assert np.allclose(h1, np.maximum(s, 0) ** 3, rtol=1e-14, atol=0)
    assert h.shape == (m, n) and np.all(np.isfinite(h))


# ------------------------------------------------------------------ 1-bit binary variant
# lpnh.cn section 2.1: binary weights sign(W) with a magnitude-compensating scale.
# Hand-derived bit positions of the binary layout (1024-byte tiles of 16 rows x 512
# columns; 16-byte slot 16 g + r; word 2 s + i / 2; bit 8 (e % 4) + 4 (i % 2) + e / 4).
def test_binary_pack_hand_derived_positions():
    n, k = 17, 1100
    assert oracle.kb_pad(k) == 1536 and oracle.packed_bytes_binary(n, k) == 32 * 1536 // 8
    expect = {
        (0, 0): (0, 0), (0, 1): (1, 0), (0, 4): (0, 1), (0, 15): (3, 3), (0, 16): (0, 4), (0, 17): (1, 4),
        (0, 32): (4, 0), (0, 63): (7, 7), (0, 64): (256, 0), (0, 256): (8, 0), (0, 300): (12, 3),
        (0, 512): (1024, 0), (1, 0): (16, 0), (16, 0): (3072, 0),
    }
    for (r, c), (byte, bit) in expect.items():
        q = -np.ones((n, k), np.int8)
        q[r, c] = 1
        packed = oracle.pack_binary(q)
        nz = np.nonzero(packed)[0]
        assert nz.tolist() == [byte] and packed[byte] == 1 << bit, ((r, c), nz, packed[nz])
        assert np.array_equal(oracle.unpack_binary(packed, n, k), q)


def test_binary_roundtrip_sizes_and_sign():
    w = np.array([[0.5, -0.5, 0.0, -0.0, 1e-30, -1e-30, 3.0, -7.0]], np.float32)
    assert oracle.binarise(w).tolist() == [[1, -1, 1, 1, 1, -1, 1, -1]]
    assert oracle.packed_bytes_binary(28672, 8192) == 28672 * 8192 // 8  # half the ternary bytes
    assert oracle.packed_bytes_binary(2560, 6912) * 2 > oracle.packed_bytes(2560, 6912)  # K pads to 512
    rng = _rng(13)
    q = np.where(rng.random((33, 777)) < 0.5, 1, -1).astype(np.int8)
    packed = oracle.pack_binary(q)
    assert np.array_equal(oracle.unpack_binary(packed, 33, 777), q)
    # bits outside the matrix are 0
    full = np.unpackbits(packed).sum()
    assert full == np.count_nonzero(q == 1)
    with pytest.raises(ValueError):
        oracle.pack_binary(np.zeros((1, 4), np.int8))
    # beta is the exact mean |W| (pinned above for gamma); the forward is the integer one
    wl = synth.latent_weights(40, 300, seed=5).numpy()
    beta, qb, _ = oracle.quantize_weights_binary(wl)
    assert beta == oracle.gamma_absmean(wl) and set(np.unique(qb)) <= {-1, 1}
    x = synth.activations(2, 300, seed=6, dtype=torch.float32).numpy()
    xq, a = oracle.quant_acts(x)
    acc, _ = oracle.forward(np.ones((1, 300), np.int8), beta, xq, a, 300)
    assert acc[:, 0].tolist() == xq[:, :300].astype(np.int64).sum(axis=1).tolist()


# ------------------------------------------------------------------ P5/P6: contraction
def test_matmul_special_cases():
    # [BH] 1.1: +1 adds the activation, -1 subtracts it, 0 skips it
    k = 300
    xq = _rng(5).integers(-127, 128, (3, 512)).astype(np.int8)
    xq[:, k:] = 0
    q = np.zeros((5, k), np.int8)
    q[0] = 1
    q[1] = -1
    q[3, 17] = 1  # one-hot row picks one activation
    q[4, ::2] = 1
    q[4, 1::2] = -1
    acc = oracle.matmul(q, xq, k)
    s = xq[:, :k].astype(np.int64).sum(1)
    assert acc.shape == (3, 5)
    assert np.array_equal(acc[:, 0], s)
    assert np.array_equal(acc[:, 1], -s)
    assert np.all(acc[:, 2] == 0)
    assert np.array_equal(acc[:, 3], xq[:, 17].astype(np.int64))
    alt = xq[:, :k:2].astype(np.int64).sum(1) - xq[:, 1:k:2].astype(np.int64).sum(1)
    assert np.array_equal(acc[:, 4], alt)
    # one-hot activation picks one column of the codes
    qr = _rng(6).integers(-1, 2, (7, k)).astype(np.int8)
    xo = np.zeros((2, k), np.int8)
    xo[1, 42] = 1
    acc = oracle.matmul(qr, xo, k)
    assert np.all(acc[0] == 0) and np.array_equal(acc[1], qr[:, 42].astype(np.int32))


def test_matmul_vs_numpy_int64():
    rng = _rng(8)
    for m, n, k in [(1, 7, 5), (4, 33, 257), (9, 64, 1000)]:
        q = rng.integers(-1, 2, (n, k)).astype(np.int8)
        xq = rng.integers(-127, 128, (m, oracle.k_pad(k))).astype(np.int8)
        ref = xq[:, :k].astype(np.int64) @ q.astype(np.int64).T
        assert np.array_equal(oracle.matmul(q, xq, k), ref)


def test_matmul_extreme_range_fits_int32():
    # |acc| <= 127 * K; the largest K of the workloads stays below 2^24, so the int32 ->
    # fp32 conversion in the rescale is exact
    assert 127 * 28672 < 2 ** 24
    k = 28672
    q = np.ones((2, k), np.int8)
    q[1] = -1
    xq = np.full((1, k), 127, np.int8)
    acc = oracle.matmul(q, xq, k)
    assert acc.tolist() == [[127 * k, -127 * k]]


def test_matmul_permutation_invariance():
    rng = _rng(9)
    k = 200
    q = rng.integers(-1, 2, (6, k)).astype(np.int8)
    xq = rng.integers(-127, 128, (3, k)).astype(np.int8)
    perm = rng.permutation(k)
    assert np.array_equal(oracle.matmul(q, xq, k), oracle.matmul(q[:, perm].copy(), xq[:, perm].copy(), k))


# ------------------------------------------------------------------ P7: brute-force float
def test_forward_within_quantisation_error_tiny():
    for seed, (m, n, k) in enumerate([(1, 8, 16), (3, 64, 256), (4, 17, 100)]):
        w = synth.latent_weights(n, k, seed=100 + seed).numpy()
        x = synth.activations(m, k, seed=600 + seed, dtype=torch.float32,
                              outlier_p=0.05, outlier_mult=20.0).numpy()
        g, q, packed = oracle.quantize_weights(w)
        xq, a = oracle.quant_acts(x)
        acc, y = oracle.forward(oracle.unpack(packed, n, k), g, xq, a, k)
        g64 = float(g)
        x64 = x.astype(np.float64)
        # against the dequantised weights: only activation rounding, |dx| <= a/254
        yq = x64 @ (g64 * q.astype(np.float64)).T
        bound_a = (a.astype(np.float64)[:, None] / 254) * g64 * np.abs(q).sum(1)[None, :]
        assert np.all(np.abs(y - yq) <= bound_a * (1 + 1e-6) + 1e-12)
        # against the latent weights: add the weight rounding term sum |W - gamma q| |x|
        yl = x64 @ w.astype(np.float64).T
        bound_w = np.abs(x64) @ np.abs(w.astype(np.float64) - g64 * q).T
        assert np.all(np.abs(y - yl) <= (bound_a + bound_w) * (1 + 1e-6) + 1e-12)


def test_rescale_closed_form():
    acc = np.array([[127, -254, 0]], np.int32)
    y = oracle.rescale(acc, np.float32(0.5), np.array([2.0], np.float32))
    assert y.tolist() == [[1.0, -2.0, 0.0]]
