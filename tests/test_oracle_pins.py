"""Pins of the CPU oracle to things other than itself (CPU only).

Sources of truth used here, per function of the oracle:
  Hadamard  - the Sylvester recursion of Eq. 5-6 built independently with
              integer block matrices (exact); scipy.linalg.hadamard (a library
              routine for the same natural-order matrix); the hand-written H~_2
              in tests/golden/hadamard_h2.txt; closed forms (H e0, H 1, spikes);
              invariants (H H = I, norm preservation, linearity); the page's own
              op count (tests/golden/fwht_opcount.txt).
  quantizer - hand-worked cases (tests/golden/quant_cases.txt); exact
              rounding ties (tests/golden/quant_ties.txt, round half to even,
              also for the ternariser and the KV quantiser); range and error
              invariants; code frequencies on Gaussian rows against the normal
              CDF (closed form).
  bf16      - torch's fp32 -> bf16 conversion and hand-worked ties.
  ternarizer- hand-worked case; idempotence on already-ternary matrices;
              alpha, zero and +-1 fractions on Gaussian weights against closed
              forms.
  packing   - hand-worked words (tests/golden/packing_cases.txt); round trips.
  int GEMM  - numpy int64 matmul; all-(+1) weights give the row sums; identity
              weights give the codes back; the library-matmul form
              (gemm_exact, fp64 BLAS, used by the large GPU parity cases)
              equals the triple loop.
  forward   - closed form: for x = H z with integer z the layer returns
              alpha * T z exactly (INT8) or alpha * T (3c/sqrt7) sign(z) (INT4).
All formulas: architecture write-up of "BitNet v2: Native 4-bit Activations
with Hadamard Transformation for 1-bit LLMs", §3.4.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
from scipy.stats import norm

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    rows, kv = [], {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.split()
            else:
                rows.append([float(t) for t in line.split()])
    return rows, kv


def sylvester(m):
    """Unnormalised H~_m from the recursion H~_0 = (1), H~_m = [[H, H], [H, -H]]."""
    h = np.ones((1, 1), np.int64)
    for _ in range(m):
        h = np.block([[h, h], [h, -h]])
    return h


# ---------------------------------------------------------------- Hadamard

def test_golden_h2_matches_recursion_and_oracle():
    rows, _ = read_golden("hadamard_h2.txt")
    h2 = np.array(rows)
    assert np.array_equal(h2, sylvester(2))
    # oracle applied to the unit vectors gives the columns of H~_2
    for j in range(4):
        e = np.zeros(4)
        e[j] = 1.0
        col, _ = oracle.fwht_unnormalized(e)
        assert np.array_equal(col, h2[:, j])


@pytest.mark.parametrize("m", range(0, 7))
def test_fwht_equals_sylvester_product_exactly(m):
    n = 1 << m
    rng = np.random.default_rng(m)
    x = rng.integers(-1000, 1000, size=(5, n)).astype(np.float64)
    h = sylvester(m)
    for row in x:
        got, ops = oracle.fwht_unnormalized(row)
        assert np.array_equal(got, h @ row)  # integer inputs: exact in fp64
        assert ops == n * m


@pytest.mark.parametrize("n", [2, 8, 64, 256, 1024])
def test_hadamard_equals_scipy(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((3, n)).astype(np.float32)
    want = x.astype(np.float64) @ (scipy.linalg.hadamard(n).T / math.sqrt(n))
    got = oracle.hadamard(x)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_fwht_opcount_matches_page():
    rows, _ = read_golden("fwht_opcount.txt")
    n, ops_page, dense = (int(v) for v in rows[0])
    _, ops = oracle.fwht_unnormalized(np.zeros(n))
    # the page counts n*log2(n) operations; a radix-2 FWHT does exactly that
    assert ops == ops_page
    assert dense == n * n and round(dense / ops) == 341


@pytest.mark.parametrize("n", [16, 256, 4096, 16384])
def test_hadamard_involution_norm_linearity(n):
    rng = np.random.default_rng(7 + n)
    x = rng.standard_normal((2, n)).astype(np.float32)
    y = oracle.hadamard(x)
    # H is symmetric and orthogonal: H(Hx) = x, |Hx| = |x|
    yy = oracle.hadamard(y.astype(np.float32))
    np.testing.assert_allclose(yy, x, atol=1e-6 * np.abs(x).max())
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x.astype(np.float64), axis=1),
                               rtol=1e-12)
    # linearity on combinations that are exact in fp32 (bf16-valued inputs)
    xb = workloads.bf16_to_f32(workloads.random_rows(8 + n, 2, n, "normal"))
    y = oracle.hadamard(xb)
    u = (np.float32(2.0) * xb[:1] + xb[1:]).astype(np.float32)
    assert np.array_equal(u.astype(np.float64), 2.0 * xb[:1].astype(np.float64) + xb[1:])
    y2 = oracle.hadamard(u)
    np.testing.assert_allclose(y2[0], 2.0 * y[0] + y[1], atol=1e-9 * np.abs(y).max())


@pytest.mark.parametrize("n", [4, 1024, 16384])
def test_hadamard_special_vectors(n):
    e0 = np.zeros((1, n), np.float32)
    e0[0, 0] = 1
    np.testing.assert_allclose(oracle.hadamard(e0)[0], np.full(n, 1 / math.sqrt(n)), rtol=1e-15)
    ones = np.ones((1, n), np.float32)
    want = np.zeros(n)
    want[0] = math.sqrt(n)
    np.testing.assert_allclose(oracle.hadamard(ones)[0], want, atol=1e-12)
    # a spike A e_j is spread evenly: |y_i| = A / sqrt(n) for every i
    spike = np.zeros((1, n), np.float32)
    spike[0, n // 3] = 50.0
    np.testing.assert_allclose(np.abs(oracle.hadamard(spike)[0]), 50.0 / math.sqrt(n), rtol=1e-15)


def test_hadamard_bf16_input_is_exact_widening():
    xb = workloads.random_rows(3, 4, 512)
    np.testing.assert_array_equal(oracle.hadamard(xb), oracle.hadamard(workloads.bf16_to_f32(xb)))


# ---------------------------------------------------------------- quantizers

def test_golden_int8_case():
    _, kv = read_golden("quant_cases.txt")
    x = np.array([kv["int8.x"]], np.float32)
    codes, scales, rowsum = oracle.quantize(x, 8, hadamard=False)
    assert codes[0].tolist() == [int(v) for v in kv["int8.codes"]]
    assert scales[0] == np.float32(float(kv["int8.scale"][0]))
    assert rowsum[0] == int(kv["int8.rowsum"][0])


def test_golden_int4_case():
    _, kv = read_golden("quant_cases.txt")
    x = np.array([kv["int4.x"]], np.float32)
    codes, scales, rowsum = oracle.quantize(x, 4, hadamard=False)
    assert oracle.unpack_int4(codes, 8)[0].tolist() == [int(v) for v in kv["int4.codes"]]
    assert scales[0] == np.float32(float(kv["int4.scale"][0]))
    assert rowsum[0] == int(kv["int4.rowsum"][0])


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("had", [True, False])
def test_quantizer_invariants(bits, had):
    x = workloads.student_t_rows(11, 0, 64, 1024, 0.01, 20.0, as_bf16=False)
    codes, s, rowsum, xr = oracle.quantize(x, bits, hadamard=had, want_xr=True)
    q = oracle.codes_int8(codes, bits, 1024).astype(np.int64)
    assert np.array_equal(q.sum(1), rowsum)
    if bits == 8:
        assert q.min() >= -127 and q.max() <= 127  # absmax never reaches -128
        assert np.all(np.abs(q).max(1) == 127)
        np.testing.assert_allclose(s, np.abs(xr).max(1) / 127, rtol=1e-6)
        # |x - s q| <= 1/(2f) + |q| |1/f - s| with 1/f - s = eps/127
        err = np.abs(xr - s[:, None] * q)
        bound = s[:, None] * 0.5 + (np.abs(q) + 1) * 1e-5 / 127 + 1e-6 * np.abs(xr)
        assert np.all(err <= bound)
    else:
        assert q.min() >= -8 and q.max() <= 7
        np.testing.assert_allclose(s, np.abs(xr).mean(1) / math.sqrt(7), rtol=1e-6)
        inside = (q > -8) & (q < 7)
        err = np.abs(xr - s[:, None] * q)
        bound = s[:, None] * 0.5 + (np.abs(q) + 1) * 1e-5 / math.sqrt(7) + 1e-6 * np.abs(xr)
        assert np.all(err[inside] <= bound[inside])
    if had:
        np.testing.assert_allclose(xr, oracle.hadamard(x).astype(np.float32), rtol=0, atol=0)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantizer_scale_invariance(bits):
    # codes(c x) = codes(x) up to eps: exact power-of-two scaling of the input
    x = workloads.random_rows(5, 32, 512, "normal", as_bf16=False)
    c1, s1, _ = oracle.quantize(x, bits)
    c2, s2, _ = oracle.quantize((x * np.float32(4.0)).astype(np.float32), bits)
    q1 = oracle.codes_int8(c1, bits, 512)
    q2 = oracle.codes_int8(c2, bits, 512)
    assert np.mean(q1 != q2) < 1e-3
    np.testing.assert_allclose(s2, 4 * s1, rtol=1e-6)


def test_int4_code_frequencies_on_gaussian_rows():
    # For x ~ N(0,1) per row, beta -> sqrt(2/pi) and q = round(x sqrt7/beta):
    #   P(q = 7) = P(x >= 6.5 beta/sqrt7), P(q = -8) = P(x < -7.5 beta/sqrt7),
    #   P(q = 0) = P(|x| <= 0.5 beta/sqrt7)  (normal CDF, closed form).
    x = workloads.random_rows(21, 512, 4096, "normal", as_bf16=False)
    codes, _, _ = oracle.quantize(x, 4, hadamard=False)
    q = oracle.unpack_int4(codes, 4096)
    b = math.sqrt(2 / math.pi) / math.sqrt(7)
    p7 = 1 - norm.cdf(6.5 * b)
    pm8 = norm.cdf(-7.5 * b)
    p0 = norm.cdf(0.5 * b) - norm.cdf(-0.5 * b)
    n = q.size
    for got, want in ((np.mean(q == 7), p7), (np.mean(q == -8), pm8), (np.mean(q == 0), p0)):
        assert abs(got - want) < 6 * math.sqrt(want * (1 - want) / n) + 2e-4
    assert abs(p7 - 0.025) < 0.001 and abs(pm8 - 0.0118) < 0.001


# ---------------------------------------------------------------- ternarizer

def test_golden_ternary_case():
    _, kv = read_golden("quant_cases.txt")
    w = np.array([kv["ternary.w"]], np.float32)
    packed, alpha, q = oracle.ternarize(w)
    assert q[0].tolist() == [int(v) for v in kv["ternary.codes"]]
    assert abs(alpha - float(kv["ternary.alpha"][0])) < 1e-7


def test_ternarizer_idempotent_on_ternary_matrices():
    rng = np.random.default_rng(3)
    t = rng.integers(-1, 2, size=(64, 256)).astype(np.int8)
    for c in (0.02, 1.0, 37.5):
        _, alpha, q = oracle.ternarize((t * np.float32(c)).astype(np.float32))
        assert np.array_equal(q, t)
        assert abs(alpha - c * np.mean(np.abs(t))) <= 1e-6 * c


def test_ternarizer_gaussian_statistics():
    # W ~ N(0, s^2): alpha -> s sqrt(2/pi); q = 0 iff |w| < alpha/2, so
    # P(q=0) = 2 Phi(sqrt(2/pi)/2) - 1 = 0.3101, P(q=+-1) = 0.3450 each.
    w = workloads.gaussian_weights(5, 0, 1024, 4096)
    _, alpha, q = oracle.ternarize(w)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    assert abs(alpha / workloads.W_STD - math.sqrt(2 / math.pi)) < 2e-3
    p0 = 2 * norm.cdf(math.sqrt(2 / math.pi) / 2) - 1
    n = q.size
    assert abs(np.mean(q == 0) - p0) < 6 * math.sqrt(p0 * (1 - p0) / n) + 1e-3
    assert abs(np.mean(q == 1) - (1 - p0) / 2) < 2e-3
    assert abs(p0 - 0.3101) < 1e-4


# ---------------------------------------------------------------- packing

def test_golden_packing_words():
    _, kv = read_golden("packing_cases.txt")
    qt = np.array([[int(v) for v in kv["ternary.codes"]]], np.int8)
    assert oracle.pack_ternary(qt)[0, 0] == int(kv["ternary.word"][0], 16)
    q4 = np.array([[int(v) for v in kv["int4.codes"]]], np.int8)
    assert oracle.pack_int4(q4)[0, 0] == int(kv["int4.word"][0], 16)


def test_pack_roundtrips():
    rng = np.random.default_rng(9)
    t = rng.integers(-1, 2, size=(17, 512)).astype(np.int8)
    back, bad = oracle.unpack_ternary(oracle.pack_ternary(t), 512)
    assert bad == 0 and np.array_equal(back, t)
    q = rng.integers(-8, 8, size=(9, 256)).astype(np.int8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(q), 256), q)


# ---------------------------------------------------------------- integer GEMM

@pytest.mark.parametrize("bits", [8, 4])
def test_gemm_equals_numpy_matmul(bits):
    rng = np.random.default_rng(bits)
    M, N, K = 13, 48, 320
    lo, hi = (-128, 128) if bits == 8 else (-8, 8)
    q = rng.integers(lo, hi, size=(M, K)).astype(np.int8)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    codes = q if bits == 8 else oracle.pack_int4(q)
    acc = oracle.gemm_i32(codes, bits, oracle.pack_ternary(t), K)
    assert np.array_equal(acc, q.astype(np.int64) @ t.astype(np.int64).T)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,N,K", [(7, 32, 64), (33, 48, 1024), (5, 16, 16384)])
def test_gemm_exact_equals_triple_loop(bits, M, N, K):
    # the library-matmul form of the oracle's matmul gives the triple loop's
    # integers, including the extreme sums (codes at the range ends against
    # all-+1 / all--1 weight rows)
    rng = np.random.default_rng(M + N + K + bits)
    lo, hi = (-128, 128) if bits == 8 else (-8, 8)
    q = rng.integers(lo, hi, size=(M, K)).astype(np.int8)
    q[0] = lo
    q[1] = hi - 1
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    t[0] = 1
    t[1] = -1
    codes = q if bits == 8 else oracle.pack_int4(q)
    packed = oracle.pack_ternary(t)
    acc = oracle.gemm_exact(codes, bits, packed, K)
    assert np.array_equal(acc, oracle.gemm_i32(codes, bits, packed, K))
    assert np.array_equal(acc, q.astype(np.int64) @ t.astype(np.int64).T)
    assert acc[0, 0] == lo * K and acc[0, 1] == -lo * K


def test_gemm_special_weights():
    rng = np.random.default_rng(1)
    K = 64
    q = rng.integers(-128, 128, size=(5, K)).astype(np.int8)
    ones = np.ones((16, K), np.int8)
    acc = oracle.gemm_i32(q, 8, oracle.pack_ternary(ones), K)
    assert np.all(acc == q.astype(np.int64).sum(1, keepdims=True))
    eye = np.eye(K, dtype=np.int8)
    assert np.array_equal(oracle.gemm_i32(q, 8, oracle.pack_ternary(eye), K), q.astype(np.int32))


# ---------------------------------------------------------------- forward

def _rotated_integer_inputs(M, K, zmax, seed):
    rng = np.random.default_rng(seed)
    z = rng.integers(-zmax, zmax + 1, size=(M, K)).astype(np.float64)
    z[:, 0] = zmax  # gamma = zmax exactly
    h = sylvester(int(math.log2(K))).astype(np.float64) / math.sqrt(K)
    x = (z @ h.T).astype(np.float32)  # x = H z, so Hadamard(x) = z (H H = I)
    return z, x


def test_forward_closed_form_int8():
    M, K, N = 6, 256, 48
    z, x = _rotated_integer_inputs(M, K, 127, 4)
    rng = np.random.default_rng(5)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    packed, alpha, q = oracle.ternarize((t * np.float32(0.25)).astype(np.float32))
    assert np.array_equal(q, t)
    y = oracle.forward(x, packed, alpha, 8, hadamard=True)
    want = float(alpha) * (z @ t.astype(np.float64).T)
    assert np.linalg.norm(y - want) <= 1e-6 * np.linalg.norm(want)


def test_forward_closed_form_int4():
    # z in {-c, +c}: beta = c, codes = round(+-sqrt7) = +-3, s = c/sqrt7,
    # so Q(X_r) = (3c/sqrt7) sign(z) and Y = alpha T Q(X_r).
    M, K, N, c = 4, 512, 32, 3.0
    rng = np.random.default_rng(6)
    z = c * rng.choice([-1.0, 1.0], size=(M, K))
    h = sylvester(9).astype(np.float64) / math.sqrt(K)
    x = (z @ h.T).astype(np.float32)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    packed, alpha, _ = oracle.ternarize(t.astype(np.float32))
    y = oracle.forward(x, packed, alpha, 4, hadamard=True)
    want = float(alpha) * (3 * c / math.sqrt(7)) * (np.sign(z) @ t.astype(np.float64).T)
    assert np.linalg.norm(y - want) <= 1e-5 * np.linalg.norm(want)


def test_forward_zero_rows_give_zero():
    x = np.zeros((3, 64), np.float32)
    w = workloads.gaussian_weights(1, 0, 16, 64)
    packed, alpha, _ = oracle.ternarize(w)
    for bits in (8, 4):
        assert np.all(oracle.forward(x, packed, alpha, bits) == 0)


def test_dequant_output_bf16_rounding():
    # the bf16 output is torch's round-to-nearest-even conversion of the
    # fp32 value (torch is an implementation independent of the oracle)
    import torch
    acc = np.array([[1, -3, 1000, 0, 257, -257, 771]], np.int32)
    s = np.array([0.1], np.float32)
    y64, yb = oracle.dequant_output(acc, s, np.float32(0.5))
    np.testing.assert_allclose(y64[0], [0.05, -0.15, 50.0, 0.0, 12.85, -12.85, 38.55], rtol=1e-7)
    want = torch.from_numpy(y64.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(yb, want)
    # acc = 257 and 771 at scale 1 land exactly halfway between bf16 values
    # (257 = 256 + 1, 771 = 768 + 3 with 8 significant bits): ties to even
    _, yt = oracle.dequant_output(np.array([[257, 771, -257]], np.int32), np.array([1.0], np.float32),
                                  np.float32(1.0))
    assert workloads.bf16_to_f32(yt)[0].tolist() == [256.0, 772.0, -256.0]


# ------------------------------------------- normalisation layer (Eq. 9 LN)
# Reading: RMSNorm y_k = x_k / sqrt(mean_j x_j^2 + eps) * g_k (the pages name
# RMSNorm without a formula).  Pins: hand-worked cases; the closed form of the
# output's mean square; scale invariance; the gain is elementwise; the codes
# of a normalised row equal those of the raw row (the quantisers are scale
# invariant up to eps), with the scale divided by the row's RMS.

def test_golden_rmsnorm_cases():
    _, kv = read_golden("rmsnorm_cases.txt")
    f = lambda key: np.array([float(v) for v in kv[key]])
    x1 = f("c1.x").astype(np.float32)[None]
    _, _, _, y1 = oracle.norm_quantize(x1, 8, hadamard=False, want_xr=True)
    np.testing.assert_allclose(y1[0], f("c1.y"), rtol=1e-7, atol=0)
    x2 = f("c2.x").astype(np.float32)[None]
    g2 = f("c2.g").astype(np.float32)
    _, _, _, y2 = oracle.norm_quantize(x2, 8, gain=g2, hadamard=False, want_xr=True)
    np.testing.assert_allclose(y2[0], f("c2.y"), rtol=1e-7, atol=0)
    codes, scales, rowsum = oracle.norm_quantize(x1, 8, hadamard=True)
    assert codes[0].tolist() == [int(v) for v in kv["c3.codes"]]
    assert abs(float(scales[0]) - float(kv["c3.scale"][0])) <= 1e-9
    assert int(rowsum[0]) == int(kv["c3.rowsum"][0])


@pytest.mark.parametrize("n", [64, 1024, 16384])
def test_rmsnorm_mean_square_closed_form(n):
    rng = np.random.default_rng(100 + n)
    # rows of very different magnitudes; the mean square of the output is
    # ms / (ms + eps) exactly (before the fp32 rounding)
    x = (rng.standard_normal((4, n)) * np.array([[1e-3], [0.1], [1.0], [30.0]])).astype(np.float32)
    _, _, _, y = oracle.norm_quantize(x, 8, hadamard=False, want_xr=True)
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    want = ms / (ms + float(oracle.EPS))
    got = (y.astype(np.float64) ** 2).mean(axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-6)
    # with the rotation the row's L2 norm is unchanged (H orthogonal)
    _, _, _, yr = oracle.norm_quantize(x, 8, hadamard=True, want_xr=True)
    np.testing.assert_allclose((yr.astype(np.float64) ** 2).mean(axis=1), want, rtol=1e-6)


def test_rmsnorm_scale_invariance_and_elementwise_gain():
    n = 4096
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((3, n)) * 5).astype(np.float32)
    g = rng.uniform(-2, 2, n).astype(np.float32)
    _, _, _, y = oracle.norm_quantize(x, 8, hadamard=False, want_xr=True)
    _, _, _, y4 = oracle.norm_quantize(np.float32(4.0) * x, 8, hadamard=False, want_xr=True)
    # ms >> eps: scaling the row by 4 changes the output by < 1e-6 relative
    np.testing.assert_allclose(y4, y, rtol=2e-6, atol=0)
    _, _, _, yg = oracle.norm_quantize(x, 8, gain=g, hadamard=False, want_xr=True)
    np.testing.assert_allclose(yg, y.astype(np.float64) * g, rtol=2e-7, atol=0)


@pytest.mark.parametrize("bits", [8, 4])
def test_rmsnorm_codes_match_raw_codes(bits):
    # RMSNorm without gain multiplies each row by one positive factor; the
    # quantisers divide by the row statistic, so the codes are those of the
    # raw row except where eps moves a value across a rounding boundary, and
    # the scale is divided by the row's RMS
    n = 4096
    rng = np.random.default_rng(11 + bits)
    x = (rng.standard_t(3, (16, n)) * 3).astype(np.float32)
    c0, s0, r0 = oracle.quantize(x, bits, hadamard=True)
    c1, s1, r1 = oracle.norm_quantize(x, bits, hadamard=True)
    q0 = oracle.codes_int8(c0, bits, n).astype(int)
    q1 = oracle.codes_int8(c1, bits, n).astype(int)
    diff = q0 != q1
    assert np.abs(q0 - q1).max() <= 1
    assert diff.mean() <= 1e-3
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=1) + float(oracle.EPS))
    np.testing.assert_allclose(s1.astype(np.float64) * rms, s0, rtol=1e-5)


# ------------------------------------------- Hadamard backward (Eq. 10)

@pytest.mark.parametrize("m", [1, 3, 6])
def test_hadamard_backward_equals_autograd(m):
    # dL/dX of L = <G, H X> by torch autograd through an explicit matrix
    # built from the Sylvester recursion (an independent route)
    import torch
    n = 1 << m
    h = torch.tensor(sylvester(m) / math.sqrt(n), dtype=torch.float64)
    rng = np.random.default_rng(m)
    x = torch.tensor(rng.standard_normal((4, n)), dtype=torch.float64, requires_grad=True)
    g = rng.standard_normal((4, n)).astype(np.float32)
    loss = ((x @ h.T) * torch.tensor(g, dtype=torch.float64)).sum()
    loss.backward()
    got = oracle.hadamard_backward(g)
    np.testing.assert_allclose(got, x.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [256, 2048])
def test_hadamard_backward_is_adjoint_and_equals_forward(n):
    rng = np.random.default_rng(n + 3)
    x = rng.standard_normal((3, n)).astype(np.float32)
    g = rng.standard_normal((3, n)).astype(np.float32)
    dx = oracle.hadamard_backward(g)
    # <H x, g> = <x, H^T g> row by row
    lhs = (oracle.hadamard(x) * g.astype(np.float64)).sum(axis=1)
    rhs = (x.astype(np.float64) * dx).sum(axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10)
    # H^T = H: the backward is the forward transform (the claim of Eq. 10)
    np.testing.assert_allclose(dx, oracle.hadamard(g), rtol=0, atol=1e-10)
    want = g.astype(np.float64) @ (scipy.linalg.hadamard(n) / math.sqrt(n))
    np.testing.assert_allclose(dx, want, rtol=0, atol=1e-10)


# ------------------------------------------- weight + activation rotation

@pytest.mark.parametrize("m", [4, 6])
def test_rotated_weights_equal_w_times_h_transpose(m):
    n = 1 << m
    rng = np.random.default_rng(20 + m)
    w = (rng.standard_normal((8, n)) * 0.02).astype(np.float32)
    packed, alpha, q, wr = oracle.ternarize_rotated(w, want_wr=True)
    want = w.astype(np.float64) @ (sylvester(m).T / math.sqrt(n))
    np.testing.assert_allclose(wr, want, rtol=1e-6, atol=1e-9)
    p2, a2, q2 = oracle.ternarize(wr)
    assert np.array_equal(q, q2) and np.array_equal(packed, p2) and alpha == a2


def test_rotation_cancels_between_weights_and_activations():
    # (W H^T)(H x) = W x: the variant computes the same unquantised product
    n = 1024
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((16, n)) * 0.02).astype(np.float32)
    x = rng.standard_normal((4, n)).astype(np.float32)
    _, _, _, wr = oracle.ternarize_rotated(w, want_wr=True)
    got = oracle.hadamard(x) @ wr.astype(np.float64).T
    want = x.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-6 * np.abs(want).max())
    # rotating the rotated rows again gives W back (H H = I)
    back = oracle.hadamard(wr)
    np.testing.assert_allclose(back, w, rtol=0, atol=1e-7)


def test_rotated_gaussian_weights_statistics():
    # rows of iid N(0, s^2) stay iid N(0, s^2) under an orthogonal rotation:
    # alpha = s sqrt(2/pi), zero fraction P(|z| < 0.5 sqrt(2/pi))
    n, s = 4096, workloads.W_STD
    w = workloads.gaussian_weights(41, 0, 256, n)
    _, alpha, q = oracle.ternarize_rotated(w)
    assert abs(alpha / (s * math.sqrt(2 / math.pi)) - 1) < 3e-3
    p0 = 2 * norm.cdf(0.5 * math.sqrt(2 / math.pi)) - 1
    assert abs((q == 0).mean() - p0) < 3e-3


# ------------------------------------------- element formats of the FP6 x FP4 path
# The test-side encoders of the MX6 / MX4 layouts derive their tables from
# the OCP MX element-format definitions; pin those against hand-worked
# values (E3M2: 7 = 1.75 * 2^2 -> exponent 5, mantissa 3 -> 0b010111).

def test_e3m2_and_e2m1_tables():
    import mx_util
    assert mx_util.E3M2_OF[7] == 0b010111 and mx_util.E3M2_OF[-8] == 0b111000
    assert mx_util.E3M2_OF[1] == 0b001100 and mx_util.E3M2_OF[3] == 0b010010
    assert mx_util.e3m2_value(0b000001) == 0.0625  # subnormal: 2^-2 * 1/4
    assert sorted(mx_util.E3M2_OF) == list(range(-8, 9))
    assert mx_util.E2M1_OF == {0: 0, 1: 0b0010, -1: 0b1010}
    assert mx_util.e2m1_value(0b0111) == 6.0


def test_mx_layout_round_trips():
    import mx_util
    rng = np.random.default_rng(17)
    q = rng.integers(-8, 8, (261, 512)).astype(np.int8)
    b = mx_util.encode_mx6(q)
    assert b.shape == (512, 384)  # two 256-row blocks
    assert np.array_equal(mx_util.decode_mx6(b, 512, 261), q.astype(np.float64))
    assert not b.reshape(-1)[mx_util._mx6_offsets(512, 512)[0][261:]].any()  # padding rows
    # row 5, group 1 of the first 128-code stage: r = 5, gi = 1; its first 16
    # bytes at 16 (4 r + (gi ^ (r >> 2 & 3))) = 16 * 20, its last 8 at
    # 16384 + 16 (2 r + (0 ^ (r >> 3 & 1))) + 8 = 16384 + 168
    flat = b.reshape(-1)
    field = int.from_bytes(bytes(flat[320:336]) + bytes(flat[16552:16560]), "little")
    assert all((field >> (6 * e)) & 63 == mx_util.E3M2_OF[int(q[5, 32 + e])] for e in range(32))
    # row 300 (second block, r = 44), group 5 (second stage, gi = 1): tile
    # 1 * 4 + 1 = 5; r >> 2 & 3 = 3 -> slot 4 r + 2; r >> 3 & 1 = 1 -> tail slot 2 r + 1
    q300 = rng.integers(-8, 8, (301, 512)).astype(np.int8)
    b300 = mx_util.encode_mx6(q300).reshape(-1)
    field = int.from_bytes(bytes(b300[5 * 24576 + 16 * 178:5 * 24576 + 16 * 178 + 16])
                           + bytes(b300[5 * 24576 + 16384 + 16 * 89 + 8:5 * 24576 + 16384 + 16 * 89 + 16]), "little")
    assert all((field >> (6 * e)) & 63 == mx_util.E3M2_OF[int(q300[300, 160 + e])] for e in range(32))
    # MX4: round trip with padding, and one word placed by hand: row 9
    # (r >> 3 & 1 = 1), k = 64 .. 79 (stage 0, half u = 1 -> slot 2 r + 0,
    # word 0) -> word 4 * 18
    t = rng.integers(-1, 2, (130, 256)).astype(np.int8)
    w = mx_util.encode_mx4(t)
    assert w.shape == (256, 16)
    assert np.array_equal(mx_util.decode_mx4(w, 256, 130), t.astype(np.float64))
    word = int(w.reshape(-1)[72])
    for n in range(8):
        for v, bit in ((int(t[9, 64 + n]), 4 * n + 1), (int(t[9, 72 + n]), 4 * n)):
            assert (word >> bit) & 1 == (v != 0) and (word >> (bit + 2)) & 1 == (v < 0)


# ------------------------------------------- QKV / KV-cache quantiser (f4)
# Reading: Eq. 7's absmax quantiser at b bits, Q = 2^(b-1) - 1, shifted into
# [0, 2^b - 1] (the pages' "unsigned integers using the absmax function").
# Pins: a hand-worked head (golden/kv_quant_cases.txt), the range and the
# position of the extreme element, zero at the zero point, the rounding
# bound |x - x_hat| <= scale / 2, the uniform-noise closed form of the mean
# squared error, and the [BOS] copy at 8 bits.

def test_golden_kv_quant_case():
    _, kv = read_golden("kv_quant_cases.txt")
    x = np.array([float(v) for v in kv["x"]], np.float32).reshape(1, 1, 1, 8)
    for b in (3, 4):
        codes, scales, _, _ = oracle.kv_quant(x, b, keep_bos8=False)
        assert codes.ravel().tolist() == [int(v) for v in kv[f"b{b}.bytes"]]
        assert abs(float(scales.ravel()[0]) - float(kv[f"b{b}.scale"][0])) < 1e-7
        # the packed bytes decode to the listed codes
        xh = oracle.kv_dequant(codes, scales, 8, b).ravel()
        u = np.rint(xh / float(scales.ravel()[0])).astype(int) + (1 << (b - 1))
        assert u.tolist() == [int(v) for v in kv[f"b{b}.codes"]]


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_kv_quant_invariants(bits):
    rng = np.random.default_rng(60 + bits)
    B, S, H, D = 2, 5, 3, 128
    x = (rng.standard_normal((B, S, H, D)) * rng.uniform(0.1, 10, (B, S, H, 1))).astype(np.float32)
    x[0, 1, 2] = 0.0                       # an all-zero head
    codes, scales, _, _ = oracle.kv_quant(x, bits, keep_bos8=False)
    half, q = 1 << (bits - 1), (1 << (bits - 1)) - 1
    xh = oracle.kv_dequant(codes, scales, D, bits)
    gamma = np.abs(x).max(axis=-1)
    np.testing.assert_allclose(scales, gamma / q, rtol=1e-6)
    u = np.rint(np.where(scales[..., None] > 0, xh / np.maximum(scales[..., None], 1e-30), 0)).astype(int) + half
    assert u.min() >= 0 and u.max() <= (1 << bits) - 1
    # the extreme element of every non-zero head sits at half +- q
    idx = np.abs(x).argmax(axis=-1)
    ext = np.take_along_axis(u, idx[..., None], axis=-1)[..., 0]
    nz = gamma > 0
    assert np.all(np.isin(ext[nz], [half - q, half + q]))
    assert np.all(u[0, 1, 2] == half) and scales[0, 1, 2] == 0
    # rounding bound (no element clips: |x f| <= q < half)
    err = np.abs(xh - x.astype(np.float64))
    assert np.all(err <= scales[..., None].astype(np.float64) * (0.5 + 1e-5) + 1e-12)


@pytest.mark.parametrize("bits", [3, 4])
def test_kv_quant_mse_closed_form(bits):
    # rounding noise uniform on [-s/2, s/2]: E|x - x_hat|^2 = s^2 / 12
    rng = np.random.default_rng(70 + bits)
    x = rng.standard_normal((4, 64, 8, 128)).astype(np.float32)
    codes, scales, _, _ = oracle.kv_quant(x, bits, keep_bos8=False)
    xh = oracle.kv_dequant(codes, scales, 128, bits)
    mse = ((xh - x) ** 2).mean(axis=-1)
    ratio = mse.mean() / (scales.astype(np.float64) ** 2 / 12).mean()
    assert abs(ratio - 1) < 0.05


def test_kv_quant_bos_kept_at_8_bits():
    rng = np.random.default_rng(80)
    B, S, H, D = 3, 4, 2, 64
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    codes, scales, bos, bos_s = oracle.kv_quant(x, 3, keep_bos8=True)
    c8, s8, _, _ = oracle.kv_quant(np.ascontiguousarray(x[:, :1]), 8, keep_bos8=False)
    assert np.array_equal(bos, c8[:, 0]) and np.array_equal(bos_s, s8[:, 0])
    # the low-bit slot of position 0 is written too
    c3, _, _, _ = oracle.kv_quant(np.ascontiguousarray(x[:, :1]), 3, keep_bos8=False)
    assert np.array_equal(codes[:, :1], c3)


# ------------------------------------------------ exact rounding ties (Eq. 2)
# Reading: RoundClip rounds an exact half to the even neighbour.  The cases
# in golden/quant_ties.txt make the fp32 product the quantiser rounds exactly
# k + 1/2 (the row statistic makes the per-row factor a power of two); the
# expected codes are worked out by hand there.  Each test first checks that
# premise in fp32, so a case cannot silently stop being a tie.

def _hexes(vals):
    return np.array([float.fromhex(v) for v in vals], np.float32)


def _tie_row(kv, key):
    x = _hexes(kv[f"{key}.x"])
    K = int(kv[f"{key}.K"][0])
    row = np.zeros((1, K), np.float32)
    row[0, :x.size] = x
    return row, x.size


def _assert_exact_halves(prod, n_min):
    """The products are exact in fp32 (checked in fp64) and at least n_min of
    them sit exactly halfway between two integers."""
    frac = np.abs(prod.astype(np.float64)) % 1.0
    assert np.sum(frac == 0.5) >= n_min


def test_golden_ties_int8():
    _, kv = read_golden("quant_ties.txt")
    row, n = _tie_row(kv, "int8")
    eps = np.float32(1e-5)
    gamma = np.abs(row).max()
    assert np.float32(gamma + eps) == np.float32(1.984375)
    f = np.float32(127.0) / np.float32(gamma + eps)
    assert f == np.float32(64.0)
    prod = row[0, :n] * f
    assert np.array_equal(prod.astype(np.float64), row[0, :n].astype(np.float64) * 64.0)
    _assert_exact_halves(prod, 5)
    codes, scales, rowsum = oracle.quantize(row, 8, hadamard=False)
    want = [int(v) for v in kv["int8.codes"]]
    assert codes[0, :n].tolist() == want and not codes[0, n:].any()
    assert rowsum[0] == int(kv["int8.rowsum"][0])


def test_golden_ties_int4():
    _, kv = read_golden("quant_ties.txt")
    row, n = _tie_row(kv, "int4")
    eps = np.float32(1e-5)
    beta = np.float32(np.abs(row.astype(np.float64)).sum() / row.shape[1])
    assert beta == np.float32(float.fromhex(kv["int4.beta"][0]))
    # the fp32 sum of |x| is exact too (every partial sum is a multiple of
    # 2^-17 below 128), so an fp32 statistic gives the same beta
    assert np.float32(np.abs(row).sum(dtype=np.float32)) == np.float32(beta * row.shape[1])
    f = np.float32(math.sqrt(7.0)) / np.float32(beta + eps)
    assert f == np.float32(2.0)
    _assert_exact_halves(row[0, :n] * f, 8)
    codes, scales, rowsum = oracle.quantize(row, 4, hadamard=False)
    q = oracle.unpack_int4(codes, row.shape[1])
    assert q[0, :n].tolist() == [int(v) for v in kv["int4.codes"]] and not q[0, n:].any()
    assert rowsum[0] == int(kv["int4.rowsum"][0])


def test_golden_ties_ternary():
    _, kv = read_golden("quant_ties.txt")
    row, n = _tie_row(kv, "ternary")
    alpha_want = np.float32(float.fromhex(kv["ternary.alpha"][0]))
    assert np.float32(np.abs(row.astype(np.float64)).sum() / row.size) == alpha_want
    d = np.float32(alpha_want + np.float32(1e-5))
    assert d == np.float32(0.25)
    _assert_exact_halves(row[0, :n] / d, 2)
    _, alpha, q = oracle.ternarize(row)
    assert alpha == alpha_want
    assert q[0, :n].tolist() == [int(v) for v in kv["ternary.codes"]] and not q[0, n:].any()


@pytest.mark.parametrize("bits", [3, 4])
def test_golden_ties_kv_quant(bits):
    _, kv = read_golden("quant_ties.txt")
    x = _hexes(kv[f"kv{bits}.x"])
    eps = np.float32(1e-5)
    gamma = np.abs(x).max()
    Q = np.float32((1 << (bits - 1)) - 1)
    f = Q / np.float32(gamma + eps)
    assert f == np.float32({3: 2.0, 4: 4.0}[bits])
    _assert_exact_halves(x * f, 4)
    codes, scales, _, _ = oracle.kv_quant(x.reshape(1, 1, 1, 8), bits, keep_bos8=False)
    # unpack the bytes by the packing contract (3-bit: bits 3j of a 24-bit
    # little-endian value; 4-bit: low nibble first)
    b = codes.ravel().astype(np.int64)
    if bits == 3:
        v = int(b[0]) | int(b[1]) << 8 | int(b[2]) << 16
        u = [(v >> (3 * j)) & 7 for j in range(8)]
    else:
        u = [int(b[j // 2] >> (4 * (j % 2))) & 15 for j in range(8)]
    assert u == [int(v) for v in kv[f"kv{bits}.codes"]]


def test_golden_bf16_ties():
    import torch
    _, kv = read_golden("quant_ties.txt")
    f = np.array([int(v, 16) for v in kv["bf16.f32"]], np.uint32).view(np.float32)
    want = [int(v, 16) for v in kv["bf16.bits"]]
    assert oracle.f32_to_bf16(f).tolist() == want
    assert torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).tolist() == want


def test_bf16_conversion_equals_torch():
    # finite fp32 patterns, a third of them forced to exact ties (low half
    # 0x8000), against torch's fp32 -> bf16 conversion
    import torch
    rng = np.random.default_rng(17)
    u = rng.integers(0, 1 << 32, size=12000, dtype=np.uint64).astype(np.uint32)
    u[::3] = (u[::3] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u = u[(u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)]          # no Inf / NaN
    u = u[(u & np.uint32(0x7FFFFFFF)) < np.uint32(0x7F7F8000)]           # no overflow to Inf
    f = u.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16(f), want)
