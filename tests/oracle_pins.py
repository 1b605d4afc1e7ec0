"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the mathematics fixes.  They are shared by
``test_oracle.py`` (run against the real oracle) and
``test_oracle_mutants.py`` (run against copies of the oracle with a planted
mistake, each of which at least one pin must reject).

What fixes each expected value:
  - exact rational arithmetic (``fractions.Fraction``) for the sum and an
    exact round-to-nearest-even to bf16 written from the IEEE definition;
  - the hand-derived tables in ``tests/golden/``;
  - closed forms (identity, zero, all-ones, permutations, exact-integer
    linearity) and an independent library product (numpy's float64 BLAS)
    within a rigorous floating-point error bound.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from pipelined_tiled_dense_amd.inputs import bits, make_operands

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# Exact bf16 arithmetic, written from the format's definition
# ----------------------------------------------------------------------------
def bf16_exact(b: int) -> Fraction:
    """Exact value of finite bf16 bits: sign, 8-bit exponent (bias 127), 7-bit
    fraction; exponent field 0 means subnormal with quantum 2^-133."""
    b = int(b)
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    assert e != 0xFF, "non-finite input in an exact computation"
    if e == 0:
        return sign * Fraction(m) * Fraction(1, 2 ** 133)
    return sign * Fraction(128 + m) * Fraction(2) ** (e - 127 - 7)


def rne_bf16_exact(x: Fraction) -> int:
    """Round an exact rational to bf16 bits, ties to even (IEEE 754)."""
    if x == 0:
        return 0x0000
    sign = 0x8000 if x < 0 else 0
    ax = abs(x)
    # binade: 2^E <= ax < 2^(E+1)
    E = ax.numerator.bit_length() - ax.denominator.bit_length()
    while Fraction(2) ** E > ax:
        E -= 1
    while Fraction(2) ** (E + 1) <= ax:
        E += 1
    qexp = max(E, -126) - 7
    n = ax / Fraction(2) ** qexp
    fl = n.numerator // n.denominator
    frac = n - fl
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * Fraction(2) ** qexp
    if v > Fraction(255) * Fraction(2) ** 120:
        return sign | 0x7F80
    if v < Fraction(2) ** -126:
        return sign | fl                     # subnormal: fraction field = fl
    # normal: fl in [128, 256]; 256 carries into the next binade
    if fl == 256:
        fl, qexp = 128, qexp + 1
    exp_field = qexp + 7 + 127
    return sign | (exp_field << 7) | (fl - 128)


def exact_product_bits(Ab: np.ndarray, Bb: np.ndarray, b_transposed: bool, K: int, N: int):
    """Brute force: exact sum of exact products, then exact RNE, per element."""
    M = Ab.shape[0]
    Av = [[bf16_exact(Ab[i, k]) for k in range(K)] for i in range(M)]
    if b_transposed:
        Bv = [[bf16_exact(Bb[j, k]) for j in range(N)] for k in range(K)]
    else:
        Bv = [[bf16_exact(Bb[k, j]) for j in range(N)] for k in range(K)]
    out = np.zeros((M, N), dtype=np.uint16)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Av[i][k] * Bv[k][j]
            out[i, j] = rne_bf16_exact(s)
    return out


def decode(bits_arr) -> np.ndarray:
    b = np.asarray(bits_arr, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_bits(values) -> np.ndarray:
    """Bits of values that are exactly representable in bf16 (asserted)."""
    t = torch.tensor(np.asarray(values, dtype=np.float32))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float32), t), "value not exact in bf16"
    return bits(b).copy()


def scaled_operands(M, N, K, b_transposed, seed, scale_a=0, scale_b=0, lda=None, ldb=None):
    """Seeded bf16 operands multiplied by powers of two (exact in binary32,
    then rounded to bf16), to reach subnormal and overflowing results."""
    A, B = make_operands(M, N, K, b_transposed=b_transposed, seed=seed, lda=lda, ldb=ldb)
    if scale_a:
        A = (A.float() * 2.0 ** scale_a).to(torch.bfloat16)
        A = _repad(A, lda)
    if scale_b:
        B = (B.float() * 2.0 ** scale_b).to(torch.bfloat16)
        B = _repad(B, ldb)
    return bits(A), bits(B)


def _repad(x, ld):
    if ld is None or ld == x.shape[1]:
        return x.contiguous()
    buf = torch.full((x.shape[0], ld), 1.0e30, dtype=torch.bfloat16)
    buf[:, : x.shape[1]] = x
    return buf[:, : x.shape[1]]


def assert_bits_equal(got, want, what):
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d mismatches, first at %s: got %#06x want %#06x" % (
        what, len(bad), tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])])


# ----------------------------------------------------------------------------
# Pins
# ----------------------------------------------------------------------------
def pin_rounding_golden(o):
    """Hand-derived fp64 -> bf16 table (tests/golden/bf16_rounding.txt)."""
    xs, want = [], []
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            xs.append(float(tok[0]) if tok[0] in ("inf", "-inf", "nan") else float.fromhex(tok[0]))
            want.append(int(tok[1], 16))
    got = o.f64_to_bf16(np.array(xs))
    for x, g, w in zip(xs, got, want):
        assert int(g) == w, "round(%r): got %#06x want %#06x" % (x, int(g), w)
        assert int(o.lib.oracle_f64_to_bf16(x)) == w


def pin_rounding_exhaustive_exact(o, seed=0, n=4000):
    """Random fp64 values over the whole bf16 range (and past it) against the
    exact rational rounding; includes values placed exactly on midpoints."""
    rng = np.random.default_rng(seed)
    vals = []
    for _ in range(n):
        e = int(rng.integers(-140, 130))
        m = rng.random() + 1.0
        vals.append(math.ldexp(m, e) * (1 if rng.random() < 0.5 else -1))
    # exact midpoints between neighbouring bf16 values (short mantissas: exact in fp64)
    for _ in range(n // 4):
        e = int(rng.integers(-133, 127))
        k = int(rng.integers(128, 256))
        vals.append(math.ldexp(2 * k + 1, e - 8))
    got = o.f64_to_bf16(np.array(vals))
    for x, g in zip(vals, got):
        w = rne_bf16_exact(Fraction(x))
        assert int(g) == w, "round(%r): got %#06x want %#06x" % (x, int(g), w)


def pin_brute_force(o):
    """Oracle == exact rational product, bitwise, on tiny shapes, both B
    layouts, padded leading dimensions, and scaled inputs that reach subnormal
    and overflowing sums."""
    shapes = [(1, 1, 1), (2, 3, 5), (3, 2, 1), (5, 8, 3), (8, 5, 17), (17, 3, 8),
              (3, 17, 2), (1, 5, 17), (17, 1, 5), (4, 4, 16)]
    scales = [(0, 0), (-60, -70), (63, 63), (-10, 5)]
    case = 0
    for (M, N, K) in shapes:
        for bt in (False, True):
            for (sa, sb) in scales:
                case += 1
                lda = K + 8
                ldb = (K if bt else N) + 8
                Ab, Bb = scaled_operands(M, N, K, bt, seed=100 + case, scale_a=sa, scale_b=sb,
                                         lda=lda, ldb=ldb)
                want = exact_product_bits(Ab, Bb, bt, K, N)
                got = o.gemm_bf16(Ab, Bb, bt, K=K, N=N)
                assert_bits_equal(got, want, "brute force M=%d N=%d K=%d bt=%s scale=%s"
                                  % (M, N, K, bt, (sa, sb)))


def pin_identity_zero(o):
    """A*I = A, I*B = B, A*0 = 0, 0*B = 0, bitwise, both layouts, non-square."""
    for bt in (False, True):
        M, K, N = 7, 12, 9
        Ab, Bb = scaled_operands(M, N, K, bt, seed=7)
        A = Ab
        B_kn = Bb.T.copy() if bt else Bb           # K x N view of B's values
        I_K = to_bf16_bits(np.eye(K))
        I_M = to_bf16_bits(np.eye(M))
        # A * I_K = A
        got = o.gemm_bf16(A, I_K, bt, K=K, N=K)
        assert_bits_equal(got, A, "A*I bt=%s" % bt)
        # I_K * B = B   (B is K x N)
        Bstore = B_kn.T.copy() if bt else B_kn
        got = o.gemm_bf16(I_K, Bstore, bt, K=K, N=N)
        assert_bits_equal(got, B_kn, "I*B bt=%s" % bt)
        # zeros
        Z_kn = np.zeros((K, N), dtype=np.uint16)
        got = o.gemm_bf16(A, Z_kn.T.copy() if bt else Z_kn, bt, K=K, N=N)
        assert_bits_equal(got, np.zeros((M, N), np.uint16), "A*0 bt=%s" % bt)
        got = o.gemm_bf16(np.zeros((M, K), np.uint16), Bstore, bt, K=K, N=N)
        assert_bits_equal(got, np.zeros((M, N), np.uint16), "0*B bt=%s" % bt)
        # I_M * A = A (left identity on a non-square operand)
        got = o.gemm_bf16(I_M, A.T.copy() if bt else A, bt, K=M, N=K)
        assert_bits_equal(got, A, "I*A bt=%s" % bt)


def pin_small_golden(o):
    """Hand-computed integer products (tests/golden/small_gemm.json)."""
    with open(os.path.join(GOLDEN, "small_gemm.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        A = to_bf16_bits(c["A"])
        B = to_bf16_bits(c["B"])
        C = to_bf16_bits(c["C"])
        K, N = B.shape
        assert_bits_equal(o.gemm_bf16(A, B, False, K=K, N=N), C, c["name"] + " (B K x N)")
        assert_bits_equal(o.gemm_bf16(A, B.T.copy(), True, K=K, N=N), C, c["name"] + " (B N x K)")
        # fp64 output equals the exact integers too
        np.testing.assert_array_equal(o.gemm_f64(A, B, False, K=K, N=N),
                                      np.array(c.get("sum", c["C"]), float))


def pin_closed_forms(o):
    """All-ones products equal K exactly (rounded once when K needs more than
    8 significant bits); permutation matrices permute exactly."""
    for K, want in [(1, 1.0), (16, 16.0), (255, 255.0), (256, 256.0), (257, 256.0),
                    (259, 260.0), (1024, 1024.0)]:
        A = to_bf16_bits(np.ones((3, K)))
        B = to_bf16_bits(np.ones((K, 5)))
        for bt, Bs in ((False, B), (True, B.T.copy())):
            got = decode(o.gemm_bf16(A, Bs, bt, K=K, N=5))
            assert np.all(got == want), ("all-ones", K, bt, got[0, 0], want)
    rng = np.random.default_rng(3)
    M, K, N = 6, 10, 8
    Ab, Bb = scaled_operands(M, N, K, False, seed=11)
    p = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), p] = 1.0                     # (A P)[:, p[i]] = A[:, i]
    Pb = to_bf16_bits(P)
    got = o.gemm_bf16(Ab, Pb, False, K=K, N=K)
    want = np.zeros_like(Ab)
    want[:, p] = Ab
    assert_bits_equal(got, want, "A*P")
    q = rng.permutation(M)
    Q = np.zeros((M, M))
    Q[np.arange(M), q] = 1.0                     # (Q A)[i] = A[q[i]]
    got = o.gemm_bf16(to_bf16_bits(Q), Ab, False, K=M, N=K)
    assert_bits_equal(got, Ab[q], "Q*A")


def pin_linearity_exact(o):
    """A(B1+B2) = AB1 + AB2 bitwise in fp64 with small-integer entries, where
    every sum is an exact integer."""
    rng = np.random.default_rng(5)
    for (M, K, N) in [(5, 64, 7), (3, 256, 4), (9, 17, 11)]:
        A = to_bf16_bits(rng.integers(-8, 9, size=(M, K)))
        B1v = rng.integers(-8, 9, size=(K, N))
        B2v = rng.integers(-8, 9, size=(K, N))
        B1, B2, B12 = to_bf16_bits(B1v), to_bf16_bits(B2v), to_bf16_bits(B1v + B2v)
        for bt in (False, True):
            t = (lambda X: X.T.copy()) if bt else (lambda X: X)
            lhs = o.gemm_f64(A, t(B12), bt, K=K, N=N)
            rhs = o.gemm_f64(A, t(B1), bt, K=K, N=N) + o.gemm_f64(A, t(B2), bt, K=K, N=N)
            np.testing.assert_array_equal(lhs, rhs)
            exact = decode(A).astype(np.int64) @ (B1v + B2v)
            np.testing.assert_array_equal(lhs, exact.astype(np.float64))


def pin_linearity_bounded(o):
    """A(B1+B2) vs AB1 + AB2 on random inputs with B1, B2 of disjoint support
    (so B1+B2 is exact in bf16): equal within the fp64 summation bound, and
    the bf16 outputs within one part in 100."""
    rng = np.random.default_rng(6)
    M, K, N = 16, 300, 24
    Ab, Bb = scaled_operands(M, N, K, False, seed=21)
    mask = rng.random((K, N)) < 0.5
    B1 = np.where(mask, Bb, 0).astype(np.uint16)
    B2 = np.where(mask, 0, Bb).astype(np.uint16)
    lhs = o.gemm_f64(Ab, Bb, False)
    rhs = o.gemm_f64(Ab, B1, False) + o.gemm_f64(Ab, B2, False)
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    bound = 3 * gamma * (np.abs(decode(Ab)) @ np.abs(decode(Bb))) + 1e-300
    assert np.all(np.abs(lhs - rhs) <= bound)
    c = decode(o.gemm_bf16(Ab, Bb, False))
    c12 = decode(o.f64_to_bf16(rhs))
    assert np.all(np.abs(c - c12) <= 1e-2 * np.maximum(1.0, np.abs(c)))


def pin_numpy_crosscheck(o):
    """numpy float64 matmul (a different summation order) agrees with the
    oracle's fp64 sums within 2 * gamma_K * |A||B|; also checks the sums
    against a direct sum of products over k for a few sampled elements."""
    for (M, N, K, bt) in [(64, 48, 512, False), (40, 72, 333, True), (256, 256, 256, False)]:
        Ab, Bb = scaled_operands(M, N, K, bt, seed=M + N + K)
        Af = decode(Ab)
        Bf = decode(Bb).T if bt else decode(Bb)
        ref = Af @ Bf
        got = o.gemm_f64(Ab, Bb, bt)
        u = 2.0 ** -53
        gamma = K * u / (1 - K * u)
        bound = 2 * gamma * (np.abs(Af) @ np.abs(Bf))
        assert np.all(np.abs(got - ref) <= bound)


def pin_layout_invariance(o):
    """The same product from B stored K x N and from B stored N x K is
    bit-identical."""
    for (M, N, K) in [(33, 40, 70), (8, 16, 256)]:
        Ab, Bb = scaled_operands(M, N, K, False, seed=31)
        a = o.gemm_bf16(Ab, Bb, False)
        b = o.gemm_bf16(Ab, Bb.T.copy(), True, K=K, N=N)
        assert_bits_equal(a, b, "layout invariance")


def pin_signed_zero_and_nan(o):
    """All-zero sums are +0 (even from -0 products); NaN inputs give 0x7FC0."""
    A = np.array([[0x8000, 0x8000]], dtype=np.uint16)        # -0, -0
    B = to_bf16_bits([[1.0], [2.0]])
    assert int(o.gemm_bf16(A, B, False)[0, 0]) == 0x0000
    A = np.array([[0x7FC0, 0x3F80]], dtype=np.uint16)        # NaN, 1
    assert int(o.gemm_bf16(A, B, False)[0, 0]) == 0x7FC0


def _module_decoder(o):
    """The Python bf16 decoder of the module that defines ``o``'s class: the
    real oracle package, or a mutated copy of it."""
    import sys
    return sys.modules[type(o).__module__].bf16_bits_to_f64


def pin_bf16_decoder(o):
    """Both bf16 decoders -- the Python one that every GPU tolerance check
    runs its operands through, and the C oracle's own -- against the format's
    definition (``bf16_exact``) on all 65536 bit patterns: finite values
    exactly, with the sign of zero; exponent field 255 with a zero fraction
    gives +-Inf, with a nonzero fraction NaN."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = np.empty(pats.size, dtype=np.float64)
    for b in range(1 << 16):
        e, m = (b >> 7) & 0xFF, b & 0x7F
        if e != 0xFF:
            want[b] = float(bf16_exact(b))
        elif m == 0:
            want[b] = -math.inf if b & 0x8000 else math.inf
        else:
            want[b] = math.nan
    neg = (pats & 0x8000) != 0
    for name, got in (("python", _module_decoder(o)(pats)), ("c", o.decode(pats))):
        assert got.shape == want.shape and got.dtype == np.float64, name
        nan_w, nan_g = np.isnan(want), np.isnan(got)
        assert np.array_equal(nan_w, nan_g), "%s decoder: NaN at %#06x" % (
            name, int(pats[np.argmax(nan_w != nan_g)]))
        ok = nan_w | (got == want)
        assert ok.all(), "%s decoder: %#06x -> %r, want %r" % (
            name, int(pats[np.argmin(ok)]), got[np.argmin(ok)], want[np.argmin(ok)])
        sign_ok = nan_w | (np.signbit(got) == neg)
        assert sign_ok.all(), "%s decoder: sign of %#06x" % (name, int(pats[np.argmin(sign_ok)]))


ALL_PINS = [pin_rounding_golden, pin_rounding_exhaustive_exact, pin_brute_force,
            pin_identity_zero, pin_small_golden, pin_closed_forms, pin_linearity_exact,
            pin_linearity_bounded, pin_numpy_crosscheck, pin_layout_invariance,
            pin_signed_zero_and_nan, pin_bf16_decoder]
