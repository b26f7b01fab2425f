"""Pins for the CPU oracle: hand-worked examples, closed forms, brute force
and invariants.  None of these re-types the oracle's formulas; each checks a
property that a dropped term, a wrong sign or index, or a transposed operand
would break.  CPU only."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line:
                key, val = line.split(":", 1)
                out[key.strip()] = val.split()
            else:
                rows.append(line.split())
    return out, rows


# ------------------------------------------------------------------ O1
def test_absmean_worked_example(orc):
    g, _ = read_golden("absmean_example.txt")
    w = np.array([[float(v) for v in g["w"]]], np.float32)
    t, s = orc.ternarize_absmean(w)
    assert s == np.float32(float(g["gamma"][0]))
    assert t.tolist() == [[int(v) for v in g["t"]]]


def _brute_ternarize(w):
    """argmin over {-1, 0, 1} of |w/gamma - t| with ties to the even value
    (0 for +-0.5); values beyond +-1.5 saturate."""
    flat = w.astype(np.float64).ravel()
    gamma = np.float32(math.fsum(abs(v) for v in flat) / flat.size)
    out = []
    for v in w.ravel():
        if gamma == 0:
            out.append(0)
            continue
        r = float(np.float32(v) / gamma)  # fp32 divide decides the trit
        best = None
        for cand in (0, -1, 1):  # 0 first: it wins exact ties at +-0.5
            d = abs(Fraction(r) - cand)
            if best is None or d < best[0]:
                best = (d, cand)
        out.append(best[1])
    return np.array(out, np.int8).reshape(w.shape), gamma


def test_absmean_brute_force(orc):
    rng = np.random.default_rng(11)
    for shape in [(1, 8), (3, 16), (7, 33)]:
        # multiples of 2^-10 in a small range: the double sum is exact
        w = (rng.integers(-900, 901, size=shape) / 1024.0).astype(np.float32)
        t, s = orc.ternarize_absmean(w)
        tb, sb = _brute_ternarize(w)
        assert s == sb
        np.testing.assert_array_equal(t, tb)


def test_absmean_idempotent_on_scaled_trits(orc):
    rng = np.random.default_rng(12)
    for s in [0.02, 0.5, 3.0, 1e-3]:
        t = rng.integers(-1, 2, size=(5, 64), dtype=np.int8)
        t[0, 0] = 1
        w = (np.float32(s) * t).astype(np.float32)
        t2, gamma = orc.ternarize_absmean(w)
        np.testing.assert_array_equal(t2, t)
        # gamma is s times the fraction of nonzero entries, not s itself
        frac = np.count_nonzero(t) / t.size
        assert gamma == pytest.approx(s * frac, rel=1e-6)


def test_absmean_odd_and_power_of_two(orc):
    rng = np.random.default_rng(13)
    w = rng.standard_normal((9, 48)).astype(np.float32)
    t, s = orc.ternarize_absmean(w)
    tn, sn = orc.ternarize_absmean(-w)
    np.testing.assert_array_equal(tn, -t)
    assert sn == s
    for j in (-3, 5):
        tj, sj = orc.ternarize_absmean(w * np.float32(2.0 ** j))
        np.testing.assert_array_equal(tj, t)
        assert sj == s * np.float32(2.0 ** j)
    assert set(np.unique(t)) <= {-1, 0, 1}


def test_absmean_all_zero(orc):
    t, s = orc.ternarize_absmean(np.zeros((2, 16), np.float32))
    assert s == 0 and not t.any()


# ------------------------------------------------------------------ O2
def test_pack_closed_forms(orc):
    for trit, byte in [(0, 0x55), (1, 0xAA), (-1, 0x00)]:
        p, bad = orc.pack_i2s(np.full((64, 128), trit, np.int8))
        assert bad == 0 and p.shape == (64 * 128 // 4,)
        assert (p == byte).all()


def test_pack_padding_rows_are_zero_trits(orc):
    # n = 70 pads to 128 rows; rows 70..127 hold code 1 (trit 0) = 0x55
    t = np.full((70, 64), 1, np.int8)
    p, bad = orc.pack_i2s(t)
    assert bad == 0 and p.size == 128 * 16
    blk1 = p[1024:].reshape(64, 16)  # second row block, one 64-k chunk
    assert (blk1[:6] == 0xAA).all() and (blk1[6:] == 0x55).all()


def test_pack_single_plus_one_golden(orc):
    _, rows = read_golden("pack_single_plus_one.txt")
    assert len(rows) >= 16
    for k, bidx, val in rows:
        t = np.zeros((1, 64), np.int8)
        t[0, int(k)] = 1
        p, _ = orc.pack_i2s(t)
        expect = np.full(1024, 0x55, np.uint8)  # row 0 + 63 padding rows
        expect[int(bidx)] = int(val, 16)
        np.testing.assert_array_equal(p, expect, err_msg=f"k={k}")


def test_pack_chunk_and_block_placement(orc):
    # single +1 entries of a 130 x 192 matrix: the one changed byte of the
    # packed image and its value, worked out by hand (golden file)
    _, rows = read_golden("pack_placement.txt")
    assert len(rows) >= 8
    n, k = 130, 192
    for r, kk, off, val in rows:
        t = np.zeros((n, k), np.int8)
        t[int(r), int(kk)] = 1
        p, _ = orc.pack_i2s(t)
        assert p.shape == (3 * 16 * k,)
        changed = np.flatnonzero(p != 0x55)
        assert changed.tolist() == [int(off)], (r, kk)
        assert p[changed[0]] == int(val, 16), (r, kk)


def test_pack_round_trip_all_81_bytes(orc):
    # positions 0, 4, 8, 12 share byte 0 of the row (one field each)
    seen = set()
    for combo in itertools.product((-1, 0, 1), repeat=4):
        t = np.zeros((1, 64), np.int8)
        t[0, [0, 4, 8, 12]] = combo
        p, bad = orc.pack_i2s(t)
        assert bad == 0
        seen.add(int(p[0]))
        back, bad2 = orc.unpack_i2s(p, 1, 64)
        assert bad2 == 0
        np.testing.assert_array_equal(back, t)
    assert len(seen) == 81
    # no valid byte holds the invalid code 3 in any 2-bit field
    for b in seen:
        assert all(((b >> s) & 3) != 3 for s in (0, 2, 4, 6))


def test_pack_round_trip_random(orc):
    rng = np.random.default_rng(14)
    t = rng.integers(-1, 2, size=(137, 320), dtype=np.int8)
    p, bad = orc.pack_i2s(t)
    assert bad == 0 and p.shape == (192 * 80,)
    back, bad2 = orc.unpack_i2s(p, 137, 320)
    assert bad2 == 0
    np.testing.assert_array_equal(back, t)


def test_pack_invalid_counted(orc):
    t = np.zeros((2, 64), np.int8)
    t[0, 3] = 2
    t[1, 7] = -2
    t[1, 9] = 5
    _, bad = orc.pack_i2s(t)
    assert bad == 3
    _, bad_unpack = orc.unpack_i2s(np.full(1024, 0xFF, np.uint8), 1, 64)
    assert bad_unpack == 64


def test_pack_size_matches_two_bits_per_weight(orc):
    # bitnet.cpp CPU tutorial §1.1: a 1B-parameter model's weights take about
    # 250 MB at 2 bits each; the packed size is n*k/4 bytes.
    t = np.zeros((128, 1024), np.int8)
    p, _ = orc.pack_i2s(t)
    assert p.nbytes * 4 == t.size
    assert orc.packed_bytes(10 ** 6, 1024) == 256_000_000  # ~1B weights


# ------------------------------------------- fewer-bytes (base-3) packing
def b3_digits(byte):
    """The five ternary digits of a stored byte, most significant first, by
    exact rational arithmetic: the byte stands for the fraction byte / 256 of
    243, so digit j is floor(byte * 3^(j+1) / 256) mod 3."""
    return [(byte * 3 ** (j + 1) // 256) % 3 for j in range(5)]


def test_b3_all_243_values(orc):
    """Every combination of five trits in one byte (inputs 0, 4, 8, 12, 16 of
    a row share byte 0): the stored byte decodes back to the same digits by
    exact arithmetic, the 243 combinations give 243 distinct bytes, larger
    base-3 numbers give larger bytes, and unpacking returns the trits."""
    seen = {}
    for combo in itertools.product((-1, 0, 1), repeat=5):
        t = np.zeros((1, 80), np.int8)
        t[0, [0, 4, 8, 12, 16]] = combo
        p, bad = orc.pack_b3(t)
        assert bad == 0 and p.size == 64 * 16
        b = int(p[0])
        assert b3_digits(b) == [c + 1 for c in combo], combo
        v = sum((c + 1) * 3 ** (4 - j) for j, c in enumerate(combo))
        seen[v] = b
        back, bad2 = orc.unpack_b3(p, 1, 80)
        assert bad2 == 0
        np.testing.assert_array_equal(back, t)
    assert len(set(seen.values())) == 243
    vals = [seen[v] for v in range(243)]
    assert vals == sorted(vals)
    # the 13 byte values no combination produces are flagged on unpacking
    unused = sorted(set(range(256)) - set(vals))
    assert len(unused) == 13
    for b in unused:
        _, bad = orc.unpack_b3(np.full(1024, b, np.uint8), 1, 80)
        assert bad == 1024, b


def test_b3_closed_forms(orc):
    # all trits 0: digits 1,1,1,1,1 (v = 121) -> byte 128; all +1 (v = 242)
    # -> 255; all -1 (v = 0) -> 0
    for trit, byte in [(0, 128), (1, 255), (-1, 0)]:
        p, bad = orc.pack_b3(np.full((64, 160), trit, np.int8))
        assert bad == 0 and p.size == 64 * 160 // 5
        assert (p == byte).all(), trit


def test_b3_padding_and_size(orc):
    """n = 70, k = 100: rows pad to 128 and inputs to 160 with trit 0 (byte
    128 where all five inputs of a byte are padding); 1.6 bits per weight,
    a fifth fewer bytes than 2 bits per weight when k is a multiple of 80."""
    t = np.full((70, 100), 1, np.int8)
    p, bad = orc.pack_b3(t)
    assert bad == 0 and p.size == 128 * 160 // 5
    back, _ = orc.unpack_b3(p, 70, 100)
    np.testing.assert_array_equal(back, t)
    assert (p == 255).sum() == 70 * 100 // 5   # all five inputs real: +1
    assert (p == 128).sum() == p.size - 70 * 100 // 5
    assert orc.b3_packed_bytes(2560, 2560) * 5 == 2560 * 2560 * 8 // 8
    assert orc.b3_packed_bytes(2560, 2560) * 10 == orc.packed_bytes(
        2560, 2560) * 8


def test_b3_round_trip_random(orc):
    rng = np.random.default_rng(15)
    for n, k in [(137, 320), (64, 6912), (3, 64), (200, 4096)]:
        t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
        p, bad = orc.pack_b3(t)
        assert bad == 0
        back, bad2 = orc.unpack_b3(p, n, k)
        assert bad2 == 0
        np.testing.assert_array_equal(back, t)


def test_b3_invalid_counted(orc):
    t = np.zeros((2, 64), np.int8)
    t[0, 3], t[1, 7] = 2, -3
    p, bad = orc.pack_b3(t)
    assert bad == 2
    back, _ = orc.unpack_b3(p, 2, 64)
    assert back[0, 3] == 0 and back[1, 7] == 0


# ------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms(orc):
    # a constant row of 2 with eps = 0 has mean square 4: the scale is 1/2
    # exactly and every output is the gain exactly
    x = np.full((1, 64), 2.0, np.float32)
    for g in (np.ones(64, np.float32),
              np.float32(2.0) ** np.arange(-8, 56, dtype=np.float32)):
        h, r64 = orc.rmsnorm(x, g, 0.0)
        assert r64[0] == 0.5
        np.testing.assert_array_equal(h[0], g)
    # an all-zero row stays zero (eps keeps the scale finite) and quantizes
    # to zeros
    q, s_a, h, r64 = orc.rmsnorm_quant(np.zeros((1, 64), np.float32),
                                       np.ones(64, np.float32), 1e-5)
    assert np.isfinite(r64).all() and not h.any() and not q.any()


def test_rmsnorm_worked_example(orc):
    # x = [3, 4], eps = 0: mean square 25 / 2, scale sqrt(2) / 5 (exactly
    # 0.28284271247461900976...), the double nearest to it
    h, r64 = orc.rmsnorm(np.array([[3.0, 4.0]], np.float32),
                         np.ones(2, np.float32), 0.0)
    exact = Fraction(28284271247461900976033774484194, 10 ** 32)
    assert abs(Fraction(r64[0]) - exact) <= Fraction(2 ** -54)
    r = np.float32(r64[0])
    assert h[0].tolist() == [float(np.float32(3 * r)), float(np.float32(4 * r))]


def test_rmsnorm_against_exact_rationals(orc):
    """Random rows: the double scale is within the rounding bound of a
    k-term double sum of the exact 1 / sqrt(sum x^2 / k + eps) (computed with
    rationals and a 60-digit square root), and each output is within two
    fp32 roundings of x * g * r."""
    import decimal
    decimal.getcontext().prec = 60
    rng = np.random.default_rng(16)
    for k, eps in [(64, 1e-5), (256, 1e-6), (1000, 0.0)]:
        x = (rng.standard_normal((3, k)) * 3).astype(np.float32)
        g = rng.uniform(0.5, 1.5, k).astype(np.float32)
        h, r64 = orc.rmsnorm(x, g, eps)
        for i in range(3):
            ss = sum(Fraction(float(v)) ** 2 for v in x[i])
            ms = ss / k + Fraction(float(np.float32(eps)))
            exact = 1 / decimal.Decimal(ms.numerator).__truediv__(
                decimal.Decimal(ms.denominator)).sqrt()
            # a sum of k doubles carries at most (k - 1) roundings of 2^-53
            # relative, the divide, add, root and reciprocal four more
            rel = abs(decimal.Decimal(float(r64[i])) - exact) / exact
            assert rel < (k + 4) * decimal.Decimal(2) ** -53, (k, i)
            r = np.float64(np.float32(r64[i]))
            ref = x[i].astype(np.float64) * g.astype(np.float64) * r
            err = np.abs(h[i].astype(np.float64) - ref)
            assert (err <= 2 * np.abs(ref) * 2.0 ** -24 + 1e-45).all()


def test_rmsnorm_invariants(orc):
    rng = np.random.default_rng(17)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 512).astype(np.float32)
    h, _ = orc.rmsnorm(x, g, 0.0)
    # scaling a row by a power of two (eps = 0) changes nothing
    for j in (-6, 3, 20):
        h2, _ = orc.rmsnorm(x * np.float32(2.0 ** j), g, 0.0)
        np.testing.assert_array_equal(h2, h)
    # negation negates
    h3, _ = orc.rmsnorm(-x, g, 0.0)
    np.testing.assert_array_equal(h3, -h)
    # with unit gains the output has mean square 1 (eps = 0)
    h4, _ = orc.rmsnorm(x, np.ones(512, np.float32), 0.0)
    ms = (h4.astype(np.float64) ** 2).mean(axis=1)
    assert np.abs(ms - 1).max() < 1e-6
    # eps only ever shrinks the scale
    _, r0 = orc.rmsnorm(x, g, 0.0)
    _, r1 = orc.rmsnorm(x, g, 1e-2)
    assert (r1 < r0).all()


# ------------------------------------------------------------------ O3
def test_quant_tie_table(orc):
    g, _ = read_golden("quant_ties.txt")
    x = np.array([[float(v) for v in g["x"]]], np.float32)
    q, s = orc.quant_act(x)
    assert q[0].tolist() == [int(v) for v in g["q"]]
    assert s[0] == np.float32(float(g["s_a"][0]))


def _brute_quant_row(x):
    """q = argmin over integers in [-127, 127] of |x * inv - q| (fp32 product
    decides), ties to even; exact rational distances."""
    amax = max(abs(float(v)) for v in x)
    a = np.float32(max(amax, float(np.float32(1e-5))))
    inv = np.float32(127.0) / a
    out = []
    for v in x:
        p = Fraction(float(np.float32(v) * inv))
        lo = math.floor(p)
        cands = [c for c in (lo, lo + 1) if -127 <= c <= 127]
        if not cands:
            cands = [max(-127, min(127, lo))]
        best = min(cands, key=lambda c: (abs(p - c), c % 2))
        out.append(best)
    return np.array(out, np.int8), np.float32(a / np.float32(127.0))


def test_quant_brute_force(orc):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 96)).astype(np.float32)
    x[1] *= 30
    x[2, ::7] *= 20
    x[3] = np.round(x[3] * 4) / 4  # many exact .5 ties after scaling
    q, s = orc.quant_act(x)
    for i in range(x.shape[0]):
        qb, sb = _brute_quant_row(x[i])
        np.testing.assert_array_equal(q[i], qb)
        assert s[i] == sb


def test_quant_invariants(orc):
    rng = np.random.default_rng(16)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    q, s = orc.quant_act(x)
    # the element of largest magnitude maps to +-127
    for i in range(6):
        j = np.argmax(np.abs(x[i]))
        assert abs(int(q[i, j])) == 127
    assert q.min() >= -127
    # odd symmetry
    qn, sn = orc.quant_act(-x)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)
    # power-of-two scaling leaves q unchanged and scales s_a exactly
    for j in (-4, 7):
        qj, sj = orc.quant_act(x * np.float32(2.0 ** j))
        np.testing.assert_array_equal(qj, q)
        np.testing.assert_array_equal(sj, s * np.float32(2.0 ** j))


def test_quant_zero_and_tiny_rows(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, 5] = 1e-30
    q, s = orc.quant_act(x)
    assert not q.any()
    assert s[0] == s[1] == np.float32(np.float32(1e-5) / np.float32(127))


# ------------------------------------------------------------------ O4
def test_gemm_matches_numpy_int64(orc):
    rng = np.random.default_rng(17)
    for n, k, m in [(5, 64, 1), (33, 128, 3), (17, 256, 8), (3, 1024, 2)]:
        t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
        q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
        p, _ = orc.pack_i2s(t)
        acc, _ = orc.gemm(p, 1.0, n, k, q, np.ones(m, np.float32))
        ref = q.astype(np.int64) @ t.astype(np.int64).T
        np.testing.assert_array_equal(acc, ref)


def test_gemm_brute_force_all_rows_of_four(orc):
    rows = np.array(list(itertools.product((-1, 0, 1), repeat=4)), np.int8)
    t = np.zeros((81, 64), np.int8)
    t[:, :4] = rows
    qs = np.zeros((3, 64), np.int8)
    qs[0, :4] = [127, 2, -4, 0]
    qs[1, :4] = [-127, -127, 127, 1]
    qs[2, :4] = [5, -3, 7, -11]
    p, _ = orc.pack_i2s(t)
    acc, _ = orc.gemm(p, 1.0, 81, 64, qs, np.ones(3, np.float32))
    for i in range(3):
        for r in range(81):
            s = 0
            for c in range(4):
                s += int(rows[r][c]) * int(qs[i][c])
            assert acc[i, r] == s


def test_gemm_closed_forms(orc):
    rng = np.random.default_rng(18)
    k = 192
    q = rng.integers(-127, 128, size=(2, k), dtype=np.int8)
    t = np.zeros((3 + k, k), np.int8)
    t[1] = 1
    t[2] = -1
    for c in range(k):
        t[3 + c, c] = 1  # one-hot rows
    p, _ = orc.pack_i2s(t)
    acc, _ = orc.gemm(p, 1.0, 3 + k, k, q, np.ones(2, np.float32))
    qs = q.astype(np.int64).sum(axis=1)
    assert (acc[:, 0] == 0).all()
    np.testing.assert_array_equal(acc[:, 1], qs)
    np.testing.assert_array_equal(acc[:, 2], -qs)
    np.testing.assert_array_equal(acc[:, 3:], q)


def test_gemm_invariants(orc):
    rng = np.random.default_rng(19)
    n, k, m = 11, 320, 4
    t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    ones = np.ones(m, np.float32)
    acc, _ = orc.gemm(orc.pack_i2s(t)[0], 1.0, n, k, q, ones)
    accn, _ = orc.gemm(orc.pack_i2s(-t)[0], 1.0, n, k, q, ones)
    np.testing.assert_array_equal(accn, -acc)
    perm = rng.permutation(k)
    accp, _ = orc.gemm(orc.pack_i2s(t[:, perm])[0], 1.0, n, k, q[:, perm],
                       ones)
    np.testing.assert_array_equal(accp, acc)
    # additivity while the sum stays ternary: split t into disjoint supports
    mask = rng.random((n, k)) < 0.5
    t1 = np.where(mask, t, 0).astype(np.int8)
    t2 = np.where(mask, 0, t).astype(np.int8)
    a1, _ = orc.gemm(orc.pack_i2s(t1)[0], 1.0, n, k, q, ones)
    a2, _ = orc.gemm(orc.pack_i2s(t2)[0], 1.0, n, k, q, ones)
    np.testing.assert_array_equal(a1 + a2, acc)


def test_gemm_threads_and_row_ranges_agree(orc):
    rng = np.random.default_rng(20)
    n, k, m = 57, 256, 3
    t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
    q = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    s_a = np.array([0.5, 0.25, 2.0], np.float32)
    p, _ = orc.pack_i2s(t)
    a1, y1 = orc.gemm(p, 0.125, n, k, q, s_a, nthreads=1)
    a7, y7 = orc.gemm(p, 0.125, n, k, q, s_a, nthreads=7)
    np.testing.assert_array_equal(a1, a7)
    np.testing.assert_array_equal(y1, y7)
    ar, yr = orc.gemm(p, 0.125, n, k, q, s_a, rows=(10, 20))
    np.testing.assert_array_equal(ar, a1[:, 10:20])
    np.testing.assert_array_equal(yr, y1[:, 10:20])


def test_gemm_extreme_accumulator(orc):
    k = 65536
    t = np.ones((1, k), np.int8)
    q = np.full((1, k), 127, np.int8)
    acc, _ = orc.gemm(orc.pack_i2s(t)[0], 1.0, 1, k, q, np.ones(1, np.float32))
    assert acc[0, 0] == 127 * k


# ------------------------------------------------------------------ O5
def test_pipeline_worked_example(orc):
    g, _ = read_golden("pipeline_example.txt")
    t4 = np.array([[int(v) for v in g["T0"]], [int(v) for v in g["T1"]]],
                  np.int8)
    for k in (64, 192):
        t = np.zeros((2, k), np.int8)
        t[:, :4] = t4
        x = np.zeros((1, k), np.float32)
        x[0, :4] = [float(v) for v in g["x"]]
        q, s_a = orc.quant_act(x)
        assert q[0, :4].tolist() == [int(v) for v in g["q"]]
        assert s_a[0] == float(g["s_a"][0])
        acc, y = orc.gemm(orc.pack_i2s(t)[0], float(g["s_w"][0]), 2, k, q,
                          s_a)
        assert acc[0].tolist() == [int(v) for v in g["acc"]]
        assert y[0].tolist() == [float(v) for v in g["y"]]


def test_rescale_close_to_exact_product(orc):
    """y (double) is within a few double roundings of the exact rational
    product acc * s_w * s_a."""
    rng = np.random.default_rng(21)
    n, k, m = 9, 128, 3
    t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
    x = rng.standard_normal((m, k)).astype(np.float32)
    q, s_a = orc.quant_act(x)
    s_w = np.float32(0.0317)
    acc, y = orc.gemm(orc.pack_i2s(t)[0], s_w, n, k, q, s_a)
    for i in range(m):
        for r in range(n):
            exact = Fraction(int(acc[i, r])) * Fraction(float(s_w)) * \
                Fraction(float(s_a[i]))
            if exact == 0:
                assert y[i, r] == 0
            else:
                err = abs((Fraction(float(y[i, r])) - exact) / exact)
                assert err < Fraction(1, 2 ** 50)


def test_rescale_f32_is_two_correctly_rounded_products(orc):
    """rescale_f32 against exact rationals: each fp32 product of two fp32
    values is exact in a double, so rounding the exact rational once to fp32
    is the correctly rounded fp32 multiply; two of them, left to right."""
    rng = np.random.default_rng(22)
    acc = rng.integers(-1_000_000, 1_000_001, size=(3, 40)).astype(np.int32)
    acc[0, :3] = [0, 1, -1]
    s_w = np.float32(0.0213)
    s_a = rng.random(3).astype(np.float32) * np.float32(0.7) + np.float32(1e-4)
    y = orc.rescale_f32(acc, s_w, s_a)
    assert y.dtype == np.float32
    for i in range(3):
        for j in range(acc.shape[1]):
            p1 = Fraction(int(acc[i, j])) * Fraction(float(s_w))
            assert Fraction(float(p1)) == p1  # exact in a double
            r1 = np.float32(float(p1))
            p2 = Fraction(float(r1)) * Fraction(float(s_a[i]))
            assert Fraction(float(p2)) == p2
            assert y[i, j] == np.float32(float(p2))


def test_rescale_f32_powers_of_two_exact(orc):
    acc = np.array([[5, -7, 0, 123456]], np.int32)
    y = orc.rescale_f32(acc, np.float32(0.25), np.array([0.125], np.float32))
    assert y.tolist() == [[5 / 32, -7 / 32, 0.0, 123456 / 32]]
