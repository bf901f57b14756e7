"""The error bound behind the deferred-row pass's rounded float64 transform.

Rows with a group whose exponents span too widely for exact float64 sums are
first transformed once in float64 (butterflies, depth log2 g). The pass keeps
an element when |y - RN32(y)| + delta stays below the half-gap h from RN32(y)
to its next rounding boundary, with delta = 2^-49 * (fp32 sum of |x|); the
fast kernel uses the smaller of 2^(E + ceil(log2 log2 g) + log2 g - 51) (E the
group's largest exponent) and 2^(e_S + ceil(log2 log2 g) - 51) (e_S the
exponent of the float64 sum of |x|). This test checks, with exact integer
arithmetic (every bf16 value is a multiple of 2^-133), that

  * the float64 transform's error never exceeds log2(g) * 2^-53 * sum |x|;
  * an accepted element always equals the correctly rounded fp32 value of the
    exact sum, and an undecided one rounds to RN32(y) or to its neighbour on
    the side of y;

on adversarial groups: GELU tails, fp32 ties broken by a tiny element, and
random spans of up to 120 binades. Pure numpy / Python; no GPU."""

import math

import numpy as np

Q = 133  # bf16 values are integer multiples of 2^-Q


def bf16(a):
    b = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def fwht_f64(x):
    v = x.astype(np.float64).copy()
    h = 1
    while h < len(v):
        for i in range(0, len(v), 2 * h):
            a = v[i:i + h].copy()
            b = v[i + h:i + 2 * h].copy()
            v[i:i + h] = a + b
            v[i + h:i + 2 * h] = a - b
        h *= 2
    return v


def fwht_int(n):
    v = list(n)
    h = 1
    while h < len(v):
        for i in range(0, len(v), 2 * h):
            for j in range(i, i + h):
                v[j], v[j + h] = v[j] + v[j + h], v[j] - v[j + h]
        h *= 2
    return v


def to_int(f):
    """exact integer N with f = N * 2^-Q (f a bf16 value or any double that
    is a multiple of 2^-Q)"""
    m, e = math.frexp(float(f))
    n = int(m * 2 ** 53)
    sh = e - 53 + Q
    return n << sh if sh >= 0 else n >> -sh if n % (1 << -sh) == 0 else None


def rn32_int(n):
    """correctly rounded fp32 of n * 2^-Q (nearest, ties to even)"""
    if n == 0:
        return 0.0
    s = -1 if n < 0 else 1
    a = abs(n)
    e = a.bit_length() - 1 - Q           # 2^e <= |value| < 2^(e+1)
    e = max(e, -126)
    sh = e - 23 + Q                       # ulp = 2^(e-23) = 2^sh units of 2^-Q
    if sh <= 0:
        return s * float(a) * 2.0 ** -Q
    fl, rem = divmod(a, 1 << sh)
    half = 1 << (sh - 1)
    if rem > half or (rem == half and fl & 1):
        fl += 1
    return s * math.ldexp(fl, e - 23)


def half_gap(r):
    rb = int(np.array(np.float32(r)).view(np.uint32))
    ef = max((rb >> 23) & 0xFF, 1)
    pow2 = 1 if (rb & 0x7FFFFF) == 0 else 0
    return 2.0 ** (ef - 151 - pow2)


def groups(g, rng):
    out = []
    for _ in range(6):   # GELU tails
        z = rng.standard_normal(g) * 3
        z[rng.random(g) < 0.03] *= 30
        out.append(bf16(0.5 * z * (1 + np.tanh(0.7978845608 * (z + 0.044715 * z ** 3)))))
    for _ in range(6):   # fp32 ties broken by a tiny element
        x = np.zeros(g, np.float32)
        x[0], x[1] = 1.0, 2.0 ** -24
        x[2] = 2.0 ** -float(rng.integers(60, 130)) * rng.choice([-1, 1])
        x[3:] = bf16(rng.standard_normal(g - 3) * 2.0 ** rng.integers(-120, -40, g - 3))
        out.append(bf16(x * 2.0 ** float(rng.integers(-20, 20))))
    for _ in range(6):   # random wide spans
        out.append(bf16(rng.standard_normal(g) * 2.0 ** rng.integers(-120, 0, g)))
    return out


def test_float64_transform_bound_and_acceptance_rule():
    rng = np.random.default_rng(20)
    accepted = undecided = 0
    for g in (16, 256):
        for x in groups(g, rng):
            y = fwht_f64(x)
            exact = fwht_int([to_int(t) for t in x])
            s_abs = sum(abs(to_int(t)) for t in x) * 2.0 ** -Q
            s32 = np.float32(0)
            for t in np.abs(x):
                s32 = np.float32(s32 + t)
            # the deferred pass's margin, and the fast kernel's (which must
            # never be the looser one here: both are twice the bound)
            delta = float(s32) * 2.0 ** -49
            logg = int(math.log2(g))
            ll = 1 if logg <= 2 else (2 if logg <= 4 else 3)
            emax = max(math.frexp(float(t))[1] - 1 for t in x if t != 0)
            s64 = 0.0
            for t in np.abs(x):
                s64 += float(t)
            e_s = math.frexp(s64)[1] - 1
            fast_delta = min(2.0 ** (emax + ll + logg - 51), 2.0 ** (e_s + ll - 51))
            bound = math.log2(g) * 2.0 ** -53 * s_abs
            assert delta > bound and fast_delta > bound, (g, delta, fast_delta, bound)
            for j in range(g):
                yj = to_int(y[j])
                assert yj is not None
                # the float64 transform's error bound (depth log2 g)
                assert abs(yj - exact[j]) * 2.0 ** -Q <= math.log2(g) * 2.0 ** -53 * s_abs
                r = float(np.float32(y[j]))
                d = y[j] - r
                h = half_gap(r)
                want = rn32_int(exact[j])
                if abs(d) + delta < h:
                    accepted += 1
                    assert r == want, (g, j)
                elif delta < h:
                    undecided += 1
                    nb = float(np.nextafter(np.float32(r), np.float32(math.copysign(np.inf, d))))
                    assert want in (r, nb), (g, j)
    assert accepted > 0 and undecided > 0


def _rn32_fraction(fr):
    """correctly rounded fp32 of an exact rational (nearest, ties to even)"""
    from fractions import Fraction
    if fr == 0:
        return 0.0
    s = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * float(fl * ulp)


def test_acceptance_margin_near_rounding_boundaries():
    """y placed just inside r's rounding interval, the exact value up to
    delta / 8 away (the transform's error is below that): whenever the rule
    accepts, the exact value rounds to r. Covers powers of two (half-gap
    ulp/4 toward zero), subnormals and zero."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    rs = [1.0, -1.0, 2.0 ** -20, 3.0, -0.75, 2.0 ** -126, 2.0 ** -140, 0.0, 1.5 * 2 ** 100]
    rs += list(rng.standard_normal(20) * 2.0 ** rng.integers(-60, 60, 20))
    checked = 0
    for r in rs:
        r = float(np.float32(r))
        up = float(np.nextafter(np.float32(r), np.float32(np.inf)))
        dn = float(np.nextafter(np.float32(r), np.float32(-np.inf)))
        for mid in ((r + up) / 2, (r + dn) / 2):          # the two rounding boundaries
            span = abs(mid - r)
            for frac in (0.5, 0.9, 0.99, 0.999999, 1 - 2.0 ** -30):
                y = r + (mid - r) * frac                   # inside r's interval
                if float(np.float32(y)) != r:
                    continue
                for delta in (span * 2.0 ** -20, span * 2.0 ** -8, span * 0.4):
                    d = y - r
                    if not (abs(d) + delta < half_gap(r)):
                        continue
                    for sgn in (-1, 1):                    # exact value within delta / 8
                        ex = Fraction(y) + sgn * Fraction(delta) / 8
                        assert _rn32_fraction(ex) == r, (r, y, delta)
                        checked += 1
    assert checked > 100
