"""Pins of the CPU oracle against facts fixed outside it: published test
vectors, closed forms, library routines and brute force on tiny inputs.

Each test would fail on a plausible mistake in the oracle: a wrong sign
placement (signs after vs before H), a transposed R, a dropped 1/sqrt(g), a
wrong rounding mode or order, an off-by-one in the exponent bound of the
exact route, a mis-scaled dequant.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as o
import synth
from exact_rounding import (EPILOGUE_ORDER_CASES, QUANT_ORDER_CASES, epilogue_scales_first,
                            epilogue_weight_first, f32, quant_divide, quant_reciprocal, rn32)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SEED = synth.ROT_SEED
GS = (4, 16, 64, 256)


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split("#")[0].strip() for ln in f if ln.split("#")[0].strip()]


# --------------------------------------------------------------------------
# P1: rotation matrix, signs
# --------------------------------------------------------------------------

def test_splitmix64_published_outputs():
    want = [int(v, 16) for v in _golden_lines("splitmix64_seed0.txt")]
    assert o.splitmix64(0, len(want)) == want


def test_hadamard_golden_and_closed_form():
    h4 = np.array([[int(t) for t in ln.split()] for ln in _golden_lines("hadamard4.txt")])
    assert np.array_equal(o.hadamard(4), h4)
    for g in GS:
        h = o.hadamard(g)
        i = np.arange(g)
        par = np.vectorize(lambda a: bin(a).count("1") & 1)(i[:, None] & i[None, :])
        assert np.array_equal(h, 1 - 2 * par)
        assert np.array_equal(h @ h.T, g * np.eye(g, dtype=np.int64))


@pytest.mark.parametrize("seed", [SEED, 0, 12345, 2 ** 64 - 1])
def test_rotation_orthogonal_exactly(seed):
    for g in GS:
        r = o.rotation_matrix(g, seed)
        k = math.log2(math.sqrt(g))
        assert np.array_equal(np.abs(r), np.full((g, g), 2.0 ** -k))
        assert np.array_equal(r @ r.T, np.eye(g))
        assert np.array_equal(r.T @ r, np.eye(g))


def test_rotation_signs_after_transform():
    # (v . R)[j] = d[j] (v . H)[j] / sqrt(g): column j of R carries sign d[j]
    for g in GS:
        d = o.rotation_signs(SEED, g)
        r = o.rotation_matrix(g, SEED)
        assert np.array_equal(np.sign(r[0, :]).astype(np.int64), d)
        assert np.all(r[:, 0] * d[0] > 0)


def test_sign_prefix_and_counts():
    d256 = o.rotation_signs(SEED, 256)
    for g in (4, 16, 64):
        assert np.array_equal(o.rotation_signs(SEED, g), d256[:g])
    # 32-bit words of the g = 256 mask (bit i set <=> d[i] = -1), LSB first
    bits = sum(1 << i for i in range(256) if d256[i] < 0)
    words = [(bits >> (32 * w)) & 0xFFFFFFFF for w in range(8)]
    assert words[0] == 0x2F06E2B7 and words[1] == 0x2CFCF23A
    assert int((d256 < 0).sum()) == 140


# --------------------------------------------------------------------------
# P2: the rotation identity (x B)(W B)^T = x W^T
# --------------------------------------------------------------------------

def test_rotation_identity_unquantized():
    x = o.bf16_to_f64(synth.TINY.x())
    w = o.bf16_to_f64(synth.TINY.w())
    for g in GS:
        b = o.block_rotation(256, g, SEED)
        lhs = (x @ b) @ (w @ b).T
        rhs = x @ w.T
        assert np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs) < 1e-13


# --------------------------------------------------------------------------
# Number-format helpers against library routines
# --------------------------------------------------------------------------

def test_round_exact_to_f32_matches_numpy():
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(4000):
        nbits = int(rng.integers(1, 53))
        n = int(rng.integers(1, 2 ** nbits))
        if rng.random() < 0.3:                     # force exact ties at 24 bits
            n = ((n >> 1) << 1) | 1
            n <<= 1
        e = int(rng.integers(-200, 60))
        if n.bit_length() + e > 127:
            continue
        cases.append((n if rng.random() < 0.5 else -n, e))
    for n, e in cases:
        ref = np.float32(np.float64(math.ldexp(float(n), e)))   # n < 2^53: exact in f64
        got = o.round_exact_to_f32(n, e)
        assert got.view(np.uint32) == ref.view(np.uint32), (n, e)


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(3)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormals
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0],
                 dtype=np.float32),                                   # exact ties
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.f32_to_bf16(a), ref)


# --------------------------------------------------------------------------
# Rotation of rows: brute force with exact rationals
# --------------------------------------------------------------------------

def _nearest_f32(fr: Fraction) -> np.float32:
    """Independent correct rounding: try the float32 neighbours of a first
    guess, pick the nearest, ties to the even significand."""
    c0 = np.float32(float(fr))
    cands = {c0, np.nextafter(c0, np.float32(np.inf)), np.nextafter(c0, np.float32(-np.inf))}
    best = sorted(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                        int(np.float32(c).view(np.uint32)) & 1))[0]
    return np.float32(best)


def _bruteforce_rotate(x_bits, g, seed):
    x = o.bf16_to_f64(x_bits)
    h = o.hadamard(g)
    d = o.rotation_signs(seed, g)
    out = np.empty(x.shape, dtype=np.float32)
    for r in range(x.shape[0]):
        for q in range(0, x.shape[1], g):
            xs = [Fraction(float(t)) for t in x[r, q:q + g]]
            for j in range(g):
                s = sum((xs[i] if h[i, j] > 0 else -xs[i]) for i in range(g))
                out[r, q + j] = _nearest_f32(s * int(d[j]) / Fraction(math.isqrt(g)))
    return out


def _wide_span_rows(rows, k, seed):
    """bf16 rows mixing ordinary values with tiny ones (exponent spans far
    beyond 53 bits) and exact cancellations."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, k)).astype(np.float32) * 3
    mask = rng.random((rows, k)) < 0.15
    tiny = (rng.standard_normal((rows, k)) * 2.0 ** rng.integers(-140, -20, (rows, k)))
    v = np.where(mask, tiny.astype(np.float32), v)
    v[0, : k // 2] = 1.0                                     # cancellations
    v[1, :] = 0.0
    v[1, 0] = 2.0 ** -130                                    # subnormal bf16
    return synth.f32_to_bf16_bits(v)


@pytest.mark.parametrize("g", [4, 16])
def test_rotate_rows_bruteforce_small_g(g):
    xb = _wide_span_rows(6, 64, 11 + g)
    want = _bruteforce_rotate(xb, g, SEED)
    got, nflag = o.rotate_rows(xb, g, SEED, return_flag_count=True)
    assert nflag > 0                      # the exact integer route is exercised
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    got2 = o.rotate_rows(xb, g, SEED, force_exact=True)
    assert np.array_equal(got2.view(np.uint32), want.view(np.uint32))


def test_rotate_rows_bruteforce_g256_rows():
    xb = np.concatenate([_wide_span_rows(2, 256, 5), synth.TINY.x()[:1]])
    want = _bruteforce_rotate(xb, 256, SEED)
    got = o.rotate_rows(xb, 256, SEED)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fast_and_exact_routes_agree_on_ordinary_data():
    xb = synth.ZIMAGE_ATTN.scaled(m=8, k=1024).x()
    for g in GS:
        a, nflag = o.rotate_rows(xb, g, SEED, return_flag_count=True)
        b = o.rotate_rows(xb, g, SEED, force_exact=True)
        assert nflag == 0
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gelu_tail_workload_has_wide_span_groups():
    # a GELU of an outlier-scaled Gaussian puts values near 1e-15 beside
    # values near 100 in the same group: the exact route must run there
    xb = synth.FLUX_MLP_DOWN.x(rows=64)
    _, nflag = o.rotate_rows(xb, 256, SEED, return_flag_count=True)
    assert nflag > 0


# --------------------------------------------------------------------------
# P3: known answers for rotate + quantize
# --------------------------------------------------------------------------

@pytest.mark.parametrize("g", GS)
def test_impulse_and_ones_known_answers(g):
    k = 512
    imp = np.zeros((1, k), dtype=np.float32)
    imp[0, ::g] = 1.0
    ones = np.ones((1, k), dtype=np.float32)
    d = o.rotation_signs(SEED, g)
    sq = math.isqrt(g)
    xr = o.rotate_rows(synth.f32_to_bf16_bits(imp), g, SEED)
    assert np.array_equal(xr[0], np.tile(d / sq, k // g).astype(np.float32))
    xq, sx = o.quantize_activations(synth.f32_to_bf16_bits(imp), g, SEED)
    assert np.array_equal(xq[0], np.tile(127 * d, k // g).astype(np.int8))
    assert sx[0] == np.float32(np.float32(1.0 / sq) / np.float32(127.0))
    xq, sx = o.quantize_activations(synth.f32_to_bf16_bits(ones), g, SEED)
    want = np.zeros(k, dtype=np.int8)
    want[::g] = 127 * d[0]
    assert np.array_equal(xq[0], want)
    assert sx[0] == np.float32(np.float32(sq) / np.float32(127.0))
    if g == 256:
        assert float(sx[0]) == float.fromhex("0x1.020408p-3")


# --------------------------------------------------------------------------
# P4: quantizer invariants
# --------------------------------------------------------------------------

def test_quantizer_invariants():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 300)).astype(np.float32)
    v[1] = 0.0
    v[2] *= np.float32(1e-30)
    v[3] *= np.float32(2.0 ** -100)                       # below the 2^-64 guard
    v[4] = (rng.standard_normal(300) * 1e-42).astype(np.float32)   # subnormal
    v[5] *= np.float32(1e30)
    amax = np.abs(v).max(axis=1).astype(np.float32)
    q, s = o.quantize_with_amax(v, amax)
    assert q.dtype == np.int8 and q.min() >= -127
    for r in range(v.shape[0]):
        if amax[r] == 0:
            assert s[r] == 0 and not q[r].any()
            continue
        assert np.abs(q[r].astype(np.int64)).max() == 127
        assert s[r] == np.float32(amax[r] / np.float32(127.0))
        if s[r] > np.float32(2.0 ** -120):                   # s itself not subnormal
            err = np.abs(v[r].astype(np.float64) - float(s[r]) * q[r].astype(np.float64))
            assert err.max() <= float(s[r]) * (0.5 + 2.0 ** -15)


def test_tiny_guard_matches_plain_formula_where_finite():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal((8, 64)) * 2.0 ** -90).astype(np.float32)
    amax = np.abs(v).max(axis=1).astype(np.float32)
    assert (amax < np.float32(2.0 ** -64)).all()
    q, _ = o.quantize_with_amax(v, amax)
    inv = (np.float32(127.0) / amax).astype(np.float32)
    assert np.isfinite(inv).all()
    plain = np.clip(np.rint((v * inv[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
    assert np.array_equal(q, plain)


# --------------------------------------------------------------------------
# P5: int32 GEMM by brute force
# --------------------------------------------------------------------------

def test_gemm_int32_bruteforce():
    rng = np.random.default_rng(1)
    xq = rng.integers(-127, 128, (64, 256)).astype(np.int8)
    wq = rng.integers(-127, 128, (256, 256)).astype(np.int8)
    want = np.einsum("mk,nk->mn", xq.astype(np.int64), wq.astype(np.int64))
    assert np.array_equal(o.gemm_int32(xq, wq).astype(np.int64), want)
    # extreme magnitudes over a long K stay exact
    xq = np.full((3, 8192), 127, dtype=np.int8)
    wq = np.full((2, 8192), -127, dtype=np.int8)
    assert (o.gemm_int32(xq, wq) == -127 * 127 * 8192).all()


def test_epilogue_closed_form():
    acc = np.array([[0, 1, -1, 2 ** 24 + 1, -(2 ** 27) - 3]], dtype=np.int32)
    s_w = np.float32(0.001)
    s_x = np.array([0.5], dtype=np.float32)
    y = o.epilogue(acc, s_w, s_x)
    t = (acc.astype(np.float32) * s_w).astype(np.float32) * np.float32(0.5)
    assert np.array_equal(y, o.f32_to_bf16(t.astype(np.float32)))
    # 2^24 + 1 is not a float32: it rounds to 2^24 before scaling
    assert acc.astype(np.float32)[0, 3] == np.float32(2 ** 24)


# --------------------------------------------------------------------------
# P4b, P5b: operation order of the quantizer and of the epilogue, pinned with
# exact rational arithmetic (fractions.Fraction) written here, not with the
# oracle's own expressions. Each case is an input where the two plausible
# readings of the same formula give different results, so a swapped order
# fails. The inputs were found by a search for such disagreements; every
# expected value below is derived in this file.
# --------------------------------------------------------------------------

def test_quantize_op_order_reciprocal_not_divide():
    """The int8 code is rint(RN32(v * RN32(127/amax))), not rint(RN32(v /
    RN32(amax/127))): the multiply-by-reciprocal reading of the quantizer's
    round(clip(Wr / s_w)) (convert_to_quant guide, "How INT8 ConvRot
    Quantization Works"; the scale itself stays s = RN32(amax/127))."""
    for vs, ams in QUANT_ORDER_CASES:
        v, amax = Fraction(float.fromhex(vs)), Fraction(float.fromhex(ams))
        want, other = quant_reciprocal(v, amax), quant_divide(v, amax)
        assert want != other, (vs, ams)
        q, s = o.quantize_with_amax(np.array([[f32(v), f32(amax)]], dtype=np.float32),
                                    np.array([f32(amax)], dtype=np.float32))
        assert int(q[0, 0]) == want, (vs, ams, int(q[0, 0]), want, other)
        assert int(q[0, 1]) == 127
        assert Fraction(float(s[0])) == rn32(amax / 127)


def test_epilogue_op_order_weight_scale_first():
    """y = RN_bf16(RN32(RN32(acc * s_w) * s_x[m])): the accumulator is scaled
    by the weight scale, then by the token's scale (Invoke docs "int8
    Compute", introduction: the int8 product is rescaled to the compute
    dtype; the pages give no order, this is the reading taken)."""
    for acc, sws, sxs in EPILOGUE_ORDER_CASES:
        sw, sx = Fraction(float.fromhex(sws)), Fraction(float.fromhex(sxs))
        want, other = epilogue_weight_first(acc, sw, sx), epilogue_scales_first(acc, sw, sx)
        assert want != other, (acc, sws, sxs)
        y = o.epilogue(np.array([[acc]], dtype=np.int32), f32(sw),
                       np.array([f32(sx)], dtype=np.float32))
        got = Fraction(float(o.bf16_to_f64(y)[0, 0]))
        assert got == want, (acc, sws, sxs, float(got), float(want), float(other))


def test_rounding_helpers_against_numpy():
    """The rational rounding above agrees with numpy's IEEE single rounding on
    random quotients (so the pins above test the oracle, not the helpers)."""
    rng = np.random.default_rng(21)
    a = rng.standard_normal(300).astype(np.float32)
    b = (rng.standard_normal(300) * 2.0 ** rng.integers(-40, 40, 300)).astype(np.float32)
    for x, y in zip(a, b):
        if y == 0:
            continue
        assert rn32(Fraction(float(x)) / Fraction(float(y))) == Fraction(float(np.float32(x / y)))
        assert rn32(Fraction(float(x)) * Fraction(float(y))) == Fraction(float(np.float32(x * y)))


# --------------------------------------------------------------------------
# P6: dequant + derotate
# --------------------------------------------------------------------------

@pytest.mark.parametrize("g", GS)
def test_dequant_integers_independent(g):
    rng = np.random.default_rng(g)
    wq = rng.integers(-127, 128, (8, 512)).astype(np.int8)
    d = o.rotation_signs(SEED, g)
    dh = np.diag(d) @ o.hadamard(g)
    dense = np.kron(np.eye(512 // g, dtype=np.int64), dh)     # blockdiag(D H)
    assert np.array_equal(o.derotation_integers(wq, g, SEED), wq.astype(np.int64) @ dense)
    assert np.abs(o.derotation_integers(wq, g, SEED)).max() <= 127 * g
    # the extreme: a row of 127 d reaches S = 127 g (and -127 d gives -127 g)
    wq[0, :g] = 127 * d
    wq[1, :g] = -127 * d
    s_int = o.derotation_integers(wq, g, SEED)
    assert s_int[0, 0] == 127 * g and s_int[1, 0] == -127 * g
    assert np.array_equal(s_int, wq.astype(np.int64) @ dense)


@pytest.mark.parametrize("g", GS)
def test_dequant_inverts_rotation_on_impulses(g):
    k = 256
    w = np.zeros((2, k), dtype=np.float32)
    w[0, 0] = 1.0
    w[1, 3] = -1.0
    wq, s_w = o.quantize_weights(synth.f32_to_bf16_bits(w), g, SEED)
    d = o.rotation_signs(SEED, g)
    assert np.array_equal(wq[0, :g], (127 * d).astype(np.int8))
    w_hat = o.bf16_to_f64(o.dequant_derotate(wq, s_w, g, SEED))
    assert np.array_equal(w_hat, w.astype(np.float64))
    ref = o.dequant_reference_f64(wq, s_w, g, SEED)
    assert np.abs(ref - w).max() < 1e-6


# --------------------------------------------------------------------------
# P7, P8: reconstruction error and derotation on/off
# --------------------------------------------------------------------------

def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.mark.parametrize("layer,g", [(synth.TINY, 256),
                                     (synth.ZIMAGE_ATTN.scaled(n=512), 256),
                                     (synth.QKV_SWEEP.scaled(n=256), 64),
                                     (synth.QKV_SWEEP.scaled(n=256), 16)])
def test_reconstruction_error_and_cosines(layer, g):
    wb = layer.w()
    w = o.bf16_to_f64(wb)
    wq, s_w = o.quantize_weights(wb, g, SEED)
    rec = o.dequant_reference_f64(wq, s_w, g, SEED)
    e = np.linalg.norm(rec - w) / np.linalg.norm(w)
    # uniform quantization noise: rms error = step / sqrt(12) (Bennett)
    pred = float(s_w) / (math.sqrt(12.0) * math.sqrt(np.mean(w * w)))
    assert abs(e / pred - 1.0) < 0.05
    assert e < 0.05
    # derotated cosine follows 1 - e^2/2; skipping derotation decorrelates
    assert abs(_cos(rec, w) - (1 - e * e / 2)) < 1e-6
    b = o.block_rotation(w.shape[1], g, SEED)
    no_derot = float(s_w) * wq.astype(np.float64)
    pred_ctrl = float(np.sum((w.T @ w) * b) / np.sum(w * w))
    assert abs(_cos(no_derot, w) - pred_ctrl) < 0.01
    assert abs(_cos(no_derot, w)) < 0.3


def test_pages_cosine_error_pairing():
    vals = dict(ln.split() for ln in _golden_lines("pages_decode_quality.txt"))
    e = float(vals["relative_error"])
    assert round(1 - e * e / 2, 5) == float(vals["cosine_derotated"])
    assert float(vals["cosine_without_derotation"]) < 0.1


# --------------------------------------------------------------------------
# P10: rotation spreads outliers before per-token quantization
# --------------------------------------------------------------------------

def test_rotation_reduces_per_token_error():
    xb = synth.ZIMAGE_ATTN.scaled(m=64, k=1024).x()
    x = o.bf16_to_f64(xb)
    xq, sx = o.quantize_activations(xb, 256, SEED)
    b = o.block_rotation(1024, 256, SEED)
    back = (sx[:, None].astype(np.float64) * xq) @ b.T
    e_rot = np.linalg.norm(back - x) / np.linalg.norm(x)
    x32 = x.astype(np.float32)
    q, s = o.quantize_with_amax(x32, np.abs(x32).max(axis=1))
    e_plain = np.linalg.norm(s[:, None] * q.astype(np.float64) - x) / np.linalg.norm(x)
    assert e_rot < e_plain / 3


# --------------------------------------------------------------------------
# The whole int8 linear on the tiny workload
# --------------------------------------------------------------------------

def test_linear_int8_tiny_tolerances():
    layer = synth.TINY
    xb, wb = layer.x(), layer.w()
    wq, s_w = o.quantize_weights(wb, 256, SEED)
    y, xq, sx, acc = o.linear_int8(xb, wq, s_w, 256, SEED)
    yb = o.bf16_to_f64(y)
    ref = o.linear_int8_reference_f64(acc, s_w, sx)
    assert o.rel_frobenius(yb, ref) < 2.0 ** -8
    true = o.bf16_to_f64(xb) @ o.bf16_to_f64(wb).T
    assert o.rel_frobenius(yb, true) < 0.05
    deq = o.dequant_linear_reference_f64(xb, wq, s_w, 256, SEED)
    assert o.rel_frobenius(deq, true) < 0.05


# --------------------------------------------------------------------------
# Per-output-channel weight scales: one fp32 scale per row of W, i.e. per
# output column of y (PR "share the int8_convrot scheme ... Krea-2 and
# Z-Image", "Z-Image: the fused QKV"; the scale-layout fix in its commits)
# --------------------------------------------------------------------------

def _rowscaled_weight(n, k, rng):
    """bf16 weight whose row magnitudes span 2^-12 .. 2^12"""
    w = rng.standard_normal((n, k)) * 0.02
    w *= 2.0 ** rng.integers(-12, 13, n)[:, None]
    return synth.f32_to_bf16_bits(w.astype(np.float32))


@pytest.mark.parametrize("g", GS)
def test_per_channel_quantize_is_per_tensor_of_each_row(g):
    rng = np.random.default_rng(30 + g)
    wb = _rowscaled_weight(12, 512, rng)
    wq, s = o.quantize_weights_per_channel(wb, g, SEED)
    assert s.shape == (12,) and s.dtype == np.float32 and wq.dtype == np.int8
    for n in range(12):
        q1, s1 = o.quantize_weights(wb[n:n + 1], g, SEED)
        assert np.array_equal(wq[n], q1[0]) and s[n] == s1
        assert np.abs(wq[n].astype(np.int64)).max() == 127


def test_per_channel_power_of_two_row_scaling():
    """rows 2^e * v quantize to the same codes with scales 2^e * s; one
    per-tensor scale flushes the small rows to zero"""
    rng = np.random.default_rng(31)
    v = o.bf16_to_f64(synth.f32_to_bf16_bits((rng.standard_normal((1, 256)) * 0.05)
                                             .astype(np.float32)))
    e = np.arange(-10, 11, 4)
    wb = synth.f32_to_bf16_bits((v * 2.0 ** e[:, None]).astype(np.float32))
    for g in GS:
        wq, s = o.quantize_weights_per_channel(wb, g, SEED)
        assert (wq == wq[0]).all()
        assert np.array_equal(s.astype(np.float64), float(s[0]) * 2.0 ** (e - e[0]))
        wq_t, _ = o.quantize_weights(wb, g, SEED)
        assert not wq_t[0].any() and np.array_equal(wq_t[-1], wq[-1])


@pytest.mark.parametrize("g", (16, 64))
def test_per_channel_dequant_recovers_row_impulses_on_square_weight(g):
    """Square W (out == in), row n one impulse of its own magnitude: the
    per-channel decode returns W exactly. Applying the scales along the input
    axis instead (the broadcast the pages' fix removed) would not."""
    k = 64
    w = np.zeros((k, k), dtype=np.float32)
    for n in range(k):
        w[n, (7 * n) % k] = (-1.0) ** n * 2.0 ** ((n % 13) - 6)
    wq, s = o.quantize_weights_per_channel(synth.f32_to_bf16_bits(w), g, SEED)
    w_hat = o.bf16_to_f64(o.dequant_derotate(wq, s, g, SEED))
    assert np.array_equal(w_hat, w.astype(np.float64))
    ref = o.dequant_reference_f64(wq, s, g, SEED)
    # float64 decode: off only by the fp32 rounding of each row's scale
    assert (np.abs(ref - w).max(axis=1) <= 2.0 ** -23 * np.abs(w).max(axis=1)).all()
    # the wrong broadcast (scales over input columns) misdecodes most rows
    k_ = int(math.log2(math.isqrt(g)))
    s_int = o.derotation_integers(wq, g, SEED).astype(np.float64)
    wrong = s_int * (s.astype(np.float64) * 2.0 ** -k_)[None, :]
    assert (np.abs(wrong - w).max(axis=1) > 0.5 * np.abs(w).max(axis=1)).sum() > k // 2


def test_per_channel_dequant_constant_scales_is_per_tensor():
    rng = np.random.default_rng(33)
    wq = rng.integers(-127, 128, (8, 512)).astype(np.int8)
    for g in GS:
        sw = np.float32(0.0123)
        assert np.array_equal(o.dequant_derotate(wq, np.full(8, sw, np.float32), g, SEED),
                              o.dequant_derotate(wq, sw, g, SEED))


def test_per_channel_epilogue_closed_form():
    """acc = 1 everywhere, s_x[m] = 2^m, s_w[n] = 2^-n: y[m, n] = 2^(m - n)
    (a scale applied along the wrong axis gives 2^(n - m) or 2^0)"""
    m = n = 6
    acc = np.ones((m, n), dtype=np.int32)
    s_x = (2.0 ** np.arange(m)).astype(np.float32)
    s_w = (2.0 ** -np.arange(n)).astype(np.float32)
    y = o.bf16_to_f64(o.epilogue(acc, s_w, s_x))
    assert np.array_equal(y, 2.0 ** (np.arange(m)[:, None] - np.arange(n)[None, :]))
    # each column is the per-tensor epilogue with that column's scale
    rng = np.random.default_rng(34)
    acc = rng.integers(-2 ** 20, 2 ** 20, (5, 7)).astype(np.int32)
    s_w = (rng.random(7) * 1e-3).astype(np.float32)
    s_x = (rng.random(5) * 1e-2).astype(np.float32)
    bias = synth.f32_to_bf16_bits(rng.standard_normal(7).astype(np.float32))
    y = o.epilogue(acc, s_w, s_x, bias)
    for j in range(7):
        assert np.array_equal(y[:, j], o.epilogue(acc[:, j:j + 1], s_w[j], s_x, bias[j:j + 1])[:, 0])
    with pytest.raises(ValueError):
        o.epilogue(acc, s_w[:5], s_x)


def test_linear_int8_per_channel_tolerances():
    """On a weight whose rows span 2^24 in magnitude, per-channel scales keep
    every output column accurate; one per-tensor scale does not."""
    rng = np.random.default_rng(35)
    layer = synth.TINY
    xb = layer.x()
    wb = _rowscaled_weight(layer.n, layer.k, rng)
    wq, s_w = o.quantize_weights_per_channel(wb, 256, SEED)
    y, xq, sx, acc = o.linear_int8(xb, wq, s_w, 256, SEED)
    yb = o.bf16_to_f64(y)
    assert o.rel_frobenius(yb, o.linear_int8_reference_f64(acc, s_w, sx)) < 2.0 ** -8
    true = o.bf16_to_f64(xb) @ o.bf16_to_f64(wb).T
    col_err = np.linalg.norm(yb - true, axis=0) / np.linalg.norm(true, axis=0)
    assert col_err.max() < 0.05
    deq = o.dequant_linear_reference_f64(xb, wq, s_w, 256, SEED)
    assert o.rel_frobenius(deq, true) < 0.05
    wq_t, s_t = o.quantize_weights(wb, 256, SEED)
    yt = o.bf16_to_f64(o.linear_int8(xb, wq_t, s_t, 256, SEED)[0])
    col_err_t = np.linalg.norm(yt - true, axis=0) / np.linalg.norm(true, axis=0)
    assert col_err_t.max() > 0.5


# --------------------------------------------------------------------------
# FP16 activations and outputs (the pages' kernels run in BF16 and FP16:
# Invoke docs "int8 Compute", the table of layers that keep unpacking)
# --------------------------------------------------------------------------

def test_f32_to_f16_known_values_and_torch():
    """IEEE 754 half, round to nearest even: printed bit patterns of the
    binary16 format, then agreement with torch's own conversion"""
    cases = [(1.0, 0x3C00), (-2.5, 0xC100), (65504.0, 0x7BFF), (65519.99, 0x7BFF),
             (65520.0, 0x7C00), (-1e6, 0xFC00), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000),
             (3 * 2.0 ** -26, 0x0001), (1 + 2.0 ** -11, 0x3C00), (1 + 3 * 2.0 ** -11, 0x3C02),
             (2.0 ** -14, 0x0400), (0.0, 0x0000), (-0.0, 0x8000)]
    got = o.f32_to_f16(np.array([c for c, _ in cases], dtype=np.float32))
    assert [int(v) for v in got] == [b for _, b in cases]
    rng = np.random.default_rng(40)
    a = (rng.standard_normal(200000) * 2.0 ** rng.integers(-30, 17, 200000)).astype(np.float32)
    want = torch.from_numpy(a).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.f32_to_f16(a), want)
    # decode is exact
    bits = np.arange(0, 0x7C00, 7, dtype=np.uint16)
    assert np.array_equal(o.f16_to_f64(bits), bits.view(np.float16).astype(np.float64))


def _f16_groups(rng, rows, k):
    """half values with the widest spans the format allows: subnormals
    (multiples of 2^-24) beside values near 65504"""
    x = rng.standard_normal((rows, k)) * 2.0 ** rng.integers(-26, 16, (rows, k))
    x = np.clip(x, -65504, 65504).astype(np.float16)
    x[:, ::17] = np.float16(2.0 ** -24)
    x[:, 5::19] = np.float16(-65504.0)
    return x.view(np.uint16)


@pytest.mark.parametrize("g", GS)
def test_f16_float64_transform_is_exact(g):
    """Every half value is a multiple of 2^-24 below 2^16, so the signed sums
    of a group are multiples of 2^-24 below 2^24: any float64 summation is
    exact. Checked against exact integer sums on the widest spans."""
    rng = np.random.default_rng(41 + g)
    xb = _f16_groups(rng, 6, 512)
    fast = o.rotate_rows(xb, g, SEED, dtype="f16")
    exact = o.rotate_rows(xb, g, SEED, dtype="f16", force_exact=True)
    assert np.array_equal(fast.view(np.uint32), exact.view(np.uint32))
    # and a float64 sum in another order (reversed terms) lands on the same values
    x = o.f16_to_f64(xb).reshape(-1, g)
    r = o.rotation_matrix(g, SEED)
    rev = (x[:, ::-1] @ r[::-1, :]).astype(np.float32).reshape(fast.shape)
    assert np.array_equal(rev.view(np.uint32), fast.view(np.uint32))


def test_f16_exact_route_uses_half_significand():
    """the integer route on half values that need all 11 significant bits"""
    g = 16
    x = np.zeros((1, g), dtype=np.float16)
    for tiny in (2.0 ** -24, 1.5):                 # smallest element tiny, or not
        x[0, 0] = np.float16(1 + 2.0 ** -10)       # 11 significant bits
        x[0, 1] = np.float16(tiny)
        xb = x.view(np.uint16)
        got = o.rotate_rows(xb, g, SEED, dtype="f16", force_exact=True)
        d = o.rotation_signs(SEED, g)
        h = o.hadamard(g)
        want = np.array([float(Fraction(1 + 2.0 ** -10) * int(h[0, j]) + Fraction(tiny)
                               * int(h[1, j])) * int(d[j]) / 4 for j in range(g)],
                        dtype=np.float32)
        assert np.array_equal(got[0], want), tiny


def test_f16_and_bf16_agree_where_both_hold_x():
    """values with at most 8 significant bits inside half's normal range are
    the same numbers in both formats: identical codes and scales"""
    rng = np.random.default_rng(42)
    v = rng.standard_normal((16, 512)) * 2.0 ** rng.integers(-10, 10, (16, 512))
    v = o.bf16_to_f64(synth.f32_to_bf16_bits(v.astype(np.float32)))
    v = np.where(np.abs(v) < 2.0 ** -14, 0.0, v)
    v = np.clip(v, -60000, 60000)
    bb = synth.f32_to_bf16_bits(v.astype(np.float32))
    hb = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(o.f16_to_f64(hb), o.bf16_to_f64(bb))
    for g in GS:
        q1, s1 = o.quantize_activations(bb, g, SEED)
        q2, s2 = o.quantize_activations(hb, g, SEED, "f16")
        assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_f16_epilogue_closed_form_and_overflow():
    acc = np.array([[1, -1, 1000, 70000, 65504, 65520]], dtype=np.int32)
    s_x = np.array([1.0], dtype=np.float32)
    y = o.epilogue(acc, np.float32(1.0), s_x, dtype="f16")
    assert [int(t) for t in y[0]] == [0x3C00, 0xBC00, 0x63D0, 0x7C00, 0x7BFF, 0x7C00]
    bias = np.array([0x3C00] * 6, dtype=np.uint16)          # +1.0 in half
    yb = o.epilogue(acc, np.float32(1.0), s_x, bias, dtype="f16")
    assert int(yb[0, 0]) == 0x4000 and int(yb[0, 1]) == 0x0000
    # bf16 bias bits read as bf16 would give a different value: the dtype decides
    assert o.f16_to_f64(np.array([0x3C00], np.uint16))[0] == 1.0
    assert o.bf16_to_f64(np.array([0x3C00], np.uint16))[0] == 2.0 ** -7


@pytest.mark.parametrize("g", GS)
def test_f16_dequant_recovers_impulses(g):
    k = 256
    w = np.zeros((2, k), dtype=np.float32)
    w[0, 0] = 1.0
    w[1, 3] = -1.0
    wq, s_w = o.quantize_weights(synth.f32_to_bf16_bits(w), g, SEED)
    w_hat = o.f16_to_f64(o.dequant_derotate(wq, s_w, g, SEED, "f16"))
    assert np.array_equal(w_hat, w.astype(np.float64))


def test_f16_linear_tolerances():
    layer = synth.TINY
    xb = o.f32_to_f16(o.bf16_to_f64(layer.x()).astype(np.float32))
    wq, s_w = o.quantize_weights(layer.w(), 256, SEED)
    bias = o.f32_to_f16(np.random.default_rng(43).standard_normal(layer.n).astype(np.float32))
    y, xq, sx, acc = o.linear_int8(xb, wq, s_w, 256, SEED, bias, "f16")
    yf = o.f16_to_f64(y)
    assert o.rel_frobenius(yf, o.linear_int8_reference_f64(acc, s_w, sx, bias, "f16")) < 2.0 ** -10
    true = o.f16_to_f64(xb) @ o.bf16_to_f64(layer.w()).T + o.f16_to_f64(bias)[None, :]
    assert o.rel_frobenius(yf, true) < 0.05
