"""CPU oracle for the int8_tensorwise "convrot" linear layer.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module. The GPU library never calls it, and
it shares no code, tables or constants with the GPU library: the two meet only
through the seeded inputs in `synth`.

What the layer computes, and where the pages say so
---------------------------------------------------
* The weight is stored int8 after a rotation of its input axis in g-wide
  groups, with one fp32 scale per tensor: convert_to_quant guide, "What is
  INT8 ConvRot?" and "How INT8 ConvRot Quantization Works" (`--int8
  --scaling_mode tensor --convrot --convrot-group-size`).
* The default path dequantizes and derotates the weight per forward as an
  [out, in/g, g] @ [g, g] block matmul, then runs a bf16 linear: PR "share the
  int8_convrot scheme ... Krea-2 and Z-Image", section "What it is worth".
* int8_compute rotates the input, quantizes it to int8 per token and
  multiplies int8 by int8: Invoke docs "int8 Compute", introduction.

What the pages leave open, and the reading taken here
-----------------------------------------------------
* R is never printed. R = H_g . D / sqrt(g): H_g the Sylvester Hadamard
  matrix, D = diag(d) with d drawn from SplitMix64 (counter form) of a seed.
* The fp32 value of a rotated element is the exact sum rounded once to fp32
  (nearest, ties to even). Products bf16 x (+-2^-k) are exact, so this is
  well defined and independent of summation order.
* Quantization is symmetric with scale s = RN(amax/127), inverse
  inv = RN(127/amax) and code q = clamp(rint_even(RN(v*inv)), -127, 127);
  amax == 0 gives s = 0 and q = 0. Where 127/amax would overflow (amax below
  2^-64), v and amax are first scaled by 2^64, which leaves every result of
  the plain formula unchanged wherever that formula is finite.
* Dequant: W_hat = RN_bf16(RN_fp32(float(S) * RN_fp32(s_w * 2^-log2(sqrt g))))
  with S = (Wq . D) . H per group in exact integers.
* GEMM epilogue: y = RN_bf16(RN_fp32(RN_fp32(float(acc) * s_w) * s_x[m])
  (+ bias[n], added in fp32)).
* Per-output-channel scales (the next step the pages point to: published int8
  convrot checkpoints carry one fp32 scale per output channel, and any weight
  scale multiplies output rows -- PR "share the int8_convrot scheme ... Krea-2
  and Z-Image", "Z-Image: the fused QKV" and the scale-layout fix in its
  commit list): s_w[n] = RN(amax_n/127) over row n of the rotated weight,
  the row quantized with it as a token row is; dequant uses RN(s_w[n]*2^-k)
  for row n; the epilogue uses s_w[n] for output column n.
* FP16 (the pages' kernels run in BF16 and FP16: Invoke docs "int8 Compute",
  the table of layers that keep unpacking): x, bias, y and W_hat may be
  IEEE half instead of bf16. Every step is the same; only the decoding of the
  inputs and the final rounding (RN to half, ties to even, overflow to inf)
  change.

Arithmetic is float64 (exact where the text says so) or exact integers.
"""

from __future__ import annotations

import math

import numpy as np

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


# ----------------------------------------------------------------------------
# Rotation: signs, Hadamard, R
# ----------------------------------------------------------------------------

def _splitmix64_mix(z: int) -> int:
    """Output function of SplitMix64 (Steele, Lea, Flood, OOPSLA 2014)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def splitmix64(seed: int, count: int) -> list[int]:
    """The first `count` outputs of SplitMix64 started from state `seed`:
    the state advances by the golden gamma before each output."""
    out = []
    state = seed & _MASK64
    for _ in range(count):
        state = (state + _GOLDEN_GAMMA) & _MASK64
        out.append(_splitmix64_mix(state))
    return out


def rotation_signs(seed: int, g: int) -> np.ndarray:
    """d[i] in {+1, -1}, i < g: -1 where bit 63 of the i-th SplitMix64 output
    (counter form: mix(seed + (i+1)*gamma)) is set."""
    return np.array([-1 if (z >> 63) & 1 else 1 for z in splitmix64(seed, g)], dtype=np.int64)


def hadamard(g: int) -> np.ndarray:
    """Sylvester's Hadamard matrix: H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    if g < 1 or g & (g - 1):
        raise ValueError("g must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(g: int, seed: int) -> np.ndarray:
    """R = H_g . diag(d) / sqrt(g) in float64. For g in {4, 16, 64, 256}
    every entry is exactly +-2^-log2(sqrt g)."""
    return hadamard(g).astype(np.float64) * rotation_signs(seed, g).astype(np.float64)[None, :] \
        / math.sqrt(g)


def block_rotation(k: int, g: int, seed: int) -> np.ndarray:
    """blockdiag(R, ..., R) of size k x k (for the float64 reference checks)."""
    if k % g:
        raise ValueError("k must be a multiple of g")
    b = np.zeros((k, k), dtype=np.float64)
    r = rotation_matrix(g, seed)
    for i in range(0, k, g):
        b[i:i + g, i:i + g] = r
    return b


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs):
    add 0x7FFF plus the kept lowest bit, drop the low 16 bits. For finite
    values the sum stays below 2^32, so uint32 arithmetic is exact."""
    u = np.array(a, dtype=np.float32).view(np.uint32)  # a private copy
    lsb = (u >> 16) & 1
    u += lsb
    u += 0x7FFF
    u >>= 16
    return u.astype(np.uint16)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE half bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f32_to_f16(a: np.ndarray) -> np.ndarray:
    """float32 -> IEEE half bits, round to nearest, ties to even; magnitudes
    from 65520 up become inf (IEEE 754 overflow under that rounding)."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


# decode, encode and significand fraction bits of each 16-bit format
_FORMATS = {"bf16": (bf16_to_f64, f32_to_bf16, 7), "f16": (f16_to_f64, f32_to_f16, 10)}


def _fmt(dtype: str):
    if dtype not in _FORMATS:
        raise ValueError(f"dtype must be one of {sorted(_FORMATS)}")
    return _FORMATS[dtype]


def to_f64(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """16-bit patterns of `dtype` -> float64 (exact)."""
    return _fmt(dtype)[0](bits)


def from_f32(a: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """float32 -> 16-bit patterns of `dtype`, round to nearest even."""
    return _fmt(dtype)[1](a)


def round_exact_to_f32(n: int, e: int) -> np.float32:
    """The float32 nearest to the exact value n * 2^e (ties to even),
    including the subnormal range. n, e are Python integers."""
    if n == 0:
        return np.float32(0.0)
    sign = -1.0 if n < 0 else 1.0
    a = -n if n < 0 else n
    nb = a.bit_length()
    top = nb - 1 + e                       # a * 2^e lies in [2^top, 2^(top+1))
    # exponent of the last kept bit: 24 significant bits, or 2^-149 at least
    keep_lsb = max(top - 23, -149)
    shift = keep_lsb - e
    if shift > 0:
        q = a >> shift
        rem = a - (q << shift)
        half = 1 << (shift - 1)
        if rem > half or (rem == half and (q & 1)):
            q += 1
        val = math.ldexp(float(q), keep_lsb)
    else:
        val = math.ldexp(float(a), e)      # exact: a has <= 24 bits here
    if val >= 2.0 ** 128:
        raise OverflowError("rotated value overflows float32")
    return np.float32(sign * val)


# ----------------------------------------------------------------------------
# Rotation of rows: exact sum, rounded once to fp32
# ----------------------------------------------------------------------------

def _group_exponent_span_ok(v: np.ndarray, g: int, frac_bits: int = 7) -> np.ndarray:
    """Per group (rows of v, shape [G, g]): True when every partial sum of
    +-v[i]*2^-k is exactly representable in float64, so any summation order
    gives the exact sum. With 2^e <= |v| < 2^(e+1) and frac_bits fraction
    bits (7 for bf16, 10 for half), every term is a multiple of
    2^(e_min-frac_bits-k) and every partial sum is below g*2^(e_max+1-k); 53
    bits cover that when e_max - e_min <= 52 - frac_bits - log2(g)."""
    a = np.abs(v)
    nz = a > 0
    _, ex = np.frexp(np.where(nz, a, 1.0))
    e = ex.astype(np.int64) - 1
    emax = np.where(nz, e, -(1 << 30)).max(axis=1)
    emin = np.where(nz, e, 1 << 30).min(axis=1)
    allzero = ~nz.any(axis=1)
    return allzero | (emax - emin <= 52 - frac_bits - int(math.log2(g)))


def _rotate_groups_exact_int(v: np.ndarray, g: int, seed: int, frac_bits: int = 7) -> np.ndarray:
    """Exact route for groups [G, g] (float64 holding 16-bit float values with
    frac_bits fraction bits): scale each group to integers, form the signed
    sums with integer arithmetic, round each sum once to float32."""
    h = hadamard(g)
    d = rotation_signs(seed, g)
    k = int(math.log2(math.isqrt(g)))      # 1/sqrt(g) = 2^-k
    out = np.empty(v.shape, dtype=np.float32)
    limb_bits = 40
    for r in range(v.shape[0]):
        row = v[r]
        nz = row != 0
        if not nz.any():
            out[r] = 0.0
            continue
        _, ex = np.frexp(np.abs(row[nz]))
        s = frac_bits - (int(ex.min()) - 1)   # every value is a multiple of 2^-s
        xs = [int(math.ldexp(float(t), s)) for t in row]   # exact integers
        # signed sums y_j = sum_i H[i, j] * xs[i], in 40-bit limbs so that a
        # plain int64 matmul is exact (|partial| < g * 2^40 < 2^63)
        mags = [abs(t) for t in xs]
        sgn = np.array([-1 if t < 0 else 1 for t in xs], dtype=np.int64)
        nlimb = max(1, (max(mags).bit_length() + limb_bits - 1) // limb_bits)
        ysum = [0] * g
        for c in range(nlimb):
            limb = np.array([(mg >> (limb_bits * c)) & ((1 << limb_bits) - 1) for mg in mags],
                            dtype=np.int64) * sgn
            yc = limb @ h                 # exact in int64
            for j in range(g):
                ysum[j] += int(yc[j]) << (limb_bits * c)
        for j in range(g):
            out[r, j] = round_exact_to_f32(int(d[j]) * ysum[j], -s - k)
    return out


def rotate_rows(x_bits: np.ndarray, g: int, seed: int, *, force_exact: bool = False,
                return_flag_count: bool = False, dtype: str = "bf16"):
    """x_r = x . blockdiag(R) per g-group of the last axis, each element the
    exact sum rounded once to float32.

    x_bits: bf16 (or, with dtype="f16", half) bit patterns [rows, K], K % g == 0.
    Groups whose exponent span keeps every float64 partial sum exact use a
    dense float64 block matmul [rows*K/g, g] @ R; the rest (and all groups
    when force_exact) use exact integer sums.
    """
    decode, _, frac_bits = _fmt(dtype)
    x = decode(x_bits)
    rows, kdim = x.shape
    if kdim % g:
        raise ValueError("K must be a multiple of g")
    v = x.reshape(-1, g)
    ok = np.zeros(v.shape[0], dtype=bool) if force_exact else \
        _group_exponent_span_ok(v, g, frac_bits)
    out = np.empty(v.shape, dtype=np.float32)
    if ok.any():
        out[ok] = (v[ok] @ rotation_matrix(g, seed)).astype(np.float32)
    bad = ~ok
    if bad.any():
        out[bad] = _rotate_groups_exact_int(v[bad], g, seed, frac_bits)
    out = out.reshape(rows, kdim)
    if return_flag_count:
        return out, int(bad.sum())
    return out


# ----------------------------------------------------------------------------
# Symmetric int8 quantization
# ----------------------------------------------------------------------------

_TWO64 = np.float32(2.0 ** 64)
_TINY = np.float32(2.0 ** -64)


def quantize_with_amax(v: np.ndarray, amax: np.ndarray):
    """q = clamp(rint_even(RN32(v * RN32(127/amax))), -127, 127) per row of v
    (float32 [rows, K]) with amax float32 [rows]; s = RN32(amax/127).
    Rows with amax == 0 get s = 0 and q = 0."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.asarray(amax, dtype=np.float32)
    pos = amax > 0
    s = np.where(pos, amax / np.float32(127.0), np.float32(0.0)).astype(np.float32)
    scale = np.where(pos & (amax < _TINY), _TWO64, np.float32(1.0)).astype(np.float32)
    vv = (v * scale[:, None]).astype(np.float32)
    aa = (amax * scale).astype(np.float32)
    inv = np.where(pos, np.float32(127.0) / np.where(pos, aa, np.float32(1.0)),
                   np.float32(0.0)).astype(np.float32)
    p = (vv * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(p), -127, 127).astype(np.int8)
    return q, s


def quantize_activations(x_bits: np.ndarray, g: int, seed: int, dtype: str = "bf16"):
    """Per-token (per-row) rotate + absmax + int8 quantize of x (bf16 or half).
    Returns xq int8 [M, K], s_x float32 [M]."""
    xr = rotate_rows(x_bits, g, seed, dtype=dtype)
    amax = np.abs(xr).max(axis=1) if xr.shape[1] else np.zeros(xr.shape[0], np.float32)
    return quantize_with_amax(xr, amax.astype(np.float32))


def quantize_weights(w_bits: np.ndarray, g: int, seed: int):
    """Per-tensor rotate + absmax + int8 quantize of W [N, K].
    Returns Wq int8 [N, K], s_w float32 (a 0-d array)."""
    wr = rotate_rows(w_bits, g, seed)
    amax = np.float32(np.abs(wr).max()) if wr.size else np.float32(0.0)
    q, s = quantize_with_amax(wr, np.full(wr.shape[0], amax, dtype=np.float32))
    return q, np.float32(s[0] if s.size else 0.0)


def quantize_weights_per_channel(w_bits: np.ndarray, g: int, seed: int):
    """Per-output-channel rotate + absmax + int8 quantize of W [N, K]: row n of
    the rotated weight gets s_w[n] = RN(amax_n/127) and is quantized with it.
    Returns Wq int8 [N, K], s_w float32 [N]."""
    wr = rotate_rows(w_bits, g, seed)
    amax = np.abs(wr).max(axis=1) if wr.shape[1] else np.zeros(wr.shape[0], np.float32)
    return quantize_with_amax(wr, amax.astype(np.float32))


def _row_scales(s_w, n: int) -> np.ndarray:
    """s_w as float32 [n]: a per-tensor scale repeated, or the per-channel
    vector itself (one scale per output row)."""
    sw = np.asarray(s_w, dtype=np.float32)
    if sw.ndim == 0:
        return np.full(n, sw, dtype=np.float32)
    if sw.shape != (n,):
        raise ValueError("a per-channel scale has one entry per output row")
    return sw


# ----------------------------------------------------------------------------
# Dequant + derotate (default path)
# ----------------------------------------------------------------------------

def derotation_integers(wq: np.ndarray, g: int, seed: int) -> np.ndarray:
    """S = (Wq . D) . H per g-group of the input axis, exact int64 [N, K].
    The product runs in float64 BLAS: every partial sum is an integer of
    magnitude <= 127 * g < 2^53, so it is exact."""
    n, kdim = wq.shape
    d = rotation_signs(seed, g)
    h = hadamard(g)
    grp = wq.reshape(-1, g).astype(np.float64) * d[None, :].astype(np.float64)
    return (grp @ h.astype(np.float64)).astype(np.int64).reshape(n, kdim)


def dequant_derotate(wq: np.ndarray, s_w, g: int, seed: int, out_dtype: str = "bf16") -> np.ndarray:
    """W_hat (bf16 bits) = RN_bf16(RN32(float(S) * c)), c = RN32(s_w*2^-k);
    with a per-channel s_w [N], row n uses c_n = RN32(s_w[n]*2^-k).
    out_dtype="f16" rounds to half instead."""
    k = int(math.log2(math.isqrt(g)))
    c = (_row_scales(s_w, wq.shape[0]) * np.float32(2.0 ** -k)).astype(np.float32)
    s_int = derotation_integers(wq, g, seed)
    return from_f32((s_int.astype(np.float32) * c[:, None]).astype(np.float32), out_dtype)


def dequant_reference_f64(wq: np.ndarray, s_w, g: int, seed: int) -> np.ndarray:
    """s_w * Wq . blockdiag(R)^T in float64 (the tolerance reference); a
    per-channel s_w scales the rows."""
    r = rotation_matrix(g, seed)
    n, kdim = wq.shape
    grp = wq.reshape(-1, g).astype(np.float64)
    sw = _row_scales(s_w, n).astype(np.float64)
    return sw[:, None] * (grp @ r.T).reshape(n, kdim)


# ----------------------------------------------------------------------------
# int8 GEMM + epilogue (int8_compute path)
# ----------------------------------------------------------------------------

def gemm_int32(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * wq[n, k], exact. Computed with float64
    BLAS: every partial sum is an integer of magnitude <= 127^2 * K < 2^53."""
    if xq.shape[1] != wq.shape[1]:
        raise ValueError("K mismatch")
    if 127 * 127 * xq.shape[1] >= 2 ** 31:
        raise ValueError("K too large for an int32 accumulator")
    acc = xq.astype(np.float64) @ wq.astype(np.float64).T
    return acc.astype(np.int64).astype(np.int32)


def epilogue(acc: np.ndarray, s_w, s_x: np.ndarray, bias_bits: np.ndarray | None = None,
             dtype: str = "bf16"):
    """y = RN_bf16(RN32(RN32(float(acc) * s_w) * s_x[m]) [+ bias[n]]) -> bf16 bits;
    a per-channel s_w [N] scales output column n. dtype="f16": bias and y are
    half (y rounded once from the same fp32 value)."""
    t = acc.astype(np.float32)
    t = (t * _row_scales(s_w, acc.shape[1])[None, :]).astype(np.float32)
    t = (t * np.asarray(s_x, dtype=np.float32)[:, None]).astype(np.float32)
    if bias_bits is not None:
        t = (t + to_f64(bias_bits, dtype).astype(np.float32)[None, :]).astype(np.float32)
    return from_f32(t, dtype)


def linear_int8(x_bits: np.ndarray, wq: np.ndarray, s_w, g: int, seed: int,
                bias_bits: np.ndarray | None = None, dtype: str = "bf16"):
    """The int8_compute forward: rotate + quantize x per token, int8 GEMM,
    scale epilogue; x, bias and y in `dtype`. Returns (y bits, xq, s_x, acc)."""
    xq, s_x = quantize_activations(x_bits, g, seed, dtype)
    acc = gemm_int32(xq, wq)
    return epilogue(acc, s_w, s_x, bias_bits, dtype), xq, s_x, acc


def linear_int8_reference_f64(acc: np.ndarray, s_w, s_x: np.ndarray,
                              bias_bits: np.ndarray | None = None,
                              dtype: str = "bf16") -> np.ndarray:
    """s_w * s_x[m] * acc (+ bias) in float64: the tolerance reference of the
    int8_compute output."""
    sw = _row_scales(s_w, acc.shape[1]).astype(np.float64)
    y = sw[None, :] * np.asarray(s_x, dtype=np.float64)[:, None] * acc.astype(np.float64)
    if bias_bits is not None:
        y = y + to_f64(bias_bits, dtype)[None, :]
    return y


def dequant_linear_reference_f64(x_bits: np.ndarray, wq: np.ndarray, s_w, g: int, seed: int,
                                 bias_bits: np.ndarray | None = None,
                                 dtype: str = "bf16") -> np.ndarray:
    """x . (s_w Wq blockdiag(R)^T)^T in float64: the tolerance reference of the
    default (dequant) path."""
    y = to_f64(x_bits, dtype) @ dequant_reference_f64(wq, s_w, g, seed).T
    if bias_bits is not None:
        y = y + to_f64(bias_bits, dtype)[None, :]
    return y


def rel_frobenius(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_F / ||ref||_F in float64."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a))
