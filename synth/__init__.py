"""Seeded synthetic inputs for the convrot int8 linear layer.

This module only draws numbers and packs them as bf16 bit patterns. It holds
none of the layer's arithmetic (no rotation, no quantization, no matmul), so
both the CPU oracle and the GPU library can be fed from it without sharing any
method code.

The pages measure on real diffusion transformers (Z-Image Turbo, FLUX.1 dev,
Wan 2.2; Invoke docs "int8 Compute", speed tables). Their trained weights are
not available, so these generators stand in for them with the layer shapes of
those models and with the value structure that motivates the rotation: a few
input channels carrying outliers ("What is INT8 ConvRot?" on the
convert_to_quant guide: the rotation spreads outliers before quantizing).

Recipe (fixed order of draws from numpy.random.Generator(PCG64(seed))):
  1. values: standard_normal(shape, float32), then scaled;
  2. outlier channel/column indices: choice(K, n_out, replace=False) with
     n_out = round(frac * K);
  3. outlier multiply (or, for Student-t columns, replacement by fresh draws);
  4. cast to bf16 with round-to-nearest-even (via float32).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

ROT_SEED = 0xC0FFEE


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Input preparation only. Inputs here are finite.
    """
    u = np.array(a, dtype=np.float32).view(np.uint32)  # a private copy
    lsb = (u >> 16) & 1
    u += lsb       # finite values stay below 2^32 (at most 0xFF7FFFFF + 0x8000)
    u += 0x7FFF
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (nearest, ties to even); return uint16
    bits. Input preparation only; inputs here stay below half's maximum."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def _n_out(frac: float, k: int) -> int:
    return int(round(frac * k))


def activations(m: int, k: int, seed: int, *, outlier_frac: float = 0.0,
                outlier_mult: float = 1.0, n_outliers: int | None = None,
                gelu: bool = False, fmt: str = "bf16") -> np.ndarray:
    """Token activations x [m, k] as bf16 bits (fmt="f16": IEEE half bits of
    the same float32 draws).

    N(0,1) values; a seeded set of input channels (columns) multiplied by
    `outlier_mult`. With `gelu=True` the tanh-approximation GELU is applied
    in float64 after the outlier multiply (a GELU of a Gaussian, as an MLP's
    second input).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal((m, k), dtype=np.float32)
    n = n_outliers if n_outliers is not None else _n_out(outlier_frac, k)
    if n > 0:
        idx = rng.choice(k, n, replace=False)
        z[:, idx] *= np.float32(outlier_mult)
    if gelu:
        zz = z.astype(np.float64)
        zz = 0.5 * zz * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (zz + 0.044715 * zz ** 3)))
        z = zz.astype(np.float32)
    return f32_to_f16_bits(z) if fmt == "f16" else f32_to_bf16_bits(z)


def weights(n: int, k: int, seed: int, *, std: float = 0.02, outlier_frac: float = 0.0,
            outlier_mult: float = 1.0, n_outliers: int | None = None,
            student_t: bool = False) -> np.ndarray:
    """Linear weight W [n, k] (out, in) as bf16 bits.

    std * N(0,1) values; a seeded set of input columns either multiplied by
    `outlier_mult` or (student_t=True) replaced by std*outlier_mult*t_3 draws.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    c = n_outliers if n_outliers is not None else _n_out(outlier_frac, k)
    if c > 0:
        idx = rng.choice(k, c, replace=False)
        if student_t:
            t = rng.standard_t(3, size=(n, c)).astype(np.float32)
            w[:, idx] = np.float32(std * outlier_mult) * t
        else:
            w[:, idx] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(w)


@dataclasses.dataclass(frozen=True)
class Layer:
    """One linear layer of a workload: y[m, n] = x[m, k] . W[n, k]^T."""
    name: str
    m: int
    n: int
    k: int
    x_seed: int
    w_seed: int
    x_outlier_frac: float = 0.0
    x_outlier_mult: float = 1.0
    x_gelu: bool = False
    w_outlier_frac: float = 0.0
    w_outlier_mult: float = 1.0
    w_student_t: bool = False
    x_n_outliers: int | None = None
    w_n_outliers: int | None = None

    def x(self, rows: int | None = None, fmt: str = "bf16") -> np.ndarray:
        """Activations (bf16 bits, or half bits with fmt="f16"). With `rows`,
        the full matrix is drawn (so the values are those of the full
        workload) and its first rows are returned."""
        a = activations(self.m, self.k, self.x_seed, outlier_frac=self.x_outlier_frac,
                        outlier_mult=self.x_outlier_mult, n_outliers=self.x_n_outliers,
                        gelu=self.x_gelu, fmt=fmt)
        return a if rows is None else a[:rows]

    def w(self) -> np.ndarray:
        return weights(self.n, self.k, self.w_seed, outlier_frac=self.w_outlier_frac,
                       outlier_mult=self.w_outlier_mult, n_outliers=self.w_n_outliers,
                       student_t=self.w_student_t)

    def scaled(self, m: int | None = None, n: int | None = None, k: int | None = None,
               suffix: str = "small") -> "Layer":
        """Same value recipe at a reduced shape (outlier counts follow the
        fractions, or stay fixed where the recipe gives a count)."""
        return dataclasses.replace(self, name=f"{self.name}-{suffix}", m=m or self.m,
                                   n=n or self.n, k=k or self.k)


# The five workloads (layer shapes of the diffusion transformers the pages
# time; group size g and rotation seed are per call).
TINY = Layer("tiny 64x256x256", 64, 256, 256, 101, 102,
             x_n_outliers=4, x_outlier_mult=20.0, w_n_outliers=2, w_outlier_mult=10.0)
ZIMAGE_ATTN = Layer("zimage-attn 4608x3840x3840", 4608, 3840, 3840, 201, 202,
                    x_outlier_frac=0.005, x_outlier_mult=30.0,
                    w_outlier_frac=0.01, w_outlier_mult=10.0)
FLUX_MLP_UP = Layer("flux-mlp-up 4608x12288x3072", 4608, 12288, 3072, 301, 302,
                    x_outlier_frac=0.005, x_outlier_mult=30.0,
                    w_outlier_frac=0.01, w_outlier_mult=10.0)
FLUX_MLP_DOWN = Layer("flux-mlp-down 4608x3072x12288", 4608, 3072, 12288, 303, 304,
                      x_outlier_frac=0.005, x_outlier_mult=30.0, x_gelu=True,
                      w_outlier_frac=0.01, w_outlier_mult=10.0)
WAN_FFN_UP = Layer("wan-ffn-up 32760x13824x5120", 32760, 13824, 5120, 401, 402,
                   w_outlier_frac=0.01, w_outlier_mult=10.0, w_student_t=True)
WAN_FFN_DOWN = Layer("wan-ffn-down 32760x5120x13824", 32760, 5120, 13824, 403, 404,
                     w_outlier_frac=0.01, w_outlier_mult=10.0, w_student_t=True)
QKV_SWEEP = Layer("fused-qkv 16384x9216x3072", 16384, 9216, 3072, 501, 502,
                  x_outlier_frac=0.005, x_outlier_mult=30.0,
                  w_outlier_frac=0.01, w_outlier_mult=10.0)
# Weights of the streamed 60-layer dequant stack (values do not matter to a
# memory-bound kernel; two base weights are copied into distinct buffers).
STACK_SQUARE = Layer("stack 3072x3072", 1, 3072, 3072, 0, 503,
                     w_outlier_frac=0.01, w_outlier_mult=10.0)
STACK_WIDE = Layer("stack 12288x3072", 1, 12288, 3072, 0, 504,
                   w_outlier_frac=0.01, w_outlier_mult=10.0)
STACK_LAYERS = 60

GROUP_SIZES = (4, 16, 64, 256)

ALL_LAYERS = (TINY, ZIMAGE_ATTN, FLUX_MLP_UP, FLUX_MLP_DOWN, WAN_FFN_UP, WAN_FFN_DOWN,
              QKV_SWEEP)
