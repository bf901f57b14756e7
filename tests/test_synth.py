"""The seeded input generators: determinism, shapes and outlier structure."""

import numpy as np

import synth


def test_deterministic_and_shaped():
    a = synth.TINY.x()
    b = synth.TINY.x()
    assert a.dtype == np.uint16 and a.shape == (64, 256)
    assert np.array_equal(a, b)
    assert synth.TINY.w().shape == (256, 256)


def test_outlier_channels_present():
    x = synth.bf16_bits_to_f32(synth.TINY.x()).astype(np.float64)
    col_rms = np.sqrt((x * x).mean(axis=0))
    assert (col_rms > 10).sum() == 4            # 4 channels x20
    w = synth.bf16_bits_to_f32(synth.TINY.w()).astype(np.float64)
    col_rms = np.sqrt((w * w).mean(axis=0))
    assert (col_rms > 0.1).sum() == 2           # 2 input columns x10


def test_student_t_columns_heavy_tailed():
    w = synth.bf16_bits_to_f32(synth.WAN_FFN_UP.scaled(n=256, k=512).w()).astype(np.float64)
    kurt = ((w - w.mean(0)) ** 4).mean(0) / (w.var(0) ** 2)
    assert (kurt > 6).sum() >= 3                # t_3 columns; Gaussian ones sit near 3


def test_bf16_round_trip():
    v = np.array([1.0, 1.0078125, -2.5, 0.0, 2.0 ** 127], dtype=np.float32)
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v)), v)


def test_f16_activations_are_the_same_draws():
    layer = synth.TINY
    hb = layer.x(fmt="f16")
    bb = layer.x()
    a = hb.view(np.float16).astype(np.float32)
    b = synth.bf16_bits_to_f32(bb)
    assert hb.dtype == np.uint16 and hb.shape == bb.shape
    assert np.isfinite(a).all()
    # both round the same float32 draws: half keeps 3 more bits
    assert np.abs(a - b).max() <= 2.0 ** -8 * np.abs(b).max()
