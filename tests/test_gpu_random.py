"""GPU: seeded random forwards against the oracle. Each case draws its own
shape (ragged M, N a multiple of 16, K a multiple of 64 and of g), group size,
scale granularity, activation format, bias and rotation seed; some inputs get
GELU-like tails, so the deferred-row pass is exercised too. The weight
quantization, the forward's output and the dequantized weight must equal the
oracle's bit for bit."""

import numpy as np
import pytest
import torch

import int8_gemm_amd as cr
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    cr.load_library()


def dev16(bits: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _case(i: int):
    rng = np.random.default_rng(1000 + i)
    g = int(rng.choice([4, 16, 64, 256]))
    k = int(rng.integers(1, 49)) * 64
    k = (k + g - 1) // g * g
    n = int(rng.integers(1, 97)) * 16
    m = int(rng.integers(1, 1200))
    while m * n * k > 1.5e9:
        m //= 2
    m = max(m, 1)
    pc = bool(rng.integers(0, 2))
    fmt = "f16" if rng.integers(0, 3) == 0 else "bf16"
    use_bias = bool(rng.integers(0, 2))
    seed = int(rng.integers(0, 2 ** 63))
    gelu = rng.integers(0, 4) == 0
    if gelu:
        m = min(m, 200)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.integers(0, k, max(1, k // 200))] *= 30.0
    if gelu:
        x = np.where(x < 0, x * np.exp(-20.0 * x * x), x).astype(np.float32)
    enc = synth.f32_to_f16_bits if fmt == "f16" else synth.f32_to_bf16_bits
    xb = enc(x)
    wb = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    bias = enc(rng.standard_normal(n).astype(np.float32)) if use_bias else None
    return dict(m=m, n=n, k=k, g=g, pc=pc, fmt=fmt, gelu=bool(gelu), seed=seed), xb, wb, bias


@pytest.mark.parametrize("i", range(24))
def test_random_forward_matches_oracle(i):
    p, xb, wb, bias = _case(i)
    print(f"random case {i}: {p}", flush=True)
    g, seed, pc, fmt = p["g"], p["seed"], p["pc"], p["fmt"]
    dtype = torch.float16 if fmt == "f16" else torch.bfloat16
    quant = cr.convrot_quantize_weights_per_channel if pc else cr.convrot_quantize_weights
    wq, s_w = quant(dev16(wb, torch.bfloat16), g, seed)
    wq_ref, s_ref = (oracle.quantize_weights_per_channel if pc else oracle.quantize_weights)(
        wb, g, seed)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert np.array_equal(np.atleast_1d(s_w.cpu().numpy()).view(np.uint32),
                          np.atleast_1d(np.asarray(s_ref, dtype=np.float32)).view(np.uint32))
    y = cr.convrot_linear_int8_ex(dev16(xb, dtype), wq, s_w, g, seed,
                                  None if bias is None else dev16(bias, dtype), per_channel=pc)
    y_ref = oracle.linear_int8(xb, wq_ref, s_ref, g, seed, bias, dtype=fmt)[0]
    assert np.array_equal(host_bits(y), y_ref)
    w_hat = cr.convrot_dequant_derotate_ex(wq, s_w, g, seed, per_channel=pc, out_dtype=dtype)
    assert np.array_equal(host_bits(w_hat),
                          oracle.dequant_derotate(wq_ref, s_ref, g, seed, out_dtype=fmt))
