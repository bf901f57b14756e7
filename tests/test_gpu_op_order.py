"""GPU kernels against the op-order pins: inputs where the two plausible
readings of the quantizer and of the epilogue give different bytes, checked
through the C ABI against values derived here with exact rational arithmetic.

* Quantizer: q = rint(RN32(v * RN32(127/amax))) (not rint(RN32(v /
  RN32(amax/127)))). Rows at g = 4 hold (a, b, 0, 0 | c, 0, 0, 0 | 0 ...):
  the rotated row is d_j (a +- b) / 2 in the first group and d_j c / 2 in the
  second, so amax = |c| / 2 and (a - b) / 2 / amax = 1/2 exactly, a tie that
  the two readings break in opposite directions. Fast kernel, exact kernel
  and both weight quantizations.
* Epilogue: y = RN_bf16(RN32(RN32(acc * s_w) * s_x[m])) (not scales
  multiplied first). The accumulator is set through crafted int8 operands;
  s_w and s_x are passed in directly.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import int8_gemm_amd as cr
import oracle
import synth
from exact_rounding import (EPILOGUE_ORDER_CASES, epilogue_scales_first, epilogue_weight_first,
                            quant_divide, quant_reciprocal, rn32)

pytestmark = pytest.mark.gpu

SEED = synth.ROT_SEED
DEV = "cuda:0"
K = 64

# bf16 (a, b, c) of the crafted rows (found by a search for ties that the
# readings round apart)
QUANT_ROWS = [
    ("0x1.72p+12", "0x1.08p+10", "0x1.3p+13"),
    ("0x1.dap+2", "0x1.3p+0", "0x1.8ep+3"),
    ("0x1.d4p+18", "0x1.cp+16", "0x1.64p+19"),
    ("0x1.e2p-20", "0x1.08p-21", "0x1.5ep-19"),
]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    cr.load_library()


def _bf16_bits(h: str) -> int:
    bits = int(np.float32(float.fromhex(h)).view(np.uint32))
    assert bits & 0xFFFF == 0, h  # exactly a bf16 value
    return bits >> 16


def _crafted_x() -> np.ndarray:
    x = np.zeros((len(QUANT_ROWS), K), dtype=np.uint16)
    for r, (a, b, c) in enumerate(QUANT_ROWS):
        x[r, 0], x[r, 1], x[r, 4] = _bf16_bits(a), _bf16_bits(b), _bf16_bits(c)
    return x


def _expected_rows(x_bits: np.ndarray, g: int):
    """Codes and scales from the rotated rows (oracle.rotate_rows, pinned
    elsewhere; exact here since a +- b is exact) with the quantizer reading
    evaluated in exact rationals; also the count of codes the other reading
    would change."""
    xr = oracle.rotate_rows(x_bits, g, SEED)
    q = np.zeros(xr.shape, dtype=np.int8)
    s = np.zeros(xr.shape[0], dtype=np.float32)
    differ = 0
    for r in range(xr.shape[0]):
        amax = Fraction(float(np.abs(xr[r]).max()))
        s[r] = np.float32(float(rn32(amax / 127)))
        for j in range(xr.shape[1]):
            v = Fraction(float(xr[r, j]))
            q[r, j] = quant_reciprocal(v, amax)
            differ += quant_reciprocal(v, amax) != quant_divide(v, amax)
    return q, s, differ


def _dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def test_quantize_op_order_on_gpu():
    print("op order: quantize", flush=True)
    g = 4
    xb = _crafted_x()
    q_want, s_want, differ = _expected_rows(xb, g)
    assert differ >= len(QUANT_ROWS)  # every row holds a code the readings disagree on
    x = _dev_bf16(xb)
    for name, fn in (("fast", cr.convrot_quantize_activations),
                     ("exact", cr.convrot_quantize_activations_exact)):
        xq, s_x = fn(x, g, SEED)
        assert np.array_equal(xq.cpu().numpy(), q_want), name
        assert np.array_equal(s_x.cpu().numpy().view(np.uint32), s_want.view(np.uint32)), name
    wq, s_w = cr.convrot_quantize_weights_per_channel(x, g, SEED)
    assert np.array_equal(wq.cpu().numpy(), q_want)
    assert np.array_equal(s_w.cpu().numpy().view(np.uint32), s_want.view(np.uint32))
    for r in range(xb.shape[0]):  # per tensor: each row a weight of its own
        wq, s_w = cr.convrot_quantize_weights(x[r:r + 1].contiguous(), g, SEED)
        assert np.array_equal(wq.cpu().numpy()[0], q_want[r]), r
        assert s_w.cpu().numpy().view(np.uint32)[0] == s_want.view(np.uint32)[r], r


def _acc_operands(acc: int):
    """int8 rows x, w [K] with x . w = acc: w = (127 x 62, 1, 0),
    x = (S spread over 62 entries, t, 0) with acc = 127 S + t."""
    s_total = int(round(acc / 127))
    t = acc - 127 * s_total
    assert abs(t) <= 127 and abs(s_total) <= 62 * 127
    x = np.zeros(K, dtype=np.int8)
    rest = s_total
    for i in range(62):
        step = max(-127, min(127, rest))
        x[i] = step
        rest -= step
    x[62] = t
    w = np.zeros(K, dtype=np.int8)
    w[:62], w[62] = 127, 1
    assert int(x.astype(np.int64) @ w.astype(np.int64)) == acc
    return x, w


def _bf16_of(fr: Fraction) -> int:
    bits = int(np.float32(float(fr)).view(np.uint32))
    assert bits & 0xFFFF == 0
    return bits >> 16


def test_epilogue_op_order_on_gpu():
    print("op order: epilogue", flush=True)
    n = 16
    # per tensor: one launch per case
    for acc, sws, sxs in EPILOGUE_ORDER_CASES:
        sw, sx = Fraction(float.fromhex(sws)), Fraction(float.fromhex(sxs))
        want = epilogue_weight_first(acc, sw, sx)
        assert want != epilogue_scales_first(acc, sw, sx)
        xr, wr = _acc_operands(acc)
        xq = torch.from_numpy(xr[None, :].copy()).to(DEV)
        wq = torch.zeros((n, K), dtype=torch.int8)
        wq[0] = torch.from_numpy(wr)
        wq = wq.to(DEV)
        s_x = torch.tensor([float(sx)], dtype=torch.float32, device=DEV)
        s_w = torch.tensor([float(sw)], dtype=torch.float32, device=DEV)
        y, a = cr.convrot_gemm_int8(xq, s_x, wq, s_w, want_acc=True)
        assert int(a[0, 0]) == acc
        got = int(y.cpu().view(torch.int16).numpy().view(np.uint16)[0, 0])
        assert got == _bf16_of(want), (acc, sws, sxs)
    # per output channel: case i on the diagonal (row i, column i, s_w[i])
    cases = EPILOGUE_ORDER_CASES
    xq = np.zeros((len(cases), K), dtype=np.int8)
    wq = np.zeros((n, K), dtype=np.int8)
    sx = np.zeros(len(cases), dtype=np.float32)
    sw = np.ones(n, dtype=np.float32)
    for i, (acc, sws, sxs) in enumerate(cases):
        xq[i], wq[i] = _acc_operands(acc)
        sx[i], sw[i] = np.float32(float.fromhex(sxs)), np.float32(float.fromhex(sws))
    y, _ = cr.convrot_gemm_int8_per_channel(
        torch.from_numpy(xq).to(DEV), torch.from_numpy(sx).to(DEV), torch.from_numpy(wq).to(DEV),
        torch.from_numpy(sw).to(DEV))
    yb = y.cpu().view(torch.int16).numpy().view(np.uint16)
    for i, (acc, sws, sxs) in enumerate(cases):
        want = epilogue_weight_first(acc, Fraction(float.fromhex(sws)), Fraction(float.fromhex(sxs)))
        assert int(yb[i, i]) == _bf16_of(want), i
