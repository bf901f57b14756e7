"""GPU parity: the HIP kernels through the C ABI against the CPU oracle, on the
same seeded inputs. Integer and bf16 outputs whose definition is exact are
compared bit for bit (Wq, s_w, xq, s_x, acc, W_hat, y of the int8 path);
float outputs are also checked against float64 references to 1e-2 relative
Frobenius error."""

import math

import numpy as np
import pytest
import torch

import int8_gemm_amd as cr
import oracle
import synth

pytestmark = pytest.mark.gpu

SEED = synth.ROT_SEED
GS = (4, 16, 64, 256)
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(cr.library_path()):
        from int8_gemm_amd import _build
        _build.build()
    cr.load_library()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _announce(msg):
    print(msg, flush=True)


def bf16_matmul_nt(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """y = x . w^T in x's 16-bit format (torch's hipBLASLt matmul): the
    caller's consumer of the dequantized weight. The transposed operand is
    made contiguous first, so the product is a plain 2-D matmul of
    contiguous operands."""
    assert x.dtype == w.dtype and x.dtype in (torch.bfloat16, torch.float16)
    return torch.matmul(x, w.t().contiguous())


# reduced shapes spanning several GEMM tiles and ragged tails, with each
# workload's K and value recipe
REDUCED = [
    (synth.TINY, 256),
    (synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256),
    (synth.FLUX_MLP_UP.scaled(m=257, n=528), 256),
    (synth.FLUX_MLP_DOWN.scaled(m=96, n=256), 256),
    (synth.WAN_FFN_UP.scaled(m=130, n=400), 256),
    (synth.WAN_FFN_DOWN.scaled(m=70, n=272), 256),
] + [(synth.QKV_SWEEP.scaled(m=260, n=288), g) for g in GS]
IDS = [f"{l.name}-g{g}" for l, g in REDUCED]


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
def test_quantize_weights_bitexact(layer, g):
    _announce(f"quantize_weights {layer.name} g={g}")
    wb = layer.w()
    wq, s_w = cr.convrot_quantize_weights(dev_bf16(wb), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert f32_bits(s_w.cpu().numpy())[0] == f32_bits(s_ref)


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
def test_dequant_bitexact_and_tolerance(layer, g):
    _announce(f"dequant {layer.name} g={g}")
    wq_ref, s_ref = oracle.quantize_weights(layer.w(), g, SEED)
    wq = torch.from_numpy(wq_ref).to(DEV)
    s_w = torch.tensor([s_ref], dtype=torch.float32, device=DEV)
    w_hat = cr.convrot_dequant_derotate(wq, s_w, g, SEED)
    got = host_bits(w_hat)
    assert np.array_equal(got, oracle.dequant_derotate(wq_ref, s_ref, g, SEED))
    ref = oracle.dequant_reference_f64(wq_ref, s_ref, g, SEED)
    assert oracle.rel_frobenius(oracle.bf16_to_f64(got), ref) < 1e-2


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
def test_quantize_activations_bitexact(layer, g):
    _announce(f"quantize_activations {layer.name} g={g}")
    xb = layer.x()
    xq_ref, sx_ref = oracle.quantize_activations(xb, g, SEED)
    for fn in (cr.convrot_quantize_activations, cr.convrot_quantize_activations_exact):
        xq, sx = fn(dev_bf16(xb), g, SEED)
        assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref)), fn.__name__
        assert np.array_equal(xq.cpu().numpy(), xq_ref), fn.__name__


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
@pytest.mark.parametrize("with_bias", [False, True])
def test_gemm_bitexact(layer, g, with_bias):
    _announce(f"gemm {layer.name} g={g} bias={with_bias}")
    xq_ref, sx_ref = oracle.quantize_activations(layer.x(), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights(layer.w(), g, SEED)
    bias_b = None
    if with_bias:
        bias_b = synth.f32_to_bf16_bits(
            np.random.default_rng(7).standard_normal(layer.n).astype(np.float32))
    y, acc = cr.convrot_gemm_int8(torch.from_numpy(xq_ref).to(DEV),
                                  torch.from_numpy(sx_ref).to(DEV),
                                  torch.from_numpy(wq_ref).to(DEV),
                                  torch.tensor([s_ref], dtype=torch.float32, device=DEV),
                                  None if bias_b is None else dev_bf16(bias_b), want_acc=True)
    acc_ref = oracle.gemm_int32(xq_ref, wq_ref)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    y_ref = oracle.epilogue(acc_ref, s_ref, sx_ref, bias_b)
    assert np.array_equal(host_bits(y), y_ref)


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
def test_linear_int8_bitexact_and_tolerances(layer, g):
    _announce(f"linear_int8 {layer.name} g={g}")
    xb, wb = layer.x(), layer.w()
    wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
    y_ref, xq_ref, sx_ref, acc_ref = oracle.linear_int8(xb, wq_ref, s_ref, g, SEED)
    x = dev_bf16(xb)
    wq = torch.from_numpy(wq_ref).to(DEV)
    s_w = torch.tensor([s_ref], dtype=torch.float32, device=DEV)
    y = cr.convrot_linear_int8(x, wq, s_w, g, SEED)
    got = host_bits(y)
    assert np.array_equal(got, y_ref)
    yf = oracle.bf16_to_f64(got)
    assert oracle.rel_frobenius(yf, oracle.linear_int8_reference_f64(acc_ref, s_ref, sx_ref)) \
        < 1e-2
    # the default (dequant) path as the caller runs it: a bf16 matmul of x
    # and W_hat (torch on ROCm), against the float64 reference; and the same
    # product in fp32
    w_hat = cr.convrot_dequant_derotate(wq, s_w, g, SEED)
    ref_deq = oracle.dequant_linear_reference_f64(xb, wq_ref, s_ref, g, SEED)
    y_bf = bf16_matmul_nt(x, w_hat)
    assert oracle.rel_frobenius(oracle.bf16_to_f64(host_bits(y_bf)), ref_deq) < 1e-2
    y_deq = (x.float() @ w_hat.float().t()).to(torch.bfloat16)
    assert oracle.rel_frobenius(oracle.bf16_to_f64(host_bits(y_deq)), ref_deq) < 1e-2


def test_slicing_invariance_and_determinism():
    layer, g = synth.ZIMAGE_ATTN.scaled(m=1030, n=256), 256
    xb = layer.x()
    wq_ref, s_ref = oracle.quantize_weights(layer.w(), g, SEED)
    x = dev_bf16(xb)
    wq = torch.from_numpy(wq_ref).to(DEV)
    s_w = torch.tensor([s_ref], dtype=torch.float32, device=DEV)
    outs = []
    for rows in (1030, 515, 258, 256, 100, 1):
        ws = torch.empty(cr.convrot_linear_int8_workspace_for_rows(rows, layer.k),
                         dtype=torch.uint8, device=DEV)
        outs.append(host_bits(cr.convrot_linear_int8(x, wq, s_w, g, SEED, workspace=ws)))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    for _ in range(10):
        assert np.array_equal(host_bits(cr.convrot_linear_int8(x, wq, s_w, g, SEED)), outs[0])


# --------------------------------------------------------------------------
# Edge cases
# --------------------------------------------------------------------------

def _edge_rows(k):
    rng = np.random.default_rng(11)
    rows = []
    rows.append(np.zeros(k))                                   # zero row
    rows.append(np.full(k, -0.0))                              # negative zeros
    imp = np.zeros(k); imp[0] = 1.0; rows.append(imp)          # impulse
    rows.append(np.ones(k))                                    # constant: cancellations
    rows.append(rng.standard_normal(k) * 2.0 ** -100)          # below the 2^-64 guard
    rows.append(rng.standard_normal(k) * 1e-42)                # subnormal bf16 values
    r = rng.standard_normal(k) * 3                             # wide exponent spans
    m = rng.random(k) < 0.2
    r[m] = rng.standard_normal(m.sum()) * 2.0 ** rng.integers(-130, -30, m.sum())
    rows.append(r)
    r = rng.standard_normal(k); r[::7] = 1e-38; rows.append(r)  # tiny normals beside O(1)
    rows.append(rng.standard_normal(k) * 1e30)                 # large
    rows.append(np.where(rng.random(k) < 0.5, 1.0, -1.0) * 2.0 ** rng.integers(-20, 20, k))
    # fp32 ties decided only by a tiny element: in every other 256-block a
    # group holds 1, 2^-24 and +-2^-100, so the float64 transform lands exactly
    # on an fp32 midpoint that the lost 2^-100 term breaks; the other blocks
    # hold 100.0 (the row absmax) or nothing (the tie group holds the absmax)
    for tiny, big in ((2.0 ** -100, 100.0), (-(2.0 ** -100), 100.0), (2.0 ** -100, 0.0)):
        r = np.zeros(k)
        for s0 in range(0, k, 512):
            r[s0], r[s0 + 1], r[s0 + 2] = 1.0, 2.0 ** -24, tiny
            if s0 + 256 < k:
                r[s0 + 256] = big
        rows.append(r)
    return synth.f32_to_bf16_bits(np.array(rows, dtype=np.float32))


@pytest.mark.parametrize("g", GS)
@pytest.mark.parametrize("k", [256, 3072])
def test_edge_rows_activations(g, k):
    _announce(f"edge rows g={g} k={k}")
    xb = _edge_rows(k)
    xq_ref, sx_ref = oracle.quantize_activations(xb, g, SEED)
    for fn in (cr.convrot_quantize_activations, cr.convrot_quantize_activations_exact):
        xq, sx = fn(dev_bf16(xb), g, SEED)
        assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref)), fn.__name__
        assert np.array_equal(xq.cpu().numpy(), xq_ref), fn.__name__


@pytest.mark.parametrize("g", GS)
def test_edge_weights(g):
    _announce(f"edge weights g={g}")
    for wb in (_edge_rows(256), np.zeros((16, 256), dtype=np.uint16),
               synth.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((16, 256))
                                      .astype(np.float32) * 2.0 ** -110)):
        wq, s_w = cr.convrot_quantize_weights(dev_bf16(wb), g, SEED)
        wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
        assert f32_bits(s_w.cpu().numpy())[0] == f32_bits(s_ref)
        assert np.array_equal(wq.cpu().numpy(), wq_ref)
        w_hat = cr.convrot_dequant_derotate(wq, s_w, g, SEED)
        assert np.array_equal(host_bits(w_hat), oracle.dequant_derotate(wq_ref, s_ref, g, SEED))


@pytest.mark.parametrize("tile", [0, 128, 192, 256, 384])
@pytest.mark.parametrize("m,n,k", [(1, 16, 64), (2, 32, 128), (255, 16, 192), (257, 272, 320),
                                   (33, 1040, 64), (512, 512, 4096), (400, 592, 384),
                                   (300, 400, 1152), (300, 400, 1088), (800, 208, 256)])
def test_gemm_shapes(m, n, k, tile):
    _announce(f"gemm shape {m}x{n}x{k} tile={tile}")
    if tile == 384 and k % 128:
        with pytest.raises(cr.ConvrotError) as e:   # the 384 x 192 tile needs K % 128 == 0
            cr.convrot_gemm_int8(torch.zeros((m, k), dtype=torch.int8, device=DEV),
                                 torch.ones(m, device=DEV),
                                 torch.zeros((n, k), dtype=torch.int8, device=DEV),
                                 torch.ones(1, device=DEV), tile=tile)
        assert e.value.status_name == "CONVROT_E_INVALID_ARG"
        return
    rng = np.random.default_rng(m * 7 + n)
    xq = rng.integers(-127, 128, (m, k)).astype(np.int8)
    wq = rng.integers(-127, 128, (n, k)).astype(np.int8)
    xq[0, :] = 127
    wq[0, :] = -127
    sx = (rng.random(m) * 1e-3).astype(np.float32)
    sw = np.float32(3e-4)
    y, acc = cr.convrot_gemm_int8(torch.from_numpy(xq).to(DEV), torch.from_numpy(sx).to(DEV),
                                  torch.from_numpy(wq).to(DEV),
                                  torch.tensor([sw], dtype=torch.float32, device=DEV),
                                  want_acc=True, tile=tile)
    acc_ref = oracle.gemm_int32(xq, wq)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert np.array_equal(host_bits(y), oracle.epilogue(acc_ref, sw, sx))


def test_m_zero_and_errors_on_device():
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    xq, sx = cr.convrot_quantize_activations(x, 256)
    assert xq.shape == (0, 256)
    with pytest.raises(cr.ConvrotError) as e:
        cr.convrot_quantize_activations(torch.zeros((4, 320), dtype=torch.bfloat16,
                                                    device=DEV), 256)
    assert e.value.status_name == "CONVROT_E_UNSUPPORTED_GROUP"


def test_wrong_rotation_gives_noise():
    # decoding with a different seed raises nothing and decorrelates the weight
    layer, g = synth.ZIMAGE_ATTN.scaled(n=256), 256
    wb = layer.w()
    wq, s_w = cr.convrot_quantize_weights(dev_bf16(wb), g, SEED)
    good = oracle.bf16_to_f64(host_bits(cr.convrot_dequant_derotate(wq, s_w, g, SEED)))
    bad = oracle.bf16_to_f64(host_bits(cr.convrot_dequant_derotate(wq, s_w, g, SEED + 1)))
    w = oracle.bf16_to_f64(wb)

    def cos(a, b):
        return float((a * b).sum() / math.sqrt((a * a).sum() * (b * b).sum()))
    assert cos(good, w) > 0.9999
    assert abs(cos(bad, w)) < 0.3


# --------------------------------------------------------------------------
# Per-output-channel weight scales (one fp32 scale per row of W)
# --------------------------------------------------------------------------

def _rowscaled(wb: np.ndarray, seed: int, span: int = 12) -> np.ndarray:
    """The weight with row r scaled by 2^e_r, e_r uniform in [-span, span]
    (exact in bf16 away from the subnormal range): row magnitudes that one
    per-tensor scale cannot serve, like the fused Q, K and V blocks."""
    e = np.random.default_rng(seed).integers(-span, span + 1, wb.shape[0])
    w = oracle.bf16_to_f64(wb) * 2.0 ** e[:, None]
    return synth.f32_to_bf16_bits(w.astype(np.float32))


def _dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
def test_per_channel_quantize_and_dequant_bitexact(layer, g):
    _announce(f"per-channel quantize+dequant {layer.name} g={g}")
    wb = _rowscaled(layer.w(), layer.n)
    wq, s_w = cr.convrot_quantize_weights_per_channel(dev_bf16(wb), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights_per_channel(wb, g, SEED)
    assert np.array_equal(f32_bits(s_w.cpu().numpy()), f32_bits(s_ref))
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    w_hat = host_bits(cr.convrot_dequant_derotate_per_channel(wq, s_w, g, SEED))
    assert np.array_equal(w_hat, oracle.dequant_derotate(wq_ref, s_ref, g, SEED))
    ref = oracle.dequant_reference_f64(wq_ref, s_ref, g, SEED)
    assert oracle.rel_frobenius(oracle.bf16_to_f64(w_hat), ref) < 1e-2
    # every row on its own scale: the smallest rows are as accurate as the largest
    w = oracle.bf16_to_f64(wb)
    row_err = np.linalg.norm(oracle.bf16_to_f64(w_hat) - w, axis=1) / np.linalg.norm(w, axis=1)
    assert row_err.max() < 0.05


@pytest.mark.parametrize("g", GS)
def test_per_channel_edge_weights(g):
    _announce(f"per-channel edge weights g={g}")
    for wb in (_edge_rows(256), _edge_rows(3072), np.zeros((16, 256), dtype=np.uint16)):
        wq, s_w = cr.convrot_quantize_weights_per_channel(dev_bf16(wb), g, SEED)
        wq_ref, s_ref = oracle.quantize_weights_per_channel(wb, g, SEED)
        assert np.array_equal(f32_bits(s_w.cpu().numpy()), f32_bits(s_ref))
        assert np.array_equal(wq.cpu().numpy(), wq_ref)
        w_hat = cr.convrot_dequant_derotate_per_channel(wq, s_w, g, SEED)
        assert np.array_equal(host_bits(w_hat), oracle.dequant_derotate(wq_ref, s_ref, g, SEED))


@pytest.mark.parametrize("g", (16, 64, 256))
def test_per_channel_square_weight_decodes_rows_not_columns(g):
    """out == in: scales applied along the wrong axis would still run; the
    decode must return every row's impulse exactly."""
    _announce(f"per-channel square impulses g={g}")
    k = 256
    w = np.zeros((k, k), dtype=np.float32)
    for r in range(k):
        w[r, (37 * r) % k] = (-1.0) ** r * 2.0 ** ((r % 29) - 14)
    wb = synth.f32_to_bf16_bits(w)
    wq, s_w = cr.convrot_quantize_weights_per_channel(dev_bf16(wb), g, SEED)
    w_hat = host_bits(cr.convrot_dequant_derotate_per_channel(wq, s_w, g, SEED))
    assert np.array_equal(oracle.bf16_to_f64(w_hat), w.astype(np.float64))


@pytest.mark.parametrize("tile", [0, 128, 192, 256, 384])
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (255, 16, 192), (257, 272, 320), (33, 1040, 64),
                                   (400, 592, 384), (300, 400, 1152), (800, 208, 256)])
def test_per_channel_gemm_shapes(m, n, k, tile):
    _announce(f"per-channel gemm shape {m}x{n}x{k} tile={tile}")
    rng = np.random.default_rng(m * 5 + n)
    xq = rng.integers(-127, 128, (m, k)).astype(np.int8)
    wq = rng.integers(-127, 128, (n, k)).astype(np.int8)
    sx = (rng.random(m) * 1e-3).astype(np.float32)
    sw = (rng.random(n) * 2.0 ** rng.integers(-20, 0, n)).astype(np.float32)
    bias = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    if tile == 384 and k % 128:
        # the 384 x 192 tile exists only for 128-byte K-steps: refused, nothing launched
        with pytest.raises(cr.ConvrotError, match="k % 128"):
            cr.convrot_gemm_int8_per_channel(
                torch.from_numpy(xq).to(DEV), _dev_f32(sx), torch.from_numpy(wq).to(DEV),
                _dev_f32(sw), None, want_acc=True, tile=tile)
        return
    for b in (None, bias):
        y, acc = cr.convrot_gemm_int8_per_channel(
            torch.from_numpy(xq).to(DEV), _dev_f32(sx), torch.from_numpy(wq).to(DEV),
            _dev_f32(sw), None if b is None else dev_bf16(b), want_acc=True, tile=tile)
        acc_ref = oracle.gemm_int32(xq, wq)
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert np.array_equal(host_bits(y), oracle.epilogue(acc_ref, sw, sx, b))


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
def test_per_channel_linear_bitexact_and_tolerances(layer, g):
    _announce(f"per-channel linear {layer.name} g={g}")
    xb = layer.x()
    wb = _rowscaled(layer.w(), layer.n + 1)
    wq_ref, s_ref = oracle.quantize_weights_per_channel(wb, g, SEED)
    bias_b = synth.f32_to_bf16_bits(
        np.random.default_rng(8).standard_normal(layer.n).astype(np.float32))
    y_ref, _, sx_ref, acc_ref = oracle.linear_int8(xb, wq_ref, s_ref, g, SEED, bias_b)
    x = dev_bf16(xb)
    wq = torch.from_numpy(wq_ref).to(DEV)
    s_w = _dev_f32(s_ref)
    got = host_bits(cr.convrot_linear_int8_per_channel(x, wq, s_w, g, SEED, dev_bf16(bias_b)))
    assert np.array_equal(got, y_ref)
    ref = oracle.linear_int8_reference_f64(acc_ref, s_ref, sx_ref, bias_b)
    assert oracle.rel_frobenius(oracle.bf16_to_f64(got), ref) < 1e-2
    # slicing invariance with per-channel scales
    ws = torch.empty(cr.convrot_linear_int8_workspace_for_rows(37, layer.k), dtype=torch.uint8,
                     device=DEV)
    sliced = cr.convrot_linear_int8_per_channel(x, wq, s_w, g, SEED, dev_bf16(bias_b),
                                                workspace=ws)
    assert np.array_equal(host_bits(sliced), y_ref)
    # the default path with per-channel scales, consumed by a bf16 matmul
    w_hat = cr.convrot_dequant_derotate_per_channel(wq, s_w, g, SEED)
    y_deq = bf16_matmul_nt(x, w_hat)
    ref_deq = oracle.dequant_linear_reference_f64(xb, wq_ref, s_ref, g, SEED)
    assert oracle.rel_frobenius(oracle.bf16_to_f64(host_bits(y_deq)), ref_deq) < 1e-2


def test_per_channel_with_constant_scales_equals_per_tensor():
    """a per-channel vector holding one value reproduces the per-tensor calls"""
    _announce("per-channel constant scales")
    layer, g = synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256
    wq, s_t = cr.convrot_quantize_weights(dev_bf16(layer.w()), g, SEED)
    s_vec = s_t.expand(layer.n).contiguous()
    x = dev_bf16(layer.x())
    assert torch.equal(cr.convrot_linear_int8_per_channel(x, wq, s_vec, g, SEED),
                       cr.convrot_linear_int8(x, wq, s_t, g, SEED))
    assert torch.equal(cr.convrot_dequant_derotate_per_channel(wq, s_vec, g, SEED),
                       cr.convrot_dequant_derotate(wq, s_t, g, SEED))


def test_per_channel_binding_rejects_wrong_scale_length():
    wq = torch.zeros((32, 256), dtype=torch.int8, device=DEV)
    with pytest.raises(ValueError):
        cr.convrot_dequant_derotate_per_channel(wq, torch.ones(31, device=DEV), 256)
    with pytest.raises(cr.ConvrotError) as e:     # 4-byte aligned only
        buf = torch.ones(40, device=DEV)
        cr.convrot_dequant_derotate_per_channel(wq, buf[1:33], 256)
    assert e.value.status_name == "CONVROT_E_MISALIGNED"


# --------------------------------------------------------------------------
# FP16 activations, bias, outputs and W_hat (the *_ex entry points)
# --------------------------------------------------------------------------

def dev_f16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(DEV)


@pytest.mark.parametrize("layer,g", REDUCED, ids=IDS)
def test_f16_quantize_activations_bitexact(layer, g):
    _announce(f"f16 quantize_activations {layer.name} g={g}")
    hb = layer.x(fmt="f16")
    xq, sx = cr.convrot_quantize_activations_ex(dev_f16(hb), g, SEED)
    xq_ref, sx_ref = oracle.quantize_activations(hb, g, SEED, "f16")
    assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("g", GS)
def test_f16_edge_rows(g):
    """the widest spans half allows, zeros, subnormals, max values, ties"""
    _announce(f"f16 edge rows g={g}")
    rng = np.random.default_rng(50 + g)
    k = 512
    rows = [np.zeros(k), np.full(k, -0.0), np.full(k, 65504.0), np.full(k, 2.0 ** -24)]
    r = rng.standard_normal(k) * 2.0 ** rng.integers(-26, 16, k)
    rows.append(np.clip(r, -65504, 65504))
    r = np.zeros(k); r[::64] = 1.0; r[1::64] = 2.0 ** -11; r[2::64] = 2.0 ** -24
    rows.append(r)
    r = rng.standard_normal(k); r[::9] = 2.0 ** -24; r[4::31] = -65504.0
    rows.append(r)
    hb = np.array(rows).astype(np.float16).view(np.uint16)
    xq, sx = cr.convrot_quantize_activations_ex(dev_f16(hb), g, SEED)
    xq_ref, sx_ref = oracle.quantize_activations(hb, g, SEED, "f16")
    assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("tile", [0, 128, 192, 256, 384])
@pytest.mark.parametrize("m,n,k", [(1, 16, 64), (257, 272, 320), (300, 400, 1152)])
def test_f16_gemm_shapes(m, n, k, tile, per_channel):
    _announce(f"f16 gemm {m}x{n}x{k} tile={tile} pc={per_channel}")
    rng = np.random.default_rng(m + 3 * n)
    xq = rng.integers(-127, 128, (m, k)).astype(np.int8)
    wq = rng.integers(-127, 128, (n, k)).astype(np.int8)
    sx = (rng.random(m) * 1e-2).astype(np.float32)
    sx[0] = np.float32(50.0)          # row 0 overflows half in places: inf
    sw = (rng.random(n) * 1e-2).astype(np.float32) if per_channel else np.float32(4e-3)
    bias = synth.f32_to_f16_bits(rng.standard_normal(n).astype(np.float32))
    if tile == 384 and k % 128:
        # the 384 x 192 tile exists only for 128-byte K-steps: refused, nothing launched
        with pytest.raises(cr.ConvrotError, match="k % 128"):
            cr.convrot_gemm_int8_ex(
                torch.from_numpy(xq).to(DEV), torch.from_numpy(sx).to(DEV),
                torch.from_numpy(wq).to(DEV),
                torch.from_numpy(np.atleast_1d(sw).astype(np.float32)).to(DEV), None,
                per_channel=per_channel, dtype=torch.float16, want_acc=True, tile=tile)
        return
    for b in (None, bias):
        y, acc = cr.convrot_gemm_int8_ex(
            torch.from_numpy(xq).to(DEV), torch.from_numpy(sx).to(DEV),
            torch.from_numpy(wq).to(DEV),
            torch.from_numpy(np.atleast_1d(sw).astype(np.float32)).to(DEV),
            None if b is None else dev_f16(b), per_channel=per_channel, dtype=torch.float16,
            want_acc=True, tile=tile)
        acc_ref = oracle.gemm_int32(xq, wq)
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert np.array_equal(host_bits(y), oracle.epilogue(acc_ref, sw, sx, b, "f16"))


@pytest.mark.parametrize("layer,g", REDUCED[:4] + REDUCED[-2:], ids=IDS[:4] + IDS[-2:])
def test_f16_linear_and_dequant(layer, g):
    _announce(f"f16 linear + dequant {layer.name} g={g}")
    hb = layer.x(fmt="f16")
    for per_channel in (False, True):
        wb = layer.w()
        wq_ref, s_ref = (oracle.quantize_weights_per_channel if per_channel
                         else oracle.quantize_weights)(wb, g, SEED)
        bias = synth.f32_to_f16_bits(
            np.random.default_rng(9).standard_normal(layer.n).astype(np.float32))
        y_ref, _, sx_ref, acc_ref = oracle.linear_int8(hb, wq_ref, s_ref, g, SEED, bias, "f16")
        wq = torch.from_numpy(wq_ref).to(DEV)
        s_w = torch.from_numpy(np.atleast_1d(s_ref).astype(np.float32)).to(DEV)
        x = dev_f16(hb)
        got = host_bits(cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED, dev_f16(bias),
                                                  per_channel=per_channel))
        assert np.array_equal(got, y_ref), per_channel
        ref = oracle.linear_int8_reference_f64(acc_ref, s_ref, sx_ref, bias, "f16")
        assert oracle.rel_frobenius(oracle.f16_to_f64(got), ref) < 1e-2
        w_hat = cr.convrot_dequant_derotate_ex(wq, s_w, g, SEED, per_channel=per_channel,
                                               out_dtype=torch.float16)
        assert np.array_equal(host_bits(w_hat),
                              oracle.dequant_derotate(wq_ref, s_ref, g, SEED, "f16"))
        # the default path in half, consumed by a half matmul
        y_deq = bf16_matmul_nt(x, w_hat)
        ref_deq = oracle.dequant_linear_reference_f64(hb, wq_ref, s_ref, g, SEED, dtype="f16")
        assert oracle.rel_frobenius(oracle.f16_to_f64(host_bits(y_deq)), ref_deq) < 1e-2


def test_ex_bf16_matches_named_entry_points():
    """the general forms with bf16 reproduce the named calls bit for bit"""
    _announce("ex bf16 vs named")
    layer, g = synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256
    x = dev_bf16(layer.x())
    wq, s_w = cr.convrot_quantize_weights(dev_bf16(layer.w()), g, SEED)
    assert torch.equal(cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED),
                       cr.convrot_linear_int8(x, wq, s_w, g, SEED))
    xq1, sx1 = cr.convrot_quantize_activations_ex(x, g, SEED)
    xq2, sx2 = cr.convrot_quantize_activations(x, g, SEED)
    assert torch.equal(xq1, xq2) and torch.equal(sx1, sx2)
    assert torch.equal(cr.convrot_dequant_derotate_ex(wq, s_w, g, SEED),
                       cr.convrot_dequant_derotate(wq, s_w, g, SEED))


# --------------------------------------------------------------------------
# Seeded random shapes through the whole forward (every format and scale
# granularity), against the oracle
# --------------------------------------------------------------------------

def _random_cases(count=12, seed=77):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        g = int(rng.choice(GS))
        k = int(rng.integers(1, 13)) * max(64, g)
        n = int(rng.integers(1, 40)) * 16
        m = int(rng.integers(1, 700))
        cases.append((m, n, k, g, bool(rng.integers(0, 2)), str(rng.choice(["bf16", "f16"])),
                      int(rng.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("m,n,k,g,pc,fmt,seed", _random_cases())
def test_random_shapes_linear(m, n, k, g, pc, fmt, seed):
    _announce(f"random linear m={m} n={n} k={k} g={g} pc={pc} {fmt}")
    rng = np.random.default_rng(seed)
    x32 = (rng.standard_normal((m, k)) * np.where(rng.random(k) < 0.01, 20.0, 1.0)).astype(np.float32)
    w32 = (rng.standard_normal((n, k)) * 0.02 * 2.0 ** rng.integers(-6, 7, n)[:, None]).astype(np.float32)
    b32 = rng.standard_normal(n).astype(np.float32)
    enc = synth.f32_to_f16_bits if fmt == "f16" else synth.f32_to_bf16_bits
    dtype = torch.float16 if fmt == "f16" else torch.bfloat16
    xb, wb, bb = enc(x32), synth.f32_to_bf16_bits(w32), enc(b32)
    wq_ref, s_ref = (oracle.quantize_weights_per_channel if pc else oracle.quantize_weights)(
        wb, g, SEED)
    y_ref = oracle.linear_int8(xb, wq_ref, s_ref, g, SEED, bb, fmt)[0]
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(DEV)
    q = cr.convrot_quantize_weights_per_channel if pc else cr.convrot_quantize_weights
    wq, s_w = q(dev_bf16(wb), g, SEED)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert np.array_equal(f32_bits(s_w.cpu().numpy()), f32_bits(np.atleast_1d(s_ref)))
    # a workspace of a random number of rows: random slicing as well
    rows = int(rng.integers(1, m + 1))
    ws = torch.empty(cr.convrot_linear_int8_workspace_for_rows(rows, k), dtype=torch.uint8,
                     device=DEV)
    y = cr.convrot_linear_int8_ex(to_dev(xb), wq, s_w, g, SEED, to_dev(bb), per_channel=pc,
                                  workspace=ws)
    assert np.array_equal(host_bits(y), y_ref)
