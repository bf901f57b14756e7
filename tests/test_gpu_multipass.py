"""Every pass of the persistent grids against the oracle, element by element.

The act-quant kernel, the exact kernel and the dequant walk their work in
persistent workgroups, each taking batch i, i + grid, i + 2 grid, ... with
the next batch prefetched into registers and per-batch LDS slots used
round-robin; after its last batch an act-quant workgroup resolves the rows it
deferred (batches marked in an LDS bitmap of 2048 passes, later ones by one
flag). At the reduced test shapes one pass covers everything, so:

* the first tests shrink the grids through convrot_set_compute_units (a
  process-wide test hook; sizing changes speed, never results) until every
  workgroup walks many batches, and compare every output with the oracle;
* the last tests use the device's own grid at shapes large enough for
  several passes (checked with convrot_plan_launch), compared in full.
"""

import numpy as np
import pytest
import torch

import int8_gemm_amd as cr
import oracle
import synth

pytestmark = pytest.mark.gpu

SEED = synth.ROT_SEED
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    cr.load_library()
    yield
    cr.convrot_set_compute_units(0)


@pytest.fixture
def few_cus(request):
    cr.convrot_set_compute_units(request.param)
    yield request.param
    cr.convrot_set_compute_units(0)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


CASES = [
    (synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256),
    (synth.FLUX_MLP_DOWN.scaled(m=40, n=256), 256),   # GELU tails: deferred rows
    (synth.WAN_FFN_UP.scaled(m=130, n=400), 256),
    (synth.QKV_SWEEP.scaled(m=260, n=288), 4),
    (synth.QKV_SWEEP.scaled(m=260, n=288), 16),
    (synth.QKV_SWEEP.scaled(m=260, n=288), 64),
]
IDS = [f"{l.name}-g{g}" for l, g in CASES]


@pytest.mark.parametrize("few_cus", [1, 3], indirect=True)
@pytest.mark.parametrize("layer,g", CASES, ids=IDS)
def test_small_grids_every_output(few_cus, layer, g):
    m, n, k = layer.m, layer.n, layer.k
    plans = {kern: cr.convrot_plan_launch(kern, m=m, n=n, k=k, g=g)
             for kern in ("act_quant", "act_quant_deferred", "exact")}
    plans["dequant"] = cr.convrot_plan_launch("dequant", n=n, k=k, g=g)
    assert all(p["compute_units"] == few_cus for p in plans.values())
    print(f"multipass cus={few_cus} {layer.name} g={g}: passes "
          + ", ".join(f"{kk} {p['passes']}" for kk, p in plans.items()), flush=True)
    assert plans["act_quant"]["passes"] >= 4 and plans["exact"]["passes"] >= 4
    xb, wb = layer.x(), layer.w()
    # weights: exact kernel, two per-tensor passes over every row
    wq, s_w = cr.convrot_quantize_weights(dev_bf16(wb), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
    assert f32_bits(s_w.cpu().numpy())[0] == f32_bits(s_ref)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    # dequant
    w_hat = cr.convrot_dequant_derotate(wq, s_w, g, SEED)
    assert np.array_equal(host_bits(w_hat), oracle.dequant_derotate(wq_ref, s_ref, g, SEED))
    # activations: fast kernel + deferred pass, and the exact kernel alone
    xq_ref, sx_ref = oracle.quantize_activations(xb, g, SEED)
    x = dev_bf16(xb)
    for fn in (cr.convrot_quantize_activations, cr.convrot_quantize_activations_exact):
        xq, sx = fn(x, g, SEED)
        assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref)), fn.__name__
        assert np.array_equal(xq.cpu().numpy(), xq_ref), fn.__name__
    # the forward (its GEMM tile chosen for the small CU count)
    y = cr.convrot_linear_int8(x, wq, s_w, g, SEED)
    acc_ref = oracle.gemm_int32(xq_ref, wq_ref)
    assert np.array_equal(host_bits(y), oracle.epilogue(acc_ref, s_ref, sx_ref))


@pytest.mark.parametrize("few_cus", [2], indirect=True)
def test_small_grids_per_channel_and_f16(few_cus):
    layer, g = synth.ZIMAGE_ATTN.scaled(m=200, n=256), 256
    xb, wb = layer.x(), layer.w()
    wq, s_w = cr.convrot_quantize_weights_per_channel(dev_bf16(wb), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights_per_channel(wb, g, SEED)
    assert np.array_equal(f32_bits(s_w.cpu().numpy()), f32_bits(s_ref))
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    w_hat = cr.convrot_dequant_derotate_per_channel(wq, s_w, g, SEED)
    assert np.array_equal(host_bits(w_hat), oracle.dequant_derotate(wq_ref, s_ref, g, SEED))
    hb = layer.x(fmt="f16")
    xh = torch.from_numpy(hb.view(np.int16)).view(torch.float16).to(DEV)
    xq, sx = cr.convrot_quantize_activations_ex(xh, g, SEED)
    xq_ref, sx_ref = oracle.quantize_activations(hb, g, SEED, dtype="f16")
    assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    y = cr.convrot_linear_int8_ex(xh, wq, s_w, g, SEED, per_channel=True)
    want = oracle.epilogue(oracle.gemm_int32(xq_ref, wq_ref), s_ref, sx_ref, dtype="f16")
    assert np.array_equal(host_bits(y), want)


def _device_passes(kern, **shape):
    return cr.convrot_plan_launch(kern, **shape)["passes"]


def test_device_grid_fast_kernel_several_passes():
    """6200 token rows at K = 3840: one row per 1-wave block, so the device's
    grid walks each block over several rows (register prefetch of the next
    row, three LDS slots in rotation); every row compared."""
    layer, g = synth.ZIMAGE_ATTN.scaled(m=6200, n=256), 256
    passes = _device_passes("act_quant", m=layer.m, k=layer.k, g=g)
    print(f"device grid: act-quant 6200x3840 passes {passes}", flush=True)
    assert passes >= 3
    xb = layer.x()
    xq, sx = cr.convrot_quantize_activations(dev_bf16(xb), g, SEED)
    xq_ref, sx_ref = oracle.quantize_activations(xb, g, SEED)
    assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)


def test_device_grid_deferred_pass_several_passes():
    """GELU-tailed rows at K = 12288, some of which the fast kernel defers:
    1100 rows give each workgroup of the device's grid several batches, so
    the rows a workgroup resolves after its last batch come from several of
    them; every row compared, and the forward on every row."""
    layer, g = synth.FLUX_MLP_DOWN.scaled(m=1100, n=256), 256
    passes = _device_passes("act_quant_deferred", m=layer.m, k=layer.k, g=g)
    print(f"device grid: deferred 1100x12288 passes {passes}", flush=True)
    assert passes >= 3
    xb, wb = layer.x(), layer.w()
    x = dev_bf16(xb)
    xq, sx = cr.convrot_quantize_activations(x, g, SEED)
    xq_ref, sx_ref = oracle.quantize_activations(xb, g, SEED)
    assert np.array_equal(f32_bits(sx.cpu().numpy()), f32_bits(sx_ref))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
    wq = torch.from_numpy(wq_ref).to(DEV)
    s_w = torch.tensor([s_ref], dtype=torch.float32, device=DEV)
    y = cr.convrot_linear_int8(x, wq, s_w, g, SEED)
    assert np.array_equal(host_bits(y),
                          oracle.epilogue(oracle.gemm_int32(xq_ref, wq_ref), s_ref, sx_ref))


@pytest.mark.parametrize("few_cus", [1], indirect=True)
def test_deferred_rows_past_the_pass_bitmap(few_cus):
    """Rows whose absmax lies below the fast kernel's scaling range (elements
    near 2^-110) are always deferred. At K = 256 on a one-CU grid every
    workgroup walks 2100 batches, so such rows sit in the bitmap's first and
    last words and past it (passes 2048 and later, found by the flag); those
    rows and a sample of the others against the oracle, and no row is left
    with the deferred marker."""
    g, k = 256, 256
    plan = cr.convrot_plan_launch("act_quant", m=1 << 20, k=k, g=g)
    grid, rpb = plan["grid"], plan["rows_per_block"]
    passes = 2100
    m = grid * rpb * passes
    print(f"deferred past the bitmap: grid {grid} rows/block {rpb} m {m}", flush=True)
    assert cr.convrot_plan_launch("act_quant", m=m, k=k, g=g)["passes"] == passes
    rng = np.random.default_rng(7)
    xf = rng.standard_normal((m, k), dtype=np.float32)
    tiny = []
    for b in sorted({0, grid - 1, grid // 2}):
        for p in (0, 5, 31, 32, 2047, 2048, 2049, passes - 1):
            tiny.append((b + p * grid) * rpb + (p % rpb))
    tiny = np.array(sorted(set(tiny)))
    xf[tiny] *= np.float32(2.0 ** -110)
    xb = synth.f32_to_bf16_bits(xf)
    del xf
    xq, sx = cr.convrot_quantize_activations(dev_bf16(xb), g, SEED)
    sx_h = sx.cpu().numpy()
    assert not np.isnan(sx_h).any()
    rest = np.setdiff1d(rng.choice(m, 3000, replace=False), tiny)
    rows = np.concatenate([tiny, rest])
    xq_ref, sx_ref = oracle.quantize_activations(xb[rows], g, SEED)
    assert np.array_equal(f32_bits(sx_h[rows]), f32_bits(sx_ref))
    assert np.array_equal(xq.cpu().numpy()[rows], xq_ref)
    assert (sx_h[tiny] < 2.0 ** -100).all()


@pytest.mark.parametrize("few_cus", [1], indirect=True)
@pytest.mark.parametrize("g", [4, 16, 64, 256])
def test_deferred_rows_every_group_size(few_cus, g):
    """Always-deferred rows (elements near 2^-110) in many batches of a
    one-CU grid, at every group size: the blocks resolve them after their
    batches with the exact row pass of that g; those rows, the rows around
    them and a sample of the rest against the oracle."""
    k = 1024
    plan = cr.convrot_plan_launch("act_quant", m=1 << 20, k=k, g=g)
    grid, rpb = plan["grid"], plan["rows_per_block"]
    m = grid * rpb * 40 + 3                      # a ragged last batch
    print(f"deferred rows g={g}: grid {grid} rows/block {rpb} m {m}", flush=True)
    rng = np.random.default_rng(100 + g)
    xf = rng.standard_normal((m, k), dtype=np.float32)
    tiny = np.unique(np.concatenate([rng.choice(m, 40, replace=False), [0, m - 1]]))
    xf[tiny] *= np.float32(2.0 ** -110)
    xb = synth.f32_to_bf16_bits(xf)
    xq, sx = cr.convrot_quantize_activations(dev_bf16(xb), g, SEED)
    sx_h = sx.cpu().numpy()
    assert not np.isnan(sx_h).any()
    near = np.clip(np.concatenate([tiny - 1, tiny + 1]), 0, m - 1)
    rows = np.unique(np.concatenate([tiny, near, rng.choice(m, 500, replace=False)]))
    xq_ref, sx_ref = oracle.quantize_activations(xb[rows], g, SEED)
    assert np.array_equal(f32_bits(sx_h[rows]), f32_bits(sx_ref))
    assert np.array_equal(xq.cpu().numpy()[rows], xq_ref)
