"""GPU parity at the full workload shapes, in the launch configurations the
benchmark times (automatic GEMM tile, convrot_linear_int8 with its default
workspace, i.e. token slices of at most 2N rows).

The GPU computes every output. The oracle then recomputes what it can one
row at a time: the weight quantization in full (it is cheap), and sampled
weight rows (dequant) and token rows (activation quantization and the whole
int8 forward). A row's result depends on no other row, so a sampled row is
the same computation as in the full call. Sampled rows include the first and
last rows, the rows around GEMM tile edges and around token-slice edges.
Over all token rows, sampled output columns of the int32 accumulator are
compared with exact float64 dot products of the GPU's own int8 operands."""

import numpy as np
import pytest
import torch

import int8_gemm_amd as cr
import oracle
import synth

pytestmark = pytest.mark.gpu

SEED = synth.ROT_SEED
DEV = "cuda:0"

FULL = [
    (synth.ZIMAGE_ATTN, 256),
    (synth.FLUX_MLP_UP, 256),
    (synth.FLUX_MLP_DOWN, 256),
    (synth.WAN_FFN_UP, 256),
    (synth.WAN_FFN_DOWN, 256),
] + [(synth.QKV_SWEEP, g) for g in synth.GROUP_SIZES]
IDS = [f"{layer.name}-g{g}" for layer, g in FULL]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    cr.load_library()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def sample_rows(count: int, extra=(), n_random: int = 8, seed: int = 11) -> np.ndarray:
    """First/last rows, rows at 128/192/256/384-row tile edges (including the
    last, ragged tile), the given extra rows and a few random ones."""
    rows = {0, 1, 127, 128, 191, 192, 255, 256, 383, 384, count - 2, count - 1}
    for t in (128, 192, 256, 384):
        last = (count - 1) // t * t
        rows.update({last - 1, last})
    rows.update(extra)
    rows.update(np.random.default_rng(seed).integers(0, count, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < count))


@pytest.mark.parametrize("layer,g", FULL, ids=IDS)
def test_fullsize(layer, g):
    m, n, k = layer.m, layer.n, layer.k
    print(f"full-size {layer.name} g={g}: inputs", flush=True)
    wb, xb = layer.w(), layer.x()

    # weight quantization: every element, bit-exact
    print(f"full-size {layer.name} g={g}: quantize_weights", flush=True)
    wq, s_w = cr.convrot_quantize_weights(dev_bf16(wb), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
    assert f32_bits(s_w.cpu().numpy())[0] == f32_bits(s_ref)
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    del wb

    # dequant + derotate: sampled weight rows, bit-exact
    print(f"full-size {layer.name} g={g}: dequant", flush=True)
    w_hat = cr.convrot_dequant_derotate(wq, s_w, g, SEED)
    nrows = sample_rows(n)
    assert np.array_equal(host_bits(w_hat[torch.from_numpy(nrows).to(DEV)]),
                          oracle.dequant_derotate(wq_ref[nrows], s_ref, g, SEED))
    del w_hat

    # activations: sampled token rows, bit-exact
    print(f"full-size {layer.name} g={g}: quantize_activations", flush=True)
    x = dev_bf16(xb)
    xq, s_x = cr.convrot_quantize_activations(x, g, SEED)
    slice_rows = 2 * n  # default workspace slices tokens at most 2N rows high
    rows = sample_rows(m, extra=(slice_rows - 1, slice_rows, 2 * slice_rows - 1, 2 * slice_rows))
    rows_t = torch.from_numpy(rows).to(DEV)
    xq_ref, sx_ref = oracle.quantize_activations(xb[rows], g, SEED)
    assert np.array_equal(f32_bits(s_x[rows_t].cpu().numpy()), f32_bits(sx_ref))
    assert np.array_equal(xq[rows_t].cpu().numpy(), xq_ref)

    # the int8 forward with the default workspace: sampled rows, every column
    print(f"full-size {layer.name} g={g}: linear_int8", flush=True)
    y = cr.convrot_linear_int8(x, wq, s_w, g, SEED)
    y_ref = oracle.epilogue(oracle.gemm_int32(xq_ref, wq_ref), s_ref, sx_ref)
    assert np.array_equal(host_bits(y[rows_t]), y_ref)
    del x, y

    # the GEMM over every token row: sampled accumulator columns, exact
    print(f"full-size {layer.name} g={g}: gemm columns", flush=True)
    y2, acc = cr.convrot_gemm_int8(xq, s_x, wq, s_w, want_acc=True)
    cols = sample_rows(n, n_random=4)
    cols_t = torch.from_numpy(cols).to(DEV)
    got = acc[:, cols_t].cpu().numpy()
    wcols = wq_ref[cols].astype(np.float64).T
    for r0 in range(0, m, 4096):  # exact: integer partial sums below 2^53
        want = xq[r0:r0 + 4096].cpu().numpy().astype(np.float64) @ wcols
        assert np.array_equal(got[r0:r0 + 4096], want.astype(np.int64)), f"rows {r0}.."
    # and the epilogue of the same launch on those columns, at the sampled
    # token rows (oracle operands only)
    y_cols = oracle.epilogue(oracle.gemm_int32(xq_ref, wq_ref[cols]), s_ref, sx_ref)
    assert np.array_equal(host_bits(y2[rows_t][:, cols_t].contiguous()), y_cols)


def test_dequant_stack_layers_0_and_59():
    """The streamed stack: each stack weight quantized once and copied into 60
    distinct device buffers; layers 0 and 59 dequantize bit-exactly (the same
    launch the benchmark's stack pass makes, per buffer)."""
    g = 256
    for lay in (synth.STACK_SQUARE, synth.STACK_WIDE):
        print(f"dequant stack {lay.name}", flush=True)
        wb = lay.w()
        wq, s_w = cr.convrot_quantize_weights(dev_bf16(wb), g, SEED)
        wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
        assert f32_bits(s_w.cpu().numpy())[0] == f32_bits(s_ref)
        copies = [wq.clone() for _ in range(synth.STACK_LAYERS)]
        want = oracle.dequant_derotate(wq_ref, s_ref, g, SEED)
        for li in (0, synth.STACK_LAYERS - 1):
            out = cr.convrot_dequant_derotate(copies[li], s_w, g, SEED)
            assert np.array_equal(host_bits(out), want), li
        del copies


def test_fullsize_per_channel_zimage_attn():
    """Per-channel scales at the full Z-Image attention shape: the weight
    quantization in full, the dequant on sampled weight rows, the int8 forward
    on sampled token rows, every column."""
    layer, g = synth.ZIMAGE_ATTN, 256
    m, n = layer.m, layer.n
    print(f"full-size per-channel {layer.name}: quantize_weights", flush=True)
    e = np.random.default_rng(5).integers(-12, 13, n)
    wb = synth.f32_to_bf16_bits((oracle.bf16_to_f64(layer.w()) * 2.0 ** e[:, None])
                                .astype(np.float32))
    wq, s_w = cr.convrot_quantize_weights_per_channel(dev_bf16(wb), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights_per_channel(wb, g, SEED)
    assert np.array_equal(f32_bits(s_w.cpu().numpy()), f32_bits(s_ref))
    assert np.array_equal(wq.cpu().numpy(), wq_ref)

    print(f"full-size per-channel {layer.name}: dequant", flush=True)
    nrows = sample_rows(n, n_random=24)
    w_hat = cr.convrot_dequant_derotate_per_channel(wq, s_w, g, SEED)
    assert np.array_equal(host_bits(w_hat[torch.from_numpy(nrows).to(DEV)]),
                          oracle.dequant_derotate(wq_ref[nrows], s_ref[nrows], g, SEED))
    del w_hat

    print(f"full-size per-channel {layer.name}: linear_int8", flush=True)
    xb = layer.x()
    y = cr.convrot_linear_int8_per_channel(dev_bf16(xb), wq, s_w, g, SEED)
    rows = sample_rows(m, extra=(2 * n - 1, 2 * n))
    xq_ref, sx_ref = oracle.quantize_activations(xb[rows], g, SEED)
    y_ref = oracle.epilogue(oracle.gemm_int32(xq_ref, wq_ref), s_ref, sx_ref)
    assert np.array_equal(host_bits(y[torch.from_numpy(rows).to(DEV)]), y_ref)
