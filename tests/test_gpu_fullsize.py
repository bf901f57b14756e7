"""GPU parity at the full workload shapes, every output compared, in the
launch configurations the benchmark times (automatic GEMM tile,
convrot_linear_int8 with its default workspace, i.e. token slices of at most
2N rows).

Per workload (pytest runs all tests of one workload before the next, so the
GPU results and the oracle's are computed once):

* weight quantization: every element of Wq and s_w;
* dequant + derotate: every row of W_hat;
* activation quantization: every row of xq and s_x (the oracle in chunks of
  4096 token rows; a row's result depends on no other row);
* the int8 forward: every row and column of y;
* the GEMM alone: the int32 accumulator at one row of every 128-row band and
  one column of every 128-column band (so every output tile of every block
  tile size is hit), and its y at those rows with each forced block tile.
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
CHUNK = 4096

FULL = [
    (synth.ZIMAGE_ATTN, 256),
    (synth.FLUX_MLP_UP, 256),
    (synth.FLUX_MLP_DOWN, 256),
    (synth.WAN_FFN_UP, 256),
    (synth.WAN_FFN_DOWN, 256),
] + [(synth.QKV_SWEEP, g) for g in synth.GROUP_SIZES]
IDS = [f"{layer.name.split()[0]}-g{g}" for layer, g in FULL]


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def band_samples(count: int, band: int = 128, salt: int = 37) -> np.ndarray:
    """One index in every band of `band` indices (its offset varies from band
    to band), plus the first and the last index."""
    idx = {0, count - 1}
    for b in range((count + band - 1) // band):
        lo, hi = b * band, min(count, (b + 1) * band)
        idx.add(lo + (b * salt + 5) % (hi - lo))
    return np.array(sorted(idx))


class Workload:
    """GPU results and oracle results of one workload, computed on first use
    and kept for the workload's other tests (so any test also runs alone)."""

    def __init__(self, layer, g):
        self.layer, self.g = layer, g
        self.name = f"{layer.name} g={g}"

    def weights(self):
        if not hasattr(self, "wq"):
            wb = self.layer.w()
            self.wq, self.s_w = cr.convrot_quantize_weights(dev_bf16(wb), self.g, SEED)
            self.wq_ref, self.s_ref = oracle.quantize_weights(wb, self.g, SEED)
        return self

    def activations(self):
        if not hasattr(self, "xq"):
            xb = self.layer.x()
            self.x = dev_bf16(xb)
            self.xq, self.s_x = cr.convrot_quantize_activations(self.x, self.g, SEED)
            self.xq_ref = np.empty((self.layer.m, self.layer.k), dtype=np.int8)
            self.sx_ref = np.empty(self.layer.m, dtype=np.float32)
            for r0 in range(0, self.layer.m, CHUNK):
                self.xq_ref[r0:r0 + CHUNK], self.sx_ref[r0:r0 + CHUNK] = \
                    oracle.quantize_activations(xb[r0:r0 + CHUNK], self.g, SEED)
        return self


@pytest.fixture(scope="module", params=FULL, ids=IDS)
def wl(request):
    cr.load_library()
    w = Workload(*request.param)
    yield w
    del w
    torch.cuda.empty_cache()


def _say(wl, what):
    print(f"full-size {wl.name}: {what}", flush=True)


def test_weights_every_element(wl):
    _say(wl, "quantize_weights")
    wl.weights()
    assert f32_bits(wl.s_w.cpu().numpy())[0] == f32_bits(wl.s_ref)
    assert np.array_equal(wl.wq.cpu().numpy(), wl.wq_ref)


def test_dequant_every_row(wl):
    _say(wl, "dequant")
    wl.weights()
    w_hat = cr.convrot_dequant_derotate(wl.wq, wl.s_w, wl.g, SEED)
    n = wl.layer.n
    step = max(1, (CHUNK * 4096) // wl.layer.k)
    for r0 in range(0, n, step):
        want = oracle.dequant_derotate(wl.wq_ref[r0:r0 + step], wl.s_ref, wl.g, SEED)
        assert np.array_equal(host_bits(w_hat[r0:r0 + step]), want), f"weight rows {r0}.."
    del w_hat


def test_act_quant_every_row(wl):
    _say(wl, "quantize_activations")
    wl.activations()
    xq_h, sx_h = wl.xq.cpu().numpy(), wl.s_x.cpu().numpy()
    for r0 in range(0, wl.layer.m, CHUNK):
        assert np.array_equal(f32_bits(sx_h[r0:r0 + CHUNK]), f32_bits(wl.sx_ref[r0:r0 + CHUNK])), \
            f"s_x rows {r0}.."
        assert np.array_equal(xq_h[r0:r0 + CHUNK], wl.xq_ref[r0:r0 + CHUNK]), f"xq rows {r0}.."


def _oracle_y(wl, r0, r1):
    acc = oracle.gemm_int32(wl.xq_ref[r0:r1], wl.wq_ref)
    return oracle.epilogue(acc, wl.s_ref, wl.sx_ref[r0:r1])


def test_linear_every_row(wl):
    _say(wl, "linear_int8 (default workspace)")
    wl.weights().activations()
    y = cr.convrot_linear_int8(wl.x, wl.wq, wl.s_w, wl.g, SEED)
    step = max(256, (CHUNK * 4096) // wl.layer.n)
    for r0 in range(0, wl.layer.m, step):
        assert np.array_equal(host_bits(y[r0:r0 + step]), _oracle_y(wl, r0, r0 + step)), \
            f"y rows {r0}.."
    del y


def test_gemm_every_tile(wl):
    _say(wl, "gemm: accumulator at every 128-band, y at those rows per tile")
    wl.weights().activations()
    m, n = wl.layer.m, wl.layer.n
    rows, cols = band_samples(m), band_samples(n, salt=53)
    rows_t, cols_t = torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)
    y_want = oracle.epilogue(oracle.gemm_int32(wl.xq_ref[rows], wl.wq_ref), wl.s_ref,
                             wl.sx_ref[rows])
    acc_want = oracle.gemm_int32(wl.xq_ref[rows], wl.wq_ref[cols])
    y, acc = cr.convrot_gemm_int8(wl.xq, wl.s_x, wl.wq, wl.s_w, want_acc=True)
    assert np.array_equal(acc[rows_t][:, cols_t].cpu().numpy(), acc_want)
    assert np.array_equal(host_bits(y[rows_t]), y_want)
    del acc
    for tile in (128, 192, 256, 384):
        if tile == 384 and wl.layer.k % 128:
            continue
        y, _ = cr.convrot_gemm_int8(wl.xq, wl.s_x, wl.wq, wl.s_w, y=y, tile=tile)
        assert np.array_equal(host_bits(y[rows_t]), y_want), tile
    del y


def test_dequant_stack_layers_0_and_59():
    """The streamed stack: each stack weight quantized once and copied into 60
    distinct device buffers; layers 0 and 59 dequantize bit-exactly (the same
    launch the benchmark's stack pass makes, per buffer)."""
    cr.load_library()
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
    """Per-channel scales at the full Z-Image attention shape, every output:
    the weight quantization, the dequant, the int8 forward."""
    cr.load_library()
    layer, g = synth.ZIMAGE_ATTN, 256
    n = layer.n
    print(f"full-size per-channel {layer.name}: quantize_weights", flush=True)
    e = np.random.default_rng(5).integers(-12, 13, n)
    wb = synth.f32_to_bf16_bits((oracle.bf16_to_f64(layer.w()) * 2.0 ** e[:, None])
                                .astype(np.float32))
    wq, s_w = cr.convrot_quantize_weights_per_channel(dev_bf16(wb), g, SEED)
    wq_ref, s_ref = oracle.quantize_weights_per_channel(wb, g, SEED)
    assert np.array_equal(f32_bits(s_w.cpu().numpy()), f32_bits(s_ref))
    assert np.array_equal(wq.cpu().numpy(), wq_ref)

    print(f"full-size per-channel {layer.name}: dequant", flush=True)
    w_hat = cr.convrot_dequant_derotate_per_channel(wq, s_w, g, SEED)
    assert np.array_equal(host_bits(w_hat), oracle.dequant_derotate(wq_ref, s_ref, g, SEED))
    del w_hat

    print(f"full-size per-channel {layer.name}: linear_int8", flush=True)
    xb = layer.x()
    y = cr.convrot_linear_int8_per_channel(dev_bf16(xb), wq, s_w, g, SEED)
    xq_ref, sx_ref = oracle.quantize_activations(xb, g, SEED)
    y_ref = oracle.epilogue(oracle.gemm_int32(xq_ref, wq_ref), s_ref, sx_ref)
    assert np.array_equal(host_bits(y), y_ref)
