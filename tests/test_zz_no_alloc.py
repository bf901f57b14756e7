"""The forward that allocates nothing (convrot_linear_int8_noalloc) against
the workspace forward it varies (convrot_linear_int8_ex), bit for bit, through
the C ABI: two calls in a row, the second with a smaller input, in each
format / scale / bias combination; the larger calls need several slices of the
library's 64 MiB per-device scratch, GELU-tailed rows take the deferred-row
pass through it. The call must not allocate through torch either."""

import gc

import numpy as np
import pytest
import torch

import int8_gemm_amd as cr
import synth

pytestmark = pytest.mark.gpu

SEED = synth.ROT_SEED
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    cr.load_library()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy()


def _inputs(layer, dtype, per_channel, with_bias):
    fmt = "f16" if dtype == torch.float16 else "bf16"
    x = torch.from_numpy(layer.x(fmt=fmt).view(np.int16)).view(dtype).to(DEV)
    w = torch.from_numpy(layer.w().view(np.int16)).view(torch.bfloat16).to(DEV)
    q = cr.convrot_quantize_weights_per_channel if per_channel else cr.convrot_quantize_weights
    wq, s_w = q(w, 256, SEED)
    bias = None
    if with_bias:
        bias = torch.from_numpy(np.random.default_rng(3).standard_normal(layer.n)
                                .astype(np.float32)).to(dtype).to(DEV)
    return x, wq, s_w, bias


# (large layer, smaller layer): the large ones exceed one scratch slice
PAIRS = [
    (synth.WAN_FFN_UP.scaled(m=20000, n=512), synth.ZIMAGE_ATTN.scaled(m=300, n=272)),
    (synth.WAN_FFN_DOWN.scaled(m=9000, n=256), synth.FLUX_MLP_DOWN.scaled(m=600, n=256)),
]
VARIANTS = [(torch.bfloat16, False, False), (torch.float16, True, True),
            (torch.bfloat16, True, True)]


def _check_layer(layer, dtype, per_channel, with_bias):
    print(f"noalloc {layer.name} {dtype} pc={per_channel} bias={with_bias}", flush=True)
    x, wq, s_w, bias = _inputs(layer, dtype, per_channel, with_bias)
    want = cr.convrot_linear_int8_ex(x, wq, s_w, 256, SEED, bias, per_channel=per_channel)
    out = torch.full_like(want, float("nan"))
    torch.cuda.synchronize()
    # nothing allocated through torch: the garbage collector stays off around
    # the call, so that it cannot free an earlier test's tensors meanwhile
    gc.collect()
    before = torch.cuda.memory_allocated()
    gc.disable()
    try:
        cr.convrot_linear_int8_noalloc(x, wq, s_w, 256, SEED, bias, per_channel=per_channel,
                                       out=out)
        after = torch.cuda.memory_allocated()
    finally:
        gc.enable()
    assert after == before
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(want)), layer.name


@pytest.mark.parametrize("dtype,per_channel,with_bias", VARIANTS,
                         ids=["bf16", "f16-pc-bias", "bf16-pc-bias"])
@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_equals_workspace_forward(pair, dtype, per_channel, with_bias):
    for layer in PAIRS[pair]:  # the second call has the smaller input
        _check_layer(layer, dtype, per_channel, with_bias)


def test_noalloc_slices_follow_the_scratch():
    """Rows per slice: floor(64 MiB / (k + 4)), in whole 256-row tiles; a
    20000 x 5120 input needs two slices, and the result does not depend on it
    (a workspace of exactly one such slice gives the same bits)."""
    layer = PAIRS[0][0]
    x, wq, s_w, _ = _inputs(layer, torch.bfloat16, False, False)
    k = layer.k
    rows = cr.NOALLOC_SCRATCH_BYTES // (k + 4)
    rows -= rows % 256
    assert rows < layer.m
    ws = torch.empty(cr.convrot_linear_int8_workspace_for_rows(rows, k), dtype=torch.uint8,
                     device=DEV)
    want = cr.convrot_linear_int8(x, wq, s_w, 256, SEED, workspace=ws)
    got = cr.convrot_linear_int8_noalloc(x, wq, s_w, 256, SEED)
    assert np.array_equal(_bits(got), _bits(want))
