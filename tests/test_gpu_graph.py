"""GPU: the int8 forward under HIP graph capture. The entry points enqueue
kernels only (no memsets, no allocation, no host synchronisation), so a
serving loop can capture a step into a graph and replay it. The captured
step is replayed several times, with eager work and synchronisations in
between, and every replay must equal the eager result bit for bit."""

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


def dev16(bits, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(DEV)


@pytest.mark.parametrize("per_channel,fmt", [(False, "bf16"), (True, "f16")])
def test_captured_linear_replays_equal_eager(per_channel, fmt):
    print(f"graph capture pc={per_channel} {fmt}", flush=True)
    layer, g = synth.ZIMAGE_ATTN.scaled(m=1030, n=512), 256
    dtype = torch.float16 if fmt == "f16" else torch.bfloat16
    xb = layer.x(fmt=fmt)
    xs = [dev16(xb, dtype), dev16(xb[::-1].copy(), dtype)]
    q = cr.convrot_quantize_weights_per_channel if per_channel else cr.convrot_quantize_weights
    wq, s_w = q(dev16(layer.w()), g, SEED)
    b32 = np.random.default_rng(4).standard_normal(layer.n).astype(np.float32)
    bias = dev16(synth.f32_to_f16_bits(b32) if fmt == "f16" else synth.f32_to_bf16_bits(b32),
                 dtype)
    # a small workspace: several token slices per step
    ws = torch.empty(cr.convrot_linear_int8_workspace_for_rows(300, layer.k), dtype=torch.uint8,
                     device=DEV)
    ys = [torch.empty((layer.m, layer.n), dtype=dtype, device=DEV) for _ in xs]

    def step():
        for x, y in zip(xs, ys):
            cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED, bias, per_channel=per_channel,
                                      workspace=ws, out=y)

    step()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for y in ys:
            y.fill_(0)
        cr.convrot_linear_int8(dev16(synth.TINY.x()), *cr.convrot_quantize_weights(
            dev16(synth.TINY.w()), 256, SEED), 256, SEED)        # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(ys, eager)):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), (rep, i)
