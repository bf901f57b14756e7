"""GPU: forwards enqueued on several streams at once. The library keeps no
state between calls (every buffer a call writes is its own workspace or
output), so layers running concurrently on different streams, the deferred
GELU-tailed rows among them, must give bit for bit what each gives alone."""

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


def dev16(bits: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(DEV)


def test_concurrent_streams_match_sequential():
    # an ordinary layer, a GELU-tailed one (some of its rows take the deferred pass)
    # with per-channel scales, and a half-precision one with g = 16
    specs = [(synth.ZIMAGE_ATTN.scaled(m=1000, n=512), 256, False, "bf16"),
             (synth.FLUX_MLP_DOWN.scaled(m=600, n=384), 256, True, "bf16"),
             (synth.QKV_SWEEP.scaled(m=900, n=640), 16, False, "f16")]
    layers = []
    for layer, g, pc, fmt in specs:
        dtype = torch.float16 if fmt == "f16" else torch.bfloat16
        x = dev16(layer.x(fmt=fmt), dtype)
        q = cr.convrot_quantize_weights_per_channel if pc else cr.convrot_quantize_weights
        wq, s_w = q(dev16(layer.w()), g, SEED)
        layers.append((layer.name, x, wq, s_w, g, pc))
    # each layer alone, on the default stream
    want = [cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED, per_channel=pc)
            for _, x, wq, s_w, g, pc in layers]
    torch.cuda.synchronize()
    reps = 4
    streams = [torch.cuda.Stream(device=DEV) for _ in layers]  # default priority
    work = [torch.empty(cr.convrot_linear_int8_workspace_size(x.shape[0], wq.shape[0],
                                                              x.shape[1]),
                        dtype=torch.uint8, device=DEV) for _, x, wq, _, _, _ in layers]
    outs = [[torch.full_like(y, float("nan")) for _ in range(reps)] for y in want]
    torch.cuda.synchronize()
    for r in range(reps):
        for i, (name, x, wq, s_w, g, pc) in enumerate(layers):
            print(f"concurrent streams rep={r} layer={name} g={g} pc={pc}", flush=True)
            with torch.cuda.stream(streams[i]):
                cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED, per_channel=pc,
                                          workspace=work[i], out=outs[i][r])
    torch.cuda.synchronize()
    for i, (name, *_rest) in enumerate(layers):
        ref = want[i].view(torch.int16)
        for r in range(reps):
            assert torch.equal(outs[i][r].view(torch.int16), ref), (name, r)
