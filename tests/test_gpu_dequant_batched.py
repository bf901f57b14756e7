"""GPU: dequant + derotate of many weights in one call
(convrot_dequant_derotate_batched), bit for bit against the oracle.

* The 60-layer stack (60 + 60 distinct buffers of the two stack shapes,
  g = 256) in one call of 120 weights, i.e. three launches of up to 48:
  layers 0 and 59 of each shape against the oracle, every other output
  against those on the GPU.
* Mixed lists: weights of different shapes (ragged tile counts, one row,
  k from 64 to 16384) in one call, per group size, per-tensor and
  per-channel scales, bf16 and half outputs, each against the oracle, with
  more weights than one launch holds.
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


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def test_stack_in_one_call():
    g = 256
    wqs, sws, want = [], [], {}
    for lay in (synth.STACK_SQUARE, synth.STACK_WIDE):
        print(f"batched dequant stack {lay.name}", flush=True)
        wb = lay.w()
        wq, s_w = cr.convrot_quantize_weights(dev_bf16(wb), g, SEED)
        wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
        want[lay.name] = oracle.dequant_derotate(wq_ref, s_ref, g, SEED)
        wqs.append([wq.clone() for _ in range(synth.STACK_LAYERS)])
        sws.append(s_w)
    # interleaved as the benchmark's pass runs them: layer i of each shape
    order = [(s, i) for i in range(synth.STACK_LAYERS) for s in range(2)]
    outs = cr.convrot_dequant_derotate_batched([wqs[s][i] for s, i in order],
                                               [sws[s] for s, i in order], g, SEED)
    torch.cuda.synchronize()
    names = [synth.STACK_SQUARE.name, synth.STACK_WIDE.name]
    first = {}
    for (s, i), out in zip(order, outs):
        if i in (0, synth.STACK_LAYERS - 1):
            assert np.array_equal(host_bits(out), want[names[s]]), (names[s], i)
        first.setdefault(s, out)
        assert torch.equal(out.view(torch.int16), first[s].view(torch.int16)), (names[s], i)


# (n, k) of a mixed list: one-row weights, ragged 32-row tiles, long rows
SHAPES = [(1, 256), (3, 512), (40, 768), (33, 16384), (257, 1024), (64, 64 * 12), (5, 3072),
          (130, 256), (2, 4096), (96, 1280)]


def _mixed(g, nweights, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(nweights):
        n, k = SHAPES[i % len(SHAPES)]
        k = max(g, k - k % g)
        out.append(synth.f32_to_bf16_bits(rng.standard_normal((n, k)).astype(np.float32)
                                          * np.float32(2.0 ** rng.integers(-8, 8))))
    return out


@pytest.mark.parametrize("g", [4, 16, 64, 256])
@pytest.mark.parametrize("per_channel,dtype", [(False, torch.bfloat16), (True, torch.float16)],
                         ids=["tensor-bf16", "channel-f16"])
def test_mixed_list(g, per_channel, dtype):
    print(f"batched dequant mixed g={g} pc={per_channel} {dtype}", flush=True)
    ws = _mixed(g, 53, 7 + g)  # more than one launch's 48
    quant = oracle.quantize_weights_per_channel if per_channel else oracle.quantize_weights
    refs = [quant(w, g, SEED) for w in ws]
    wqs = [torch.from_numpy(q).to(DEV) for q, _ in refs]
    sws = [torch.from_numpy(np.atleast_1d(np.asarray(s, dtype=np.float32))).to(DEV)
           for _, s in refs]
    outs = cr.convrot_dequant_derotate_batched(wqs, sws, g, SEED, per_channel=per_channel,
                                               out_dtype=dtype)
    fmt = "f16" if dtype == torch.float16 else "bf16"
    for i, ((q, s), out) in enumerate(zip(refs, outs)):
        assert np.array_equal(host_bits(out), oracle.dequant_derotate(q, s, g, SEED, fmt)), i
    # and equal to the single calls
    for i in (0, 17, 52):
        one = cr.convrot_dequant_derotate_ex(wqs[i], sws[i], g, SEED, per_channel=per_channel,
                                             out_dtype=dtype)
        assert torch.equal(one.view(torch.int16), outs[i].view(torch.int16)), i


def test_shared_inputs_and_empty_list():
    """One weight decoded into two outputs in the same call; an empty call."""
    g = 64
    q, s = oracle.quantize_weights(_mixed(g, 1, 3)[0], g, SEED)
    wq = torch.from_numpy(q).to(DEV)
    sw = torch.tensor([s], dtype=torch.float32, device=DEV)
    a, b = cr.convrot_dequant_derotate_batched([wq, wq], [sw, sw], g, SEED)
    want = oracle.dequant_derotate(q, s, g, SEED)
    assert np.array_equal(host_bits(a), want) and np.array_equal(host_bits(b), want)
    assert cr.convrot_dequant_derotate_batched([], [], g, SEED) == []
