"""GPU: host-streamed int8 layers (convrot_streamer). Every streamed forward
must equal the resident forward on a device copy of the same weight bit for
bit (the pages report the streamed image bit-identical to the resident one:
Invoke docs "int8 Compute", the streamed-from-RAM table), and one layer is
checked against the CPU oracle as well."""

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


def dev16(bits: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _layers():
    """(x, wq_dev, wq_host_pinned, s_w, per_channel, g) over several shapes,
    scale modes and formats"""
    out = []
    specs = [(synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256, False, "bf16"),
             (synth.FLUX_MLP_UP.scaled(m=257, n=528), 256, True, "bf16"),
             (synth.QKV_SWEEP.scaled(m=260, n=288), 64, False, "f16"),
             (synth.WAN_FFN_UP.scaled(m=130, n=400), 256, True, "f16"),
             (synth.TINY, 16, False, "bf16")]
    for layer, g, pc, fmt in specs:
        dtype = torch.float16 if fmt == "f16" else torch.bfloat16
        x = dev16(layer.x(fmt=fmt), dtype)
        w = dev16(layer.w())
        q = cr.convrot_quantize_weights_per_channel if pc else cr.convrot_quantize_weights
        wq, s_w = q(w, g, SEED)
        out.append((x, wq, wq.cpu().pin_memory(), s_w, pc, g))
    return out


@pytest.mark.parametrize("slots", [1, 2, 3])
def test_streamed_equals_resident(slots):
    print(f"streamer slots={slots}", flush=True)
    layers = _layers()
    slot_bytes = max(wq.numel() for _, wq, _, _, _, _ in layers)
    want = [cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED, per_channel=pc)
            for x, wq, _, s_w, pc, g in layers]
    with cr.Streamer(slot_bytes, slots) as st:
        for rep in range(2):                     # every slot is reused
            got = [st.linear(x, wh, s_w, g, SEED, per_channel=pc)
                   for x, _, wh, s_w, pc, g in layers]
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(zip(got, want)):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, i)


def test_streamed_against_oracle():
    layer, g = synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256
    xb, wb = layer.x(), layer.w()
    wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
    y_ref = oracle.linear_int8(xb, wq_ref, s_ref, g, SEED)[0]
    wh = torch.from_numpy(wq_ref).pin_memory()
    with cr.Streamer(wq_ref.nbytes, 2) as st:
        y = st.linear(dev16(xb), wh, torch.tensor([s_ref], dtype=torch.float32, device=DEV), g,
                      SEED)
        assert np.array_equal(host_bits(y), y_ref)


def test_slot_reuse_waits_for_the_forward():
    """forwards slower than the copies (many tokens, small weights): a slot
    must not be refilled while its forward still reads it. Ten distinct
    weights through two slots, synchronised only at the end."""
    print("streamer slot reuse", flush=True)
    m, n, k, g = 32768, 1024, 1024, 256
    gen = torch.Generator(device=DEV)
    gen.manual_seed(3)
    x = (torch.randn((m, k), device=DEV, generator=gen)).to(torch.bfloat16)
    ws, outs, want = [], [], []
    for i in range(10):
        w = (torch.randn((n, k), device=DEV, generator=gen) * 0.02).to(torch.bfloat16)
        wq, s_w = cr.convrot_quantize_weights(w, g, SEED)
        ws.append((wq.cpu().pin_memory(), s_w))
        want.append(cr.convrot_linear_int8(x, wq, s_w, g, SEED))
    torch.cuda.synchronize()
    with cr.Streamer(n * k, 2) as st:
        for wh, s_w in ws:
            outs.append(st.linear(x, wh, s_w, g, SEED))
        torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs, want)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), i


def test_streamer_pageable_weight_and_errors():
    layer, g = synth.TINY, 256
    x = dev16(layer.x())
    wq, s_w = cr.convrot_quantize_weights(dev16(layer.w()), g, SEED)
    want = cr.convrot_linear_int8(x, wq, s_w, g, SEED)
    with cr.Streamer(wq.numel(), 2) as st:
        got = st.linear(x, wq.cpu(), s_w, g, SEED)          # pageable host memory
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        got = st.linear(x, wq, s_w, g, SEED)                # device memory
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        big = torch.zeros((layer.n * 2, layer.k), dtype=torch.int8).pin_memory()
        with pytest.raises(cr.ConvrotError) as e:
            st.linear(x, big, torch.ones(1, device=DEV), g, SEED)
        assert e.value.status_name == "CONVROT_E_WORKSPACE"
        empty = st.linear(torch.zeros((0, layer.k), dtype=torch.bfloat16, device=DEV),
                          wq.cpu(), s_w, g, SEED)
        assert empty.shape == (0, layer.n)
        torch.cuda.synchronize()
