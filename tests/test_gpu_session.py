"""GPU: sessions (first-call tile tuning and check against the default path).

On the pages, the int8 forward of each new layer shape and token range is
compared once with the dequant path, and a mismatch switches that GPU back to
the dequant path (Invoke docs "int8 Compute", "When something goes wrong"). Here:
the session's forward equals the plain forward bit for bit whatever tile it
kept; the check's error equals an independent float64 computation of the
same quantity from the oracle; a failing check (forced from the host with a
tolerance below the quantization noise) latches the session, and a latched
session enqueues nothing."""

import numpy as np
import pytest
import torch

import int8_gemm_amd as cr
import oracle
import synth

pytestmark = pytest.mark.gpu

SEED = synth.ROT_SEED
DEV = "cuda:0"
TILES = {128, 192, 256, 384}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    cr.load_library()


def dev16(bits: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


CASES = [(synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256, False, "bf16"),
         (synth.FLUX_MLP_UP.scaled(m=257, n=528), 256, True, "bf16"),
         (synth.QKV_SWEEP.scaled(m=260, n=288), 64, False, "f16"),
         (synth.WAN_FFN_DOWN.scaled(m=70, n=272), 256, True, "f16")]


@pytest.mark.parametrize("layer,g,pc,fmt", CASES, ids=[c[0].name + "-" + c[3] for c in CASES])
def test_session_forward_and_check(layer, g, pc, fmt):
    print(f"session {layer.name} g={g} pc={pc} {fmt}", flush=True)
    dtype = torch.float16 if fmt == "f16" else torch.bfloat16
    xb, wb = layer.x(fmt=fmt), layer.w()
    wq_ref, s_ref = (oracle.quantize_weights_per_channel if pc else oracle.quantize_weights)(
        wb, g, SEED)
    bias = np.random.default_rng(12).standard_normal(layer.n).astype(np.float32)
    bias_b = oracle.from_f32(bias, fmt)
    x, wq = dev16(xb, dtype), torch.from_numpy(wq_ref).to(DEV)
    s_w = torch.from_numpy(np.atleast_1d(s_ref).astype(np.float32)).to(DEV)
    bias_t = dev16(bias_b, dtype)
    want = cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED, bias_t, per_channel=pc)
    with cr.Session() as ses:
        for _ in range(2):                                   # the first call, then the kept tile
            y = ses.linear(x, wq, s_w, g, SEED, bias_t, per_channel=pc)
            assert torch.equal(y.view(torch.int16), want.view(torch.int16))
        tile, err, latched = ses.lookup(layer.m, layer.n, layer.k, g, dtype, pc)
        assert tile in TILES and not latched
        # the same quantity from the oracle: int8 path vs x . W_hat^T (+ bias)
        # on the first min(m, 256) rows, W_hat the default path's decode
        r = min(layer.m, 256)
        y8 = oracle.to_f64(oracle.linear_int8(xb, wq_ref, s_ref, g, SEED, bias_b, fmt)[0], fmt)[:r]
        w_hat = oracle.to_f64(oracle.dequant_derotate(wq_ref, s_ref, g, SEED, fmt), fmt)
        y_def = oracle.to_f64(xb[:r], fmt) @ w_hat.T + oracle.to_f64(bias_b, fmt)[None, :]
        want_err = oracle.rel_frobenius(y8, y_def)
        assert abs(err - want_err) <= 1e-4 + 1e-3 * want_err, (err, want_err)
        assert err < 0.05
        # another m in the same token bucket, ceil(log2 m), reuses the key
        b = (layer.m - 1).bit_length()
        m2 = max(2 ** (b - 1) + 1, layer.m - 7)
        y2 = ses.linear(x[:m2], wq, s_w, g, SEED, bias_t, per_channel=pc)
        assert torch.equal(y2.view(torch.int16), want[:m2].view(torch.int16))
        assert ses.lookup(m2, layer.n, layer.k, g, dtype, pc)[0] == tile


def test_failed_check_latches_and_latched_session_enqueues_nothing():
    print("session latch", flush=True)
    layer, g = synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256
    x = dev16(layer.x())
    wq, s_w = cr.convrot_quantize_weights(dev16(layer.w()), g, SEED)
    with cr.Session(check_tolerance=1e-9) as ses:   # below any quantization noise
        with pytest.raises(cr.ConvrotError) as e:
            ses.linear(x, wq, s_w, g, SEED)
        assert e.value.status_name == "CONVROT_E_SELFCHECK"
        tile, err, latched = ses.lookup(layer.m, layer.n, layer.k, g)
        assert latched and err > 1e-9 and tile in TILES
        # latched: another shape fails at once and its output stays untouched
        out = torch.full((64, layer.n), 7.0, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(cr.ConvrotError) as e:
            ses.linear(x[:64], wq, s_w, g, SEED, out=out)
        assert e.value.status_name == "CONVROT_E_SELFCHECK"
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())


def test_session_on_a_workload_shape():
    """one first call at the full Z-Image attention shape (tuning over all
    four tiles, the check on 256 rows); the kept tile gives the plain bits"""
    layer, g = synth.ZIMAGE_ATTN, 256
    x = dev16(layer.x())
    wq, s_w = cr.convrot_quantize_weights(dev16(layer.w()), g, SEED)
    want = cr.convrot_linear_int8(x, wq, s_w, g, SEED)
    with cr.Session() as ses:
        y = ses.linear(x, wq, s_w, g, SEED)
        tile, err, latched = ses.lookup(layer.m, layer.n, layer.k, g)
        print(f"zimage-attn session: tile {tile}, check error {err:.4g}", flush=True)
        assert torch.equal(y.view(torch.int16), want.view(torch.int16))
        assert tile in TILES and err < 0.05 and not latched


def test_check_over_column_chunks():
    """At k = 16384 the session buffer holds the check's W_hat for 7936
    weight rows at a time: n = 8256 takes two chunks (the second ragged), with
    a bias; the check's error still equals the oracle's over all n columns,
    and the first call allocates no device memory (the buffer was made by
    convrot_session_create)."""
    g, m, n, k = 256, 8, 8256, 16384
    print(f"session check in column chunks {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(21)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    wb = synth.f32_to_bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    bias_b = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    wq_ref, s_ref = oracle.quantize_weights(wb, g, SEED)
    x, wq, bias_t = dev16(xb), torch.from_numpy(wq_ref).to(DEV), dev16(bias_b)
    s_w = torch.tensor([s_ref], dtype=torch.float32, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    with cr.Session() as ses:
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        ses.linear(x, wq, s_w, g, SEED, bias_t, out=y)
        torch.cuda.synchronize()
        # a first call that allocated would take >= 256 MB + 2nk (528 MB) here
        assert torch.cuda.mem_get_info()[0] >= free0 - (64 << 20)
        tile, err, latched = ses.lookup(m, n, k, g)
    y_bits = oracle.linear_int8(xb, wq_ref, s_ref, g, SEED, bias_b)[0]
    assert np.array_equal(host_bits(y), y_bits)
    y8 = oracle.to_f64(y_bits, "bf16")
    w_hat = oracle.to_f64(oracle.dequant_derotate(wq_ref, s_ref, g, SEED), "bf16")
    y_def = oracle.to_f64(xb, "bf16") @ w_hat.T + oracle.to_f64(bias_b, "bf16")[None, :]
    want_err = oracle.rel_frobenius(y8, y_def)
    assert abs(err - want_err) <= 1e-4 + 1e-3 * want_err, (err, want_err)
    assert not latched and tile in TILES


def test_tiles_exported_and_imported():
    """A session's tuned tiles as text, read by another session: an imported
    key's first call runs with the imported tile (a tile the timing would
    not pick is kept as given) and still runs the check; its results equal
    the plain forward's; the text of the second session lists the same keys;
    malformed text imports nothing."""
    cases = [(synth.ZIMAGE_ATTN.scaled(m=300, n=272), 256, False, torch.bfloat16),
             (synth.QKV_SWEEP.scaled(m=260, n=288), 64, True, torch.float16)]
    inputs = []
    for layer, g, pc, dtype in cases:
        fmt = "f16" if dtype == torch.float16 else "bf16"
        wq_ref, s_ref = (oracle.quantize_weights_per_channel if pc else oracle.quantize_weights)(
            layer.w(), g, SEED)
        x = dev16(layer.x(fmt=fmt), dtype)
        wq = torch.from_numpy(wq_ref).to(DEV)
        s_w = torch.from_numpy(np.atleast_1d(s_ref).astype(np.float32)).to(DEV)
        want = cr.convrot_linear_int8_ex(x, wq, s_w, g, SEED, per_channel=pc)
        inputs.append((layer, g, pc, dtype, x, wq, s_w, want))
    with cr.Session() as a:
        for layer, g, pc, dtype, x, wq, s_w, want in inputs:
            assert torch.equal(a.linear(x, wq, s_w, g, SEED, per_channel=pc).view(torch.int16),
                               want.view(torch.int16))
        text = a.export_tiles()
        tiles_a = [a.lookup(l.m, l.n, l.k, g, dt, pc)[0] for l, g, pc, dt, *_ in inputs]
    lines = text.splitlines()
    assert lines[0] == "convrot-session-tiles 1" and len(lines) == 3
    print("exported:", lines[1:], flush=True)
    # the first key's tile replaced by one the timing did not keep
    f = lines[1].split()
    other = 128 if f[6] != "128" else 192
    lines[1] = " ".join(f[:6] + [str(other)])
    with cr.Session() as b:
        b.import_tiles("\n".join(lines) + "\n")
        with pytest.raises(cr.ConvrotError):     # imported, but no first call yet
            b.lookup(inputs[0][0].m, inputs[0][0].n, inputs[0][0].k, inputs[0][1],
                     inputs[0][3], inputs[0][2])
        assert b.export_tiles() == "\n".join(lines) + "\n"
        for i, (layer, g, pc, dtype, x, wq, s_w, want) in enumerate(inputs):
            y = b.linear(x, wq, s_w, g, SEED, per_channel=pc)
            assert torch.equal(y.view(torch.int16), want.view(torch.int16))
            tile, err, latched = b.lookup(layer.m, layer.n, layer.k, g, dtype, pc)
            assert tile == (other if i == 0 else tiles_a[1]) and not latched
            assert 0.0 < err < 0.05
        # malformed text: nothing imported, entries unchanged
        bad = ["", "convrot-session-tiles 2\n",
               "convrot-session-tiles 1\n272 3840 9 256 0 0 384 7\n",
               "convrot-session-tiles 1\n272 3840 9 256 0 0 320\n",
               "convrot-session-tiles 1\n272 3904 9 64 0 0 384\n",   # 384 needs k % 128 == 0
               "convrot-session-tiles 1\n270 3840 9 256 0 0 256\n",  # n % 16 != 0
               "convrot-session-tiles 1\n272 3840 9 48 0 0 256\n",
               "convrot-session-tiles 1\n272 3840 9 256 2 0 256\n"]
        before = b.export_tiles()
        for t in bad:
            with pytest.raises(cr.ConvrotError):
                b.import_tiles(t)
        assert b.export_tiles() == before
