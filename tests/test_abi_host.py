"""The C-ABI library without a GPU: it loads, exports every symbol that
include/convrot.h declares, rejects bad arguments before touching HIP, and its
host-side sign generator agrees with the oracle's independent one."""

import ctypes
import os
import re
import subprocess

import pytest

import int8_gemm_amd as cr
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cr.library_path()):
        from int8_gemm_amd import _build
        _build.build()
    return cr.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert sorted(cr.EXPORTED_SYMBOLS) == _declared_functions()


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", cr.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(convrot_[a-z0-9_]+)\b", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version_and_status_strings(lib):
    assert cr.convrot_abi_version() == 7
    for s in range(8):
        assert cr.convrot_status_string(s)
    assert cr.convrot_status_string(7).startswith("first-call check")


@pytest.mark.parametrize("seed", [synth.ROT_SEED, 0, 1, 2 ** 64 - 1, 0x123456789ABCDEF])
@pytest.mark.parametrize("g", [4, 16, 64, 256])
def test_signs_match_oracle(lib, seed, g):
    assert cr.convrot_rotation_signs(seed, g) == list(oracle.rotation_signs(seed, g))


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced on error paths
FAKE_MIS = ctypes.c_void_p((1 << 20) + 4)


def _status(lib, fn, *args):
    return getattr(lib, fn)(*args)


@pytest.mark.parametrize("g,k,want", [(512, 256, 2), (0, 256, 2), (3, 192, 2), (256, 320, 2),
                                      (4, 100, 3), (64, 32832, 3), (256, 0, 1)])
def test_rotating_entry_points_reject_bad_group_and_shape(lib, g, k, want):
    for fn in ("convrot_quantize_activations", "convrot_quantize_activations_exact"):
        assert _status(lib, fn, FAKE, 8, k, g, 1, FAKE, ctypes.c_void_p(1 << 24), None) == want
    assert _status(lib, "convrot_quantize_weights", FAKE, 8, k, g, 1, ctypes.c_void_p(1 << 24),
                   ctypes.c_void_p(1 << 28), None) == want
    assert _status(lib, "convrot_dequant_derotate", FAKE, ctypes.c_void_p(1 << 24), 8, k, g, 1,
                   ctypes.c_void_p(1 << 28), None) == want
    assert _status(lib, "convrot_quantize_weights_per_channel", FAKE, 8, k, g, 1,
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 28), None) == want
    assert _status(lib, "convrot_dequant_derotate_per_channel", FAKE, ctypes.c_void_p(1 << 24), 8,
                   k, g, 1, ctypes.c_void_p(1 << 28), None) == want
    assert lib.convrot_last_error_string()


@pytest.mark.parametrize("tile,k,why", [(100, 256, "not supported"), (-1, 256, "not supported"),
                                        (512, 256, "not supported"), (384, 320, "k % 128"),
                                        (384, 192, "k % 128"), (384, 256, "null pointer"),
                                        (128, 320, "null pointer"), (0, 320, "null pointer")])
def test_forced_tile_is_checked_before_launch(lib, tile, k, why):
    """Unsupported tiles, and the 384 x 192 tile without 128-byte K-steps, are
    refused before any HIP call; accepted tiles get as far as the null-output
    check (m = 8, y = acc = null), which also refuses before any launch."""
    calls = [("convrot_gemm_int8_tile", (FAKE, FAKE, FAKE, FAKE, None, 8, 16, k, None, None,
                                         tile, None)),
             ("convrot_gemm_int8_per_channel_tile", (FAKE, FAKE, FAKE, FAKE, None, 8, 16, k, None,
                                                     None, tile, None))]
    calls += [("convrot_gemm_int8_ex", (FAKE, FAKE, FAKE, FAKE, 0, None, 8, 16, k, None, None, dt,
                                        tile, None)) for dt in (0, 1)]
    for fn, args in calls:
        assert _status(lib, fn, *args) == 1, fn
        assert why in lib.convrot_last_error_string().decode(), fn


def test_null_and_misaligned_and_overlap(lib):
    assert _status(lib, "convrot_quantize_activations", None, 8, 256, 256, 1, FAKE, FAKE,
                   None) == 1
    assert _status(lib, "convrot_quantize_activations", FAKE_MIS, 8, 256, 256, 1,
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 28), None) == 4
    # xq overlapping x
    assert _status(lib, "convrot_quantize_activations", FAKE, 8, 256, 256, 1,
                   ctypes.c_void_p((1 << 20) + 256), ctypes.c_void_p(1 << 28), None) == 1
    # gemm: no output at all
    assert _status(lib, "convrot_gemm_int8", FAKE, FAKE, FAKE, FAKE, None, 8, 16, 64, None,
                   None, None) == 1
    # gemm: more output tiles than a 32-bit grid holds
    assert _status(lib, "convrot_gemm_int8", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26), None, 1 << 30, 1 << 30,
                   64, ctypes.c_void_p(1 << 28), None, None) == 3
    # gemm: n % 16, k % 64
    assert _status(lib, "convrot_gemm_int8", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26), None, 8, 24, 64,
                   ctypes.c_void_p(1 << 28), None, None) == 3
    assert _status(lib, "convrot_gemm_int8", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26), None, 8, 32, 96,
                   ctypes.c_void_p(1 << 28), None, None) == 3
    # gemm: K beyond the int32 accumulator bound
    assert _status(lib, "convrot_gemm_int8", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26), None, 8, 32, 133184,
                   ctypes.c_void_p(1 << 36), None, None) == 3


def test_linear_workspace_rules(lib):
    k = 3840
    assert cr.convrot_linear_int8_workspace_for_rows(1, k) == 3840 + 4
    assert cr.convrot_linear_int8_workspace_for_rows(3, 320) == 1024 + 12
    assert cr.convrot_linear_int8_workspace_size(4608, 3840, k) == \
        cr.convrot_linear_int8_workspace_for_rows(4608, k)
    assert cr.convrot_linear_int8_workspace_size(100000, 16, k) == \
        cr.convrot_linear_int8_workspace_for_rows(32, k)
    # too small for one row
    st = _status(lib, "convrot_linear_int8", FAKE, ctypes.c_void_p(1 << 24),
                 ctypes.c_void_p(1 << 26), None, 8, 16, k, 256, 1, ctypes.c_void_p(1 << 28),
                 ctypes.c_void_p(1 << 32), 1000, None)
    assert st == 5
    # misaligned workspace
    st = _status(lib, "convrot_linear_int8", FAKE, ctypes.c_void_p(1 << 24),
                 ctypes.c_void_p(1 << 26), None, 8, 16, k, 256, 1, ctypes.c_void_p(1 << 28),
                 ctypes.c_void_p((1 << 32) + 16), 1 << 20, None)
    assert st == 4


def test_m_zero_is_a_noop(lib):
    # no HIP call happens for M == 0 (this container has no GPU)
    assert _status(lib, "convrot_quantize_activations", FAKE, 0, 256, 256, 1,
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 28), None) == 0
    assert _status(lib, "convrot_gemm_int8", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26), None, 0, 32, 64,
                   ctypes.c_void_p(1 << 28), None, None) == 0


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cr.convrot_quantize_activations(x, 256)


def test_per_channel_scale_vector_checks(lib):
    """A per-channel s_w is n floats, 16-byte aligned, and may not overlap an
    output; every check fires before any HIP call."""
    sw_mis = ctypes.c_void_p((1 << 26) + 4)     # 4-byte aligned only
    n, k = 64, 256
    assert _status(lib, "convrot_quantize_weights_per_channel", FAKE, n, k, 256, 1,
                   ctypes.c_void_p(1 << 24), sw_mis, None) == 4
    assert _status(lib, "convrot_dequant_derotate_per_channel", FAKE, sw_mis, n, k, 256, 1,
                   ctypes.c_void_p(1 << 28), None) == 4
    for fn in ("convrot_gemm_int8_per_channel",):
        assert _status(lib, fn, FAKE, ctypes.c_void_p(1 << 22), ctypes.c_void_p(1 << 24), sw_mis,
                       None, 8, n, k, ctypes.c_void_p(1 << 28), None, None) == 4
    assert _status(lib, "convrot_gemm_int8_per_channel_tile", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), sw_mis, None, 8, n, k, ctypes.c_void_p(1 << 28),
                   None, 192, None) == 4
    assert _status(lib, "convrot_linear_int8_per_channel", FAKE, ctypes.c_void_p(1 << 24), sw_mis,
                   None, 8, n, k, 256, 1, ctypes.c_void_p(1 << 28), ctypes.c_void_p(1 << 32),
                   1 << 20, None) == 4
    # the n-float vector overlapping y (y at 1 << 28, s_w n*4 bytes just below its end)
    y_end = (1 << 28) + 8 * n * 2
    sw_in_y = ctypes.c_void_p(y_end - 16)
    assert _status(lib, "convrot_gemm_int8_per_channel", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), sw_in_y, None, 8, n, k, ctypes.c_void_p(1 << 28),
                   None, None) == 1
    # ... and starting just below y: only the vector's length makes it overlap
    sw_before_y = ctypes.c_void_p((1 << 28) - 16)
    assert _status(lib, "convrot_gemm_int8_per_channel", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), sw_before_y, None, 8, n, k,
                   ctypes.c_void_p(1 << 28), None, None) == 1
    # the per-channel quantize writes n scales: overlapping wq is rejected
    assert _status(lib, "convrot_quantize_weights_per_channel", FAKE, n, k, 256, 1,
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p((1 << 24) + n * k - 16), None) == 1
    # m == 0 is a no-op here too
    assert _status(lib, "convrot_gemm_int8_per_channel", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26), None, 0, n, k,
                   ctypes.c_void_p(1 << 28), None, None) == 0


def test_ex_entry_points_reject_unknown_enums(lib):
    """dtype and scale_mode values outside their enums fail before any HIP call"""
    n, k = 64, 256
    assert _status(lib, "convrot_quantize_activations_ex", FAKE, 2, 8, k, 256, 1,
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 28), None) == 1
    assert _status(lib, "convrot_dequant_derotate_ex", FAKE, ctypes.c_void_p(1 << 24), 2, n, k,
                   256, 1, ctypes.c_void_p(1 << 28), 0, None) == 1
    assert _status(lib, "convrot_dequant_derotate_ex", FAKE, ctypes.c_void_p(1 << 24), 0, n, k,
                   256, 1, ctypes.c_void_p(1 << 28), -1, None) == 1
    assert _status(lib, "convrot_gemm_int8_ex", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26), 0, None, 8, n, k,
                   ctypes.c_void_p(1 << 28), None, 7, 0, None) == 1
    assert _status(lib, "convrot_linear_int8_ex", FAKE, ctypes.c_void_p(1 << 24),
                   ctypes.c_void_p(1 << 26), 5, None, 8, n, k, 256, 1, ctypes.c_void_p(1 << 28),
                   1, ctypes.c_void_p(1 << 32), 1 << 20, None) == 1
    # valid enums reach the ordinary checks (here: a bad group, and a
    # per-channel scale that is only 4-byte aligned)
    assert _status(lib, "convrot_quantize_activations_ex", FAKE, 1, 8, k, 512, 1,
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 28), None) == 2
    assert _status(lib, "convrot_gemm_int8_ex", FAKE, ctypes.c_void_p(1 << 22),
                   ctypes.c_void_p(1 << 24), ctypes.c_void_p((1 << 26) + 4), 1, None, 8, n, k,
                   ctypes.c_void_p(1 << 28), None, 1, 0, None) == 4
    # m == 0 with half: a no-op
    assert _status(lib, "convrot_linear_int8_ex", FAKE, ctypes.c_void_p(1 << 24),
                   ctypes.c_void_p(1 << 26), 0, None, 0, n, k, 256, 1, ctypes.c_void_p(1 << 28),
                   1, ctypes.c_void_p(1 << 32), 1 << 20, None) == 0


def test_streamer_argument_checks_without_gpu(lib):
    """rejected before any HIP call: a null streamer or output, bad slot counts"""
    h = ctypes.c_void_p()
    assert lib.convrot_streamer_create(1 << 20, 0, ctypes.byref(h)) == 1
    assert lib.convrot_streamer_create(1 << 20, 9, ctypes.byref(h)) == 1
    assert lib.convrot_streamer_create(0, 2, ctypes.byref(h)) == 1
    assert lib.convrot_streamer_create(1 << 20, 2, None) == 1
    assert lib.convrot_streamer_destroy(None) == 1
    assert lib.convrot_streamer_linear_int8(None, FAKE, 0, FAKE, FAKE, 0, None, 8, 64, 256, 256, 1,
                                            FAKE, FAKE, 1 << 20, None) == 1


def test_session_argument_checks_without_gpu(lib):
    h = ctypes.c_void_p()
    assert lib.convrot_session_create(float("nan"), ctypes.byref(h)) == 1
    assert lib.convrot_session_create(0.1, None) == 1
    assert lib.convrot_session_destroy(None) == 1
    assert lib.convrot_session_linear_int8(None, FAKE, 0, FAKE, FAKE, 0, None, 8, 64, 256, 256, 1,
                                           FAKE, FAKE, 1 << 20, None) == 1
    t, e, lt = ctypes.c_int(), ctypes.c_double(), ctypes.c_int()
    assert lib.convrot_session_lookup(None, 8, 64, 256, 256, 0, 0, ctypes.byref(t),
                                      ctypes.byref(e), ctypes.byref(lt)) == 1
    assert lib.convrot_session_export(None, None, 0) == 0
    assert lib.convrot_session_import(None, b"convrot-session-tiles 1\n") == 1
    assert lib.convrot_session_import(FAKE, None) == 1


def test_header_compiles_and_links_as_c99(lib, tmp_path):
    """include/convrot.h from plain C99 (gcc -std=c99 -pedantic), every entry
    point referenced with its declared types, linked against the library"""
    import shutil
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    src = os.path.join(ROOT, "tests", "c", "header_c99.c")
    obj = tmp_path / "header_c99.so"
    r = subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Werror", "-fPIC", "-shared",
                        "-I", os.path.join(ROOT, "include"), src, "-o", str(obj),
                        cr.library_path(), "-Wl,--no-undefined",
                        "-Wl,--unresolved-symbols=ignore-in-shared-libs"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


# --------------------------------------------------------------------------
# Launch sizing from the device's compute units (host only)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cus", [256, 128, 64, 32, 3])
def test_launch_plans_follow_compute_units(lib, cus):
    """Persistent grids hold at most a fixed number of workgroups per CU, the
    GEMM's tile order spreads over CUs / 32 XCDs, and a plan covers the shape."""
    # act-quant at K = 3840: two 60-lane rows per 2-wave block, 4 per CU
    # (a block holds at least two rows, i.e. one row of the exact pass's
    # 120-lane team for the rows it defers)
    p = cr.convrot_plan_launch("act_quant", m=4608, k=3840, g=256, compute_units=cus)
    assert p["compute_units"] == cus and p["block"] == 128 and p["rows_per_block"] == 2
    assert p["grid"] == min(4608 // 2, 4 * cus)
    assert p["grid"] * p["passes"] >= 2304 > p["grid"] * (p["passes"] - 1)
    # deferred rows: the fast kernel's grid and blocks, one 384-lane exact row
    # per step at K = 12288 (two 192-lane fast rows in a 6-wave block)
    p = cr.convrot_plan_launch("act_quant_deferred", m=4608, k=12288, g=256, compute_units=cus)
    f = cr.convrot_plan_launch("act_quant", m=4608, k=12288, g=256, compute_units=cus)
    assert p["block"] == f["block"] == 384 and p["grid"] == f["grid"] == min(2304, cus)
    assert f["rows_per_block"] == 2 and p["rows_per_block"] == 1 and p["passes"] == f["passes"]
    # dequant: 2 blocks per CU at g = 256, 4 at g <= 64
    for g, per_cu in ((256, 2), (64, 4), (4, 4)):
        p = cr.convrot_plan_launch("dequant", n=3840, k=3840, g=g, compute_units=cus)
        tiles = 3840 * 3840 // max(g, 32) // 32
        steps = tiles if g == 256 else tiles // 4
        assert p["grid"] == min(steps, per_cu * cus), g
        assert p["grid"] * p["passes"] >= steps
    # GEMM: a tile that covers the output, the XCD count of the tile order
    p = cr.convrot_plan_launch("gemm", m=32760, n=13824, k=5120, compute_units=cus)
    assert p["xcds"] == (cus // 32 if cus >= 64 else 1)
    tm, tn = p["tile_m"], p["tile_n"]
    assert p["grid"] == -(-32760 // tm) * -(-13824 // tn)


def test_act_quant_blocks_fit_a_deferred_row_at_every_k(lib):
    """A fast-kernel block resolves the rows it defers with a team of K/32
    lanes, so every bf16 act-quant block holds at least two K/64-lane rows;
    the deferred-row plan runs in the same grid with whole K/32-lane rows."""
    for cus in (256, 7):
        for k in range(64, 16384 + 1, 64):
            p = cr.convrot_plan_launch("act_quant", m=100000, k=k, g=4, compute_units=cus)
            d = cr.convrot_plan_launch("act_quant_deferred", m=100000, k=k, g=4, compute_units=cus)
            assert p["block"] % 64 == 0 and p["block"] <= 512, k
            assert p["rows_per_block"] >= 2 and p["rows_per_block"] * (k // 64) <= p["block"], k
            assert (d["grid"], d["block"], d["passes"]) == (p["grid"], p["block"], p["passes"]), k
            assert d["rows_per_block"] == p["block"] // (k // 32) >= 1, k


def test_gemm_tile_choice_counts_rounds_over_the_cus(lib):
    """The 384 x 192 tile covers 4608 x 3840 in 240 tiles, one round on 256
    CUs; on 128 CUs that takes two rounds, where the 256 x 256 tile's 270
    tiles take three and the 192 tile's 480 four (a 384 x 192 round lasts 1.6
    of a 192 round, a 256 round 1.336): the 384 tile stays the choice."""
    for cus in (256, 128):
        p = cr.convrot_plan_launch("gemm", m=4608, n=3840, k=3840, compute_units=cus)
        assert (p["tile_m"], p["tile_n"], p["grid"]) == (384, 192, 240), cus
    # with K % 128 != 0 the 384 tile does not exist
    p = cr.convrot_plan_launch("gemm", m=4608, n=3840, k=3840 + 64, compute_units=256)
    assert p["tile_m"] != 384
    # a single CU: every tile is a round of its own; the fewest-bytes-per-op
    # tiles win on round count
    p1 = cr.convrot_plan_launch("gemm", m=4096, n=4096, k=4096, compute_units=1)
    assert p1["tile_m"] in (256, 384)


def test_gemm_tile_choice_on_the_workload_layers_and_slices(lib):
    """The tile the chooser takes on 256 CUs for each workload layer and for
    the token slices the linear cuts them into (at most 2N rows), as measured
    fastest on an MI355X (HIP events, every tile forced in turn)."""
    want = {(4608, 3840, 3840): 384, (4608, 12288, 3072): 384, (4608, 3072, 12288): 256,
            (32760, 13824, 5120): 256, (27648, 13824, 5120): 256, (5112, 13824, 5120): 384,
            (32760, 5120, 13824): 256, (10240, 5120, 13824): 384, (2040, 5120, 13824): 256,
            (16384, 9216, 3072): 256}
    for (m, n, k), tile in want.items():
        p = cr.convrot_plan_launch("gemm", m=m, n=n, k=k, compute_units=256)
        assert p["tile_m"] == tile, (m, n, k)


def test_plan_launch_checks_shapes(lib):
    with pytest.raises(cr.ConvrotError, match="UNSUPPORTED_GROUP"):
        cr.convrot_plan_launch("act_quant", m=8, k=96, g=64, compute_units=8)
    with pytest.raises(cr.ConvrotError, match="UNSUPPORTED_SHAPE"):
        cr.convrot_plan_launch("gemm", m=8, n=24, k=64, compute_units=8)
    with pytest.raises(cr.ConvrotError, match="INVALID_ARG"):
        cr.convrot_set_compute_units(-1)
    assert cr.convrot_plan_launch("act_quant", m=0, k=256, g=256, compute_units=8)["grid"] == 0


def test_noalloc_argument_checks_without_gpu(lib):
    """The no-allocation forward checks its arguments before any HIP call,
    like the workspace forward; m == 0 is a no-op."""
    P = FAKE
    fn = lib.convrot_linear_int8_noalloc
    # bad group, bad shape, null pointers, unknown enums
    assert fn(P, P, P, 0, None, 8, 16, 96, 64, 1, P, 0, None) == 2
    assert fn(P, P, P, 0, None, 8, 24, 64, 4, 1, P, 0, None) == 3
    assert fn(None, P, P, 0, None, 8, 16, 64, 4, 1, P, 0, None) == 1
    assert fn(P, P, P, 7, None, 8, 16, 64, 4, 1, P, 0, None) == 1
    assert fn(P, P, P, 0, None, 8, 16, 64, 4, 1, P, 9, None) == 1
    assert fn(P, P, P, 0, None, 0, 16, 64, 4, 1, P, 0, None) == 0
    assert cr.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_batched_dequant_argument_checks_without_gpu(lib):
    """Every job is checked before anything is launched; outputs may not
    overlap another job's buffers, inputs may be shared; no jobs is a no-op."""
    J = cr._DequantJob
    fn = lib.convrot_dequant_derotate_batched

    def call(*jobs, g=256, mode=0, dt=0):
        arr = (J * max(len(jobs), 1))(*jobs)
        return fn(arr, len(jobs), mode, g, 1, dt, None)

    a, b, c, d = (1 << 24), (1 << 26), (1 << 28), (1 << 30)
    assert fn(None, 0, 0, 256, 1, 0, None) == 0
    assert fn(None, 2, 0, 256, 1, 0, None) == 1                     # null list
    assert call(J(a, b, c, 16, 256), g=3) == 2                      # group
    assert call(J(a, b, c, 16, 320)) == 2                           # k % g
    assert call(J(a, b, c, 16, 256), J(a, b, c + 4, 16, 256)) == 4  # misaligned output
    assert call(J(a, b, c, 16, 256), J(a, b, c + 4096, 16, 256)) == 1  # outputs overlap
    assert call(J(a, b, c, 16, 256), J(c, b, d, 16, 256)) == 1      # output is an input
    assert call(J(a, b, c, 16, 256), J(0, b, d, 16, 256)) == 1      # null weight
    assert call(J(a, b, c, 16, 256), mode=5) == 1                   # unknown enum
    assert lib.convrot_last_error_string()
