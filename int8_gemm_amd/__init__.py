"""MI355X (gfx950) int8_tensorwise "convrot" linear layer.

A thin binding of libconvrot.so (the C ABI declared in include/convrot.h):
each function checks its torch tensors (device, dtype, contiguity), passes raw
device pointers and the current HIP stream, and raises ConvrotError on a
non-OK status. Every step of the computation runs in the library's HIP
kernels; there is no other code path. The names follow the C entry points.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "ConvrotError", "ROT_SEED", "load_library", "library_path",
    "convrot_quantize_weights", "convrot_dequant_derotate", "convrot_quantize_activations",
    "convrot_quantize_activations_exact", "convrot_gemm_int8", "convrot_linear_int8",
    "convrot_linear_int8_workspace_size", "convrot_linear_int8_workspace_for_rows",
    "convrot_rotation_signs", "convrot_abi_version", "convrot_status_string",
    "convrot_quantize_weights_per_channel", "convrot_dequant_derotate_per_channel",
    "convrot_gemm_int8_per_channel", "convrot_linear_int8_per_channel",
    "convrot_quantize_activations_ex", "convrot_dequant_derotate_ex", "convrot_gemm_int8_ex",
    "convrot_linear_int8_ex", "convrot_streamer_create", "convrot_streamer_destroy",
    "convrot_streamer_linear_int8", "Streamer", "convrot_session_create",
    "convrot_session_destroy", "convrot_session_linear_int8", "convrot_session_lookup",
    "convrot_session_export", "convrot_session_import",
    "Session", "EXPORTED_SYMBOLS", "convrot_compute_units", "convrot_set_compute_units",
    "convrot_plan_launch", "KERNELS", "convrot_linear_int8_noalloc", "NOALLOC_SCRATCH_BYTES",
    "convrot_dequant_derotate_batched",
]

ROT_SEED = 0xC0FFEE
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libconvrot.so")
_lib = None
_lock = threading.Lock()

# every extern "C" symbol that include/convrot.h declares
EXPORTED_SYMBOLS = (
    "convrot_quantize_weights", "convrot_dequant_derotate", "convrot_quantize_activations",
    "convrot_quantize_activations_exact", "convrot_gemm_int8", "convrot_gemm_int8_tile",
    "convrot_linear_int8", "convrot_linear_int8_workspace_for_rows",
    "convrot_linear_int8_workspace_size", "convrot_rotation_signs", "convrot_status_string",
    "convrot_last_error_string", "convrot_abi_version",
    "convrot_quantize_weights_per_channel", "convrot_dequant_derotate_per_channel",
    "convrot_gemm_int8_per_channel", "convrot_gemm_int8_per_channel_tile",
    "convrot_linear_int8_per_channel",
    "convrot_quantize_activations_ex", "convrot_dequant_derotate_ex", "convrot_gemm_int8_ex",
    "convrot_linear_int8_ex", "convrot_streamer_create", "convrot_streamer_destroy",
    "convrot_streamer_linear_int8", "convrot_session_create", "convrot_session_destroy",
    "convrot_session_linear_int8", "convrot_session_lookup", "convrot_session_export",
    "convrot_session_import", "convrot_compute_units",
    "convrot_set_compute_units", "convrot_plan_launch", "convrot_linear_int8_noalloc",
    "convrot_dequant_derotate_batched",
)

# bytes of the per-device scratch array behind convrot_linear_int8_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

# convrot_kernel values (convrot_plan_launch)
KERNELS = {"act_quant": 0, "act_quant_deferred": 1, "exact": 2, "dequant": 3, "gemm": 4}


class _DequantJob(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("s_w", ctypes.c_void_p), ("w_out", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64)]


class _LaunchPlan(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int64), ("passes", ctypes.c_int64), ("block", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("xcds", ctypes.c_int32),
                ("compute_units", ctypes.c_int32)]

# convrot_dtype and convrot_scale_mode values
_DTYPES = {torch.bfloat16: 0, torch.float16: 1}
_SCALE_PER_TENSOR, _SCALE_PER_CHANNEL = 0, 1

_STATUS = {0: "CONVROT_OK", 1: "CONVROT_E_INVALID_ARG", 2: "CONVROT_E_UNSUPPORTED_GROUP",
           3: "CONVROT_E_UNSUPPORTED_SHAPE", 4: "CONVROT_E_MISALIGNED", 5: "CONVROT_E_WORKSPACE",
           6: "CONVROT_E_HIP", 7: "CONVROT_E_SELFCHECK"}


class ConvrotError(RuntimeError):
    """A non-OK status from libconvrot (argument check or HIP launch error)."""

    def __init__(self, status: int, detail: str):
        self.status = status
        self.status_name = _STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libconvrot.so (built in-tree by __graft_entry__.build() or
    int8_gemm_amd/_build.py). Raises if it is missing: there is no fallback."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libconvrot.so is not built ({_LIB_PATH}); run "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I, U64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, \
            ctypes.c_size_t
        sig = {
            "convrot_quantize_weights": [P, I64, I64, I, U64, P, P, P],
            "convrot_dequant_derotate": [P, P, I64, I64, I, U64, P, P],
            "convrot_quantize_activations": [P, I64, I64, I, U64, P, P, P],
            "convrot_quantize_activations_exact": [P, I64, I64, I, U64, P, P, P],
            "convrot_gemm_int8": [P, P, P, P, P, I64, I64, I64, P, P, P],
            "convrot_gemm_int8_tile": [P, P, P, P, P, I64, I64, I64, P, P, I, P],
            "convrot_linear_int8": [P, P, P, P, I64, I64, I64, I, U64, P, P, SZ, P],
            "convrot_rotation_signs": [U64, I, P],
            "convrot_quantize_weights_per_channel": [P, I64, I64, I, U64, P, P, P],
            "convrot_dequant_derotate_per_channel": [P, P, I64, I64, I, U64, P, P],
            "convrot_gemm_int8_per_channel": [P, P, P, P, P, I64, I64, I64, P, P, P],
            "convrot_gemm_int8_per_channel_tile": [P, P, P, P, P, I64, I64, I64, P, P, I, P],
            "convrot_linear_int8_per_channel": [P, P, P, P, I64, I64, I64, I, U64, P, P, SZ, P],
            "convrot_quantize_activations_ex": [P, I, I64, I64, I, U64, P, P, P],
            "convrot_dequant_derotate_ex": [P, P, I, I64, I64, I, U64, P, I, P],
            "convrot_gemm_int8_ex": [P, P, P, P, I, P, I64, I64, I64, P, P, I, I, P],
            "convrot_linear_int8_ex": [P, P, P, I, P, I64, I64, I64, I, U64, P, I, P, SZ, P],
            "convrot_streamer_create": [SZ, I, ctypes.POINTER(P)],
            "convrot_streamer_destroy": [P],
            "convrot_streamer_linear_int8": [P, P, I, P, P, I, P, I64, I64, I64, I, U64, P, P, SZ,
                                             P],
            "convrot_session_create": [ctypes.c_double, ctypes.POINTER(P)],
            "convrot_session_destroy": [P],
            "convrot_session_linear_int8": [P, P, I, P, P, I, P, I64, I64, I64, I, U64, P, P, SZ,
                                            P],
            "convrot_session_lookup": [P, I64, I64, I64, I, I, I, ctypes.POINTER(I),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I)],
            "convrot_session_import": [P, ctypes.c_char_p],
            "convrot_set_compute_units": [I],
            "convrot_linear_int8_noalloc": [P, P, P, I, P, I64, I64, I64, I, U64, P, I, P],
            "convrot_dequant_derotate_batched": [ctypes.POINTER(_DequantJob), I, I, I, U64, I, P],
            "convrot_plan_launch": [I, I64, I64, I64, I, I, ctypes.POINTER(_LaunchPlan)],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.convrot_linear_int8_workspace_for_rows.argtypes = [I64, I64]
        lib.convrot_linear_int8_workspace_for_rows.restype = SZ
        lib.convrot_linear_int8_workspace_size.argtypes = [I64, I64, I64]
        lib.convrot_linear_int8_workspace_size.restype = SZ
        lib.convrot_status_string.argtypes = [I]
        lib.convrot_status_string.restype = ctypes.c_char_p
        lib.convrot_last_error_string.argtypes = []
        lib.convrot_last_error_string.restype = ctypes.c_char_p
        lib.convrot_abi_version.argtypes = []
        lib.convrot_abi_version.restype = I
        lib.convrot_compute_units.argtypes = []
        lib.convrot_compute_units.restype = I
        lib.convrot_session_export.argtypes = [P, ctypes.c_char_p, SZ]
        lib.convrot_session_export.restype = SZ
        _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise ConvrotError(status, lib.convrot_last_error_string().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {devs}")


def convrot_abi_version() -> int:
    return load_library().convrot_abi_version()


def convrot_status_string(status: int) -> str:
    return load_library().convrot_status_string(status).decode()


def convrot_compute_units() -> int:
    """CUs that launches on the current device size their grids for."""
    return int(load_library().convrot_compute_units())


def convrot_set_compute_units(compute_units: int) -> None:
    """Process-wide override of that count (tests and tuning); 0 restores the
    device's count."""
    _check(load_library().convrot_set_compute_units(compute_units))


def convrot_plan_launch(kernel: str, m: int = 0, n: int = 0, k: int = 0, g: int = 256,
                        compute_units: int = 0) -> dict:
    """Launch geometry of `kernel` (a KERNELS key) for a shape on
    `compute_units` CUs (0 = the current device's). Host only when
    compute_units > 0."""
    plan = _LaunchPlan()
    _check(load_library().convrot_plan_launch(KERNELS[kernel], m, n, k, g, compute_units,
                                              ctypes.byref(plan)))
    return {f: int(getattr(plan, f)) for f, _ in _LaunchPlan._fields_}


def convrot_rotation_signs(rot_seed: int, g: int) -> list[int]:
    """Host-only: the rotation signs d[0..g) as +1/-1 ints."""
    buf = (ctypes.c_int8 * g)()
    _check(load_library().convrot_rotation_signs(rot_seed, g, buf))
    return list(buf)


def _need_sw(s_w: torch.Tensor, per_channel: bool, n: int):
    _need(s_w, "s_w", torch.float32, 1 if per_channel else None)
    if per_channel and s_w.shape[0] != n:
        raise ValueError(f"per-channel s_w needs {n} entries (got {s_w.shape[0]})")


def _quant_w(fn_name, per_channel, w, g, rot_seed, wq, s_w):
    _need(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    wq = torch.empty((n, k), dtype=torch.int8, device=w.device) if wq is None else wq
    if s_w is None:
        s_w = torch.empty(n if per_channel else 1, dtype=torch.float32, device=w.device)
    _need(wq, "wq", torch.int8, 2)
    _need_sw(s_w, per_channel, n)
    _same_device(w, wq, s_w)
    _check(getattr(load_library(), fn_name)(_ptr(w), n, k, g, rot_seed, _ptr(wq), _ptr(s_w),
                                            _stream(w)))
    return wq, s_w


def convrot_quantize_weights(w: torch.Tensor, g: int, rot_seed: int = ROT_SEED, *,
                             wq: torch.Tensor | None = None, s_w: torch.Tensor | None = None):
    """W bf16 [n, k] -> (Wq int8 [n, k], s_w fp32 [1])."""
    return _quant_w("convrot_quantize_weights", False, w, g, rot_seed, wq, s_w)


def convrot_quantize_weights_per_channel(w: torch.Tensor, g: int, rot_seed: int = ROT_SEED, *,
                                         wq: torch.Tensor | None = None,
                                         s_w: torch.Tensor | None = None):
    """W bf16 [n, k] -> (Wq int8 [n, k], s_w fp32 [n]), one scale per output row."""
    return _quant_w("convrot_quantize_weights_per_channel", True, w, g, rot_seed, wq, s_w)


def _dequant(fn_name, per_channel, wq, s_w, g, rot_seed, out):
    _need(wq, "wq", torch.int8, 2)
    n, k = wq.shape
    _need_sw(s_w, per_channel, n)
    out = torch.empty((n, k), dtype=torch.bfloat16, device=wq.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    _same_device(wq, s_w, out)
    _check(getattr(load_library(), fn_name)(_ptr(wq), _ptr(s_w), n, k, g, rot_seed, _ptr(out),
                                            _stream(wq)))
    return out


def convrot_dequant_derotate(wq: torch.Tensor, s_w: torch.Tensor, g: int,
                             rot_seed: int = ROT_SEED, *, out: torch.Tensor | None = None):
    """Wq int8 [n, k], s_w fp32 [1] -> W_hat bf16 [n, k]."""
    return _dequant("convrot_dequant_derotate", False, wq, s_w, g, rot_seed, out)


def convrot_dequant_derotate_per_channel(wq: torch.Tensor, s_w: torch.Tensor, g: int,
                                         rot_seed: int = ROT_SEED, *,
                                         out: torch.Tensor | None = None):
    """Wq int8 [n, k], s_w fp32 [n] -> W_hat bf16 [n, k] (row r scaled by s_w[r])."""
    return _dequant("convrot_dequant_derotate_per_channel", True, wq, s_w, g, rot_seed, out)


def _quant_act(fn_name, x, g, rot_seed, xq, s_x):
    _need(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device) if xq is None else xq
    s_x = torch.empty(m, dtype=torch.float32, device=x.device) if s_x is None else s_x
    _need(xq, "xq", torch.int8, 2)
    _need(s_x, "s_x", torch.float32, 1)
    _same_device(x, xq, s_x)
    _check(getattr(load_library(), fn_name)(_ptr(x), m, k, g, rot_seed, _ptr(xq), _ptr(s_x),
                                            _stream(x)))
    return xq, s_x


def convrot_quantize_activations(x: torch.Tensor, g: int, rot_seed: int = ROT_SEED, *,
                                 xq: torch.Tensor | None = None,
                                 s_x: torch.Tensor | None = None):
    """x bf16 [m, k] -> (xq int8 [m, k], s_x fp32 [m]), per-token scales."""
    return _quant_act("convrot_quantize_activations", x, g, rot_seed, xq, s_x)


def convrot_quantize_activations_exact(x: torch.Tensor, g: int, rot_seed: int = ROT_SEED, *,
                                       xq: torch.Tensor | None = None,
                                       s_x: torch.Tensor | None = None):
    """Test hook: the same result through the exact (banded) kernel only."""
    return _quant_act("convrot_quantize_activations_exact", x, g, rot_seed, xq, s_x)


def _gemm(per_channel, xq, s_x, wq, s_w, bias, want_y, want_acc, y, acc, tile):
    _need(xq, "xq", torch.int8, 2)
    _need(wq, "wq", torch.int8, 2)
    _need(s_x, "s_x", torch.float32, 1)
    m, k = xq.shape
    n = wq.shape[0]
    _need_sw(s_w, per_channel, n)
    if wq.shape[1] != k:
        raise ValueError(f"K mismatch: xq {tuple(xq.shape)} vs wq {tuple(wq.shape)}")
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
    if want_y and y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=xq.device)
    if y is not None:
        _need(y, "y", torch.bfloat16, 2)
    if acc is not None:
        _need(acc, "acc", torch.int32, 2)
    _same_device(xq, s_x, wq, s_w, bias, y, acc)
    lib = load_library()
    name = "convrot_gemm_int8_per_channel" if per_channel else "convrot_gemm_int8"
    args = [_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), _ptr(bias), m, n, k, _ptr(y), _ptr(acc)]
    if tile:
        st = getattr(lib, name + "_tile")(*args, tile, _stream(xq))
    else:
        st = getattr(lib, name)(*args, _stream(xq))
    _check(st)
    return y, acc


def convrot_gemm_int8(xq: torch.Tensor, s_x: torch.Tensor, wq: torch.Tensor, s_w: torch.Tensor,
                      bias: torch.Tensor | None = None, *, want_y: bool = True,
                      want_acc: bool = False, y: torch.Tensor | None = None,
                      acc: torch.Tensor | None = None, tile: int = 0):
    """int8 GEMM + epilogue. Returns (y bf16 [m, n] or None, acc int32 [m, n] or None).
    `tile` != 0 forces the block tile (test / tuning hook convrot_gemm_int8_tile)."""
    return _gemm(False, xq, s_x, wq, s_w, bias, want_y, want_acc, y, acc, tile)


def convrot_gemm_int8_per_channel(xq: torch.Tensor, s_x: torch.Tensor, wq: torch.Tensor,
                                  s_w: torch.Tensor, bias: torch.Tensor | None = None, *,
                                  want_y: bool = True, want_acc: bool = False,
                                  y: torch.Tensor | None = None, acc: torch.Tensor | None = None,
                                  tile: int = 0):
    """convrot_gemm_int8 with s_w fp32 [n]: column n of y uses s_w[n]. `tile` != 0
    calls the hook convrot_gemm_int8_per_channel_tile."""
    return _gemm(True, xq, s_x, wq, s_w, bias, want_y, want_acc, y, acc, tile)


def convrot_linear_int8_workspace_size(m: int, n: int, k: int) -> int:
    return int(load_library().convrot_linear_int8_workspace_size(m, n, k))


def convrot_linear_int8_workspace_for_rows(rows: int, k: int) -> int:
    return int(load_library().convrot_linear_int8_workspace_for_rows(rows, k))


def _linear(fn_name, per_channel, x, wq, s_w, g, rot_seed, bias, workspace, out):
    _need(x, "x", torch.bfloat16, 2)
    _need(wq, "wq", torch.int8, 2)
    m, k = x.shape
    n = wq.shape[0]
    _need_sw(s_w, per_channel, n)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
    if workspace is None:
        workspace = torch.empty(max(convrot_linear_int8_workspace_size(m, n, k), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(out, "out", torch.bfloat16, 2)
    _same_device(x, wq, s_w, bias, workspace, out)
    _check(getattr(load_library(), fn_name)(_ptr(x), _ptr(wq), _ptr(s_w), _ptr(bias), m, n, k,
                                            g, rot_seed, _ptr(out), _ptr(workspace),
                                            workspace.numel(), _stream(x)))
    return out


def convrot_linear_int8(x: torch.Tensor, wq: torch.Tensor, s_w: torch.Tensor, g: int,
                        rot_seed: int = ROT_SEED, bias: torch.Tensor | None = None, *,
                        workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """The int8_compute forward: x bf16 [m, k] -> y bf16 [m, n]. `workspace`
    (uint8 on the device) defaults to the library's default size."""
    return _linear("convrot_linear_int8", False, x, wq, s_w, g, rot_seed, bias, workspace, out)


def convrot_linear_int8_per_channel(x: torch.Tensor, wq: torch.Tensor, s_w: torch.Tensor, g: int,
                                    rot_seed: int = ROT_SEED, bias: torch.Tensor | None = None, *,
                                    workspace: torch.Tensor | None = None,
                                    out: torch.Tensor | None = None):
    """convrot_linear_int8 with per-channel weight scales s_w fp32 [n]."""
    return _linear("convrot_linear_int8_per_channel", True, x, wq, s_w, g, rot_seed, bias,
                   workspace, out)


# ---------------------------------------------------------------------------
# General forms: bf16 or fp16 activations / outputs, per-tensor or per-channel
# weight scales
# ---------------------------------------------------------------------------

def _need16(t: torch.Tensor, name: str, ndim: int | None = None) -> int:
    if not isinstance(t, torch.Tensor) or t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be a bfloat16 or float16 tensor")
    _need(t, name, t.dtype, ndim)
    return _DTYPES[t.dtype]


def convrot_quantize_activations_ex(x: torch.Tensor, g: int, rot_seed: int = ROT_SEED, *,
                                    xq: torch.Tensor | None = None,
                                    s_x: torch.Tensor | None = None):
    """x bf16 or fp16 [m, k] -> (xq int8 [m, k], s_x fp32 [m])."""
    dt = _need16(x, "x", 2)
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device) if xq is None else xq
    s_x = torch.empty(m, dtype=torch.float32, device=x.device) if s_x is None else s_x
    _need(xq, "xq", torch.int8, 2)
    _need(s_x, "s_x", torch.float32, 1)
    _same_device(x, xq, s_x)
    _check(load_library().convrot_quantize_activations_ex(_ptr(x), dt, m, k, g, rot_seed,
                                                          _ptr(xq), _ptr(s_x), _stream(x)))
    return xq, s_x


def convrot_dequant_derotate_ex(wq: torch.Tensor, s_w: torch.Tensor, g: int,
                                rot_seed: int = ROT_SEED, *, per_channel: bool = False,
                                out_dtype: torch.dtype = torch.bfloat16,
                                out: torch.Tensor | None = None):
    """Wq int8 [n, k], s_w fp32 [1] or [n] -> W_hat [n, k] in out_dtype (bf16 or fp16)."""
    _need(wq, "wq", torch.int8, 2)
    n, k = wq.shape
    _need_sw(s_w, per_channel, n)
    out = torch.empty((n, k), dtype=out_dtype, device=wq.device) if out is None else out
    dt = _need16(out, "out", 2)
    _same_device(wq, s_w, out)
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_dequant_derotate_ex(_ptr(wq), _ptr(s_w), mode, n, k, g,
                                                      rot_seed, _ptr(out), dt, _stream(wq)))
    return out


def convrot_gemm_int8_ex(xq: torch.Tensor, s_x: torch.Tensor, wq: torch.Tensor,
                         s_w: torch.Tensor, bias: torch.Tensor | None = None, *,
                         per_channel: bool = False, dtype: torch.dtype = torch.bfloat16,
                         want_y: bool = True, want_acc: bool = False,
                         y: torch.Tensor | None = None, acc: torch.Tensor | None = None,
                         tile: int = 0):
    """int8 GEMM + epilogue with bias and y in `dtype` (bf16 or fp16)."""
    if dtype not in _DTYPES:
        raise TypeError("dtype must be torch.bfloat16 or torch.float16")
    _need(xq, "xq", torch.int8, 2)
    _need(wq, "wq", torch.int8, 2)
    _need(s_x, "s_x", torch.float32, 1)
    m, k = xq.shape
    n = wq.shape[0]
    _need_sw(s_w, per_channel, n)
    if wq.shape[1] != k:
        raise ValueError(f"K mismatch: xq {tuple(xq.shape)} vs wq {tuple(wq.shape)}")
    if bias is not None:
        _need(bias, "bias", dtype, 1)
    if want_y and y is None:
        y = torch.empty((m, n), dtype=dtype, device=xq.device)
    if want_acc and acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=xq.device)
    if y is not None:
        _need(y, "y", dtype, 2)
    if acc is not None:
        _need(acc, "acc", torch.int32, 2)
    _same_device(xq, s_x, wq, s_w, bias, y, acc)
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_gemm_int8_ex(_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), mode,
                                               _ptr(bias), m, n, k, _ptr(y), _ptr(acc),
                                               _DTYPES[dtype], tile, _stream(xq)))
    return y, acc


def convrot_linear_int8_ex(x: torch.Tensor, wq: torch.Tensor, s_w: torch.Tensor, g: int,
                           rot_seed: int = ROT_SEED, bias: torch.Tensor | None = None, *,
                           per_channel: bool = False, workspace: torch.Tensor | None = None,
                           out: torch.Tensor | None = None):
    """The int8_compute forward in x's format (bf16 or fp16): bias and y too."""
    dt = _need16(x, "x", 2)
    _need(wq, "wq", torch.int8, 2)
    m, k = x.shape
    n = wq.shape[0]
    _need_sw(s_w, per_channel, n)
    if bias is not None:
        _need(bias, "bias", x.dtype, 1)
    if workspace is None:
        workspace = torch.empty(max(convrot_linear_int8_workspace_size(m, n, k), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8)
    out = torch.empty((m, n), dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out", x.dtype, 2)
    _same_device(x, wq, s_w, bias, workspace, out)
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_linear_int8_ex(_ptr(x), _ptr(wq), _ptr(s_w), mode, _ptr(bias),
                                                 m, n, k, g, rot_seed, _ptr(out), dt,
                                                 _ptr(workspace), workspace.numel(),
                                                 _stream(x)))
    return out


# ---------------------------------------------------------------------------
# Host-streamed int8 layers
# ---------------------------------------------------------------------------

def convrot_streamer_create(slot_bytes: int, slots: int = 2) -> ctypes.c_void_p:
    """A streamer with `slots` device staging buffers of slot_bytes each, on
    the current device. Free it with convrot_streamer_destroy."""
    h = ctypes.c_void_p()
    _check(load_library().convrot_streamer_create(slot_bytes, slots, ctypes.byref(h)))
    return h


def convrot_streamer_destroy(streamer: ctypes.c_void_p) -> None:
    _check(load_library().convrot_streamer_destroy(streamer))


def convrot_streamer_linear_int8(streamer: ctypes.c_void_p, x: torch.Tensor,
                                 wq_host: torch.Tensor, s_w: torch.Tensor, g: int,
                                 rot_seed: int = ROT_SEED, bias: torch.Tensor | None = None, *,
                                 per_channel: bool = False, workspace: torch.Tensor | None = None,
                                 out: torch.Tensor | None = None):
    """convrot_linear_int8_ex with the int8 weight in host memory (pinned for
    an asynchronous copy): copied into the streamer's next slot, then used."""
    dt = _need16(x, "x", 2)
    if not isinstance(wq_host, torch.Tensor) or wq_host.dtype != torch.int8 or wq_host.dim() != 2:
        raise TypeError("wq_host must be a 2-D int8 tensor")
    if not wq_host.is_contiguous():
        raise ValueError("wq_host must be contiguous")
    m, k = x.shape
    n = wq_host.shape[0]
    if wq_host.shape[1] != k:
        raise ValueError(f"K mismatch: x {tuple(x.shape)} vs wq_host {tuple(wq_host.shape)}")
    _need_sw(s_w, per_channel, n)
    if bias is not None:
        _need(bias, "bias", x.dtype, 1)
    if workspace is None:
        workspace = torch.empty(max(convrot_linear_int8_workspace_size(m, n, k), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8)
    out = torch.empty((m, n), dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out", x.dtype, 2)
    _same_device(x, s_w, bias, workspace, out)
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_streamer_linear_int8(
        streamer, _ptr(x), dt, _ptr(wq_host), _ptr(s_w), mode, _ptr(bias), m, n, k, g, rot_seed,
        _ptr(out), _ptr(workspace), workspace.numel(), _stream(x)))
    return out


class Streamer:
    """Owns a convrot_streamer: `with Streamer(slot_bytes) as s: s.linear(...)`."""

    def __init__(self, slot_bytes: int, slots: int = 2):
        self.handle = convrot_streamer_create(slot_bytes, slots)

    def linear(self, x, wq_host, s_w, g, rot_seed=ROT_SEED, bias=None, **kw):
        return convrot_streamer_linear_int8(self.handle, x, wq_host, s_w, g, rot_seed, bias, **kw)

    def close(self):
        if self.handle is not None:
            convrot_streamer_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


# ---------------------------------------------------------------------------
# Sessions: first-call tile tuning and check against the default path
# ---------------------------------------------------------------------------

def convrot_session_create(check_tolerance: float = 0.0) -> ctypes.c_void_p:
    """A session on the current device (check_tolerance <= 0: 0.1)."""
    h = ctypes.c_void_p()
    _check(load_library().convrot_session_create(check_tolerance, ctypes.byref(h)))
    return h


def convrot_session_destroy(session: ctypes.c_void_p) -> None:
    _check(load_library().convrot_session_destroy(session))


def convrot_session_linear_int8(session: ctypes.c_void_p, x: torch.Tensor, wq: torch.Tensor,
                                s_w: torch.Tensor, g: int, rot_seed: int = ROT_SEED,
                                bias: torch.Tensor | None = None, *, per_channel: bool = False,
                                workspace: torch.Tensor | None = None,
                                out: torch.Tensor | None = None):
    """convrot_linear_int8_ex through a session: the first call for each
    (shape, token bucket) tunes the GEMM tile and checks the result against
    the default path; a failed check raises ConvrotError (CONVROT_E_SELFCHECK)
    now and on every later call."""
    dt = _need16(x, "x", 2)
    _need(wq, "wq", torch.int8, 2)
    m, k = x.shape
    n = wq.shape[0]
    _need_sw(s_w, per_channel, n)
    if bias is not None:
        _need(bias, "bias", x.dtype, 1)
    if workspace is None:
        workspace = torch.empty(max(convrot_linear_int8_workspace_size(m, n, k), 1),
                                dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8)
    out = torch.empty((m, n), dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out", x.dtype, 2)
    _same_device(x, wq, s_w, bias, workspace, out)
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_session_linear_int8(
        session, _ptr(x), dt, _ptr(wq), _ptr(s_w), mode, _ptr(bias), m, n, k, g, rot_seed,
        _ptr(out), _ptr(workspace), workspace.numel(), _stream(x)))
    return out


def convrot_session_lookup(session: ctypes.c_void_p, m: int, n: int, k: int, g: int,
                           dtype: torch.dtype = torch.bfloat16, per_channel: bool = False):
    """(tile, check_error, latched) kept for a key; ConvrotError if the key
    has had no first call."""
    tile, err, latched = ctypes.c_int(), ctypes.c_double(), ctypes.c_int()
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_session_lookup(session, m, n, k, g, _DTYPES[dtype], mode,
                                                 ctypes.byref(tile), ctypes.byref(err),
                                                 ctypes.byref(latched)))
    return tile.value, err.value, bool(latched.value)


def convrot_session_export(session: ctypes.c_void_p) -> str:
    """The session's tuned tiles as text (one line per key), for
    convrot_session_import in a later process."""
    lib = load_library()
    need = lib.convrot_session_export(session, None, 0)
    if need == 0:
        raise ConvrotError(1, lib.convrot_last_error_string().decode())
    buf = ctypes.create_string_buffer(need)
    lib.convrot_session_export(session, buf, need)
    return buf.value.decode("ascii")


def convrot_session_import(session: ctypes.c_void_p, text: str) -> None:
    """Give the keys of exported text their tiles: their first calls skip the
    timing (the check still runs). Malformed text raises, importing nothing."""
    _check(load_library().convrot_session_import(session, text.encode("ascii")))


class Session:
    """Owns a convrot_session: `with Session() as s: s.linear(...)`."""

    def __init__(self, check_tolerance: float = 0.0):
        self.handle = convrot_session_create(check_tolerance)

    def linear(self, x, wq, s_w, g, rot_seed=ROT_SEED, bias=None, **kw):
        return convrot_session_linear_int8(self.handle, x, wq, s_w, g, rot_seed, bias, **kw)

    def lookup(self, m, n, k, g, dtype=torch.bfloat16, per_channel=False):
        return convrot_session_lookup(self.handle, m, n, k, g, dtype, per_channel)

    def export_tiles(self) -> str:
        return convrot_session_export(self.handle)

    def import_tiles(self, text: str) -> None:
        convrot_session_import(self.handle, text)

    def close(self):
        if self.handle is not None:
            convrot_session_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def convrot_linear_int8_noalloc(x: torch.Tensor, wq: torch.Tensor, s_w: torch.Tensor, g: int,
                                rot_seed: int = ROT_SEED, bias: torch.Tensor | None = None, *,
                                per_channel: bool = False, out: torch.Tensor | None = None):
    """convrot_linear_int8_ex without a workspace: the library's per-device
    scratch array holds the token slices, so the call allocates nothing (pass
    `out` to allocate nothing on this side either). Calls that overlap in time
    on one device race on the scratch."""
    dt = _need16(x, "x", 2)
    _need(wq, "wq", torch.int8, 2)
    m, k = x.shape
    n = wq.shape[0]
    _need_sw(s_w, per_channel, n)
    if bias is not None:
        _need(bias, "bias", x.dtype, 1)
    out = torch.empty((m, n), dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out", x.dtype, 2)
    _same_device(x, wq, s_w, bias, out)
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_linear_int8_noalloc(_ptr(x), _ptr(wq), _ptr(s_w), mode,
                                                      _ptr(bias), m, n, k, g, rot_seed,
                                                      _ptr(out), dt, _stream(x)))
    return out


def convrot_dequant_derotate_batched(wqs, s_ws, g: int, rot_seed: int = ROT_SEED, *,
                                     per_channel: bool = False,
                                     out_dtype: torch.dtype = torch.bfloat16, outs=None):
    """W_hat of every (wq, s_w) pair in one batched call (launches of up to 48
    weights): the list of each weight's int8 [n, k] and scale; returns the
    list of outputs [n, k] in out_dtype (or fills `outs`)."""
    if len(wqs) != len(s_ws):
        raise ValueError("one scale per weight")
    if outs is None:
        outs = [torch.empty(w.shape, dtype=out_dtype, device=w.device) for w in wqs]
    if len(outs) != len(wqs):
        raise ValueError("one output per weight")
    jobs = (_DequantJob * max(len(wqs), 1))()
    dt = None
    for i, (wq, s_w, out) in enumerate(zip(wqs, s_ws, outs)):
        _need(wq, "wq", torch.int8, 2)
        n, k = wq.shape
        _need_sw(s_w, per_channel, n)
        d = _need16(out, "out", 2)
        if dt is not None and d != dt:
            raise TypeError("every output has the same format")
        dt = d
        if tuple(out.shape) != (n, k):
            raise ValueError(f"output {i} has shape {tuple(out.shape)}, want {(n, k)}")
        _same_device(wq, s_w, out, wqs[0])
        jobs[i] = _DequantJob(wq.data_ptr(), s_w.data_ptr(), out.data_ptr(), n, k)
    if not wqs:
        return outs
    mode = _SCALE_PER_CHANNEL if per_channel else _SCALE_PER_TENSOR
    _check(load_library().convrot_dequant_derotate_batched(jobs, len(wqs), mode, g, rot_seed, dt,
                                                           _stream(wqs[0])))
    return outs
