"""ctypes binding of libtf_exl3.so (the C ABI declared in include/tf_exl3.h).

Marshalling only: torch tensors supply device memory and the current HIP
stream; every step of the projection runs in the library's kernels. If the
library is missing, loading fails loudly: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libtf_exl3.so"
HEADER = PKG.parent / "include" / "tf_exl3.h"

TF_DT_F32, TF_DT_F16, TF_DT_BF16 = 0, 1, 2
TF_OK = 0
STATUS = {
    0: "TF_OK", -1: "TF_E_BITS", -2: "TF_E_SHAPE", -3: "TF_E_ROWS", -4: "TF_E_DTYPE",
    -5: "TF_E_NULL", -6: "TF_E_ALIGN", -7: "TF_E_ALIAS", -8: "TF_E_WAVES", -9: "TF_E_LAUNCH",
}


class Exl3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [
        ("width_index", ctypes.c_int),
        ("waves", ctypes.c_int),
        ("threads", ctypes.c_int),
        ("grid_x", ctypes.c_int),
        ("passes", ctypes.c_int),
        ("rows_last_pass", ctypes.c_int),
        ("rows_kernel", ctypes.c_int),
        ("lds_bytes", ctypes.c_int),
        ("column_split", ctypes.c_int),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "tf_exl3_rot_in": (_I, [_P, _I, _P, _P, _I, _I, _P]),
    "tf_exl3_linear": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P]),
    "tf_exl3_linear_mfma": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P]),
    "tf_exl3_linear_prompt": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P]),
    "tf_exl3_linear_strips": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P]),
    "tf_exl3_repack_strips": (_I, [_I, _I, _I, _P, _P, _P]),
    "tf_exl3_debug_linear_split": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _I, _P]),
    "tf_exl3_debug_linear_mfma_split": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _I, _P]),
    "tf_exl3_project": (_I, [_I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _I, _I, _P]),
    "tf_exl3_project_pass_rows": (_I, [_I, _I, _I, _I]),
    "tf_exl3_linear_plan": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(Plan)]),
    "tf_exl3_trellis_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "tf_exl3_status_string": (ctypes.c_char_p, [_I]),
    "tf_exl3_debug_decode_states": (_I, [_P, _P, _I, _P]),
    "tf_exl3_debug_decode_tiles": (_I, [_I, _I, _I, _P, _P, _P]),
    "tf_exl3_calib_copy": (_I, [_P, _P, ctypes.c_size_t, _I, _P]),
    "tf_exl3_calib_stream_read": (_I, [_P, ctypes.c_size_t, _P, _I, _P]),
}

_lib = None


def load(path: str | os.PathLike | None = None) -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise ImportError(
            f"{p} is missing: build it with __graft_entry__.build() or "
            "python trellis_quantized_linear_tf_amd/_build.py (hipcc, gfx950)"
        )
    lib = ctypes.CDLL(str(p))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/tf_exl3.h declares."""
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-zA-Z_][\w\s\*]*?\b(tf_exl3_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return load().tf_exl3_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != TF_OK:
        raise Exl3Error(status, status_string(status))


def trellis_bytes(bits: int, in_dim: int, out_dim: int) -> int:
    return int(load().tf_exl3_trellis_bytes(bits, in_dim, out_dim))


def linear_plan(bits: int, rows: int, in_dim: int, out_dim: int, waves: int = 0) -> dict:
    p = Plan()
    _check(load().tf_exl3_linear_plan(bits, rows, in_dim, out_dim, waves, ctypes.byref(p)))
    return p.as_dict()


# ---------------------------------------------------------------------------
# Tensor entry points (torch supplies memory and the stream).


def _torch():
    import torch

    return torch


# Element types, built once on first use (torch is imported lazily).
_DTYPES = None


def _dtypes():
    global _DTYPES
    if _DTYPES is None:
        torch = _torch()
        _DTYPES = (
            (torch.float16, torch.int16),  # fp16 bit patterns (z, suh, svh)
            (torch.float32, torch.float16, torch.bfloat16),  # rows and outputs
            {torch.float32: TF_DT_F32, torch.float16: TF_DT_F16, torch.bfloat16: TF_DT_BF16},
        )
    return _DTYPES


def _dt_code(dtype) -> int:
    code = _dtypes()[2].get(dtype)
    if code is None:
        raise ValueError(f"unsupported element type {dtype}")
    return code


def _ptr(t) -> int | None:
    """Device address of a tensor that _same_gpu has accepted (None stays NULL)."""
    return None if t is None else t.data_ptr()


# Argument checks. The C ABI sees plain pointers, not buffer sizes, so a short
# stream or a wrong-shaped output would become an out-of-bounds device access,
# and an fp32 tensor passed where fp16 bits are read would be misread silently.
# Every wrapper checks element types, shapes and byte sizes first (these checks
# need no GPU), then that all tensors are contiguous and on one GPU. They run on
# every call, so they are kept to attribute reads and comparisons.


def _half_bits_dtypes():
    return _dtypes()[0]


def _row_dtypes():
    return _dtypes()[1]


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need(name: str, t, dtypes=None, shape=None, nbytes=None) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must have element type {' or '.join(map(str, dtypes))}, not {t.dtype}")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if nbytes is not None and t.numel() * t.element_size() != nbytes:
        raise ValueError(f"{name} must hold {nbytes} bytes, not {_nbytes(t)}")


def _need_2d(name: str, t) -> tuple:
    if t is None or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor [rows][dim]")
    return tuple(t.shape)


_WIDTH_SET = frozenset((2, 3, 4, 5, 6, 8))


def _stream_bytes(bits: int, in_dim: int, out_dim: int) -> int | None:
    """Stream size the library expects (tf_exl3_trellis_bytes' rule, evaluated here so
    that a call costs no extra library round trip; a host test checks the two agree),
    or None where the library refuses the shape (it then returns its status before any
    launch)."""
    if bits not in _WIDTH_SET or in_dim < 128 or out_dim < 128 or in_dim % 128 or out_dim % 128:
        return None
    n = in_dim * out_dim * bits // 8
    return n if n < (1 << 32) else None


def _same_gpu(*tensors) -> None:
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        d = t.get_device()
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError("all tensors must be on one GPU")


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.get_device()).cuda_stream


def rot_in(x, suh, z=None):
    """z[rows][in_dim] fp16 = rot_in(x, suh); x is fp32/fp16/bf16 [rows][in_dim], suh fp16 [in_dim]."""
    torch = _torch()
    rows, in_dim = _need_2d("x", x)
    _need("x", x, _row_dtypes())
    _need("suh", suh, _half_bits_dtypes(), (in_dim,))
    if z is not None:
        _need("z", z, _half_bits_dtypes(), (rows, in_dim))
    _same_gpu(x, suh, z)
    if z is None:
        z = torch.empty((rows, in_dim), dtype=torch.float16, device=x.device)
    _check(load().tf_exl3_rot_in(_ptr(x), _dt_code(x.dtype), _ptr(suh), _ptr(z), rows, in_dim, _stream(x)))
    return z


ENGINES = ("dot2", "mfma", "prompt", "strips")


def _check_linear_args(z, trellis, svh, bits: int, out_dim: int, y, out_dtype) -> tuple:
    """Shapes, element types and the stream's size of a linear call; returns (rows, in_dim)."""
    rows, in_dim = _need_2d("z", z)
    _need("z", z, _half_bits_dtypes())
    _need("trellis", trellis, nbytes=_stream_bytes(bits, in_dim, out_dim))
    _need("svh", svh, _half_bits_dtypes(), (out_dim,))
    if y is not None:
        _need("y", y, _row_dtypes(), (rows, out_dim))
    elif out_dtype is not None and out_dtype not in _row_dtypes():
        raise ValueError(f"out_dtype must be one of {_row_dtypes()}")
    _same_gpu(z, trellis, svh, y)
    return rows, in_dim


def linear(z, trellis, svh, bits: int, out_dim: int, y=None, out_dtype=None, waves: int = 0,
           engine: str = "dot2"):
    """y[rows][out_dim] = the trellis linear of fp16 z [rows][in_dim] (trellis: uint8/int32 stream).
    engine "dot2" runs tf_exl3_linear, "mfma" tf_exl3_linear_mfma, "prompt"
    tf_exl3_linear_prompt (32-row passes, bit-equal to "dot2") and "strips"
    tf_exl3_linear_strips (trellis in the strips layout, see repack_strips)."""
    torch = _torch()
    if engine not in ENGINES:
        raise ValueError(f"engine must be one of {ENGINES}")
    rows, in_dim = _check_linear_args(z, trellis, svh, bits, out_dim, y, out_dtype)
    if y is None:
        y = torch.empty((rows, out_dim), dtype=out_dtype or torch.float32, device=z.device)
    lib = load()
    fn = {"dot2": lib.tf_exl3_linear, "mfma": lib.tf_exl3_linear_mfma, "prompt": lib.tf_exl3_linear_prompt,
          "strips": lib.tf_exl3_linear_strips}[engine]
    _check(fn(bits, rows, in_dim, out_dim, _ptr(z), _ptr(trellis), _ptr(svh), _ptr(y), _dt_code(y.dtype), waves,
              _stream(z)))
    return y


def repack_strips(trellis, bits: int, in_dim: int, out_dim: int, out=None):
    """The strips-layout image of a tile-layout stream (tf_exl3_repack_strips)."""
    torch = _torch()
    n = _stream_bytes(bits, in_dim, out_dim)
    _need("trellis", trellis, nbytes=n)
    if out is not None:
        _need("out", out, nbytes=n)
    _same_gpu(trellis, out)
    if out is None:
        out = torch.empty_like(trellis)
    _check(load().tf_exl3_repack_strips(bits, in_dim, out_dim, _ptr(trellis), _ptr(out), _stream(trellis)))
    return out


def project(x, suh, trellis, svh, bits: int, out_dim: int, y=None, out_dtype=None, waves: int = 0):
    """y = linear(rot_in(x)) in one launch (bit-identical to rot_in then linear with engine "dot2")."""
    torch = _torch()
    rows, in_dim = _need_2d("x", x)
    _need("x", x, _row_dtypes())
    _need("suh", suh, _half_bits_dtypes(), (in_dim,))
    _need("trellis", trellis, nbytes=_stream_bytes(bits, in_dim, out_dim))
    _need("svh", svh, _half_bits_dtypes(), (out_dim,))
    if y is not None:
        _need("y", y, _row_dtypes(), (rows, out_dim))
    elif out_dtype is not None and out_dtype not in _row_dtypes():
        raise ValueError(f"out_dtype must be one of {_row_dtypes()}")
    _same_gpu(x, suh, trellis, svh, y)
    if y is None:
        y = torch.empty((rows, out_dim), dtype=out_dtype or torch.float32, device=x.device)
    _check(load().tf_exl3_project(bits, rows, in_dim, out_dim, _ptr(x), _dt_code(x.dtype), _ptr(suh),
                                  _ptr(trellis), _ptr(svh), _ptr(y), _dt_code(y.dtype), waves, _stream(x)))
    return y


def project_pass_rows(rows: int, in_dim: int, out_dim: int, waves: int = 0) -> int:
    r = load().tf_exl3_project_pass_rows(rows, in_dim, out_dim, waves)
    _check(min(r, 0))
    return r


def debug_decode_states(states):
    """fp16 weights (as int16 bits) of uint16 states given as an int16/int32 tensor of 16-bit values."""
    torch = _torch()
    _same_gpu(states)
    s = states.to(torch.int16) if states.dtype != torch.int16 else states
    w = torch.empty_like(s)
    _check(load().tf_exl3_debug_decode_states(_ptr(s), _ptr(w), s.numel(), _stream(s)))
    return w


def debug_decode_tiles(trellis, bits: int, in_dim: int, out_dim: int):
    """W[in_dim][out_dim] as fp16 decoded by the linear's own decode path."""
    torch = _torch()
    _need("trellis", trellis, nbytes=_stream_bytes(bits, in_dim, out_dim))
    _same_gpu(trellis)
    w = torch.empty((in_dim, out_dim), dtype=torch.float16, device=trellis.device)
    _check(load().tf_exl3_debug_decode_tiles(bits, in_dim, out_dim, _ptr(trellis), _ptr(w), _stream(trellis)))
    return w


def debug_linear_split(z, trellis, svh, bits: int, out_dim: int, split: int, y=None, out_dtype=None,
                       waves: int = 0):
    """tf_exl3_linear with every launch forced to the regular (split 0) or the
    column-split (split 1) kernels (tf_exl3_debug_linear_split)."""
    torch = _torch()
    rows, in_dim = _check_linear_args(z, trellis, svh, bits, out_dim, y, out_dtype)
    if y is None:
        y = torch.empty((rows, out_dim), dtype=out_dtype or torch.float32, device=z.device)
    _check(load().tf_exl3_debug_linear_split(bits, rows, in_dim, out_dim, _ptr(z), _ptr(trellis), _ptr(svh), _ptr(y),
                                             _dt_code(y.dtype), waves, split, _stream(z)))
    return y


def debug_linear_mfma_split(z, trellis, svh, bits: int, out_dim: int, split: int, y=None, out_dtype=None,
                            waves: int = 0):
    """tf_exl3_linear_mfma with its form forced: split 0 (one workgroup's waves per strip)
    or split 1 (the column-split form, 4 waves only) (tf_exl3_debug_linear_mfma_split)."""
    torch = _torch()
    rows, in_dim = _check_linear_args(z, trellis, svh, bits, out_dim, y, out_dtype)
    if y is None:
        y = torch.empty((rows, out_dim), dtype=out_dtype or torch.float32, device=z.device)
    _check(load().tf_exl3_debug_linear_mfma_split(bits, rows, in_dim, out_dim, _ptr(z), _ptr(trellis), _ptr(svh),
                                                  _ptr(y), _dt_code(y.dtype), waves, split, _stream(z)))
    return y


def calib_copy(src, dst, blocks: int = 2048):
    """dst <- src byte for byte (both contiguous device tensors of equal byte size)."""
    nbytes = _nbytes(src)
    _need("dst", dst, nbytes=nbytes)
    _same_gpu(src, dst)
    _check(load().tf_exl3_calib_copy(_ptr(src), _ptr(dst), nbytes, blocks, _stream(src)))


def calib_stream_read(src, out):
    """Reads all of src; out is an int32 tensor of blocks * 256 entries."""
    torch = _torch()
    nbytes = _nbytes(src)
    _need("out", out, (torch.int32,))
    if out.numel() < 256 or out.numel() % 256:
        raise ValueError("out must hold a positive multiple of 256 int32 words (one per thread)")
    blocks = out.numel() // 256
    _same_gpu(src, out)
    _check(load().tf_exl3_calib_stream_read(_ptr(src), nbytes, _ptr(out), blocks, _stream(src)))
