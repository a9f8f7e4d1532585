"""MI355X-native FP16 grouped-query-attention single-token decode.

Thin Python binding over the C ABI of ``libgqa_decode.so``
(``include/gqa_decode.h``): argument checks and marshalling only. Every step
of the decode runs in the library's HIP kernels; there is no fallback. If
the library has not been built, calls raise ``RuntimeError``.

PyTorch supplies device memory and the current stream; the decode itself
never goes through torch operators.

Public API (names and keyword arguments follow the ``sm110_gqa_decode``
entry point documented on the FlashInfer PR #5052 analysis page, section 1;
bf16 tensors and the K/V scales are this library's extension):
    gqa_decode(q, kv, sequence_lengths, *, out=None, q_scale=1.0, chunk_len=0,
               k_scale=1.0, v_scale=1.0)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # must load before the library so both share one HIP runtime

__all__ = ["gqa_decode", "workspace_bytes", "release_workspace", "library_path",
           "load_library", "KernelTimer", "GqaDecodeError",
           "NUM_Q_HEADS", "NUM_KV_HEADS", "HEAD_DIM"]

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 128

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgqa_decode.so"
_lib = None


class GqaDecodeError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"gqa_decode failed with status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG_DIR, _LIB_NAME)


def load_library():
    """Load (once) and return the ctypes handle of libgqa_decode.so."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m gqa_token_decode_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, f32, i32, i32, vp]
    lib.gqa_decode.restype = i32
    lib.gqa_decode_chunked.argtypes = [vp, vp, vp, vp, f32, i32, i32, i32, vp]
    lib.gqa_decode_chunked.restype = i32
    lib.gqa_decode_typed.argtypes = [vp, vp, vp, vp, i32, f32, f32, f32, i32, i32, i32, vp]
    lib.gqa_decode_typed.restype = i32
    lib.gqa_decode_workspace_bytes.argtypes = [i32, i32]
    lib.gqa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.gqa_decode_release_workspace.argtypes = []
    lib.gqa_decode_release_workspace.restype = None
    lib.gqa_decode_status_string.argtypes = [i32]
    lib.gqa_decode_status_string.restype = ctypes.c_char_p
    lib.gqa_decode_last_error.argtypes = []
    lib.gqa_decode_last_error.restype = ctypes.c_char_p
    lib.gqa_decode_profile_begin.argtypes = []
    lib.gqa_decode_profile_begin.restype = i32
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gqa_decode_profile_end.argtypes = [dp, dp, ctypes.POINTER(i32)]
    lib.gqa_decode_profile_end.restype = i32
    _lib = lib
    return lib


def _raise(lib, status: int):
    msg = lib.gqa_decode_last_error().decode() or lib.gqa_decode_status_string(status).decode()
    raise GqaDecodeError(status, msg)


def _check_tensor(name, t, dtype, shape_len):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.dim() != shape_len:
        raise ValueError(f"{name} must have {shape_len} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_device(name, t):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")


_DTYPES = {torch.float16: 0, torch.bfloat16: 1}   # gqa_dtype codes
_E4M3_KV = 2
_FP8_KV_DTYPES = tuple(t for t in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if t is not None)


def gqa_decode(q: torch.Tensor, kv: torch.Tensor, sequence_lengths: torch.Tensor, *,
               out: Optional[torch.Tensor] = None, q_scale: float = 1.0,
               chunk_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Decode one token of GQA (32 query heads, 8 KV heads, dim 128).

    q: fp16 or bf16 [batch, 32, 128]; kv: same dtype [batch, 2, 8, capacity,
    128] with K at index 0 and V at index 1 of axis 1, or, with fp16 q, an
    OCP FP8 E4M3 cache (torch.float8_e4m3fn, or uint8 holding E4M3 bytes)
    dequantised by k_scale and v_scale; sequence_lengths:
    int32 [batch] on the same device (values clamped to [0, capacity]).
    ``out`` (optional, caller-owned, q's dtype and shape) receives the result
    and is returned; otherwise a new tensor is allocated. Scores are scaled by
    ``q_scale * k_scale / sqrt(128)`` and the output by ``v_scale``.
    ``chunk_len`` > 0 fixes the split-KV piece length (0 = automatic).
    Enqueued on the current stream of q's device.
    """
    if isinstance(q, torch.Tensor) and q.dtype in _DTYPES:
        dtype = q.dtype
    else:
        dtype = torch.float16
    fp8_kv = (dtype == torch.float16 and isinstance(kv, torch.Tensor)
              and kv.dtype in _FP8_KV_DTYPES)
    _check_tensor("q", q, dtype, 3)
    _check_tensor("kv", kv, kv.dtype if fp8_kv else dtype, 5)
    _check_tensor("sequence_lengths", sequence_lengths, torch.int32, 1)
    B = q.shape[0]
    kshape = kv.shape
    if q.shape[1] != NUM_Q_HEADS or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must have shape [batch, 32, 128], got {tuple(q.shape)}")
    if kshape[0] != B or kshape[1] != 2 or kshape[2] != NUM_KV_HEADS or kshape[4] != HEAD_DIM:
        raise ValueError(f"kv must have shape [{B}, 2, 8, capacity, 128], got {tuple(kshape)}")
    if sequence_lengths.shape[0] != B:
        raise ValueError(f"sequence_lengths must have shape [{B}], got {tuple(sequence_lengths.shape)}")
    dev = q.device
    if dev.type != "cuda":
        _check_device("q", q)
    if kv.device != dev or sequence_lengths.device != dev:
        for name, t in (("kv", kv), ("sequence_lengths", sequence_lengths)):
            _check_device(name, t)
        raise ValueError("q, kv and sequence_lengths must be on the same device")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, dtype, 3)
        if out.shape != q.shape or out.device != dev:
            _check_device("out", out)
            raise ValueError("out must have q's shape and device")
    if chunk_len.__class__ is not int or chunk_len < 0:
        raise ValueError("chunk_len must be a non-negative int")
    lib = _lib if _lib is not None else load_library()
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    stream = torch._C._cuda_getCurrentRawStream(index)
    if fp8_kv or dtype != torch.float16 or k_scale != 1.0 or v_scale != 1.0:
        code = _E4M3_KV if fp8_kv else _DTYPES[dtype]
        st = lib.gqa_decode_typed(q.data_ptr(), kv.data_ptr(), sequence_lengths.data_ptr(),
                                  out.data_ptr(), code, float(q_scale), float(k_scale),
                                  float(v_scale), B, kshape[3], chunk_len, stream)
    elif chunk_len:
        st = lib.gqa_decode_chunked(q.data_ptr(), kv.data_ptr(), sequence_lengths.data_ptr(),
                                    out.data_ptr(), float(q_scale), B, kshape[3], chunk_len,
                                    stream)
    else:
        st = lib.gqa_decode(q.data_ptr(), kv.data_ptr(), sequence_lengths.data_ptr(),
                            out.data_ptr(), float(q_scale), B, kshape[3], stream)
    if st != 0:
        _raise(lib, st)
    return out


def workspace_bytes(batch: int, capacity: int) -> int:
    return int(load_library().gqa_decode_workspace_bytes(batch, capacity))


def release_workspace() -> None:
    load_library().gqa_decode_release_workspace()


class KernelTimer:
    """Context manager: HIP-event timing of the decode kernels launched inside.

    After exit, ``pieces_ms`` and ``combine_ms`` hold the summed durations of
    the split-KV pieces kernel and of the combine kernel (events recorded by
    the library on each call's stream), and ``calls`` the number of calls.
    """

    def __enter__(self):
        lib = load_library()
        st = lib.gqa_decode_profile_begin()
        if st != 0:
            _raise(lib, st)
        return self

    def __exit__(self, *exc):
        lib = load_library()
        p, c, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
        st = lib.gqa_decode_profile_end(ctypes.byref(p), ctypes.byref(c), ctypes.byref(n))
        self.pieces_ms, self.combine_ms, self.calls = p.value, c.value, n.value
        if st != 0 and exc[0] is None:
            _raise(lib, st)
        return False
