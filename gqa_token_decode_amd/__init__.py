"""MI355X-native FP16 grouped-query-attention single-token decode.

Thin Python binding over the C ABI of ``libgqa_decode.so``
(``include/gqa_decode.h``): argument checks and marshalling only. Every step
of the decode runs in the library's HIP kernels; there is no fallback. If
the library has not been built, calls raise ``RuntimeError``.

PyTorch supplies device memory and the current stream; the decode itself
never goes through torch operators.

Public API (names and keyword arguments follow the ``sm110_gqa_decode``
entry point documented on the FlashInfer PR #5052 analysis page, section 1;
bf16 tensors, the K/V scales, other head counts and paged caches are this
library's extension):
    gqa_decode(q, kv, sequence_lengths, *, out=None, q_scale=1.0, chunk_len=0,
               k_scale=1.0, v_scale=1.0)
    gqa_decode_paged(q, kv_pages, block_table, sequence_lengths, *, ...)
    gqa_decode_fp4(q, kv_codes, kv_scales, sequence_lengths, *, block_table=None, ...)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # must load before the library so both share one HIP runtime

__all__ = ["gqa_decode", "gqa_decode_paged", "gqa_decode_fp4", "gqa_decode_noalloc",
           "workspace_bytes", "release_workspace", "library_path",
           "load_library", "KernelTimer", "GqaDecodeError",
           "NUM_Q_HEADS", "NUM_KV_HEADS", "HEAD_DIM"]

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 128
MAX_GROUP = 8          # query heads per KV head, at most

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
    lib.gqa_decode_ex.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(_Layout), f32, f32, f32,
                                  i32, i32, i32, vp]
    lib.gqa_decode_ex.restype = i32
    lib.gqa_decode_ex_noalloc.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(_Layout), f32, f32,
                                          f32, i32, i32, i32, vp]
    lib.gqa_decode_ex_noalloc.restype = i32
    lib.gqa_decode_fp4.argtypes = [vp, vp, ctypes.POINTER(_BlockScales), vp, vp,
                                   ctypes.POINTER(_Layout), f32, f32, f32, i32, i32, i32, vp]
    lib.gqa_decode_fp4.restype = i32
    lib.gqa_decode_workspace_bytes.argtypes = [i32, i32]
    lib.gqa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.gqa_decode_release_workspace.argtypes = []
    lib.gqa_decode_release_workspace.restype = None
    lib.gqa_decode_status_string.argtypes = [i32]
    lib.gqa_decode_status_string.restype = ctypes.c_char_p
    lib.gqa_decode_last_error.argtypes = []
    lib.gqa_decode_last_error.restype = ctypes.c_char_p
    lib.gqa_decode_set_launch_form.argtypes = [i32]
    lib.gqa_decode_set_launch_form.restype = i32
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


class _Layout(ctypes.Structure):
    """struct gqa_layout of the C ABI (strides in elements)."""

    _fields_ = [("q_stride_batch", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
                ("kv_stride_batch", ctypes.c_int64), ("kv_stride_kind", ctypes.c_int64),
                ("kv_stride_head", ctypes.c_int64), ("kv_stride_row", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int),
                ("page_size", ctypes.c_int), ("num_pages", ctypes.c_int),
                ("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int)]


class _BlockScales(ctypes.Structure):
    """struct gqa_block_scales of the C ABI (strides in bytes)."""

    _fields_ = [("scales", ctypes.c_void_p), ("stride_batch", ctypes.c_int64),
                ("stride_kind", ctypes.c_int64), ("stride_head", ctypes.c_int64),
                ("stride_row", ctypes.c_int64)]


FP4_SCALES_PER_ROW = 8      # E4M3 block scales per head row (one per 16 elements)


def _check_view(name, t, dtype, shape_len):
    """A tensor whose innermost (head-dim) axis is contiguous; other axes may
    be strided (views into larger buffers)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.dim() != shape_len:
        raise ValueError(f"{name} must have {shape_len} dimensions, got shape {tuple(t.shape)}")
    if t.stride(-1) != 1 or any(st < 0 for st in t.stride()):
        raise ValueError(f"{name} must have a contiguous last axis and non-negative strides")


def _prepare(q, kv, sequence_lengths, out, kv_shape_check):
    """Type/shape/device checks shared by the entry points. Returns
    (dtype code, fp8 cache flag, out)."""
    if isinstance(q, torch.Tensor) and q.dtype in _DTYPES:
        dtype = q.dtype
    else:
        dtype = torch.float16
    fp8_kv = (dtype == torch.float16 and isinstance(kv, torch.Tensor)
              and kv.dtype in _FP8_KV_DTYPES)
    _check_view("q", q, dtype, 3)
    _check_view("kv", kv, kv.dtype if fp8_kv else dtype, 5)
    _check_tensor("sequence_lengths", sequence_lengths, torch.int32, 1)
    B, Hq = q.shape[0], q.shape[1]
    if q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must have shape [batch, heads, 128], got {tuple(q.shape)}")
    kv_shape_check(B)
    Hkv = kv.shape[2]
    if Hkv < 1 or Hq < 1 or Hq % Hkv != 0 or Hq // Hkv > MAX_GROUP:
        raise ValueError(f"{Hq} query heads over {Hkv} KV heads: need a positive multiple with "
                         f"at most {MAX_GROUP} query heads per KV head")
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
        out = torch.empty(q.shape, dtype=dtype, device=dev)
    else:
        _check_tensor("out", out, dtype, 3)
        if out.shape != q.shape or out.device != dev:
            _check_device("out", out)
            raise ValueError("out must have q's shape and device")
    return (_E4M3_KV if fp8_kv else _DTYPES[dtype]), fp8_kv, out


def _stream_of(dev):
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    return torch._C._cuda_getCurrentRawStream(index)


def _check_chunk(chunk_len):
    if chunk_len.__class__ is not int or chunk_len < 0:
        raise ValueError("chunk_len must be a non-negative int")


def gqa_decode(q: torch.Tensor, kv: torch.Tensor, sequence_lengths: torch.Tensor, *,
               out: Optional[torch.Tensor] = None, q_scale: float = 1.0,
               chunk_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Decode one token of GQA (32 query heads over 8 KV heads, dim 128, on
    the page; other head counts too).

    q: fp16 or bf16 [batch, Hq, 128]; kv: same dtype [batch, 2, Hkv,
    capacity, 128] with K at index 0 and V at index 1 of axis 1 (Hq a
    multiple of Hkv, at most 8 query heads per KV head; query head h reads
    KV head h // (Hq // Hkv)), or, with fp16 q, an
    OCP FP8 E4M3 cache (torch.float8_e4m3fn, or uint8 holding E4M3 bytes)
    dequantised by k_scale and v_scale; sequence_lengths:
    int32 [batch] on the same device (values clamped to [0, capacity]).
    q and kv may be strided views whose last axis is contiguous (e.g. q
    sliced from a packed projection, or an NHD cache [batch, capacity, 2, 8,
    128] permuted to this shape); no copy is made.
    ``out`` (optional, caller-owned, contiguous, q's dtype and shape)
    receives the result and is returned; otherwise a new tensor is allocated.
    Scores are scaled by ``q_scale * k_scale / sqrt(128)`` and the output by
    ``v_scale``. ``chunk_len`` > 0 fixes the split-KV piece length (0 =
    automatic). Enqueued on the current stream of q's device.
    """
    def kv_shape(B):
        ks = kv.shape
        if ks[0] != B or ks[1] != 2 or ks[4] != HEAD_DIM:
            raise ValueError(f"kv must have shape [{B}, 2, kv_heads, capacity, 128], "
                             f"got {tuple(ks)}")

    code, fp8_kv, out = _prepare(q, kv, sequence_lengths, out, kv_shape)
    _check_chunk(chunk_len)
    B, C = q.shape[0], kv.shape[3]
    Hq, Hkv = q.shape[1], kv.shape[2]
    lib = _lib if _lib is not None else load_library()
    stream = _stream_of(q.device)
    args = (q.data_ptr(), kv.data_ptr(), sequence_lengths.data_ptr(), out.data_ptr())
    if (not (q.is_contiguous() and kv.is_contiguous())
            or (Hq, Hkv) != (NUM_Q_HEADS, NUM_KV_HEADS)):
        lay = _Layout(q.stride(0), q.stride(1), kv.stride(0), kv.stride(1), kv.stride(2),
                      kv.stride(3), None, 0, 0, 0, Hq, Hkv)
        st = lib.gqa_decode_ex(*args, code, ctypes.byref(lay), float(q_scale), float(k_scale),
                               float(v_scale), B, C, chunk_len, stream)
    elif code != 0 or k_scale != 1.0 or v_scale != 1.0:
        st = lib.gqa_decode_typed(*args, code, float(q_scale), float(k_scale), float(v_scale),
                                  B, C, chunk_len, stream)
    elif chunk_len:
        st = lib.gqa_decode_chunked(*args, float(q_scale), B, C, chunk_len, stream)
    else:
        st = lib.gqa_decode(*args, float(q_scale), B, C, stream)
    if st != 0:
        _raise(lib, st)
    return out


def gqa_decode_noalloc(q: torch.Tensor, kv: torch.Tensor, sequence_lengths: torch.Tensor, *,
                       out: torch.Tensor, q_scale: float = 1.0, chunk_len: int = 0,
                       k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """gqa_decode through the allocation-free entry point
    (gqa_decode_ex_noalloc): the library takes its fixed device scratch
    instead of a cached workspace, and ``out`` must be given. Same tensors,
    results (bitwise) and errors as gqa_decode, except that shapes whose
    partial results do not fit the scratch raise GqaDecodeError
    (GQA_ERR_BAD_SHAPE). Calls on one device must not overlap.
    """
    def kv_shape(B):
        ks = kv.shape
        if ks[0] != B or ks[1] != 2 or ks[4] != HEAD_DIM:
            raise ValueError(f"kv must have shape [{B}, 2, kv_heads, capacity, 128], "
                             f"got {tuple(ks)}")

    if out is None:
        raise ValueError("gqa_decode_noalloc needs a caller-allocated out")
    code, _, out = _prepare(q, kv, sequence_lengths, out, kv_shape)
    _check_chunk(chunk_len)
    B, C, Hq, Hkv = q.shape[0], kv.shape[3], q.shape[1], kv.shape[2]
    lay = _Layout(q.stride(0), q.stride(1), kv.stride(0), kv.stride(1), kv.stride(2),
                  kv.stride(3), None, 0, 0, 0, Hq, Hkv)
    lib = _lib if _lib is not None else load_library()
    st = lib.gqa_decode_ex_noalloc(q.data_ptr(), kv.data_ptr(), sequence_lengths.data_ptr(),
                                   out.data_ptr(), code, ctypes.byref(lay), float(q_scale),
                                   float(k_scale), float(v_scale), B, C, chunk_len,
                                   _stream_of(q.device))
    if st != 0:
        _raise(lib, st)
    return out


def gqa_decode_paged(q: torch.Tensor, kv_pages: torch.Tensor, block_table: torch.Tensor,
                     sequence_lengths: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                     q_scale: float = 1.0, chunk_len: int = 0, k_scale: float = 1.0,
                     v_scale: float = 1.0) -> torch.Tensor:
    """Decode one token of GQA from a paged KV cache.

    kv_pages: [num_pages, 2, Hkv, page_size, 128] (HND pages; fp16, bf16 or an
    E4M3 cache as for gqa_decode; strided views with a contiguous last axis
    allowed), page_size a power of two >= 16. block_table: int32 [batch,
    max_pages] on the same device; position i of sequence b lives in page
    block_table[b, i // page_size]. Entries for positions at or beyond a
    sequence's length are never read. Lengths are clamped to
    max_pages * page_size. Other arguments as for gqa_decode.
    """
    def kv_shape(B):
        ks = kv_pages.shape
        if ks[1] != 2 or ks[4] != HEAD_DIM:
            raise ValueError(f"kv_pages must have shape [num_pages, 2, kv_heads, page_size, "
                             f"128], got {tuple(ks)}")
        _check_tensor("block_table", block_table, torch.int32, 2)
        if block_table.shape[0] != B:
            raise ValueError(f"block_table must have {B} rows, got {tuple(block_table.shape)}")

    code, _, out = _prepare(q, kv_pages, sequence_lengths, out, kv_shape)
    if block_table.device != q.device:
        _check_device("block_table", block_table)
        raise ValueError("block_table must be on q's device")
    _check_chunk(chunk_len)
    B = q.shape[0]
    num_pages, page_size = kv_pages.shape[0], kv_pages.shape[3]
    max_pages = block_table.shape[1]
    lay = _Layout(q.stride(0), q.stride(1), kv_pages.stride(0), kv_pages.stride(1),
                  kv_pages.stride(2), kv_pages.stride(3), block_table.data_ptr(), max_pages,
                  page_size, num_pages, q.shape[1], kv_pages.shape[2])
    lib = _lib if _lib is not None else load_library()
    st = lib.gqa_decode_ex(q.data_ptr(), kv_pages.data_ptr(), sequence_lengths.data_ptr(),
                           out.data_ptr(), code, ctypes.byref(lay), float(q_scale),
                           float(k_scale), float(v_scale), B, max_pages * page_size, chunk_len,
                           _stream_of(q.device))
    if st != 0:
        _raise(lib, st)
    return out


def gqa_decode_fp4(q: torch.Tensor, kv_codes: torch.Tensor, kv_scales: torch.Tensor,
                   sequence_lengths: torch.Tensor, *, block_table: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, q_scale: float = 1.0, chunk_len: int = 0,
                   k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Decode one token of GQA from a block-scaled FP4 cache.

    q: fp16 [batch, Hq, 128]. kv_codes: uint8 [batch, 2, Hkv, capacity, 64]
    (or pages [num_pages, 2, Hkv, page_size, 64] with ``block_table``): per
    head row, 64 bytes of E2M1 codes, element 2m in the low nibble of byte
    m. kv_scales: uint8 (or torch.float8_e4m3fn) with kv_codes' leading
    shape and a last axis of 8: the E4M3 scale of each block of 16
    elements. Element value = E2M1 value x its block's scale; k_scale and
    v_scale are per-tensor scales on top. Paged caches: page_size a power of
    two >= 32, block_table int32 [batch, max_pages] as for gqa_decode_paged.
    Strided views with contiguous last axes are taken without copies. Other
    arguments as for gqa_decode; fp16 output.
    """
    paged = block_table is not None
    if not isinstance(kv_scales, torch.Tensor):
        raise TypeError(f"kv_scales must be a torch.Tensor, got {type(kv_scales).__name__}")
    sc_dtype = kv_scales.dtype if kv_scales.dtype in _FP8_KV_DTYPES else torch.uint8

    def kv_shape(B):
        ks = kv_codes.shape
        if (not paged and ks[0] != B) or ks[1] != 2 or ks[4] != HEAD_DIM // 2:
            lead = "num_pages" if paged else str(B)
            raise ValueError(f"kv_codes must have shape [{lead}, 2, kv_heads, "
                             f"{'page_size' if paged else 'capacity'}, 64], got {tuple(ks)}")
        _check_view("kv_scales", kv_scales, sc_dtype, 5)
        if tuple(kv_scales.shape) != tuple(ks[:4]) + (FP4_SCALES_PER_ROW,):
            raise ValueError(f"kv_scales must have shape {tuple(ks[:4]) + (FP4_SCALES_PER_ROW,)}, "
                             f"got {tuple(kv_scales.shape)}")
        if paged:
            _check_tensor("block_table", block_table, torch.int32, 2)
            if block_table.shape[0] != B:
                raise ValueError(f"block_table must have {B} rows, got {tuple(block_table.shape)}")

    if not isinstance(kv_codes, torch.Tensor) or kv_codes.dtype != torch.uint8:
        raise TypeError("kv_codes must be a uint8 torch.Tensor of packed E2M1 codes")
    if not isinstance(q, torch.Tensor) or q.dtype != torch.float16:
        raise TypeError("q must be a float16 torch.Tensor")
    _, _, out = _prepare(q, kv_codes, sequence_lengths, out, kv_shape)
    for name, t in (("kv_scales", kv_scales),) + ((("block_table", block_table),) if paged else ()):
        if t.device != q.device:
            _check_device(name, t)
            raise ValueError(f"{name} must be on q's device")
    _check_chunk(chunk_len)
    B, Hq, Hkv = q.shape[0], q.shape[1], kv_codes.shape[2]
    if paged:
        num_pages, page_size, max_pages = kv_codes.shape[0], kv_codes.shape[3], block_table.shape[1]
        capacity = max_pages * page_size
        lay = _Layout(q.stride(0), q.stride(1), kv_codes.stride(0), kv_codes.stride(1),
                      kv_codes.stride(2), kv_codes.stride(3), block_table.data_ptr(), max_pages,
                      page_size, num_pages, Hq, Hkv)
    else:
        capacity = kv_codes.shape[3]
        lay = _Layout(q.stride(0), q.stride(1), kv_codes.stride(0), kv_codes.stride(1),
                      kv_codes.stride(2), kv_codes.stride(3), None, 0, 0, 0, Hq, Hkv)
    scl = _BlockScales(kv_scales.data_ptr(), kv_scales.stride(0), kv_scales.stride(1),
                       kv_scales.stride(2), kv_scales.stride(3))
    lib = _lib if _lib is not None else load_library()
    st = lib.gqa_decode_fp4(q.data_ptr(), kv_codes.data_ptr(), ctypes.byref(scl),
                            sequence_lengths.data_ptr(), out.data_ptr(), ctypes.byref(lay),
                            float(q_scale), float(k_scale), float(v_scale), B, capacity,
                            chunk_len, _stream_of(q.device))
    if st != 0:
        _raise(lib, st)
    return out


def workspace_bytes(batch: int, capacity: int) -> int:
    return int(load_library().gqa_decode_workspace_bytes(batch, capacity))


def release_workspace() -> None:
    load_library().gqa_decode_release_workspace()


_LAUNCH_FORMS = {"auto": 0, "single": 1, "two": 2}


def set_launch_form(form: str) -> None:
    """Select how later calls run the combine step: "single" (one kernel; the
    last workgroup of each cut segment merges it), "two" (pieces kernel, then
    combine kernel) or "auto" (single launch for capacities up to 512 with at
    most 131072 cache rows, batch x KV heads x capacity, in all, or up to 1024
    with at most 32768 rows). The forms
    return the same bits."""
    if form not in _LAUNCH_FORMS:
        raise ValueError(f"launch form must be one of {sorted(_LAUNCH_FORMS)}, got {form!r}")
    lib = load_library()
    st = lib.gqa_decode_set_launch_form(_LAUNCH_FORMS[form])
    if st != 0:
        _raise(lib, st)


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
