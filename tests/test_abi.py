"""Host-side checks of the C ABI (no GPU needed).

* libgqa_decode.so loads and exports every function declared in
  include/gqa_decode.h.
* Argument errors are reported with the documented status codes before any
  device work; with no device visible a valid-looking call reports
  GQA_ERR_NO_DEVICE instead of crashing.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_decode.h")

OK, NULL, BAD_SHAPE, MISALIGNED, ALIAS, NO_DEVICE, ARCH, ALLOC, LAUNCH, BAD_ARG, MISMATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(gqa_\w+)\s*\(", text, flags=re.M)))


def _status_codes():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(GQA_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    import gqa_token_decode_amd as g
    from gqa_token_decode_amd import build as b

    srcs = [os.path.join(b.CSRC, s) for s in b.SOURCES] + [HEADER, os.path.join(b.CSRC, "launch.h")]
    if (not os.path.exists(b.LIB_PATH)
            or os.path.getmtime(b.LIB_PATH) < max(os.path.getmtime(s) for s in srcs)):
        b.build()
    return g.load_library()


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


def test_header_declares_the_documented_entry_points():
    names = _declared_functions()
    assert names == sorted([
        "gqa_decode", "gqa_decode_chunked", "gqa_decode_typed", "gqa_decode_ex",
        "gqa_decode_ex_noalloc", "gqa_decode_fp4", "gqa_decode_workspace_bytes", "gqa_decode_set_launch_form",
        "gqa_decode_release_workspace", "gqa_decode_status_string", "gqa_decode_last_error",
        "gqa_decode_profile_begin", "gqa_decode_profile_end"])


def test_library_exports_every_declared_symbol(lib):
    from gqa_token_decode_amd import build as b

    nm = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", nm, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_codes_match_header_and_have_text(lib):
    codes = _status_codes()
    assert codes["GQA_OK"] == OK and codes["GQA_ERR_NO_DEVICE"] == NO_DEVICE
    assert codes["GQA_ERR_DEVICE_MISMATCH"] == MISMATCH and codes["GQA_ERR_BAD_ARG"] == BAD_ARG
    texts = set()
    for v in codes.values():
        t = lib.gqa_decode_status_string(v).decode()
        assert t and t != "unknown status"
        texts.add(t)
    assert len(texts) == len(codes)
    assert lib.gqa_decode_status_string(12345).decode() == "unknown status"


def _call(lib, q=0x10000, kv=0x20000000, lens=0x30000, out=0x40000, scale=1.0, B=2, C=64,
          chunk=None):
    if chunk is None:
        return lib.gqa_decode(q, kv, lens, out, scale, B, C, None)
    return lib.gqa_decode_chunked(q, kv, lens, out, scale, B, C, chunk, None)


def test_argument_errors_are_reported_before_device_work(lib):
    assert _call(lib, q=None) == NULL
    assert _call(lib, kv=None) == NULL
    assert _call(lib, lens=None) == NULL
    assert _call(lib, out=None) == NULL
    assert "non-NULL" in lib.gqa_decode_last_error().decode()
    assert _call(lib, B=0) == BAD_SHAPE
    assert _call(lib, C=0) == BAD_SHAPE
    assert _call(lib, B=-3) == BAD_SHAPE
    assert _call(lib, B=(1 << 24) + 1) == BAD_SHAPE
    # one (sequence, KV head) block of K must stay addressable with 32-bit offsets
    assert _call(lib, B=1, C=(1 << 22) + 1) == BAD_SHAPE
    assert "capacity" in lib.gqa_decode_last_error().decode()
    assert lib.gqa_decode_workspace_bytes(1, (1 << 22) + 1) == 0
    assert _call(lib, q=0x10008) == MISALIGNED
    assert _call(lib, out=0x40004) == MISALIGNED
    assert _call(lib, lens=0x30002) == MISALIGNED
    # out inside q (q is 2 * 8 KiB long), inside kv, or covering seq_lens
    assert _call(lib, out=0x10000 + 0x2000) == ALIAS
    assert _call(lib, out=0x20000000 + 4096 * 64) == ALIAS
    assert _call(lib, out=0x30000 - 0x10) == ALIAS
    assert _call(lib, chunk=-1) == BAD_ARG
    assert _call(lib, scale=float("nan")) == BAD_ARG
    assert _call(lib, scale=float("inf")) == BAD_ARG


def _call_typed(lib, dtype=1, ks=1.0, vs=1.0, **kw):
    a = dict(q=0x10000, kv=0x20000000, lens=0x30000, out=0x40000, scale=1.0, B=2, C=64, chunk=0)
    a.update(kw)
    return lib.gqa_decode_typed(a["q"], a["kv"], a["lens"], a["out"], dtype, a["scale"], ks, vs,
                                a["B"], a["C"], a["chunk"], None)


def test_typed_entry_point_argument_errors(lib):
    assert _call_typed(lib, q=None) == NULL
    assert _call_typed(lib, B=0) == BAD_SHAPE
    assert _call_typed(lib, out=0x40004) == MISALIGNED
    assert _call_typed(lib, out=0x10000 + 0x2000) == ALIAS
    assert _call_typed(lib, dtype=7) == BAD_ARG
    assert "dtype" in lib.gqa_decode_last_error().decode()
    assert _call_typed(lib, dtype=-1) == BAD_ARG
    assert _call_typed(lib, ks=float("nan")) == BAD_ARG
    assert _call_typed(lib, vs=float("inf")) == BAD_ARG
    assert _call_typed(lib, chunk=-2) == BAD_ARG
    expected = MISMATCH if _gpu_visible() else NO_DEVICE
    for dt in (0, 1):
        assert _call_typed(lib, dtype=dt, ks=0.5, vs=2.0) == expected


def test_valid_looking_call_without_device_memory(lib):
    # No GPU here: the library must say so. With a GPU, these made-up
    # addresses are not device memory.
    expected = MISMATCH if _gpu_visible() else NO_DEVICE
    assert _call(lib) == expected
    assert _call(lib, chunk=7) == expected
    assert lib.gqa_decode_last_error().decode()


def test_helpers_without_device(lib):
    if _gpu_visible():
        pytest.skip("host-only behaviour")
    assert lib.gqa_decode_workspace_bytes(4, 256) == 0
    assert lib.gqa_decode_workspace_bytes(0, 256) == 0
    lib.gqa_decode_release_workspace()          # no-op, must not crash
    p, c, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    assert lib.gqa_decode_profile_begin() == OK
    assert lib.gqa_decode_profile_end(ctypes.byref(p), ctypes.byref(c), ctypes.byref(n)) == OK
    assert n.value == 0


def test_launch_form_selection(lib):
    # needs no device: the form is a library-wide setting
    for form in (1, 2, 0):
        assert lib.gqa_decode_set_launch_form(form) == OK
    assert lib.gqa_decode_set_launch_form(3) == BAD_ARG
    assert lib.gqa_decode_set_launch_form(-1) == BAD_ARG
    assert "form" in lib.gqa_decode_last_error().decode()


def test_python_binding_rejects_bad_tensors_before_the_library():
    import torch

    import gqa_token_decode_amd as g

    q = torch.zeros(2, 32, 128, dtype=torch.float16)
    kv = torch.zeros(2, 2, 8, 16, 128, dtype=torch.float16)
    lens = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        g.gqa_decode(q, kv, lens)
    with pytest.raises(TypeError):
        g.gqa_decode(q.float(), kv, lens)
    with pytest.raises(TypeError):
        g.gqa_decode(q, kv, lens.long())
    with pytest.raises(ValueError):
        g.gqa_decode(q[:, :16], kv, lens)
    with pytest.raises(ValueError):
        g.gqa_decode(q, kv.transpose(3, 4), lens)


def test_product_path_never_imports_the_oracle():
    # The binding, the build script and the C/HIP sources must not reach
    # the oracle package.
    pkg = os.path.join(ROOT, "gqa_token_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f


def _layout(**kw):
    from gqa_token_decode_amd import _Layout

    C = kw.pop("C", 64)
    d = dict(q_stride_batch=4096, q_stride_head=128, kv_stride_batch=2 * 8 * C * 128,
             kv_stride_kind=8 * C * 128, kv_stride_head=C * 128, kv_stride_row=128,
             block_table=None, max_pages=0, page_size=0, num_pages=0)
    d.update(kw)
    return _Layout(**d)


def _call_ex(lib, lay, dtype=0, B=2, C=64, chunk=0, q=0x10000, kv=0x20000000, out=0x40000):
    return lib.gqa_decode_ex(q, kv, 0x30000, out, dtype, ctypes.byref(lay) if lay else None,
                             1.0, 1.0, 1.0, B, C, chunk, None)


def test_layout_argument_errors(lib):
    expected = MISMATCH if _gpu_visible() else NO_DEVICE
    assert _call_ex(lib, None) == expected                      # contiguous
    assert _call_ex(lib, _layout()) == expected
    assert _call_ex(lib, _layout(q_stride_head=-128)) == BAD_ARG
    assert _call_ex(lib, _layout(kv_stride_row=132)) == BAD_ARG  # rows not 16-byte aligned
    assert _call_ex(lib, _layout(q_stride_batch=4100)) == BAD_ARG
    assert _call_ex(lib, _layout(kv_stride_row=64)) == BAD_ARG   # does not cover a row
    assert "row" in lib.gqa_decode_last_error().decode()
    # E4M3 rows are 128 B: strides count bytes there
    assert _call_ex(lib, _layout(kv_stride_row=64), dtype=2) == BAD_ARG
    assert _call_ex(lib, _layout(kv_stride_row=136), dtype=2) == BAD_ARG
    assert _call_ex(lib, _layout(kv_stride_row=144), dtype=2) == expected
    # 32-bit buffer offsets: row stride times capacity
    assert _call_ex(lib, _layout(kv_stride_row=1 << 20, C=4096), C=4096) == BAD_ARG
    assert _call_ex(lib, _layout(q_stride_head=1 << 29)) == BAD_ARG
    # paged caches
    bt = 0x50000
    assert _call_ex(lib, _layout(block_table=bt, max_pages=4, page_size=16, num_pages=9)) == expected
    assert _call_ex(lib, _layout(block_table=bt, max_pages=4, page_size=24, num_pages=9)) == BAD_ARG
    assert _call_ex(lib, _layout(block_table=bt, max_pages=4, page_size=8, num_pages=9)) == BAD_ARG
    assert _call_ex(lib, _layout(block_table=bt, max_pages=3, page_size=16, num_pages=9)) == BAD_ARG
    assert "capacity" in lib.gqa_decode_last_error().decode()
    assert _call_ex(lib, _layout(block_table=bt, max_pages=4, page_size=16, num_pages=0)) == BAD_ARG
    assert _call_ex(lib, _layout(block_table=bt + 2, max_pages=4, page_size=16, num_pages=9)) == MISALIGNED
    # out overlapping q under q's strides, or the block table
    assert _call_ex(lib, _layout(q_stride_batch=1 << 20), out=0x10000 + (1 << 20)) == ALIAS
    assert _call_ex(lib, _layout(block_table=0x40000 + 4096, max_pages=4, page_size=16,
                                 num_pages=9)) == ALIAS


def test_noalloc_entry_point_argument_errors(lib):
    # the allocation-free variant validates like gqa_decode_ex, before any
    # device work or scratch lookup
    f = lib.gqa_decode_ex_noalloc
    lay = _layout()
    args = lambda **k: dict(dict(q=0x10000, kv=0x20000000, lens=0x30000, out=0x40000, dtype=0,
                                 B=2, C=64, chunk=0), **k)
    call = lambda a: f(a["q"], a["kv"], a["lens"], a["out"], a["dtype"], ctypes.byref(lay), 1.0,
                       1.0, 1.0, a["B"], a["C"], a["chunk"], None)
    assert call(args(q=None)) == NULL
    assert call(args(B=0)) == BAD_SHAPE
    assert call(args(out=0x40004)) == MISALIGNED
    assert call(args(chunk=-1)) == BAD_ARG
    assert call(args(dtype=3)) == BAD_ARG                       # FP4 goes through gqa_decode_fp4
    assert "gqa_decode_fp4" in lib.gqa_decode_last_error().decode()
    assert call(args()) == (MISMATCH if _gpu_visible() else NO_DEVICE)


def test_head_count_argument_errors(lib):
    expected = MISMATCH if _gpu_visible() else NO_DEVICE
    for hq, hkv in [(64, 8), (28, 4), (16, 16), (8, 1), (1, 1), (0, 0)]:
        lay = _layout(num_q_heads=hq, num_kv_heads=hkv, q_stride_batch=max(hq, 1) * 128)
        assert _call_ex(lib, lay) == expected, (hq, hkv)
    for hq, hkv in [(72, 8), (30, 4), (4, 8), (32, 0), (0, 8), (-32, -8), (9, 1), (2048, 2048)]:
        lay = _layout(num_q_heads=hq, num_kv_heads=hkv)
        assert _call_ex(lib, lay) == BAD_ARG, (hq, hkv)
        assert "heads" in lib.gqa_decode_last_error().decode()
    # batch * KV heads is bounded
    lay = _layout(num_q_heads=256, num_kv_heads=256, q_stride_batch=256 * 128)
    assert _call_ex(lib, lay, B=1 << 20) == BAD_SHAPE
    # out extends over Hq rows per sequence: it must not reach kv
    lay = _layout(num_q_heads=64, num_kv_heads=8, q_stride_batch=64 * 128)
    assert _call_ex(lib, lay, out=0x20000000 - 2 * 64 * 128 * 2 + 256) == ALIAS


def _fp4_layout(**kw):
    C = kw.pop("C", 64)
    d = dict(kv_stride_batch=2 * 8 * C * 64, kv_stride_kind=8 * C * 64, kv_stride_head=C * 64,
             kv_stride_row=64)
    d.update(kw)
    return _layout(C=C, **d)


def _call_fp4(lib, lay="default", scales=0x60000, strides=(0, 0, 0, 0), B=2, C=64, chunk=0,
              out=0x40000, ks=1.0):
    from gqa_token_decode_amd import _BlockScales

    lay = _fp4_layout(C=C) if lay == "default" else lay
    sc = None if scales is None else _BlockScales(scales, *strides)
    return lib.gqa_decode_fp4(0x10000, 0x20000000, ctypes.byref(sc) if sc else None, 0x30000, out,
                              ctypes.byref(lay) if lay else None, 1.0, ks, 1.0, B, C, chunk, None)


def test_fp4_entry_point_argument_errors(lib):
    expected = MISMATCH if _gpu_visible() else NO_DEVICE
    assert _call_fp4(lib) == expected                        # contiguous codes and scales
    assert _call_fp4(lib, lay=None) == expected              # layout NULL: 64-byte rows
    assert _call_fp4(lib, strides=(2 * 8 * 64 * 8, 8 * 64 * 8, 64 * 8, 8)) == expected
    assert _call_fp4(lib, scales=None) == NULL
    assert _call_fp4(lib, scales=0) == NULL
    assert _call_fp4(lib, scales=0x60002) == MISALIGNED
    assert _call_fp4(lib, strides=(2 * 8 * 64 * 8, 8 * 64 * 8, 64 * 8, 6)) == BAD_ARG   # not a multiple of 4
    assert _call_fp4(lib, strides=(2 * 8 * 64 * 4, 8 * 64 * 4, 64 * 4, 4)) == BAD_ARG   # under 8 bytes
    assert "8 bytes" in lib.gqa_decode_last_error().decode()
    assert _call_fp4(lib, strides=(0, 0, 0, 1 << 26), C=64) == BAD_ARG                  # 32-bit offsets
    assert _call_fp4(lib, lay=_fp4_layout(kv_stride_row=48)) == BAD_ARG                 # does not cover 64 B
    assert _call_fp4(lib, lay=_fp4_layout(kv_stride_row=80)) == expected
    assert _call_fp4(lib, ks=float("inf")) == BAD_ARG
    # out overlapping the scales
    assert _call_fp4(lib, scales=0x40000 + 1024) == ALIAS
    # paged: pages of at least 32 rows
    bt = 0x50000
    paged = dict(block_table=bt, max_pages=4, num_pages=9)
    assert _call_fp4(lib, lay=_fp4_layout(page_size=32, C=32, **paged), C=128) == expected
    assert _call_fp4(lib, lay=_fp4_layout(page_size=16, C=16, **paged), C=64) == BAD_ARG
    assert ">= 32" in lib.gqa_decode_last_error().decode()
    # the other entry points take no FP4 cache
    assert _call_typed(lib, dtype=3) == BAD_ARG
    assert "gqa_decode_fp4" in lib.gqa_decode_last_error().decode()
    assert _call_ex(lib, _layout(), dtype=3) == BAD_ARG


def test_fp4_binding_rejects_bad_tensors_before_the_library():
    import torch
    import gqa_token_decode_amd as g

    q = torch.zeros((2, 32, 128), dtype=torch.float16)
    codes = torch.zeros((2, 2, 8, 64, 64), dtype=torch.uint8)
    scales = torch.zeros((2, 2, 8, 64, 8), dtype=torch.uint8)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(TypeError):
        g.gqa_decode_fp4(q, codes.to(torch.int8), scales, lens)
    with pytest.raises(TypeError):
        g.gqa_decode_fp4(q.to(torch.bfloat16), codes, scales, lens)
    with pytest.raises(ValueError, match="kv_codes must have shape"):
        g.gqa_decode_fp4(q, torch.zeros((2, 2, 8, 64, 128), dtype=torch.uint8), scales, lens)
    with pytest.raises(ValueError, match="kv_scales must have shape"):
        g.gqa_decode_fp4(q, codes, torch.zeros((2, 2, 8, 64, 16), dtype=torch.uint8), lens)
    with pytest.raises(TypeError):
        g.gqa_decode_fp4(q, codes, scales.to(torch.int32), lens)
    with pytest.raises(ValueError, match="GPU"):                  # CPU tensors
        g.gqa_decode_fp4(q, codes, scales, lens)


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    # no fallback: a missing library is an error, never a silent CPU path
    import torch

    import gqa_token_decode_amd as g

    monkeypatch.setattr(g, "_lib", None)
    monkeypatch.setattr(g, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="build"):
        g.load_library()
    if not torch.cuda.is_available():
        q = torch.zeros(1, 32, 128, dtype=torch.float16)
        with pytest.raises((RuntimeError, ValueError)):
            g.gqa_decode(q, torch.zeros(1, 2, 8, 4, 128, dtype=torch.float16),
                         torch.ones(1, dtype=torch.int32))


def _c_abi_helper():
    import importlib.util

    path = os.path.join(ROOT, "tests", "c_abi", "build.py")
    spec = importlib.util.spec_from_file_location("gqa_c_abi_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_c_program_reaches_the_abi_without_python(lib, tmp_path):
    # A plain C11 program built against include/gqa_decode.h alone links to
    # the library and gets its argument errors back (no device needed).
    prog = _c_abi_helper().ensure_c_program()
    res = subprocess.run([prog, "--bad-shape"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert f"status {BAD_SHAPE}" in res.stdout and "batch" in res.stdout
    missing = str(tmp_path / "nothing.bin")
    res = subprocess.run([prog, missing, missing, missing, missing, "1", "16", "1.0"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "could not read" in res.stderr
