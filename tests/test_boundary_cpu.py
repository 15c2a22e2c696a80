"""C-ABI boundary checks that need no GPU: the product library loads and
exports every function include/siglip.h declares (and none of the test
hooks), the test build also exports those of include/siglip_test_hooks.h,
and both reject malformed blobs, unsupported dimensions, bad options and null
pointers with the documented status before any HIP call."""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

import synthetic as S
import vision_transformer_so400m_amd as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "siglip.h")
HOOKS_HEADER = os.path.join(ROOT, "include", "siglip_test_hooks.h")


def _declared(path=HEADER):
    text = open(path).read()
    return sorted(set(re.findall(r"SIGLIP_API\s+[\w\s\*]+?\b(siglip_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(V.EXPORTED)
    assert _declared(HOOKS_HEADER) == sorted(V.TEST_HOOKS)


def _exports(lib, name):
    try:
        return bool(ctypes.cast(getattr(lib, name), ctypes.c_void_p).value)
    except AttributeError:
        return False


def test_product_library_exports_every_declared_symbol_and_no_hook():
    lib = V.load_library(V.LIB_PATH)
    for name in _declared():
        assert _exports(lib, name), name
    for name in _declared(HOOKS_HEADER):
        assert not _exports(lib, name), name


def test_test_library_exports_the_hooks_too():
    lib = V.load_library(V.TEST_LIB_PATH)
    for name in _declared() + _declared(HOOKS_HEADER):
        assert _exports(lib, name), name


def test_status_strings():
    assert V.status_name(V.SIGLIP_OK) == "SIGLIP_OK"
    assert V.status_name(V.SIGLIP_E_BAD_BLOB) == "SIGLIP_E_BAD_BLOB"
    assert V.status_name(12345) == "SIGLIP_E_UNKNOWN"


@pytest.fixture(scope="module")
def blob1():
    d = S.SO400M.with_depth(1)
    return bytes(S.pack_blob(d, S.make_weights(d, 0)))


def _create(blob, **kw):
    with pytest.raises(V.SiglipError) as ei:
        V.Model(blob, **kw)
    return ei.value


def _patched(blob, off, fmt, value):
    b = bytearray(blob)
    struct.pack_into(fmt, b, off, value)
    return bytes(b)


@pytest.mark.parametrize("case,mutate,status,msg", [
    ("magic", lambda b: b"XXXX" + b[4:], V.SIGLIP_E_BAD_BLOB, "magic"),
    ("version", lambda b: _patched(b, 4, "<I", 2), V.SIGLIP_E_BAD_BLOB, "version"),
    ("dtype", lambda b: _patched(b, 36, "<I", 1), V.SIGLIP_E_BAD_BLOB, "dtype"),
    ("zero_dim", lambda b: _patched(b, 28, "<I", 0), V.SIGLIP_E_BAD_BLOB, "zero"),
    ("heads_x_dim", lambda b: _patched(b, 16, "<I", 15), V.SIGLIP_E_BAD_BLOB, "heads"),
    ("truncated", lambda b: b[:-64], V.SIGLIP_E_BAD_BLOB, "size"),
    ("total_mismatch", lambda b: _patched(b, 40, "<Q", len(b) + 64) , V.SIGLIP_E_BAD_BLOB, "total_bytes"),
    ("short", lambda b: b[:32], V.SIGLIP_E_BAD_BLOB, "header"),
])
def test_bad_blobs_are_rejected_on_cpu(blob1, case, mutate, status, msg):
    e = _create(mutate(blob1))
    assert e.status == status, e
    assert msg in e.message


def test_truncated_with_consistent_header(blob1):
    # header claims the shorter size: the tensor walk must find the truncation
    b = bytearray(blob1[:-4096])
    struct.pack_into("<Q", b, 40, len(b))
    e = _create(bytes(b))
    assert e.status == V.SIGLIP_E_BAD_BLOB and "truncated" in e.message


def test_depth_mismatch_is_truncation(blob1):
    b = _patched(blob1, 12, "<I", 2)   # claims 2 layers, holds 1
    e = _create(b)
    assert e.status == V.SIGLIP_E_BAD_BLOB


def test_trailing_bytes(blob1):
    b = bytearray(blob1) + bytes(64)
    struct.pack_into("<Q", b, 40, len(b))
    e = _create(bytes(b))
    assert e.status == V.SIGLIP_E_BAD_BLOB and "trailing" in e.message


@pytest.mark.parametrize("kw,msg", [
    (dict(max_batch=0), "max_batch"),
    (dict(max_batch=5000), "max_batch"),
    (dict(layers=2), "layers"),
    (dict(layers=-1), "layers"),
    (dict(fp8=True, fp8_scale_exp=9), "fp8_scale_exp"),
])
def test_bad_options(blob1, kw, msg):
    e = _create(blob1, **kw)
    assert e.status == V.SIGLIP_E_INVALID_ARG and msg in e.message


def test_options_struct_matches_header():
    """The binding's siglip_options has the header's fields, in order."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} siglip_options;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"int32_t\s+(\w+)\s*;", body)
    assert fields == [f[0] for f in V.siglip_options._fields_]
    assert all(f[1] is ctypes.c_int32 for f in V.siglip_options._fields_)


def test_bad_separate_qkv_value(blob1):
    lib = V.load_library()
    out = ctypes.c_void_p()
    opt = V.siglip_options(0, 1, 0, -4, 2)
    st = lib.siglip_create(blob1, len(blob1), ctypes.byref(opt), ctypes.byref(out))
    assert st == V.SIGLIP_E_INVALID_ARG and not out.value
    assert b"separate_qkv" in lib.siglip_last_error()


def test_bad_map_explicit_kv_value(blob1):
    lib = V.load_library()
    out = ctypes.c_void_p()
    opt = V.siglip_options(0, 1, 0, -4, 0, 3)
    st = lib.siglip_create(blob1, len(blob1), ctypes.byref(opt), ctypes.byref(out))
    assert st == V.SIGLIP_E_INVALID_ARG and not out.value
    assert b"map_explicit_kv" in lib.siglip_last_error()


def test_bad_attention_fp8_value(blob1):
    lib = V.load_library()
    out = ctypes.c_void_p()
    for bad in (4, -1):  # bits 0 (PV) and 1 (QK) only
        opt = V.siglip_options(0, 1, 0, -4, 0, 0, bad)
        st = lib.siglip_create(blob1, len(blob1), ctypes.byref(opt), ctypes.byref(out))
        assert st == V.SIGLIP_E_INVALID_ARG and not out.value
        assert b"attention_fp8" in lib.siglip_last_error()
    # its scale exponent is checked even with F16 GEMM operands, for either product
    for mode in (1, 2, 3):
        opt = V.siglip_options(0, 1, 0, 9, 0, 0, mode)
        st = lib.siglip_create(blob1, len(blob1), ctypes.byref(opt), ctypes.byref(out))
        assert st == V.SIGLIP_E_INVALID_ARG and not out.value
        assert b"fp8_scale_exp" in lib.siglip_last_error()


def test_bad_layernorm_fold_value(blob1):
    lib = V.load_library()
    out = ctypes.c_void_p()
    for bad in (2, -1):
        opt = V.siglip_options(0, 1, 0, -4, 0, 0, 0, bad)
        st = lib.siglip_create(blob1, len(blob1), ctypes.byref(opt), ctypes.byref(out))
        assert st == V.SIGLIP_E_INVALID_ARG and not out.value
        assert b"layernorm_fold" in lib.siglip_last_error()


def test_layernorm_fold_needs_width_1152_before_the_device():
    # width 1280 (16 heads of 80) is otherwise supported
    d = S.ModelDims(width=1280, heads=16, head_dim=80, depth=1, mlp=288, tokens=4)
    blob = bytes(S.pack_blob(d, S.make_weights(d, 0)))
    lib = V.load_library()
    out = ctypes.c_void_p()
    opt = V.siglip_options(0, 1, 0, -4, 0, 0, 0, 1)
    st = lib.siglip_create(blob, len(blob), ctypes.byref(opt), ctypes.byref(out))
    assert st == V.SIGLIP_E_UNSUPPORTED and not out.value
    assert b"layernorm_fold" in lib.siglip_last_error()


def test_unsupported_width_is_reported_before_the_device():
    d = S.small_dims(1)   # width 144: not a multiple of 128
    e = _create(bytes(S.pack_blob(d, S.make_weights(d, 0))))
    assert e.status == V.SIGLIP_E_UNSUPPORTED and "128" in e.message


def test_null_pointers_and_bad_attention_args():
    lib = V.load_library()
    out = ctypes.c_void_p()
    opt = V.siglip_options(0, 1, 0, -4)
    assert lib.siglip_create(None, 0, ctypes.byref(opt), ctypes.byref(out)) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_create(b"x" * 64, 64, None, ctypes.byref(out)) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_create(b"x" * 64, 64, ctypes.byref(opt), None) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_encode(None, None, 1, None, None) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_destroy(None) == V.SIGLIP_OK
    assert lib.siglip_debug_capture(None, 0) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_debug_fill_workspace(None, 0) == V.SIGLIP_E_INVALID_ARG
    # attention argument checks: every call below fails validation, so no
    # kernel is ever launched on the bogus pointer
    p = 4096
    assert lib.siglip_attention(None, p, p, 1152, p, 1, 16, 729, 72, 0.1, None) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_attention(p, p, p, 2048, p, 1, 16, 729, 128, 0.1, None) == V.SIGLIP_E_UNSUPPORTED
    assert lib.siglip_attention(p, p, p, 1152, p, 1, 16, 729, 76, 0.1, None) == V.SIGLIP_E_UNSUPPORTED
    assert lib.siglip_attention(p, p, p, 1000, p, 1, 16, 729, 72, 0.1, None) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_attention(p, p, p, 1152, p, 0, 16, 729, 72, 0.1, None) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_attention(p + 8, p, p, 1152, p, 1, 16, 729, 72, 0.1, None) == V.SIGLIP_E_INVALID_ARG
    assert lib.siglip_attention(p, p, p, 1152, p, 1, 16, 729, 72, -1.0, None) == V.SIGLIP_E_INVALID_ARG
    assert "scale" in V.last_error()


def test_e4m3_decode_helper_matches_oracle_rounding():
    import oracle as O
    from e4m3_codes import e4m3_decode
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes, scale_exp=0)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    np.testing.assert_array_equal(O.e4m3_round(vals[finite]), vals[finite])
    # a few codes decoded by hand: 0x38 = 1.0, 0x7E = 448, 0x01 = 2^-9, 0xB8 = -1.0
    np.testing.assert_array_equal(e4m3_decode(np.array([0x38, 0x7E, 0x01, 0xB8], np.uint8), 0),
                                  [1.0, 448.0, 2.0 ** -9, -1.0])
