"""ctypes binding of libsiglip (include/siglip.h), same names as the C ABI.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of libsiglip.so. PyTorch supplies device memory and the stream.
There is no CPU fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsiglip.so")
TEST_LIB_PATH = os.path.join(_PKG, "libsiglip_test.so")   # + include/siglip_test_hooks.h

SIGLIP_OK = 0
SIGLIP_E_INVALID_ARG = -1
SIGLIP_E_BAD_BLOB = -2
SIGLIP_E_UNSUPPORTED = -3
SIGLIP_E_OUT_OF_MEMORY = -4
SIGLIP_E_HIP = -5

STAGES = ["EMBED", "LN1", "QKV", "ATTN", "H_ATTN", "LN2", "MLP_HIDDEN", "H_OUT",
          "FINAL_LN", "MAP_KV", "MAP_ATTN", "MAP_Y", "MAP_LN", "MAP_HIDDEN", "MAP_Q", "V_T"]
STAGE = {n: i for i, n in enumerate(STAGES)}

EXPORTED = ["siglip_create", "siglip_encode", "siglip_attention", "siglip_attention_noalloc", "siglip_destroy",
            "siglip_status_string", "siglip_last_error", "siglip_model_info",
            "siglip_debug_timing", "siglip_debug_timing_read"]
TEST_HOOKS = ["siglip_debug_capture", "siglip_debug_stage_info", "siglip_debug_stage",
              "siglip_debug_fill_workspace"]

KERNEL_CLASSES = ["INPUT", "EMBED", "LAYERNORM", "QKV", "ATTENTION", "OUT_PROJ", "MLP_UP",
                  "MLP_DOWN", "MAP_KV", "MAP_ATTENTION", "MAP_TAIL"]
KCLASS = {n: i for i, n in enumerate(KERNEL_CLASSES)}


class SiglipError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status
        self.message = message


class siglip_options(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("gemm_precision", ctypes.c_int32), ("fp8_scale_exp", ctypes.c_int32),
                ("separate_qkv", ctypes.c_int32), ("map_explicit_kv", ctypes.c_int32),
                ("attention_fp8", ctypes.c_int32), ("layernorm_fold", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None
_path = LIB_PATH


def use_test_hooks() -> None:
    """Load the test build (libsiglip_test.so: the product library plus the
    stage-capture and workspace-poisoning hooks) instead of libsiglip.so.
    Must be called before the library is first loaded in this process."""
    global _path
    if _lib is not None and _path != TEST_LIB_PATH:
        raise RuntimeError("the product library is already loaded in this process")
    _path = TEST_LIB_PATH


def has_test_hooks() -> bool:
    return _path == TEST_LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the library (built in-tree by build.build()); raises if absent.
    Without a path: libsiglip.so, or libsiglip_test.so after use_test_hooks().
    With a path: that file, loaded on its own (not cached)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _path
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with "
                           "`python -m vision_transformer_so400m_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    P = ctypes.POINTER
    lib.siglip_create.argtypes = [vp, ctypes.c_size_t, P(siglip_options), P(vp)]
    lib.siglip_encode.argtypes = [vp, vp, i32, vp, vp]
    lib.siglip_attention.argtypes = [vp, vp, vp, i64, vp, i32, i32, i32, i32, ctypes.c_float, vp]
    lib.siglip_attention_noalloc.argtypes = [vp, vp, vp, i64, vp, i32, i32, i32, i32, ctypes.c_float, vp]
    lib.siglip_destroy.argtypes = [vp]
    lib.siglip_status_string.argtypes = [ctypes.c_int]
    lib.siglip_status_string.restype = ctypes.c_char_p
    lib.siglip_last_error.argtypes = []
    lib.siglip_last_error.restype = ctypes.c_char_p
    lib.siglip_model_info.argtypes = [vp] + [P(i32)] * 9
    lib.siglip_debug_timing.argtypes = [vp, ctypes.c_uint32]
    lib.siglip_debug_timing_read.argtypes = [vp, i32, P(ctypes.c_double), P(i64)]
    names = list(EXPORTED)
    if hasattr(lib, "siglip_debug_capture"):
        lib.siglip_debug_capture.argtypes = [vp, i32]
        lib.siglip_debug_stage_info.argtypes = [vp, i32, P(i64), P(i64), P(i64), P(i32)]
        lib.siglip_debug_stage.argtypes = [vp, i32, vp, ctypes.c_size_t]
        lib.siglip_debug_fill_workspace.argtypes = [vp, ctypes.c_uint16]
        names += TEST_HOOKS
    for name in names:
        getattr(lib, name).restype = getattr(lib, name).restype or ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _hooks():
    lib = load_library()
    if not hasattr(lib, "siglip_debug_capture"):
        raise RuntimeError("stage capture and workspace poisoning are test hooks: call "
                           "use_test_hooks() before the library is first loaded")
    return lib


def status_name(status: int) -> str:
    return load_library().siglip_status_string(status).decode()


def last_error() -> str:
    return load_library().siglip_last_error().decode()


def _check(status: int) -> None:
    if status != SIGLIP_OK:
        raise SiglipError(status, last_error())


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _host_ptr(buf) -> tuple:
    arr = np.frombuffer(buf, dtype=np.uint8)
    return arr, arr.ctypes.data, arr.nbytes


class Model:
    """A resident encoder: weights uploaded once by siglip_create."""

    def __init__(self, blob, layers: int = 0, max_batch: int = 1, fp8: bool = False,
                 fp8_scale_exp: int = -4, separate_qkv: bool = False, map_explicit_kv: bool = False,
                 attention_fp8=0, layernorm_fold: bool = False):
        """attention_fp8: e4m3 attention products, siglip_options bits (1 = PV,
        2 = QK, 3 = both); True means PV. layernorm_fold: LayerNorms 1 and 2
        folded into the QKV and MLP-up GEMMs (width 1152 only)."""
        lib = load_library()
        keep, ptr, n = _host_ptr(blob)
        afp8 = 1 if attention_fp8 is True else int(attention_fp8)
        opt = siglip_options(layers, max_batch, 1 if fp8 else 0, fp8_scale_exp, 1 if separate_qkv else 0,
                             1 if map_explicit_kv else 0, afp8, 1 if layernorm_fold else 0)
        h = ctypes.c_void_p()
        _check(lib.siglip_create(ptr, n, ctypes.byref(opt), ctypes.byref(h)))
        self._h = h
        del keep
        vals = [ctypes.c_int32() for _ in range(9)]
        _check(lib.siglip_model_info(self._h, *[ctypes.byref(v) for v in vals]))
        (self.width, self.layers, self.heads, self.head_dim, self.mlp, self.tokens,
         self.patch_dim, self.max_batch, prec) = [v.value for v in vals]
        self.fp8 = prec == 1
        self.fp8_scale_exp = fp8_scale_exp

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("model is closed")
        return self._h

    def encode(self, pixels, out=None, stream=None):
        """pixels: CUDA float16 [B, tokens, patch_dim] -> float16 [B, 1, width]."""
        import torch
        if pixels.device.type != "cuda" or pixels.dtype != torch.float16 or not pixels.is_contiguous():
            raise ValueError("pixels must be a contiguous CUDA float16 tensor")
        if pixels.dim() != 3 or tuple(pixels.shape[1:]) != (self.tokens, self.patch_dim):
            raise ValueError(f"pixels must be [B, {self.tokens}, {self.patch_dim}]")
        b = pixels.shape[0]
        if out is None:
            out = torch.empty((b, 1, self.width), dtype=torch.float16, device=pixels.device)
        elif (out.dtype != torch.float16 or not out.is_contiguous()
              or tuple(out.shape) != (b, 1, self.width)):
            raise ValueError("out must be a contiguous float16 [B, 1, width] tensor")
        elif out.device != pixels.device:
            raise ValueError(f"out is on {out.device}, pixels on {pixels.device}: both must be on the same GPU")
        _check(load_library().siglip_encode(self.handle, pixels.data_ptr(), b, out.data_ptr(),
                                            _stream_ptr(stream)))
        return out

    # ---- diagnostics
    def debug_capture(self, layer: int) -> None:
        _check(_hooks().siglip_debug_capture(self.handle, layer))

    def debug_stage_info(self, stage):
        s = STAGE[stage] if isinstance(stage, str) else stage
        r, c, l, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(_hooks().siglip_debug_stage_info(self.handle, s, ctypes.byref(r), ctypes.byref(c),
                                                      ctypes.byref(l), ctypes.byref(e)))
        return r.value, c.value, l.value, e.value

    def debug_stage(self, stage, full: bool = False) -> np.ndarray:
        """Captured stage as a numpy array [rows, cols] ([rows, ld] with
        full=True, padding columns included): float16, or uint8 e4m3 codes
        (value = code * 2^fp8_scale_exp) for FP8 operand stages."""
        s = STAGE[stage] if isinstance(stage, str) else stage
        rows, cols, ld, eb = self.debug_stage_info(s)
        buf = np.empty(rows * ld * eb, np.uint8)
        _check(_hooks().siglip_debug_stage(self.handle, s, buf.ctypes.data, buf.nbytes))
        arr = buf.view(np.float16 if eb == 2 else np.uint8).reshape(rows, ld)
        return arr if full else arr[:, :cols]

    def debug_fill_workspace(self, pattern: int) -> None:
        _check(_hooks().siglip_debug_fill_workspace(self.handle, pattern))

    def debug_timing(self, classes) -> None:
        """Per-launch HIP-event timing of later encode calls for the given
        kernel classes (names or indices; True = all, False/None/() = off).
        Resets the totals."""
        if classes is True:
            mask = (1 << len(KERNEL_CLASSES)) - 1
        elif not classes:
            mask = 0
        else:
            mask = 0
            for c in classes:
                mask |= 1 << (KCLASS[c] if isinstance(c, str) else int(c))
        _check(load_library().siglip_debug_timing(self.handle, mask))

    def debug_timing_read(self, kclass) -> tuple:
        """(total ms, launches) of one kernel class since timing was enabled."""
        k = KCLASS[kclass] if isinstance(kclass, str) else kclass
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(load_library().siglip_debug_timing_read(self.handle, k, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            load_library().siglip_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _span_ok(x, elems: int) -> bool:
    """x's storage holds `elems` elements of its dtype from x.data_ptr() on."""
    st = x.untyped_storage()
    avail = st.nbytes() - (x.data_ptr() - st.data_ptr())
    return elems * x.element_size() <= avail


def attention(q, k, v, heads: int, head_dim: int, scale: float, out=None, row_stride: Optional[int] = None,
              tokens: Optional[int] = None, batch: Optional[int] = None, stream=None, noalloc: bool = False):
    """siglip_attention on CUDA float16 tensors or views; q/k/v rows hold
    heads*head_dim values at row_stride elements apart (default
    heads*head_dim). batch and tokens default to q.shape[0] and q.shape[1].
    noalloc=True calls siglip_attention_noalloc (the library's fixed scratch
    array instead of its allocated staging buffer; out must be given, so
    nothing is allocated). Raises ValueError, before any launch, if a tensor
    is not on q's GPU or its storage does not cover the rows the call reads
    or writes."""
    import torch
    b = batch if batch is not None else q.shape[0]
    t = tokens if tokens is not None else q.shape[1]
    w = heads * head_dim
    if row_stride is None:
        row_stride = w
    if out is None:
        if noalloc:
            raise ValueError("noalloc=True needs out")
        out = torch.empty((b, t, w), dtype=torch.float16, device=q.device)
    for x in (q, k, v, out):
        if x.device.type != "cuda" or x.dtype != torch.float16:
            raise ValueError("q, k, v, out must be CUDA float16")
        if x.device != q.device:
            raise ValueError("q, k, v and out must be on the same GPU")
    if b < 1 or t < 1 or row_stride < w:
        raise ValueError("batch, tokens >= 1 and row_stride >= heads*head_dim required")
    span = (b * t - 1) * row_stride + w
    for name, x in (("q", q), ("k", k), ("v", v)):
        if not _span_ok(x, span):
            raise ValueError(f"{name}: its storage does not hold the {span} elements the call reads")
    if not out.is_contiguous() or out.numel() < b * t * w or not _span_ok(out, b * t * w):
        raise ValueError("out must be a contiguous tensor of at least batch*tokens*heads*head_dim elements")
    lib = load_library()
    fn = lib.siglip_attention_noalloc if noalloc else lib.siglip_attention
    _check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), row_stride, out.data_ptr(), b, heads, t, head_dim,
              float(scale), _stream_ptr(stream)))
    return out
