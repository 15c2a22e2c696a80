"""Seeded synthetic inputs for the SigLIP So400m/14 image encoder.

This module is the only code that both the CPU oracle's tests and the GPU
library's tests share. It holds none of the encoder's arithmetic: it draws
random weights and pixels, names the workload configurations, packs weights
into the weight-blob byte format the C library reads, and rearranges a raw
image into patch order. It never normalises, multiplies or adds model tensors.

Sources (page "Single-layer SigLIP vision benchmark", intro):
  * So400m/14 dims: 378x378 RGB, 14x14 patches -> 729 tokens, width 1152,
    16 heads of width 72, MLP width 4304; depth 27 (reduced to 1 in the
    single-layer benchmark).
  * Gaussian Xavier-style weights, positional embedding std 1/sqrt(width),
    layernorm scale one, tiny Gaussian biases; one shared learned probe.
  * The reduced "small" model: 28x28 image, width 144, two 72-wide heads,
    MLP width 288 (intro, "--vit-small" paragraph).
  * Input binding [batch, patch_y, patch_x, y, x, channel] -> [batch, 729, 588].
Same page, section "Fused encoder QKV and MAP KV": the fused projections keep
the initialisation variance of the individual projections.

Readings where the pages are silent (all listed in the design notes):
  * biases N(0, 1e-3^2); probe std sqrt(2/(1+width)) (Xavier with fan_in 1);
  * RNG: numpy PCG64 `default_rng([seed, 0])` draws every random weight tensor
    in blob order as `standard_normal(shape, float32) * std`;
    `default_rng([seed, 1])` draws the pixels, rounded to F16.
"""
from __future__ import annotations

import dataclasses
import struct
from typing import Dict, Iterator, List, Tuple

import numpy as np

__all__ = [
    "ModelDims", "SO400M", "small_dims", "four_token_dims", "CONFIGS",
    "tensor_specs", "make_weights", "make_pixels", "make_attention_inputs",
    "pack_blob", "blob_size", "image_to_patches", "BLOB_MAGIC", "BLOB_VERSION",
    "BLOB_HEADER_BYTES", "BLOB_ALIGN",
]

BLOB_MAGIC = b"SGLP"
BLOB_VERSION = 1
BLOB_HEADER_BYTES = 64
BLOB_ALIGN = 64
DTYPE_F32 = 0


@dataclasses.dataclass(frozen=True)
class ModelDims:
    """Shape of one encoder instance (all sizes in elements)."""
    width: int = 1152      # token embedding width
    depth: int = 27        # encoder layers
    heads: int = 16
    head_dim: int = 72
    mlp: int = 4304        # MLP hidden width (encoder and MAP head)
    tokens: int = 729      # patches per image: (378/14)^2
    patch_dim: int = 588   # 14*14*3 values per patch
    patch: int = 14        # patch side in pixels
    channels: int = 3

    def with_depth(self, depth: int) -> "ModelDims":
        return dataclasses.replace(self, depth=depth)

    @property
    def grid(self) -> int:
        g = int(round(self.tokens ** 0.5))
        assert g * g == self.tokens
        return g

    @property
    def image_side(self) -> int:
        return self.grid * self.patch


SO400M = ModelDims()


def small_dims(depth: int = 1) -> ModelDims:
    """The reduced complete graph: 28x28 image (4 tokens), width 144,
    two 72-wide heads, MLP 288."""
    return ModelDims(width=144, depth=depth, heads=2, head_dim=72, mlp=288,
                     tokens=4, patch_dim=588)


def four_token_dims(depth: int = 1) -> ModelDims:
    """Four tokens at the full 1152/4304 widths and 16 heads (the pages'
    full-width diagnostic)."""
    return ModelDims(width=1152, depth=depth, heads=16, head_dim=72,
                     mlp=4304, tokens=4, patch_dim=588)


# Workload configurations: name -> recipe. "fp8" selects e4m3 operands for
# every weight GEMM; everything else is F16 storage with F32 statistics.
CONFIGS: Dict[str, dict] = {
    "c0_1layer_b1_f16": dict(layers=1, batch=1, seed=0, fp8=False),
    "c1_1layer_b8_f16": dict(layers=1, batch=8, seed=0, fp8=False),
    "c2_attention_b32": dict(batch=32, heads=16, tokens=729, head_dim=72,
                             seeds=((0, 2), (0, 3), (0, 4))),
    "c3_27layer_b1_f16": dict(layers=27, batch=1, seed=1, fp8=False),
    "c3_27layer_b2_f16": dict(layers=27, batch=2, seed=1, fp8=False),
    "c4_27layer_b64_fp8": dict(layers=27, batch=64, seed=2, fp8=True),
}


def _xavier_std(fan_in: int, fan_out: int) -> float:
    return (2.0 / (fan_in + fan_out)) ** 0.5


BIAS_STD = 1e-3


def tensor_specs(d: ModelDims) -> List[Tuple[str, Tuple[int, ...], str, float]]:
    """Every parameter in blob order: (name, shape, init kind, std).

    init kind: "normal" (drawn with the given std), "ones", "zeros".
    Weight matrices are [in, out] row-major so that y = x @ W.
    """
    W, F, T, P = d.width, d.mlp, d.tokens, d.patch_dim
    xs = _xavier_std
    specs: List[Tuple[str, Tuple[int, ...], str, float]] = [
        ("embed.w", (P, W), "normal", xs(P, W)),
        ("embed.b", (W,), "normal", BIAS_STD),
        ("pos", (T, W), "normal", W ** -0.5),
    ]
    for i in range(d.depth):
        p = f"layer{i}."
        specs += [
            (p + "ln1.g", (W,), "ones", 0.0),
            (p + "ln1.b", (W,), "zeros", 0.0),
            # three [W, W] projections side by side; each keeps its own
            # Xavier variance, which is the same std for all three
            (p + "qkv.w", (W, 3 * W), "normal", xs(W, W)),
            (p + "qkv.b", (3 * W,), "normal", BIAS_STD),
            (p + "out.w", (W, W), "normal", xs(W, W)),
            (p + "out.b", (W,), "normal", BIAS_STD),
            (p + "ln2.g", (W,), "ones", 0.0),
            (p + "ln2.b", (W,), "zeros", 0.0),
            (p + "mlp1.w", (W, F), "normal", xs(W, F)),
            (p + "mlp1.b", (F,), "normal", BIAS_STD),
            (p + "mlp2.w", (F, W), "normal", xs(F, W)),
            (p + "mlp2.b", (W,), "normal", BIAS_STD),
        ]
    specs += [
        ("final_ln.g", (W,), "ones", 0.0),
        ("final_ln.b", (W,), "zeros", 0.0),
        ("map.probe", (1, W), "normal", xs(1, W)),
        ("map.q.w", (W, W), "normal", xs(W, W)),
        ("map.q.b", (W,), "normal", BIAS_STD),
        ("map.kv.w", (W, 2 * W), "normal", xs(W, W)),
        ("map.kv.b", (2 * W,), "normal", BIAS_STD),
        ("map.out.w", (W, W), "normal", xs(W, W)),
        ("map.out.b", (W,), "normal", BIAS_STD),
        ("map.ln.g", (W,), "ones", 0.0),
        ("map.ln.b", (W,), "zeros", 0.0),
        ("map.mlp1.w", (W, F), "normal", xs(W, F)),
        ("map.mlp1.b", (F,), "normal", BIAS_STD),
        ("map.mlp2.w", (F, W), "normal", xs(F, W)),
        ("map.mlp2.b", (W,), "normal", BIAS_STD),
    ]
    return specs


def make_weights(d: ModelDims, seed: int) -> Dict[str, np.ndarray]:
    """Draw all parameters (float32) in blob order from default_rng([seed, 0])."""
    rng = np.random.default_rng([seed, 0])
    out: Dict[str, np.ndarray] = {}
    for name, shape, kind, std in tensor_specs(d):
        if kind == "normal":
            a = rng.standard_normal(shape, dtype=np.float32)
            a *= np.float32(std)
        elif kind == "ones":
            a = np.ones(shape, np.float32)
        else:
            a = np.zeros(shape, np.float32)
        out[name] = a
    return out


def make_pixels(d: ModelDims, batch: int, seed: int) -> np.ndarray:
    """Patch-ordered input [batch, tokens, patch_dim], N(0,1) rounded to F16.

    Drawn in C order from default_rng([seed, 1]), so image 0 of a larger
    batch equals the single-image input of the same seed.
    """
    rng = np.random.default_rng([seed, 1])
    x = rng.standard_normal((batch, d.tokens, d.patch_dim), dtype=np.float32)
    return x.astype(np.float16)


def make_attention_inputs(batch: int = 32, tokens: int = 729, heads: int = 16,
                          head_dim: int = 72,
                          seeds=((0, 2), (0, 3), (0, 4))) -> Tuple[np.ndarray, ...]:
    """Q, K, V as [batch, tokens, heads*head_dim] F16 from N(0,1)."""
    outs = []
    for s in seeds:
        rng = np.random.default_rng(list(s))
        a = rng.standard_normal((batch, tokens, heads * head_dim), dtype=np.float32)
        outs.append(a.astype(np.float16))
    return tuple(outs)


def image_to_patches(img: np.ndarray, patch: int = 14) -> np.ndarray:
    """Host patch packing: [B, H, W, C] -> [B, (H/p)*(W/p), p*p*C] in
    [batch, patch_y, patch_x, y, x, channel] order (a pure rearrangement)."""
    b, h, w, c = img.shape
    gy, gx = h // patch, w // patch
    x = img[:, : gy * patch, : gx * patch, :]
    x = x.reshape(b, gy, patch, gx, patch, c).transpose(0, 1, 3, 2, 4, 5)
    return np.ascontiguousarray(x.reshape(b, gy * gx, patch * patch * c))


# ---------------------------------------------------------------- blob format
#
# Little-endian. A 64-byte header, then every tensor of tensor_specs() in that
# order as raw float32, each starting at a 64-byte aligned offset (zero fill in
# between). Header layout:
#   0  char[4]  magic "SGLP"
#   4  u32      version (1)
#   8  u32 x 8  width, depth, heads, head_dim, mlp, tokens, patch_dim, dtype(0=F32)
#   40 u64      total blob bytes (header included)
#   48 u8[16]   reserved, zero

_HDR = struct.Struct("<4sI8IQ16s")
assert _HDR.size == BLOB_HEADER_BYTES


def _align(n: int) -> int:
    return (n + BLOB_ALIGN - 1) // BLOB_ALIGN * BLOB_ALIGN


def _layout(d: ModelDims) -> Iterator[Tuple[str, Tuple[int, ...], int]]:
    off = BLOB_HEADER_BYTES
    for name, shape, _, _ in tensor_specs(d):
        off = _align(off)
        yield name, shape, off
        off += int(np.prod(shape)) * 4


def blob_size(d: ModelDims) -> int:
    end = BLOB_HEADER_BYTES
    for name, shape, off in _layout(d):
        end = off + int(np.prod(shape)) * 4
    return _align(end)


def pack_blob(d: ModelDims, weights: Dict[str, np.ndarray]) -> bytearray:
    """Serialise weights (float32) into the blob byte format."""
    total = blob_size(d)
    buf = bytearray(total)
    _HDR.pack_into(buf, 0, BLOB_MAGIC, BLOB_VERSION, d.width, d.depth, d.heads,
                   d.head_dim, d.mlp, d.tokens, d.patch_dim, DTYPE_F32, total,
                   b"\0" * 16)
    mv = memoryview(buf)
    for name, shape, off in _layout(d):
        a = np.ascontiguousarray(weights[name], dtype="<f4")
        assert a.shape == tuple(shape), (name, a.shape, shape)
        n = a.nbytes
        mv[off: off + n] = a.reshape(-1).view(np.uint8)
    return buf
