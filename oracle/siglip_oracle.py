"""CPU oracle for the SigLIP So400m/14 image-encoder forward pass.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module. The product (the HIP library
and its Python binding) never imports it, and it imports nothing from the
product. It is deliberately plain and slow: numpy, float64 by default, the
steps in the order the pages give them, no blocking, fusion or reordering
beyond what the definitions state. A numpy matmul is used as a library step.

Page citations below use these short names for the source pages:
  [SLB] "Single-layer SigLIP vision benchmark" (intro, mermaid figure,
        "Performance follow-up", "Fused encoder QKV and MAP KV (2026-09-09)")
  [PVN] "SigLIP optimized execution and PV padding -- 12 September 2026"
        ("Cause and fix", "Full-model results")
  [CAP] "Capacity-first baseline -- September 12, 2026"
        ("Correctness fixes exposed by the new layouts": blocked attention)
  [FP8] "FP8 attention and resident image/embedding transfers"
        (intro, "Full 27-layer ViT", "Host transfer mechanism")

Where the pages leave a step open, the reading taken is stated at the
function. Every function here is pinned by the CPU tests to something other
than itself (brute force, closed forms, library routines, printed sizes);
none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

LN_EPS = 1e-6          # [SLB] intro: layernorm epsilon 1e-6
FP8_SCALE_EXP = -4     # [SLB] intro example "--fp8-scale=-4"; [PVN] "scale -4"
E4M3_MAX = 448.0


# ----------------------------------------------------------------- primitives

def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """y = x @ w + b with w stored [in, out]. [SLB] intro: every projection is a
    GEMM followed by a bias addition."""
    y = np.matmul(x, w)
    if b is not None:
        y = y + b
    return y


def layer_norm(h: np.ndarray, g: np.ndarray, b: np.ndarray,
               eps: float = LN_EPS) -> np.ndarray:
    """[SLB] intro, layernorm paragraph: separate sum, centered-variance and
    affine passes with epsilon 1e-6. Reading: population variance (divide by
    the width), epsilon inside the square root, scale and shift after
    normalisation."""
    n = h.shape[-1]
    mu = h.sum(axis=-1, keepdims=True) / n                    # pass 1: sum
    c = h - mu
    var = (c * c).sum(axis=-1, keepdims=True) / n              # pass 2: centered
    return c / np.sqrt(var + eps) * g + b                      # pass 3: affine


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU on the MLP hidden tensor ([SLB] intro: "GELU"; the tanh form is
    the reading taken, the published tanh approximation of the Gaussian
    error linear unit)."""
    k = math.sqrt(2.0 / math.pi)
    return 0.5 * x * (1.0 + np.tanh(k * (x + 0.044715 * x * x * x)))


def softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis: subtract the row maximum, exponentiate,
    divide by the row sum ([PVN] "Cause and fix": the softmax keeps a maximum
    and a denominator per row)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Scaled dot-product attention: softmax(q k^T * scale) v over the last two
    axes (any leading batch axes). [SLB] intro: Q/K/V projections ->
    self-attention; the scale 1/sqrt(head width) is the reading taken."""
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * scale
    return np.matmul(softmax(s), v)


def split_heads(x: np.ndarray, heads: int) -> np.ndarray:
    """[..., T, heads*D] -> [..., heads, T, D]: head h owns the D consecutive
    columns starting at h*D ([SLB] "Fused encoder QKV and MAP KV": last-axis
    slices composed with head views)."""
    *lead, t, w = x.shape
    d = w // heads
    return np.swapaxes(x.reshape(*lead, t, heads, d), -3, -2)


def merge_heads(x: np.ndarray) -> np.ndarray:
    """Inverse of split_heads: heads concatenated in order along the width."""
    *lead, h, t, d = x.shape
    return np.swapaxes(x, -3, -2).reshape(*lead, t, h * d)


# ------------------------------------------------------------ FP8 (e4m3) mode

def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest OCP e4m3fn value (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits, no infinities), ties to even, saturating at +-448.
    The pages name the format "F143" ([SLB] intro, FP8 paragraph); saturation
    is the reading taken (the pages are silent on overflow)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # binade exponent e with 2^e <= a < 2^(e+1); below 2^-6 the spacing is
    # fixed at 2^-9 (subnormals)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    e = e - 1
    e = np.maximum(e, -6)
    quantum = np.ldexp(1.0, e - 3)
    r = np.rint(a / quantum) * quantum          # np.rint: ties to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def fp8_operand(x: np.ndarray, scale_exp: int = FP8_SCALE_EXP) -> np.ndarray:
    """Value an e4m3 operand at power-of-two scale 2^scale_exp represents:
    2^scale_exp * e4m3(2^-scale_exp * x) ([SLB] intro: "--fp8-scale=-4";
    [FP8] intro: both operands of a product use that scale)."""
    s = 2.0 ** (-scale_exp)
    return e4m3_round(x * s) / s


# ------------------------------------------------------------------ the model

def weight_gemm(x, w, b, fp8: bool):
    """A weight GEMM. In FP8 mode both operands are first replaced by their
    e4m3 values at scale 2^-4 ([SLB] intro, FP8 paragraph: the pages' host
    reference applies the same operand quantization at every GEMM it checks);
    the products, their sum and the bias stay exact. Pinned exactly against
    torch's float8_e4m3fn casts composed by hand, a hand-worked case at
    rounding midpoints and saturation, and an independent torch model."""
    if fp8:
        return linear(fp8_operand(x), fp8_operand(w), b)
    return linear(x, w, b)


def patch_embed(x: np.ndarray, wt: Dict[str, np.ndarray], fp8: bool = False) -> np.ndarray:
    """[SLB] intro: the VALID 14x14/14 patch convolution is the 588->width
    embedding GEMM plus bias on patch-ordered pixels, then the learned
    positional embedding is added per token."""
    return weight_gemm(x, wt["embed.w"], wt["embed.b"], fp8) + wt["pos"]


def encoder_layer(h: np.ndarray, wt: Dict[str, np.ndarray], i: int, heads: int,
                  fp8: bool = False, stages: Optional[dict] = None) -> np.ndarray:
    """One pre-norm encoder block ([SLB] intro and mermaid figure):
    h += out_proj(attention(LN1(h))); h += MLP(LN2(h)), with the fused
    1152->3456 QKV projection sliced Q | K | V along the last axis
    ([SLB] "Fused encoder QKV and MAP KV")."""
    p = f"layer{i}."
    w = h.shape[-1]
    d = w // heads
    a = layer_norm(h, wt[p + "ln1.g"], wt[p + "ln1.b"])
    qkv = weight_gemm(a, wt[p + "qkv.w"], wt[p + "qkv.b"], fp8)
    q, k, v = qkv[..., :w], qkv[..., w:2 * w], qkv[..., 2 * w:]
    o = merge_heads(attention(split_heads(q, heads), split_heads(k, heads),
                              split_heads(v, heads), 1.0 / math.sqrt(d)))
    h1 = h + weight_gemm(o, wt[p + "out.w"], wt[p + "out.b"], fp8)
    a2 = layer_norm(h1, wt[p + "ln2.g"], wt[p + "ln2.b"])
    u = gelu_tanh(weight_gemm(a2, wt[p + "mlp1.w"], wt[p + "mlp1.b"], fp8))
    h2 = h1 + weight_gemm(u, wt[p + "mlp2.w"], wt[p + "mlp2.b"], fp8)
    if stages is not None:
        stages.update({p + "ln1": a, p + "qkv": qkv, p + "attn": o,
                       p + "h_attn": h1, p + "ln2": a2, p + "mlp_hidden": u,
                       p + "h_out": h2})
    return h2


def map_head(z: np.ndarray, wt: Dict[str, np.ndarray], heads: int,
             fp8: bool = False, stages: Optional[dict] = None) -> np.ndarray:
    """MAP pooling ([SLB] intro and mermaid figure; "Fused encoder QKV and
    MAP KV"): one learned probe shared by every image has its own query
    projection; one fused width->2*width KV projection of the encoder output
    (K first, then V); multi-head cross-attention; output projection; then
    out = y + MLP(LN(y)). Returns [B, 1, width] (the probe axis is kept)."""
    w = z.shape[-1]
    d = w // heads
    q = weight_gemm(wt["map.probe"], wt["map.q.w"], wt["map.q.b"], fp8)    # [1, W]
    kv = weight_gemm(z, wt["map.kv.w"], wt["map.kv.b"], fp8)               # [B, T, 2W]
    k, v = kv[..., :w], kv[..., w:]
    qh = split_heads(np.broadcast_to(q, (z.shape[0], 1, w)), heads)  # [B,H,1,D]
    o = merge_heads(attention(qh, split_heads(k, heads), split_heads(v, heads),
                              1.0 / math.sqrt(d)))                   # [B,1,W]
    y = weight_gemm(o, wt["map.out.w"], wt["map.out.b"], fp8)
    a = layer_norm(y, wt["map.ln.g"], wt["map.ln.b"])
    u = gelu_tanh(weight_gemm(a, wt["map.mlp1.w"], wt["map.mlp1.b"], fp8))
    out = y + weight_gemm(u, wt["map.mlp2.w"], wt["map.mlp2.b"], fp8)
    if stages is not None:
        stages.update({"map.q": q, "map.kv": kv, "map.attn": o, "map.y": y,
                       "map.ln": a, "map.mlp_hidden": u, "out": out})
    return out


def encode(wt: Dict[str, np.ndarray], pixels: np.ndarray, heads: int,
           layers: Optional[int] = None, fp8: bool = False,
           dtype=np.float64, stages: Optional[dict] = None) -> np.ndarray:
    """The whole forward pass: patch-ordered pixels [B, T, 588] -> [B, 1, W].

    [SLB] intro: patch GEMM + bias, positional embedding, `layers` pre-norm
    blocks, final encoder layernorm, MAP pooling. `layers` defaults to the
    number of blocks present in `wt`. `fp8` quantizes every weight GEMM's
    operands (a diagnostic; the accuracy bar of the FP8 path is measured
    against the unquantized computation, as the pages do in [FP8]
    "Full 27-layer ViT"). `dtype` is the arithmetic type (float64 default;
    float32 mirrors the pages' FP32 host reference).
    """
    if layers is None:
        layers = 0
        while f"layer{layers}.qkv.w" in wt:
            layers += 1
    wt = {k: np.asarray(v, dtype=dtype) for k, v in wt.items()
          if not k.startswith("layer") or int(k[5:k.index(".")]) < layers}
    x = np.asarray(pixels, dtype=dtype)
    h = patch_embed(x, wt, fp8)
    if stages is not None:
        stages["embed"] = h
    for i in range(layers):
        h = encoder_layer(h, wt, i, heads, fp8, stages)
    z = layer_norm(h, wt["final_ln.g"], wt["final_ln.b"])
    if stages is not None:
        stages["final_ln"] = z
    return map_head(z, wt, heads, fp8, stages)
