"""Pins of the CPU oracle to things other than itself.

Each test checks an oracle function against brute force written differently
(plain Python loops), a closed form, an invariant of the definition, or an
independent library implementation (torch float64 on the CPU). A plausible
slip in the oracle (dropped term, wrong sign, transposed operand, swapped
Q/K/V slice, wrong head split, wrong patch order) fails at least one test.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synthetic as S

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- linear

def test_linear_matches_triple_loop():
    x = RNG.standard_normal((3, 5))
    w = RNG.standard_normal((5, 4))
    b = RNG.standard_normal(4)
    y = O.linear(x, w, b)
    for i in range(3):
        for j in range(4):
            acc = b[j]
            for k in range(5):
                acc += x[i, k] * w[k, j]
            assert abs(y[i, j] - acc) < 1e-12


# ---------------------------------------------------------------- layer norm

def test_layer_norm_zero_mean_and_shrunk_unit_variance():
    h = RNG.standard_normal((16, 1152)) * RNG.uniform(0.01, 5, (16, 1)) + 3.0
    y = O.layer_norm(h, np.ones(1152), np.zeros(1152))
    var_in = h.var(axis=-1)
    np.testing.assert_allclose(y.mean(axis=-1), 0, atol=1e-12)
    # population variance of the output is sigma^2 / (sigma^2 + eps)
    np.testing.assert_allclose(y.var(axis=-1), var_in / (var_in + 1e-6), rtol=1e-12)


def test_layer_norm_two_value_row_closed_form():
    # row of +a and -a: mean 0, variance a^2 -> outputs +-a/sqrt(a^2+eps)
    a = 0.002
    h = np.array([a, -a] * 8)
    y = O.layer_norm(h, np.ones(16), np.zeros(16))
    np.testing.assert_allclose(y, h / math.sqrt(a * a + 1e-6), rtol=1e-13)


def test_layer_norm_affine_and_library():
    h = RNG.standard_normal((4, 144))
    g = RNG.standard_normal(144)
    b = RNG.standard_normal(144)
    y = O.layer_norm(h, g, b)
    ref = F.layer_norm(torch.from_numpy(h), (144,), torch.from_numpy(g),
                       torch.from_numpy(b), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- softmax

def test_softmax_rows_sum_to_one_and_shift_invariant():
    s = RNG.standard_normal((7, 729)) * 10
    p = O.softmax(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-13)
    assert (p > 0).all()
    np.testing.assert_allclose(O.softmax(s + 123.0), p, rtol=1e-12)
    np.testing.assert_allclose(O.softmax(np.zeros((2, 5))), 0.2, rtol=1e-15)


# ---------------------------------------------------------------- attention

def _attention_loops(q, k, v, scale):
    t_q, d = q.shape
    t_k = k.shape[0]
    out = np.zeros((t_q, v.shape[1]))
    for i in range(t_q):
        logits = [scale * sum(q[i, c] * k[j, c] for c in range(d)) for j in range(t_k)]
        m = max(logits)
        e = [math.exp(z - m) for z in logits]
        den = sum(e)
        for c in range(v.shape[1]):
            out[i, c] = sum(e[j] * v[j, c] for j in range(t_k)) / den
    return out


@pytest.mark.parametrize("t", [1, 2, 3, 4, 7, 64, 65])
def test_attention_matches_brute_force(t):
    d = 8 if t > 7 else 72
    q, k, v = (RNG.standard_normal((t, d)) for _ in range(3))
    scale = 1 / math.sqrt(d)
    np.testing.assert_allclose(O.attention(q, k, v, scale),
                               _attention_loops(q, k, v, scale), rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    t, d = 729, 72
    k = RNG.standard_normal((t, d))
    v = RNG.standard_normal((t, d))
    # zero query -> uniform weights -> column mean of V
    np.testing.assert_allclose(O.attention(np.zeros((3, d)), k, v, 0.1),
                               np.broadcast_to(v.mean(0), (3, d)), rtol=1e-11, atol=1e-13)
    # identical keys -> uniform weights whatever the query
    kk = np.broadcast_to(k[0], (t, d))
    np.testing.assert_allclose(O.attention(RNG.standard_normal((2, d)), kk, v, 0.1),
                               np.broadcast_to(v.mean(0), (2, d)), rtol=1e-11, atol=1e-13)
    # one dominant logit -> that row of V
    q = np.zeros((1, d)); q[0, 0] = 1.0
    k2 = np.zeros((t, d)); k2[37, 0] = 1e4
    np.testing.assert_allclose(O.attention(q, k2, v, 1.0)[0], v[37], rtol=1e-12)


def test_multi_head_split_matches_torch_mha():
    # fused QKV slices + head views vs torch's MultiheadAttention (library)
    w, h, t = 144, 2, 5
    x = RNG.standard_normal((2, t, w))
    wqkv = RNG.standard_normal((w, 3 * w)) * 0.1
    bqkv = RNG.standard_normal(3 * w) * 0.1
    wo = RNG.standard_normal((w, w)) * 0.1
    bo = RNG.standard_normal(w) * 0.1
    qkv = O.linear(x, wqkv, bqkv)
    q, k, v = qkv[..., :w], qkv[..., w:2 * w], qkv[..., 2 * w:]
    o = O.merge_heads(O.attention(O.split_heads(q, h), O.split_heads(k, h),
                                  O.split_heads(v, h), 1 / math.sqrt(w // h)))
    ours = O.linear(o, wo, bo)
    mha = torch.nn.MultiheadAttention(w, h, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(torch.from_numpy(wqkv.T))
        mha.in_proj_bias.copy_(torch.from_numpy(bqkv))
        mha.out_proj.weight.copy_(torch.from_numpy(wo.T))
        mha.out_proj.bias.copy_(torch.from_numpy(bo))
        xt = torch.from_numpy(x)
        ref = mha(xt, xt, xt, need_weights=False)[0].numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- GELU

def test_gelu_tanh_library_and_identities():
    x = np.linspace(-12, 12, 20001)
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(x), ref, rtol=1e-13, atol=1e-15)
    # gelu(x) - gelu(-x) = x for the tanh form (tanh is odd)
    np.testing.assert_allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, rtol=1e-12, atol=1e-13)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.gelu_tanh(np.array([1.0])), [0.8411919906082768], rtol=1e-14)


# ---------------------------------------------------------------- e4m3

def _e4m3_code_values():
    vals = []
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            continue  # NaN encodings
        v = s * (m / 8.0) * 2.0 ** -6 if e == 0 else s * (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append((code, v))
    return vals


def test_e4m3_every_code_is_a_fixed_point_and_ties_go_even():
    vals = _e4m3_code_values()
    assert len(vals) == 254
    arr = np.array([v for _, v in vals])
    np.testing.assert_array_equal(O.e4m3_round(arr), arr)
    pos = sorted({(abs(v), c & 0x7F) for c, v in vals})
    for (a, ca), (b, cb) in zip(pos, pos[1:]):
        mid = (a + b) / 2
        even = a if ca % 2 == 0 else b
        assert O.e4m3_round(np.array([mid]))[0] == even
        assert O.e4m3_round(np.array([np.nextafter(mid, 0)]))[0] == a
        assert O.e4m3_round(np.array([np.nextafter(mid, 1e9)]))[0] == b
    assert pos[-1][0] == 448.0
    np.testing.assert_array_equal(O.e4m3_round(np.array([449.0, 464.0, 500.0, 1e6, -1e6])),
                                  [448, 448, 448, 448, -448])
    np.testing.assert_array_equal(O.e4m3_round(np.array([2.0 ** -10, 1.5 * 2.0 ** -10])),
                                  [0.0, 2.0 ** -9])


def test_e4m3_matches_torch_in_range():
    x = np.concatenate([RNG.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 100)])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e4m3_round(x), ref)
    np.testing.assert_array_equal(O.fp8_operand(x / 16), ref / 16)


# ---------------------------------------------------------------- model level

def _torch_model(wt, image, dims, layers):
    """Independent float64 implementation from torch library routines:
    conv2d for the VALID patch convolution on the raw image, layer_norm,
    MultiheadAttention and tanh-GELU."""
    W, H = dims.width, dims.heads
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    img = t(image).permute(0, 3, 1, 2)                            # [B,C,H,W]
    conv_w = t(wt["embed.w"]).reshape(dims.patch, dims.patch, dims.channels, W)
    conv_w = conv_w.permute(3, 2, 0, 1)                           # [W,C,p,p]
    x = F.conv2d(img, conv_w, t(wt["embed.b"]), stride=dims.patch)
    x = x.flatten(2).transpose(1, 2) + t(wt["pos"])               # [B,T,W]

    def mha(q_in, kv_in, wq, bq, wk, bk, wv, bv, wo, bo):
        m = torch.nn.MultiheadAttention(W, H, batch_first=True, dtype=torch.float64)
        with torch.no_grad():
            m.in_proj_weight.copy_(torch.cat([t(wq), t(wk), t(wv)], 1).T)
            m.in_proj_bias.copy_(torch.cat([t(bq), t(bk), t(bv)]))
            m.out_proj.weight.copy_(t(wo).T)
            m.out_proj.bias.copy_(t(bo))
            return m(q_in, kv_in, kv_in, need_weights=False)[0]

    ln = lambda a, p: F.layer_norm(a, (W,), t(wt[p + ".g"]), t(wt[p + ".b"]), eps=1e-6)
    mlp = lambda a, p: F.gelu(a @ t(wt[p + "1.w"]) + t(wt[p + "1.b"]),
                              approximate="tanh") @ t(wt[p + "2.w"]) + t(wt[p + "2.b"])
    with torch.no_grad():
        for i in range(layers):
            p = f"layer{i}."
            a = ln(x, p + "ln1")
            wqkv, bqkv = wt[p + "qkv.w"], wt[p + "qkv.b"]
            x = x + mha(a, a, wqkv[:, :W], bqkv[:W], wqkv[:, W:2 * W], bqkv[W:2 * W],
                        wqkv[:, 2 * W:], bqkv[2 * W:], wt[p + "out.w"], wt[p + "out.b"])
            x = x + mlp(ln(x, p + "ln2"), p + "mlp")
        z = ln(x, "final_ln")
        probe = t(wt["map.probe"]).expand(z.shape[0], 1, W)
        wkv, bkv = wt["map.kv.w"], wt["map.kv.b"]
        y = mha(probe, z, wt["map.q.w"], wt["map.q.b"], wkv[:, :W], bkv[:W],
                wkv[:, W:], bkv[W:], wt["map.out.w"], wt["map.out.b"])
        return (y + mlp(ln(y, "map.ln"), "map.mlp")).numpy()


@pytest.mark.parametrize("dims", [S.small_dims(2), S.four_token_dims(2)],
                         ids=["small_w144_t4", "fourtoken_w1152"])
def test_whole_model_matches_torch_from_raw_image(dims):
    wt = S.make_weights(dims, seed=5)
    rng = np.random.default_rng(7)
    side = dims.image_side
    image = rng.standard_normal((2, side, side, 3))
    pixels = S.image_to_patches(image, dims.patch)
    ours = O.encode(wt, pixels, dims.heads)
    ref = _torch_model(wt, image, dims, dims.depth)
    assert ours.shape == (2, 1, dims.width)
    np.testing.assert_allclose(ours, ref, rtol=1e-9, atol=1e-10)


def test_permutation_invariance_without_position_embedding():
    dims = S.small_dims(2).__class__(width=144, depth=2, heads=2, head_dim=72,
                                     mlp=288, tokens=9, patch_dim=588)
    wt = S.make_weights(dims, seed=3)
    wt["pos"] = np.zeros_like(wt["pos"])
    x = np.random.default_rng(0).standard_normal((1, 9, 588))
    perm = np.random.default_rng(1).permutation(9)
    a = O.encode(wt, x, dims.heads)
    b = O.encode(wt, x[:, perm], dims.heads)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    # with the positional embedding the order matters
    wt2 = S.make_weights(dims, seed=3)
    assert np.abs(O.encode(wt2, x, 2) - O.encode(wt2, x[:, perm], 2)).max() > 1e-4


def test_batch_independence_and_shape():
    dims = S.SO400M.with_depth(1)
    wt = S.make_weights(dims, seed=0)
    x8 = S.make_pixels(dims, 3, seed=0)
    x1 = S.make_pixels(dims, 1, seed=0)
    np.testing.assert_array_equal(x8[:1], x1)   # generator prefix property
    y3 = O.encode(wt, x8, 16)
    y1 = O.encode(wt, x1, 16)
    assert y3.shape == (3, 1, 1152)
    np.testing.assert_allclose(y3[:1], y1, rtol=1e-12, atol=1e-13)
    assert np.abs(y3[0] - y3[1]).max() > 1e-3


def test_map_with_zero_query_pools_the_mean_value():
    dims = S.small_dims(1)
    wt = S.make_weights(dims, seed=2)
    wt["map.q.w"] = np.zeros_like(wt["map.q.w"])
    wt["map.q.b"] = np.zeros_like(wt["map.q.b"])
    st = {}
    x = S.make_pixels(dims, 2, seed=2).astype(np.float64)
    O.encode(wt, x, dims.heads, stages=st)
    v = st["map.kv"][..., dims.width:]
    np.testing.assert_allclose(st["map.attn"][:, 0], v.mean(axis=1), rtol=1e-12, atol=1e-14)


def test_fp32_arithmetic_agrees_with_fp64():
    dims = S.SO400M.with_depth(1)
    wt = S.make_weights(dims, seed=0)
    x = S.make_pixels(dims, 1, seed=0)
    y64 = O.encode(wt, x, 16)
    y32 = O.encode(wt, x, 16, dtype=np.float32)
    assert np.abs(y64 - y32).max() < 1e-4


def _torch_e4m3_operand(a):
    """Independent e4m3 operand value: torch's float8_e4m3fn cast (round to
    nearest even) of 2^4 a after clipping to +-448 (torch gives NaN above the
    range instead of saturating), divided back by 2^4."""
    a = torch.as_tensor(np.asarray(a, np.float64))
    return torch.clamp(a * 16.0, -448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64) / 16.0


def test_fp8_gemm_equals_scaled_code_product():
    # float32 inputs, so 2^4 x is exact and there is no double rounding on
    # torch's side; a few values past the e4m3 range exercise saturation
    x = (RNG.standard_normal((5, 64)) * 0.5).astype(np.float32)
    w = (RNG.standard_normal((64, 7)) * 0.05).astype(np.float32)
    x[0, :3] = [40.0, -35.0, 1e-5]
    b = RNG.standard_normal(7)
    y = O.weight_gemm(x.astype(np.float64), w.astype(np.float64), b, True)
    cx = torch.clamp(torch.from_numpy(x.astype(np.float64)) * 16, -448, 448).to(torch.float8_e4m3fn)
    cw = torch.clamp(torch.from_numpy(w.astype(np.float64)) * 16, -448, 448).to(torch.float8_e4m3fn)
    ref = (cx.to(torch.float64).numpy() @ cw.to(torch.float64).numpy()) / 256.0 + b
    np.testing.assert_array_equal(y, ref)
    # quantizing only the weights, or quantizing without the 2^4 scale,
    # gives other numbers
    assert not np.array_equal(O.linear(x.astype(np.float64), O.fp8_operand(w), b), ref)
    unscaled = (torch.from_numpy(x.astype(np.float64)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
                @ torch.from_numpy(w.astype(np.float64)).to(torch.float8_e4m3fn).to(torch.float64).numpy()) + b
    assert not np.allclose(unscaled, ref, rtol=1e-3, atol=1e-6)


def test_fp8_gemm_hand_worked_midpoints_and_saturation():
    # 2^4 x = [[1.0625, 1.1875], [500, -0.016]]: 1.0625 is the midpoint of
    # 1 and 1.125 (ties to the even mantissa: 1), 1.1875 the midpoint of
    # 1.125 and 1.25 (even: 1.25), 500 saturates to 448, -0.016 is
    # -8.192 subnormal steps of 2^-9 -> -8 * 2^-9 = -0.015625.
    # 2^4 w = [[2, 0.5], [1, 3]] are e4m3 values.
    x = np.array([[1.0625, 1.1875], [500.0, -0.016]]) / 16
    w = np.array([[2.0, 0.5], [1.0, 3.0]]) / 16
    b = np.array([0.5, -0.25])
    # codes product [[1*2 + 1.25*1, 1*0.5 + 1.25*3], [448*2 - 0.015625, 448*0.5 - 0.015625*3]]
    #             = [[3.25, 4.25], [895.984375, 223.953125]], times 2^-8, plus b
    expect = np.array([[3.25, 4.25], [895.984375, 223.953125]]) / 256 + b
    np.testing.assert_array_equal(O.weight_gemm(x, w, b, True), expect)
    assert expect[0, 0] == 0.5126953125 and expect[1, 1] == 0.62481689453125


def _torch_fp8_model(wt, pixels, dims, layers):
    """Independent float64 model in which every weight GEMM (patch, QKV,
    out-projection, MLP, MAP q, K/V, out-projection and MLP) multiplies torch
    e4m3 casts of both operands; attention, layernorm, GELU and residuals
    exact. Works on patch vectors."""
    W, H, D = dims.width, dims.heads, dims.head_dim
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    q8 = _torch_e4m3_operand

    def lin(a, wn, bn):
        return q8(a) @ q8(wt[wn]) + t(wt[bn])

    def heads_attn(q, k, v):
        B, Tq, Tk = q.shape[0], q.shape[1], k.shape[1]
        qh = q.reshape(B, Tq, H, D).transpose(1, 2)
        kh = k.reshape(B, Tk, H, D).transpose(1, 2)
        vh = v.reshape(B, Tk, H, D).transpose(1, 2)
        p = torch.softmax(qh @ kh.transpose(-1, -2) / math.sqrt(D), dim=-1)
        return (p @ vh).transpose(1, 2).reshape(B, Tq, W)

    ln = lambda a, p: F.layer_norm(a, (W,), t(wt[p + ".g"]), t(wt[p + ".b"]), eps=1e-6)
    gelu = lambda a: F.gelu(a, approximate="tanh")
    x = lin(t(pixels), "embed.w", "embed.b") + t(wt["pos"])
    for i in range(layers):
        p = f"layer{i}."
        qkv = lin(ln(x, p + "ln1"), p + "qkv.w", p + "qkv.b")
        o = heads_attn(qkv[..., :W], qkv[..., W:2 * W], qkv[..., 2 * W:])
        x = x + lin(o, p + "out.w", p + "out.b")
        x = x + lin(gelu(lin(ln(x, p + "ln2"), p + "mlp1.w", p + "mlp1.b")), p + "mlp2.w", p + "mlp2.b")
    z = ln(x, "final_ln")
    q = lin(t(wt["map.probe"]), "map.q.w", "map.q.b").expand(z.shape[0], 1, W)
    kv = lin(z, "map.kv.w", "map.kv.b")
    y = lin(heads_attn(q, kv[..., :W], kv[..., W:]), "map.out.w", "map.out.b")
    return (y + lin(gelu(lin(ln(y, "map.ln"), "map.mlp1.w", "map.mlp1.b")), "map.mlp2.w", "map.mlp2.b")).numpy()


@pytest.mark.parametrize("dims", [S.small_dims(2), S.four_token_dims(2)],
                         ids=["small_w144_t4", "fourtoken_w1152"])
def test_fp8_whole_model_matches_torch_e4m3_model(dims):
    wt = S.make_weights(dims, seed=8)
    x = S.make_pixels(dims, 2, seed=9)
    ours = O.encode(wt, x, dims.heads, fp8=True)
    ref = _torch_fp8_model(wt, x, dims, dims.depth)
    np.testing.assert_allclose(ours, ref, rtol=1e-9, atol=1e-10)
    # and it is not the unquantized model
    assert np.abs(ours - O.encode(wt, x, dims.heads)).max() > 1e-3
