"""The synthetic model's shapes against the sizes the pages print
(tests/golden/page_sizes.json, each value cited there)."""
import json
import os

import numpy as np

import synthetic as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")))


def g(k):
    return GOLD[k]["value"]


def test_io_bytes():
    d = S.SO400M
    x = S.make_pixels(d, 1, 0)
    assert x.nbytes == g("input_bytes_per_image")
    assert d.width * 2 == g("output_bytes_per_image")
    assert (d.image_side, d.tokens, d.patch_dim) == (378, g("tokens"), 588)


def test_weight_shapes_and_fp8_bytes():
    specs = {n: s for n, s, _, _ in S.tensor_specs(S.SO400M.with_depth(1))}
    one_byte = lambda n: int(np.prod(specs[n]))
    # q, k, v (fused) + out projection: four width x width matrices
    assert one_byte("layer0.qkv.w") + one_byte("layer0.out.w") == g("fp8_bytes_four_1152_projections")
    assert one_byte("layer0.mlp1.w") == g("fp8_bytes_mlp_up")
    assert one_byte("embed.w") == g("fp8_bytes_input_projection_logical")
    assert specs["layer0.qkv.w"][1] == g("fused_qkv_out")
    assert specs["map.kv.w"][1] == g("map_kv_out")
    assert specs["layer0.mlp1.w"][1] == g("mlp")
    assert S.SO400M.heads * S.SO400M.head_dim == g("width") and S.SO400M.heads == g("heads")
    # one layer, fused: embed, qkv, out, mlp1, mlp2, map q, map kv, map out, map mlp1, map mlp2
    n_gemm = sum(1 for n, s in specs.items() if n.endswith(".w") and len(s) == 2)
    assert n_gemm == g("gemms_fused")


def test_small_model_dims():
    d = S.small_dims()
    sm = g("small_model")
    assert (d.image_side, d.width, d.heads, d.head_dim, d.mlp) == (
        sm["image"], sm["width"], sm["heads"], sm["head_dim"], sm["mlp"])
    assert d.tokens == 4


def test_blob_roundtrip_layout():
    d = S.small_dims(2)
    wt = S.make_weights(d, 9)
    blob = S.pack_blob(d, wt)
    assert len(blob) == S.blob_size(d) and len(blob) % 64 == 0
    assert bytes(blob[:4]) == b"SGLP"
    # every tensor is recoverable at its aligned offset
    off = S.BLOB_HEADER_BYTES
    for name, shape, _, _ in S.tensor_specs(d):
        off = (off + 63) // 64 * 64
        n = int(np.prod(shape))
        got = np.frombuffer(bytes(blob[off:off + 4 * n]), "<f4").reshape(shape)
        np.testing.assert_array_equal(got, wt[name])
        off += 4 * n
    # 27-layer parameter count
    total = sum(int(np.prod(s)) for _, s, _, _ in S.tensor_specs(S.SO400M))
    assert total == 428_225_600
