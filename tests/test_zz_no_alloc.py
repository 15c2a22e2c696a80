"""siglip_attention_noalloc (the attention entry point that allocates
nothing: its V^T staging is the library's fixed 64 MiB device array)
against siglip_attention (library-allocated staging), through the C ABI:
same arguments, same kernels, so the outputs must be the same bits. Two
calls in a row, the second with a smaller input, so the second reads a
scratch array that still holds the first call's larger V^T."""
import ctypes
import math

import numpy as np
import pytest

import synthetic as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import vision_transformer_so400m_amd as lib
    lib.use_test_hooks()
    lib.load_library()
    return lib


def _pair(V, q, k, v, heads, d, t, b, row_stride=None):
    w = heads * d
    out_a = torch.full((b, t, w), float("nan"), dtype=torch.float16, device="cuda")
    out_n = torch.full((b, t, w), float("nan"), dtype=torch.float16, device="cuda")
    V.attention(q, k, v, heads, d, 1 / math.sqrt(d), out=out_a, row_stride=row_stride, tokens=t, batch=b)
    V.attention(q, k, v, heads, d, 1 / math.sqrt(d), out=out_n, row_stride=row_stride, tokens=t, batch=b,
                noalloc=True)
    torch.cuda.synchronize()
    return out_a, out_n


def test_noalloc_matches_allocating_entry_point_twice_shrinking(V):
    # 1) the full attention workload [32, 729, 16 x 72] (56.6 MB of V^T)
    cfg = S.CONFIGS["c2_attention_b32"]
    b, t, heads, d = cfg["batch"], cfg["tokens"], cfg["heads"], cfg["head_dim"]
    print(f"noalloc: [{b}, {t}, {heads} x {d}]", flush=True)
    q, k, v = (torch.from_numpy(a).cuda() for a in S.make_attention_inputs(b, t, heads, d, cfg["seeds"]))
    a, n = _pair(V, q, k, v, heads, d, t, b)
    assert torch.isfinite(a).all()
    assert torch.equal(a.view(torch.int16), n.view(torch.int16))
    # 2) a smaller, ragged call right after: 3 images of 300 tokens read as
    # strided views of a fused row (zeros past token 299 must come from this
    # call's transpose, not from the larger V^T left in the array)
    b2, t2 = 3, 300
    print(f"noalloc: [{b2}, {t2}, {heads} x {d}] fused views", flush=True)
    w = heads * d
    rng = np.random.default_rng(21)
    fused = torch.from_numpy(rng.standard_normal((b2 * t2, 3 * w), dtype=np.float32).astype(np.float16)).cuda()
    flat = fused.reshape(-1)
    a2, n2 = _pair(V, flat[0:], flat[w:], flat[2 * w:], heads, d, t2, b2, row_stride=3 * w)
    assert torch.isfinite(a2).all()
    assert torch.equal(a2.view(torch.int16), n2.view(torch.int16))
    # 3) other head widths of the streaming kernel, and one that needs no staging
    for hd, hh in ((64, 18), (80, 16), (8, 4)):
        print(f"noalloc: head_dim {hd}", flush=True)
        qq, kk, vv = (torch.from_numpy(rng.standard_normal((2, 65, hh * hd), dtype=np.float32)
                                       .astype(np.float16)).cuda() for _ in range(3))
        a3, n3 = _pair(V, qq, kk, vv, hh, hd, 65, 2)
        assert torch.equal(a3.view(torch.int16), n3.view(torch.int16))


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_launch(V):
    lib = V.load_library()
    p = 4096   # never dereferenced: the size check fails first
    # 40 images x 1152 x 768 x 2 bytes = 70.8 MB > 64 MiB
    st = lib.siglip_attention_noalloc(p, p, p, 1152, p, 40, 16, 729, 72, 0.1, None)
    assert st == V.SIGLIP_E_INVALID_ARG
    assert "64 MiB" in V.last_error()
    # the allocating entry point has no such limit; the no-alloc one still
    # works after the refusal
    cfg = S.CONFIGS["c2_attention_b32"]
    q, k, v = (torch.from_numpy(a[:2]).cuda() for a in S.make_attention_inputs(4, 729, 16, 72, cfg["seeds"]))
    a, n = _pair(V, q, k, v, 16, 72, 729, 2)
    assert torch.equal(a.view(torch.int16), n.view(torch.int16))


def test_noalloc_runs_under_graph_capture(V):
    """A call captured into a HIP graph (where allocation is not allowed)
    and replayed three times, with other calls on the same scratch between
    the replays: every replay gives the eager bits."""
    heads, d, t, b = 16, 72, 729, 4
    rng = np.random.default_rng(5)
    q, k, v = (torch.from_numpy(rng.standard_normal((b, t, heads * d), dtype=np.float32).astype(np.float16)).cuda()
               for _ in range(3))
    eager = torch.empty((b, t, heads * d), dtype=torch.float16, device="cuda")
    V.attention(q, k, v, heads, d, 1 / math.sqrt(d), out=eager, noalloc=True)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    other = torch.empty((2, t, heads * d), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            V.attention(q, k, v, heads, d, 1 / math.sqrt(d), out=out, noalloc=True, stream=s)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        V.attention(k[:2], q[:2], v[:2], heads, d, 1 / math.sqrt(d), out=other, noalloc=True)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
    del g
