"""CPU checks of the algebraic readings the GPU path relies on (float64,
numpy only; no HIP code is involved).

The MAP head's K/V projection is folded on the GPU (page "Single-layer
SigLIP vision benchmark", intro: one shared learned probe, one fused K/V
projection of the final-LN tokens): per head h the probe's scores are
Z (W_k,h q_h) + b_k,h . q_h, where the constant term cancels in the softmax,
and the head output is (sum_t p_t Z_t) W_v,h + b_v,h because the
probabilities sum to one. Both are identities in the reals; this test shows
they hold to float64 rounding, including with a large key bias."""
import numpy as np


def _softmax(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_map_kv_fold_is_the_plain_probe_attention():
    rng = np.random.default_rng(7)
    T, W, H = 37, 48, 4
    D = W // H
    z = rng.standard_normal((T, W))
    wk, wv = rng.standard_normal((W, W)) * 0.2, rng.standard_normal((W, W)) * 0.2
    bk, bv = rng.standard_normal(W) * 3.0, rng.standard_normal(W)
    q = rng.standard_normal(W)
    scale = 1 / np.sqrt(D)
    k, v = z @ wk + bk, z @ wv + bv
    for h in range(H):
        sl = slice(h * D, (h + 1) * D)
        p_plain = _softmax(scale * (k[:, sl] @ q[sl]))
        o_plain = p_plain @ v[:, sl]
        u = wk[:, sl] @ q[sl]                       # W_k,h q_h
        p_fold = _softmax(scale * (z @ u))          # b_k,h . q_h dropped
        o_fold = (p_fold @ z) @ wv[:, sl] + bv[sl]  # (sum_t p_t Z_t) W_v,h + b_v,h
        np.testing.assert_allclose(p_fold, p_plain, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(o_fold, o_plain, rtol=1e-11, atol=1e-12)
        # the check is sensitive to plausible slips: a dropped value bias, or
        # the key bias applied per token instead of cancelling
        assert not np.allclose((p_fold @ z) @ wv[:, sl], o_plain, rtol=1e-6)
        assert not np.allclose(_softmax(scale * (z @ u + (z @ np.ones(W)) * (bk[sl] @ q[sl]))), p_plain, rtol=1e-6)
