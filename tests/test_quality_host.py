"""The quality harness's host parts (CPU): the uncompressed reference attention and
the metrics, against scipy and closed forms; the needle queries' construction."""
import math

import numpy as np
import scipy.special

from kv_cache_quantization_block_amd import quality


def test_reference_is_dense_softmax_attention():
    rng = np.random.default_rng(3)
    B, Hkv, G, T, D = 2, 2, 3, 50, 128
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float16)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float16)
    s, out = quality.reference(k, v, q, 0.2)
    for b in range(B):
        for h in range(Hkv * G):
            kk, vv = k[b, h // G].astype(np.float64), v[b, h // G].astype(np.float64)
            sr = 0.2 * kk @ q[b, h].astype(np.float64)
            np.testing.assert_allclose(s[b, h], sr, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(out[b, h], scipy.special.softmax(sr) @ vv, rtol=1e-11, atol=1e-13)


def test_metrics_closed_forms():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((2, 4, 128))
    s = rng.standard_normal((2, 4, 100))
    m = quality.metrics(o, o, s, s)
    assert m["rel_l2_max"] == 0.0 and abs(m["cos_min"] - 1.0) < 1e-15 and m["score_rel_mean"] == 0.0
    assert m["top1_min"] == m["top8_min"] == m["top32_min"] == 1.0
    m = quality.metrics(1.01 * o, o, 1.02 * s, s)            # a pure scale
    assert abs(m["rel_l2_mean"] - 0.01) < 1e-12 and abs(m["cos_min"] - 1.0) < 1e-12
    assert abs(m["score_rel_mean"] - 0.02) < 1e-12 and m["top32_min"] == 1.0
    m = quality.metrics(-o, o, -s, s)                          # everything reversed
    assert abs(m["rel_l2_mean"] - 2.0) < 1e-12 and abs(m["cos_mean"] + 1.0) < 1e-12
    assert m["top1_mean"] == 0.0


def test_needle_queries_point_at_their_row():
    """Needle queries put the softmax's largest weight on their target row."""
    k, v, q = quality.make_inputs(5, 1, 2, 4, 300, "needle", device="cpu")
    s, _ = quality.reference(k.numpy(), v.numpy(), q.numpy(), 1 / math.sqrt(128))
    p = scipy.special.softmax(s, axis=-1)
    assert np.mean(p.max(axis=-1) > 0.5) > 0.9
