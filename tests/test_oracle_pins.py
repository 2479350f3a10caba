"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: the
article's printed sizes, the published Gaussian Lloyd-Max levels, closed
forms of the Hadamard algebra, scipy's Hadamard matrix and numerical
integration, numpy's binary16 conversion, and brute force on small inputs.
The article is openalchemy.io "llama.cpp に TurboQuant を実装 -- 2bit・3bit の
KV キャッシュ圧縮"; the section each test follows is named in its docstring.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats

import oracle

H128 = scipy.linalg.hadamard(128).astype(np.float64)   # Sylvester construction, natural order


def _golden(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _unpack(codes, bits):
    """Independent unpacking: little-endian bit stream, code i at bits [b*i, b*i+b)."""
    codes = np.asarray(codes, np.uint8).reshape(-1, 16 * bits)
    stream = np.unpackbits(codes, axis=1, bitorder="little").reshape(-1, 128, bits)
    return (stream * (1 << np.arange(bits))).sum(axis=2)


def _pack(code, bits):
    code = np.asarray(code).reshape(-1, 128)
    stream = ((code[:, :, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(code.shape[0], -1)
    return np.packbits(stream, axis=1, bitorder="little")


def _rng_blocks(seed, nb, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((nb, 128))
    if outliers:
        x[:, rng.choice(128, 4, replace=False)] *= 20
    x *= np.exp(rng.uniform(np.log(0.5), np.log(4.0), (nb, 1)))
    return x.astype(np.float16)


# ---------------------------------------------------------------- binary16

def test_half_to_double_all_patterns():
    """fp16 decoding of every bit pattern matches numpy's binary16."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_double_to_half_matches_numpy():
    """Round-to-nearest-even into fp16: normals, subnormals, exact midpoints, overflow."""
    rng = np.random.default_rng(0)
    vals = [0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, -70000.0, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
            1.0 + 3 * 2.0 ** -11, 0.1, 1e-9, float("inf"), -float("inf")]
    # exact midpoints between adjacent fp16 values (ties to even)
    h = rng.integers(0, 0x7BFF, 2000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    vals += list((lo + hi) / 2) + list(-(lo + hi) / 2)
    vals += list(rng.standard_normal(5000) * 10.0 ** rng.uniform(-9, 5, 5000))
    vals = np.array(vals, dtype=np.float64)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_half_bits(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- rotation (FWHT)

def test_fwht_equals_dense_sylvester_hadamard():
    """Section "TurboQuant の何が違うのか": the add/sub transform is the Hadamard matrix.
    Butterflies vs scipy's dense Sylvester H: exact on integers, 1e-12 on doubles."""
    rng = np.random.default_rng(1)
    xi = rng.integers(-1000, 1000, (16, 128)).astype(np.float64)
    assert np.array_equal(oracle.fwht128(xi), xi @ H128.T)
    xd = rng.standard_normal((16, 128))
    ref = xd @ H128.T
    assert np.max(np.abs(oracle.fwht128(xd) - ref)) <= 1e-12 * np.max(np.abs(ref))
    # unit vectors give the columns of H; the all-ones vector gives 128 e_0
    assert np.array_equal(oracle.fwht128(np.eye(128)), H128)
    e0 = np.zeros(128)
    e0[0] = 128
    assert np.array_equal(oracle.fwht128(np.ones(128))[0], e0)


def test_hadamard_algebra():
    """Self-inverse up to 128 (H H = 128 I), norm preserving once scaled by 1/sqrt(128),
    Sylvester recursion H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    H = oracle.fwht128(np.eye(128))
    assert np.array_equal(H @ H, 128 * np.eye(128))
    assert np.array_equal(oracle.fwht128(H), 128 * np.eye(128))   # transform applied twice
    Hs = np.array([[1.0]])
    while Hs.shape[0] < 128:
        Hs = np.block([[Hs, Hs], [Hs, -Hs]])
    assert np.array_equal(H, Hs)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128))
    y = oracle.fwht128(x) / math.sqrt(128)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


# ---------------------------------------------------------------- Lloyd-Max codebook

@pytest.mark.parametrize("bits", [1, 2, 3])
def test_lloyd_max_optimality_conditions(bits):
    """Section "TurboQuant の何が違うのか": optimal (Lloyd-Max) scalar quantiser.
    Centroid condition by independent numerical integration (scipy.quad), midpoint
    condition, symmetry, strictly increasing levels."""
    lv, th, _ = oracle.codebook(bits)
    L = 1 << bits
    assert lv.shape == (L,) and th.shape == (L - 1,)
    assert np.all(np.diff(lv) > 0)
    np.testing.assert_array_equal(lv, -lv[::-1])
    np.testing.assert_allclose(th, (lv[:-1] + lv[1:]) / 2, rtol=0, atol=1e-15)
    assert th[L // 2 - 1] == 0.0
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    pdf = scipy.stats.norm.pdf
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        mass = scipy.integrate.quad(pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        mean = scipy.integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(mean / mass - lv[k]) < 1e-10


def test_lloyd_max_one_bit_closed_form():
    """One bit: the optimal levels are +-E|X| = +-sqrt(2/pi)."""
    lv, th, _ = oracle.codebook(1)
    np.testing.assert_allclose(lv, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=1e-14)
    assert th[0] == 0.0


def test_lloyd_max_matches_published_gaussian_levels(golden_dir):
    """The solver reproduces the tabulated Gaussian Lloyd-Max levels to 1e-3."""
    for row in _golden(golden_dir, "gaussian_lloyd_max_levels.txt"):
        bits, pos = int(row[0]), np.array([float(v) for v in row[1:]])
        lv, _, _ = oracle.codebook(bits)
        np.testing.assert_allclose(lv[len(lv) // 2:], pos, atol=1e-3, rtol=0)


@pytest.mark.parametrize("bits", [2, 3])
def test_lloyd_max_is_a_local_minimum_of_distortion(bits):
    """Distortion D = E[(X - Q(X))^2] by quad; any small move of a level or a threshold
    raises it, and D equals 1 - sum_k P_k c_k^2 (orthogonality at the centroids)."""
    lv, th, _ = oracle.codebook(bits)
    pdf = scipy.stats.norm.pdf

    def distortion(levels, thr):
        edges = np.concatenate([[-np.inf], thr, [np.inf]])
        return sum(scipy.integrate.quad(lambda x, c=c: (x - c) ** 2 * pdf(x), a, b,
                                        epsabs=1e-14, epsrel=1e-13)[0]
                   for c, a, b in zip(levels, edges[:-1], edges[1:]))

    D = distortion(lv, th)
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    P = np.diff(scipy.stats.norm.cdf(edges))
    assert abs(D - (1 - np.sum(P * lv ** 2))) < 1e-10
    for k in range(len(lv)):
        for eps in (1e-3, -1e-3):
            l2 = lv.copy()
            l2[k] += eps
            assert distortion(l2, th) > D
    for k in range(len(th)):
        for eps in (1e-3, -1e-3):
            t2 = th.copy()
            t2[k] += eps
            assert distortion(lv, t2) > D


# ---------------------------------------------------------------- sizes

def test_block_sizes_match_article(golden_dir):
    """Section "どこまで小さくなるのか": 128 values + one FP16 norm per block;
    0.39 / 0.27 B per value, about 1/5 and 1/7 of FP16, smaller than q4_0."""
    rows = _golden(golden_dir, "block_sizes.txt")
    comp = {r[0]: float(r[1]) for r in rows if len(r) == 2}
    for r in rows:
        if len(r) != 5:
            continue
        name, bits, nval, printed, frac = r[0], int(r[1]), int(r[2]), float(r[3]), r[4]
        block_bytes = oracle.code_bytes(bits) + 2            # codes + one fp16 norm
        assert block_bytes == {3: 50, 2: 34}[bits]
        per_value = block_bytes / nval
        assert round(per_value, 2) == printed
        ratio = comp["fp16"] / per_value
        assert abs(ratio - int(frac.split("/")[1])) < 0.6      # "about 1/5", "about 1/7"
        assert per_value < comp["q4_0"]


def test_head_dim_blocks(golden_dir):
    """Section "実モデルでの数値": head_dim 256 is two stacked 128-blocks (each with its
    own norm): encoding a [.., 256] row equals encoding its two halves."""
    rows = _golden(golden_dir, "head_dim.txt")
    rng = np.random.default_rng(3)
    for hd, nblk in ((int(a), int(b)) for a, b in rows):
        assert hd // 128 == nblk and hd % 128 == 0
        x = rng.standard_normal((1, 2, 5, hd)).astype(np.float16)
        codes = np.zeros((1, 2, 5, nblk, 48), np.uint8)
        norms = np.zeros((1, 2, 5, nblk), np.float16)
        oracle.encode(3, x, codes, norms)
        c2, n2, _ = oracle.encode_blocks(3, x.reshape(-1, 128))
        assert np.array_equal(codes.reshape(-1, 48), c2)
        assert np.array_equal(norms.reshape(-1).view(np.uint16), n2.view(np.uint16))


# ---------------------------------------------------------------- encode / decode

@pytest.mark.parametrize("bits", [2, 3])
def test_encode_brute_force(bits):
    """Encode = norm, rotate, normalise, nearest Lloyd-Max level, pack.  Checked by
    brute force: dense H (scipy), nearest level by argmin distance, numpy bit packing,
    norm by numpy.linalg.norm rounded by numpy to fp16."""
    x = _rng_blocks(4, 3000)
    codes, norms, dist = oracle.encode_blocks(bits, x, want_dist=True)
    lv, th, _ = oracle.codebook(bits)
    x64 = x.astype(np.float64)
    n = np.linalg.norm(x64, axis=1)
    t = (x64 @ H128.T) / n[:, None]
    near = np.argmin(np.abs(t[:, :, None] - lv[None, None, :]), axis=2)
    got = _unpack(codes, bits)
    clear = dist > 1e-12
    assert clear.mean() > 0.999
    assert np.array_equal(got[clear], near[clear])
    assert np.array_equal(norms.view(np.uint16), n.astype(np.float16).view(np.uint16))
    # the reported distance is the distance to the nearest threshold
    np.testing.assert_allclose(dist, np.min(np.abs(t[:, :, None] - th[None, None, :]), axis=2),
                               rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3])
def test_decode_brute_force(bits):
    """Decode = unpack, look up, transform again, rescale by n16/128 (dense H here)."""
    rng = np.random.default_rng(5)
    code = rng.integers(0, 1 << bits, (500, 128))
    norms = (rng.uniform(0.1, 500, 500)).astype(np.float16)
    xhat, x16 = oracle.decode_blocks(bits, _pack(code, bits), norms)
    lv, _, _ = oracle.codebook(bits)
    ref = (lv[code] @ H128.T) * (norms.astype(np.float64)[:, None] / 128.0)
    np.testing.assert_allclose(xhat, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    assert np.array_equal(x16.view(np.uint16), xhat.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("bits", [2, 3])
def test_decode_closed_forms(bits):
    """All codes k decode to n16*c_k*e_0; codes tracing +-c_k along Hadamard row r
    (code k where the row is +1, code L-1-k where it is -1) decode to n16*c_k*e_r."""
    lv, _, _ = oracle.codebook(bits)
    L = 1 << bits
    n16 = np.float16(3.5)
    for k in range(L):
        xhat, _ = oracle.decode_blocks(bits, _pack(np.full(128, k), bits), np.array([n16]))
        ref = np.zeros(128)
        ref[0] = float(n16) * lv[k]
        np.testing.assert_allclose(xhat[0], ref, atol=1e-13)
        for r in (1, 37, 127):
            code = np.where(H128[r] > 0, k, L - 1 - k)
            xhat, _ = oracle.decode_blocks(bits, _pack(code, bits), np.array([n16]))
            ref = np.zeros(128)
            ref[r] = float(n16) * lv[k]
            np.testing.assert_allclose(xhat[0], ref, atol=1e-13)


def test_one_hot_round_trip_closed_form():
    """x = a e_j: t = sign(a) * column j of H (all +-1), so every code is the level
    just above / below 1 and the round trip is n16 * c e_j exactly:
    0.756005 e_j for turbo3, 1.510418 e_j for turbo2 (a = 1)."""
    for bits, gain, cpos, cneg in ((3, 0.75600528, 5, 2), (2, 1.51041761, 3, 0)):
        for j in (0, 5, 127):
            for a in (1.0, -2.0):
                x = np.zeros((1, 128), np.float16)
                x[0, j] = a
                codes, norms, _ = oracle.encode_blocks(bits, x)
                code = _unpack(codes, bits)[0]
                col = H128[:, j] * np.sign(a)
                assert np.array_equal(code, np.where(col > 0, cpos, cneg))
                assert float(norms[0]) == abs(a)
                xhat, _ = oracle.decode_blocks(bits, codes, norms)
                ref = np.zeros(128)
                ref[j] = a * gain
                np.testing.assert_allclose(xhat[0], ref, atol=1e-7)


def test_exact_zero_ties_go_to_upper_cell():
    """x = e_0 + e_1: t = sqrt(2) on even rows and exactly 0 on odd rows; a value on a
    threshold goes to the upper cell, so the zeros take code 2^bits / 2."""
    x = np.zeros((1, 128), np.float16)
    x[0, 0] = 1
    x[0, 1] = 1
    for bits, even_code in ((3, 6), (2, 3)):
        codes, norms, dist = oracle.encode_blocks(bits, x, want_dist=True)
        code = _unpack(codes, bits)[0]
        assert np.all(code[1::2] == (1 << bits) // 2)
        assert np.all(dist[0, 1::2] == 0.0)
        assert np.all(code[0::2] == even_code)


@pytest.mark.parametrize("bits", [2, 3])
def test_zero_block(bits):
    x = np.zeros((2, 128), np.float16)
    x[1] = -0.0
    codes, norms, _ = oracle.encode_blocks(bits, x)
    assert np.all(_unpack(codes, bits) == (1 << bits) // 2)
    assert np.all(norms.view(np.uint16) == 0)
    xhat, x16 = oracle.decode_blocks(bits, codes, norms)
    assert np.all(xhat == 0)


@pytest.mark.parametrize("bits", [2, 3])
def test_norm_saturates_at_fp16_max(bits):
    """Reading R7 (the page stores one FP16 norm per block and is silent on overflow):
    a norm beyond the largest fp16 value is stored as 65504 (0x7BFF), not +inf, and the
    codes are those of the unsaturated block (the normalisation uses the exact norm).
    A norm at or beyond the rounding midpoint to infinity (65520) is the case that
    separates saturation from plain rounding (nearest-even rounding alone would give
    +inf there); norms below the midpoint round to nearest even as usual, and the
    stored norm's decode scales the levels by 65504."""
    x = np.stack([np.full(128, v, np.float16) for v in (6188.0, 5792.0, 5788.0, 5745.0)])
    x[2, 0] = 6100.0                            # norm 65512.06: inside (65504, 65520)
    x[:, 1::2] *= -1                            # not a Hadamard row of H alone: mixed codes
    codes, norms, _ = oracle.encode_blocks(bits, x)
    exact = np.linalg.norm(x.astype(np.float64), axis=1)
    assert exact[0] > exact[1] > 65520 > exact[2] > 65504 > exact[3]
    expect = [0x7BFF, 0x7BFF, 0x7BFF, int(np.float16(exact[3]).view(np.uint16))]
    with np.errstate(over="ignore"):
        assert np.float16(exact[1]) == np.inf and np.float16(exact[2]) == 65504.0
    assert norms.view(np.uint16).tolist() == expect
    assert not np.isinf(norms.astype(np.float64)).any()
    # same direction, a norm far inside the range: identical codes
    small, _, _ = oracle.encode_blocks(bits, (x.astype(np.float64) / 64).astype(np.float16))
    assert np.array_equal(codes, small)
    # decode of the saturated block: (65504 / 128) * H * levels, dense H (scipy)
    lv, _, _ = oracle.codebook(bits)
    y = lv[_unpack(codes[:1], bits)[0]]
    xhat, _ = oracle.decode_blocks(bits, codes[:1], norms[:1])
    assert np.allclose(xhat[0], 65504.0 / 128.0 * (H128 @ y), rtol=1e-12, atol=0)


@pytest.mark.parametrize("bits", [2, 3])
def test_scale_and_sign_invariance(bits):
    """encode(2x): same codes, norm doubled exactly.  encode(-x): code -> L-1-code
    wherever t is not exactly on a threshold."""
    x = _rng_blocks(6, 400)
    c1, n1, d1 = oracle.encode_blocks(bits, x, want_dist=True)
    c2, n2, _ = oracle.encode_blocks(bits, (x.astype(np.float32) * 2).astype(np.float16))
    assert np.array_equal(c1, c2)
    assert np.array_equal(n2.astype(np.float64), 2 * n1.astype(np.float64))
    c3, n3, _ = oracle.encode_blocks(bits, -x)
    u1, u3 = _unpack(c1, bits), _unpack(c3, bits)
    off = d1 > 0
    assert np.array_equal(u3[off], (1 << bits) - 1 - u1[off])
    assert np.array_equal(n3, n1)


@pytest.mark.parametrize("bits", [2, 3])
def test_gaussian_distortion_statistics(bits):
    """On 20000 N(0,1) blocks the relative squared error of a round trip sits just under
    the Gaussian Lloyd-Max distortion D (computed here by quad): the rotated coordinates
    of a Gaussian vector are Gaussian, normalised by the block's own norm."""
    lv, th, _ = oracle.codebook(bits)
    edges = np.concatenate([[-np.inf], th, [np.inf]])
    pdf = scipy.stats.norm.pdf
    D = sum(scipy.integrate.quad(lambda x, c=c: (x - c) ** 2 * pdf(x), a, b)[0]
            for c, a, b in zip(lv, edges[:-1], edges[1:]))
    rng = np.random.default_rng(7)
    x = rng.standard_normal((20000, 128)).astype(np.float16)
    codes, norms, _ = oracle.encode_blocks(bits, x)
    xhat, _ = oracle.decode_blocks(bits, codes, norms)
    x64 = x.astype(np.float64)
    rel = np.sum((xhat - x64) ** 2, axis=1) / np.sum(x64 ** 2, axis=1)
    assert 0.95 * D <= rel.mean() <= 1.0 * D


# ---------------------------------------------------------------- tensor addressing

@pytest.mark.parametrize("bits", [2, 3])
def test_tensor_encode_decode_addressing(bits):
    """Cache rows [t0, t0+T) of [L,H,Tc,D/128] receive x's rows; other rows untouched;
    decode of the same rows returns the blockwise decode (numpy indexing as reference)."""
    rng = np.random.default_rng(8)
    L, H, T, D, Tc, t0 = 2, 3, 7, 256, 12, 4
    m = D // 128
    x = rng.standard_normal((L, H, T, D)).astype(np.float16)
    codes = np.full((L, H, Tc, m, 16 * bits), 0xAB, np.uint8)
    norms = np.full((L, H, Tc, m), 7.0, np.float16)
    oracle.encode(bits, x, codes, norms, t0=t0)
    cb, nb, _ = oracle.encode_blocks(bits, x.reshape(-1, 128))
    assert np.array_equal(codes[:, :, t0:t0 + T].reshape(-1, 16 * bits), cb)
    assert np.array_equal(norms[:, :, t0:t0 + T].reshape(-1), nb)
    assert np.all(codes[:, :, :t0] == 0xAB) and np.all(codes[:, :, t0 + T:] == 0xAB)
    assert np.all(norms[:, :, :t0] == 7.0) and np.all(norms[:, :, t0 + T:] == 7.0)
    xhat, x16 = oracle.decode(bits, codes, norms, t0, T)
    xb, _ = oracle.decode_blocks(bits, cb, nb)
    assert np.array_equal(xhat.reshape(-1, 128), xb)


@pytest.mark.parametrize("bits", [2, 3])
def test_qk_against_dense_dot(bits):
    """Scores = scale * q . k_hat with grouped heads (q head h reads kv head h // G);
    k_hat rebuilt here from the packed cache with numpy unpacking and dense H."""
    rng = np.random.default_rng(9)
    B, Hkv, G, Tc, T, D = 2, 2, 3, 9, 7, 256
    m = D // 128
    k = rng.standard_normal((B, Hkv, Tc, D)).astype(np.float16)
    codes = np.zeros((B, Hkv, Tc, m, 16 * bits), np.uint8)
    norms = np.zeros((B, Hkv, Tc, m), np.float16)
    oracle.encode(bits, k, codes, norms)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float16)
    scale = 1 / math.sqrt(D)
    s = oracle.qk_scores(bits, codes, norms, q, scale, T=T)
    lv, _, _ = oracle.codebook(bits)
    y = lv[_unpack(codes, bits)].reshape(B, Hkv, Tc, m, 128)
    khat = (y @ H128.T) * (norms.astype(np.float64)[..., None] / 128)
    khat = khat.reshape(B, Hkv, Tc, D)[:, :, :T]
    ref = np.einsum("bgrd,bgtd->bgrt", q.astype(np.float64).reshape(B, Hkv, G, D), khat)
    ref = scale * ref.reshape(B, Hkv * G, T)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- decode attention

def _attn_inputs(bits, seed, B, Hkv, Tc, D, G):
    rng = np.random.default_rng(seed)
    m = D // 128
    caches = []
    for _ in range(2):   # K, V
        x = (rng.standard_normal((B, Hkv, Tc, D)) * np.exp(rng.uniform(-1, 1, (B, Hkv, Tc, 1))))
        codes = np.zeros((B, Hkv, Tc, m, 16 * bits), np.uint8)
        norms = np.zeros((B, Hkv, Tc, m), np.float16)
        oracle.encode(bits, x.astype(np.float16), codes, norms)
        caches.append((codes, norms))
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float16)
    return caches, q


def _dense_hat(bits, codes, norms):
    """Decoded cache rebuilt here: numpy unpacking, codebook lookup, dense H."""
    B, Hkv, Tc, m, _ = codes.shape
    lv, _, _ = oracle.codebook(bits)
    y = lv[_unpack(codes, bits)].reshape(B, Hkv, Tc, m, 128)
    return ((y @ H128.T) * (norms.astype(np.float64)[..., None] / 128)).reshape(B, Hkv, Tc, m * 128)


@pytest.mark.parametrize("bits", [2, 3])
def test_attn_decode_against_dense_softmax(bits):
    """out = softmax(scale q . k_hat) v_hat with grouped heads, against scipy's softmax
    over keys and values rebuilt densely from the packed caches."""
    import scipy.special
    B, Hkv, G, Tc, T, D = 2, 2, 3, 11, 9, 256
    (kc, kn), (vc, vn) = _attn_inputs(bits, 21, B, Hkv, Tc, D, G)[0]
    q = _attn_inputs(bits, 21, B, Hkv, Tc, D, G)[1]
    scale = 1 / math.sqrt(D)
    out = oracle.attn_decode(bits, kc, kn, vc, vn, q, scale, T=T)
    kh = _dense_hat(bits, kc, kn)[:, :, :T]
    vh = _dense_hat(bits, vc, vn)[:, :, :T]
    qd = q.astype(np.float64).reshape(B, Hkv, G, D)
    s = scale * np.einsum("bgrd,bgtd->bgrt", qd, kh)
    p = scipy.special.softmax(s, axis=-1)
    ref = np.einsum("bgrt,bgtd->bgrd", p, vh).reshape(B, Hkv * G, D)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("bits", [2, 3])
def test_attn_decode_special_cases(bits):
    """T = 1: the weight is exactly 1, out = v_hat of row 0.  q = 0: equal weights,
    out = the mean of v_hat over the rows.  A huge scale: the weights become one-hot
    on the highest-scoring row (exp underflows to 0 for the others)."""
    B, Hkv, G, Tc, D = 1, 2, 2, 8, 128
    (kc, kn), (vc, vn) = _attn_inputs(bits, 22, B, Hkv, Tc, D, G)[0]
    q = _attn_inputs(bits, 22, B, Hkv, Tc, D, G)[1]
    vh = _dense_hat(bits, vc, vn)
    out1 = oracle.attn_decode(bits, kc, kn, vc, vn, q, 0.3, T=1)
    np.testing.assert_allclose(out1, np.repeat(vh[:, :, 0], G, axis=1), rtol=1e-13, atol=1e-14)
    out0 = oracle.attn_decode(bits, kc, kn, vc, vn, np.zeros_like(q), 0.3, T=Tc)
    np.testing.assert_allclose(out0, np.repeat(vh.mean(axis=2), G, axis=1), rtol=1e-12,
                               atol=1e-13 * np.abs(vh).max())
    big = 1e6
    outb = oracle.attn_decode(bits, kc, kn, vc, vn, q, big, T=Tc)
    s = oracle.qk_scores(bits, kc, kn, q, 1.0, T=Tc)          # [B, Hq, T]
    top = s.argmax(axis=-1)
    srt = np.sort(s, axis=-1)
    assert np.all((srt[..., -1] - srt[..., -2]) * big > 800)     # exp(-800) == 0 in binary64
    vdec, _ = oracle.decode(bits, vc, vn, 0, Tc)                 # the oracle's own decode
    for h in range(Hkv * G):
        np.testing.assert_array_equal(outb[0, h], vdec[0, h // G, top[0, h]])
        np.testing.assert_allclose(outb[0, h], vh[0, h // G, top[0, h]], rtol=1e-13, atol=1e-14)


def test_attn_decode_grouping_equals_repeated_heads():
    """Grouped-query attention equals ordinary multi-head attention over K and V caches
    repeated G times along the head axis (the GQA mapping kv head = h // G)."""
    bits, B, Hkv, G, Tc, D = 3, 2, 2, 4, 10, 128
    (kc, kn), (vc, vn) = _attn_inputs(bits, 23, B, Hkv, Tc, D, G)[0]
    q = _attn_inputs(bits, 23, B, Hkv, Tc, D, G)[1]
    a = oracle.attn_decode(bits, kc, kn, vc, vn, q, 0.2, T=Tc)
    rep = lambda z: np.repeat(z, G, axis=1)
    b = oracle.attn_decode(bits, rep(kc), rep(kn), rep(vc), rep(vn), q, 0.2, T=Tc)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- randomised rotation H D

def _signs(seed):
    return np.where(np.random.default_rng(seed).random(128) < 0.5, -1.0, 1.0)


def test_rotation_is_orthogonal_for_any_signs():
    """(H D)^T (H D) = 128 I for every diagonal of signs, so the norm, the unit mean
    square of t and the decode's 1/128 are unchanged ("何が違う": any orthogonal
    rotation spreads the energy; TurboQuant's is a random one)."""
    for seed in range(5):
        M = H128 @ np.diag(_signs(seed))
        np.testing.assert_array_equal(M.T @ M, 128.0 * np.eye(128))


@pytest.mark.parametrize("bits", [2, 3])
def test_rotation_all_plus_signs_is_the_plain_codec(bits):
    """D = I gives exactly the plain transform: codes, norms, decodes, scores, attention."""
    ones = np.ones(128)
    x = _rng_blocks(11, 400)
    c0, n0, _ = oracle.encode_blocks(bits, x)
    c1, n1, _ = oracle.encode_blocks(bits, x, signs=ones)
    assert np.array_equal(c0, c1) and np.array_equal(n0.view(np.uint16), n1.view(np.uint16))
    assert np.array_equal(oracle.decode_blocks(bits, c0, n0)[0], oracle.decode_blocks(bits, c0, n0, signs=ones)[0])
    (kc, kn), (vc, vn) = _attn_inputs(bits, 12, 1, 2, 6, 128, 2)[0]
    q = _attn_inputs(bits, 12, 1, 2, 6, 128, 2)[1]
    assert np.array_equal(oracle.qk_scores(bits, kc, kn, q, 0.1), oracle.qk_scores(bits, kc, kn, q, 0.1, signs=ones))
    assert np.array_equal(oracle.attn_decode(bits, kc, kn, vc, vn, q, 0.1),
                          oracle.attn_decode(bits, kc, kn, vc, vn, q, 0.1, signs=ones))


@pytest.mark.parametrize("bits", [2, 3])
def test_rotation_encode_decode_brute_force(bits):
    """Encode with signs d: t = H D x / ||x||, nearest level; decode: D H C[code] n16/128.
    Both checked with the dense matrix H diag(d) (scipy), argmin and numpy packing."""
    d = _signs(13)
    M = H128 @ np.diag(d)
    x = _rng_blocks(14, 2000)
    codes, norms, dist = oracle.encode_blocks(bits, x, want_dist=True, signs=d)
    lv, _, _ = oracle.codebook(bits)
    x64 = x.astype(np.float64)
    n = np.linalg.norm(x64, axis=1)
    t = (x64 @ M.T) / n[:, None]
    near = np.argmin(np.abs(t[:, :, None] - lv[None, None, :]), axis=2)
    clear = dist > 1e-12
    assert clear.mean() > 0.999
    assert np.array_equal(_unpack(codes, bits)[clear], near[clear])
    assert np.array_equal(norms.view(np.uint16), n.astype(np.float16).view(np.uint16))
    rng = np.random.default_rng(15)
    code = rng.integers(0, 1 << bits, (300, 128))
    nn = rng.uniform(0.1, 500, 300).astype(np.float16)
    xhat, x16 = oracle.decode_blocks(bits, _pack(code, bits), nn, signs=d)
    ref = (lv[code] @ M) * (nn.astype(np.float64)[:, None] / 128.0)     # (H D)^-1 = D H / 128
    np.testing.assert_allclose(xhat, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    assert np.array_equal(x16.view(np.uint16), xhat.astype(np.float16).view(np.uint16))


def test_rotation_spreads_hadamard_rows_but_not_one_hots():
    """What a seeded sign diagonal changes.  An input along a Hadamard row is the plain
    transform's worst case: H maps it onto one coordinate (t = sqrt(128) e_k), which
    clamps to the outermost level, and the round trip loses most of the block.  With
    random signs the same input is spread over all coordinates and reconstructs like
    a Gaussian block.  A one-hot input stays flat under any H D (t = +-1 everywhere),
    so its round trip is the plain one: gain 0.756005 for turbo3."""
    bits = 3
    d = _signs(16)
    rel = {}
    for name, signs in (("plain", None), ("rot", d)):
        x = H128[[3, 40, 77]].astype(np.float16)
        c, n, _ = oracle.encode_blocks(bits, x, signs=signs)
        xh, _ = oracle.decode_blocks(bits, c, n, signs=signs)
        rel[name] = np.sum((xh - x.astype(np.float64)) ** 2, axis=1) / np.sum(x.astype(np.float64) ** 2, axis=1)
    assert np.all(rel["plain"] > 0.5)
    assert np.all(rel["rot"] < 0.1)
    x = np.zeros((1, 128), np.float16)
    x[0, 9] = 1.0
    c, n, _ = oracle.encode_blocks(bits, x, signs=d)
    xh, _ = oracle.decode_blocks(bits, c, n, signs=d)
    ref = np.zeros(128)
    ref[9] = 0.75600528
    np.testing.assert_allclose(xh[0], ref, atol=1e-7)


@pytest.mark.parametrize("bits", [2, 3])
def test_rotation_qk_and_attention_against_dense(bits):
    """Scores and attention over caches encoded with signs d, against keys and values
    rebuilt densely as D H C[code] n16/128 and scipy's softmax."""
    import scipy.special
    d = _signs(17)
    M = H128 @ np.diag(d)
    rng = np.random.default_rng(18)
    B, Hkv, G, Tc, T, D = 1, 2, 3, 10, 8, 256
    m = D // 128
    caches = []
    for _ in range(2):
        x = rng.standard_normal((B, Hkv, Tc, D)).astype(np.float16)
        codes = np.zeros((B, Hkv, Tc, m, 16 * bits), np.uint8)
        norms = np.zeros((B, Hkv, Tc, m), np.float16)
        oracle.encode(bits, x, codes, norms, signs=d)
        caches.append((codes, norms))
    (kc, kn), (vc, vn) = caches
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float16)
    scale = 0.2
    lv, _, _ = oracle.codebook(bits)

    def dense(codes, norms):
        y = lv[_unpack(codes, bits)].reshape(B, Hkv, Tc, m, 128)
        return ((y @ M) * (norms.astype(np.float64)[..., None] / 128)).reshape(B, Hkv, Tc, D)[:, :, :T]

    kh, vh = dense(kc, kn), dense(vc, vn)
    qd = q.astype(np.float64).reshape(B, Hkv, G, D)
    s = scale * np.einsum("bgrd,bgtd->bgrt", qd, kh)
    got = oracle.qk_scores(bits, kc, kn, q, scale, T=T, signs=d)
    np.testing.assert_allclose(got, s.reshape(B, Hkv * G, T), rtol=1e-12, atol=1e-12 * np.abs(s).max())
    ref = np.einsum("bgrt,bgtd->bgrd", scipy.special.softmax(s, axis=-1), vh).reshape(B, Hkv * G, D)
    out = oracle.attn_decode(bits, kc, kn, vc, vn, q, scale, T=T, signs=d)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- interleaved records

@pytest.mark.parametrize("bits", [2, 3])
def test_records_match_a_block_struct(bits, golden_dir):
    """Records are the block struct {fp16 d; uint8 qs[16*bits]} in block order: checked
    against numpy's packed structured dtype of that struct, whose item size is the
    article's bytes per block (50 / 34, "どこまで小さくなるのか")."""
    cb = 16 * bits
    rec_t = np.dtype([("d", "<f2"), ("qs", "u1", (cb,))])
    printed = {r[0]: float(r[3]) for r in _golden(golden_dir, "block_sizes.txt") if r[0].startswith("turbo")}
    assert rec_t.itemsize == 2 + cb
    assert round(rec_t.itemsize / 128, 2) == printed[f"turbo{bits}"]   # 0.39 / 0.27 B per value
    rng = np.random.default_rng(30 + bits)
    nb = 777
    codes = rng.integers(0, 256, (nb, cb), dtype=np.uint8)
    norms = rng.uniform(0, 300, nb).astype(np.float16)
    rec = oracle.pack_records(bits, codes, norms)
    view = rec.reshape(-1).view(rec_t)
    assert np.array_equal(view["d"].view(np.uint16), norms.view(np.uint16))
    assert np.array_equal(view["qs"], codes)
    c2, n2 = oracle.unpack_records(bits, rec)
    assert np.array_equal(c2, codes) and np.array_equal(n2.view(np.uint16), norms.view(np.uint16))
    # built independently: records from the struct, unpacked by the oracle
    s = np.zeros(nb, rec_t)
    s["d"], s["qs"] = norms, codes
    c3, n3 = oracle.unpack_records(bits, s.view(np.uint8))
    assert np.array_equal(c3, codes) and np.array_equal(n3.view(np.uint16), norms.view(np.uint16))
