"""Randomised rotation H D (the _rot entry points) vs the CPU oracle with the same
signs (GPU).

The signs are an input drawn here with numpy; both sides receive the same 128
values.  Every check mirrors the plain path's: codes bit-exact up to threshold
ties, norms exact, decode / scores / attention within their tolerances, rows
outside the written range untouched.
"""
import math

import numpy as np
import pytest
import torch

import gen
import kv_cache_quantization_block_amd as tq
import oracle
from _parity import check_attn, check_codes, check_decode, check_norms, check_scores

pytestmark = pytest.mark.gpu

SENT_CODE = 0xA5
SENT_NORM = 7.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    tq.lib()


def _signs(seed):
    return np.where(np.random.default_rng(seed).random(128) < 0.5, -1.0, 1.0)


def _rand_kv(seed, L, H, T, D):
    return gen.kv_tensor(seed, "K", gen.KVSpec(n_outliers=3, row_scale=True), L, H, T, D)


def _encode(bits, x, Tc, t0, d):
    L, H, T, D = x.shape
    codes, norms = tq.empty_cache(bits, L, H, Tc, D)
    codes.fill_(SENT_CODE)
    norms.fill_(SENT_NORM)
    tq.tq_encode(bits, x.cuda(), codes, norms, t0, signs=d)
    return codes, norms


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("shape", [
    (2, 3, 37, 128, 50, 5),     # 222 blocks: ragged last tile, t0 > 0
    (1, 2, 65, 256, 65, 0),     # head_dim 256, odd T
    (3, 1, 1, 128, 9, 8),       # single-token append at the last row
    (2, 2, 300, 128, 300, 0),   # several tiles per (l, h)
])
def test_rot_encode_decode(bits, shape):
    L, H, T, D, Tc, t0 = shape
    d = _signs(100 + T)
    x = _rand_kv(31 + T + D, L, H, T, D)
    codes, norms = _encode(bits, x, Tc, t0, d)
    out = torch.empty((L, H, T, D), dtype=torch.float16, device="cuda")
    tq.tq_decode(bits, codes, norms, t0, out, signs=d)
    torch.cuda.synchronize()
    gc, gn, gx = codes.cpu().numpy(), norms.cpu().numpy(), out.cpu().numpy()
    xn = x.numpy()
    oc = np.full(gc.shape, SENT_CODE, np.uint8)
    on = np.full(gn.shape, SENT_NORM, np.float16)
    dist = oracle.encode(bits, xn, oc, on, t0=t0, want_dist=True, signs=d)
    rows = slice(t0, t0 + T)
    what = f"rot shape {shape}"
    st = check_codes(bits, gc[:, :, rows], oc[:, :, rows], dist.reshape(L, H, T, D // 128, 128), what)
    st.update(check_norms(gn[:, :, rows], on[:, :, rows], xn, what))
    assert np.all(gc[:, :, :t0] == SENT_CODE) and np.all(gc[:, :, t0 + T:] == SENT_CODE)
    assert np.all(gn[:, :, :t0] == SENT_NORM) and np.all(gn[:, :, t0 + T:] == SENT_NORM)
    ref, _ = oracle.decode(bits, gc, gn, t0, T, signs=d)
    st.update(check_decode(gx, ref, what))
    print(st)


@pytest.mark.parametrize("bits", [3, 2])
def test_rot_signs_change_the_cache(bits):
    """The same input under two sign vectors: different codes, and each cache decodes
    back (within the decode tolerance) only with its own signs."""
    x = _rand_kv(7, 1, 2, 64, 128)
    d1, d2 = _signs(1), _signs(2)
    c1, n1 = _encode(bits, x, 64, 0, d1)
    c2, n2 = _encode(bits, x, 64, 0, d2)
    assert not torch.equal(c1, c2)
    assert torch.equal(n1, n2)          # the norm does not depend on the rotation
    out = torch.empty((1, 2, 64, 128), dtype=torch.float16, device="cuda")
    tq.tq_decode(bits, c1, n1, 0, out, signs=d1)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(bits, c1.cpu().numpy(), n1.cpu().numpy(), 0, 64, signs=d1)
    check_decode(out.cpu().numpy(), ref, "own signs")


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("case", [
    (2, 2, 4, 100, 97, 128),     # GQA group 4, ragged T < Tc
    (1, 1, 12, 40, 40, 128),     # group 12: passes of eight and four heads
    (1, 2, 3, 50, 50, 256),      # odd group, head_dim 256
])
def test_rot_qk(bits, case):
    B, Hkv, G, Tc, T, D = case
    d = _signs(200 + G)
    k = _rand_kv(41 + G, B, Hkv, Tc, D)
    codes, norms = _encode(bits, k, Tc, 0, d)
    q = gen.queries(42 + G, B, Hkv * G, D)
    scale = 1.0 / math.sqrt(D)
    scores = torch.empty((B, Hkv * G, T), dtype=torch.float32, device="cuda")
    tq.tq_qk_scores(bits, codes, norms, q.cuda(), scale, scores, signs=d)
    torch.cuda.synchronize()
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    ref = oracle.qk_scores(bits, gc, gn, q.numpy(), scale, T=T, signs=d)
    khat, _ = oracle.decode(bits, gc, gn, 0, T, signs=d)
    kn = np.repeat(np.linalg.norm(khat, axis=-1), G, axis=1)
    qn = np.linalg.norm(q.numpy().astype(np.float64), axis=-1)
    print(check_scores(scores.cpu().numpy(), ref, qn[:, :, None] * scale, kn, f"rot qk {case}"))


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("case", [
    (1, 2, 4, 100, 97, 128),      # GQA group 4, ragged T < Tc
    (2, 1, 8, 40, 33, 128),       # group 8: two head sets
    (1, 2, 4, 5000, 4999, 128),   # many row chunks and waves
    (1, 2, 4, 3000, 2999, 256),   # head_dim 256: the signs apply to each block
    (2, 1, 8, 40, 33, 256),
])
def test_rot_attention(bits, case):
    B, Hkv, G, Tc, T, D = case
    d = _signs(300 + T % 97)
    k = _rand_kv(51 + G, B, Hkv, Tc, D)
    v = gen.kv_tensor(52 + G, "V", gen.KVSpec(n_outliers=3, row_scale=True), B, Hkv, Tc, D)
    kc, kn = _encode(bits, k, Tc, 0, d)
    vc, vn = _encode(bits, v, Tc, 0, d)
    q = gen.queries(53 + G, B, Hkv * G, D)
    scale = 1.0 / math.sqrt(D)
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device="cuda")
    tq.tq_attn_decode(bits, kc, kn, vc, vn, q.cuda(), scale, out, T=T, signs=d)
    torch.cuda.synchronize()
    vcn, vnn = vc.cpu().numpy(), vn.cpu().numpy()
    ref = oracle.attn_decode(bits, kc.cpu().numpy(), kn.cpu().numpy(), vcn, vnn, q.numpy(), scale,
                             T=T, signs=d)
    vhat = oracle.decode_blocks(bits, vcn[:, :, :T].reshape(-1, 16 * bits), vnn[:, :, :T].reshape(-1),
                                signs=d)[0]
    vmax = np.repeat(np.abs(vhat).reshape(B, Hkv, -1).max(axis=-1), G, axis=1)
    print(check_attn(out.cpu().numpy(), ref, vmax, T, f"rot attn {case}"))
