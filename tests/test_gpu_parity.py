"""HIP path vs the CPU oracle on small inputs (GPU).

Every case feeds the same fp16 bytes to the library (through the C ABI via the
Python binding) and to the oracle, then compares element by element under the
rules in _parity.py.  Sizes span several 32-block wave tiles with ragged tails.
"""
import math

import numpy as np
import pytest
import torch

import gen
import kv_cache_quantization_block_amd as tq
import oracle
from _parity import check_attn, check_codes, check_decode, check_norms, check_scores, unpack_codes

pytestmark = pytest.mark.gpu

SENT_CODE = 0xA5
SENT_NORM = 7.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    tq.lib()


def _rand_kv(seed, L, H, T, D, n_out=3, row_scale=True, t3=False):
    spec = gen.KVSpec(n_outliers=n_out, row_scale=row_scale, student_t3=t3)
    return gen.kv_tensor(seed, "K", spec, L, H, T, D)


def _gpu_encode(bits, x, Tc, t0):
    L, H, T, D = x.shape
    codes, norms = tq.empty_cache(bits, L, H, Tc, D)
    codes.fill_(SENT_CODE)
    norms.fill_(SENT_NORM)
    tq.tq_encode(bits, x.cuda(), codes, norms, t0)
    return codes, norms


def _check_roundtrip(bits, x, Tc, t0, what):
    """Encode on both sides, compare the written rows, untouched rows, then decode."""
    L, H, T, D = x.shape
    m = D // 128
    codes, norms = _gpu_encode(bits, x, Tc, t0)
    out = torch.empty((L, H, T, D), dtype=torch.float16, device="cuda")
    tq.tq_decode(bits, codes, norms, t0, out)
    torch.cuda.synchronize()
    gc, gn, gx = codes.cpu().numpy(), norms.cpu().numpy(), out.cpu().numpy()

    xn = x.numpy()
    oc = np.full(gc.shape, SENT_CODE, np.uint8)
    on = np.full(gn.shape, SENT_NORM, np.float16)
    dist = oracle.encode(bits, xn, oc, on, t0=t0, want_dist=True)
    rows = slice(t0, t0 + T)
    st = check_codes(bits, gc[:, :, rows], oc[:, :, rows], dist.reshape(L, H, T, m, 128), what)
    st.update(check_norms(gn[:, :, rows], on[:, :, rows], xn, what))
    # rows outside [t0, t0+T) untouched
    assert np.all(gc[:, :, :t0] == SENT_CODE) and np.all(gc[:, :, t0 + T:] == SENT_CODE)
    assert np.all(gn[:, :, :t0] == SENT_NORM) and np.all(gn[:, :, t0 + T:] == SENT_NORM)
    # decode of the GPU's own cache vs the oracle's binary64 decode of it
    ref, _ = oracle.decode(bits, gc, gn, t0, T)
    st.update(check_decode(gx, ref, what))
    return st


@pytest.mark.parametrize("bits", [3, 2])
def test_single_head_workload(bits):
    """1 x 1 x 1024 x 128, N(0,1) with 4 fixed x20 outlier channels (1024 blocks)."""
    w = gen.WORKLOADS["single_head"]
    x = gen.kv_tensor(w.seed, "K", w.spec, w.L, w.H, w.T, w.D)
    st = _check_roundtrip(bits, x, w.T, 0, "single_head")
    print(st)


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("shape", [
    (2, 3, 37, 128, 50, 5),     # 222 blocks: ragged last tile, t0 > 0
    (1, 2, 65, 256, 65, 0),     # head_dim 256, odd T
    (3, 1, 1, 128, 9, 8),       # single-token append at the last row
    (1, 1, 64, 384, 70, 6),     # three blocks per row
    (2, 2, 300, 128, 300, 0),   # several tiles per (l, h)
])
def test_ragged_shapes(bits, shape):
    L, H, T, D, Tc, t0 = shape
    x = _rand_kv(11 + T + D, L, H, T, D)
    _check_roundtrip(bits, x, Tc, t0, f"shape {shape}")


def _special_blocks():
    rows = []
    z = np.zeros(128, np.float32)
    rows.append(z.copy())                               # zero block
    rows.append(-z)                                     # -0.0 block
    for j, a in ((0, 1.0), (5, -2.0), (127, 0.5), (64, 300.0)):
        r = z.copy(); r[j] = a; rows.append(r)         # one-hots
    r = z.copy(); r[0] = r[1] = 1.0; rows.append(r)    # exact zero ties
    rows.append(np.ones(128, np.float32))               # constant
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(128)] for i in range(128)], np.float32)
    rows.append(H[37] * 3.0)                             # a Hadamard row
    rows.append(np.full(128, 65504.0, np.float32))      # saturating norm
    rows.append(np.full(128, 2.0 ** -24, np.float32))   # subnormal values
    r = np.random.default_rng(0).standard_normal(128).astype(np.float32) * 1e-3
    r[3] = 60000.0; rows.append(r)                      # one huge outlier
    return np.stack(rows).astype(np.float16)


@pytest.mark.parametrize("bits", [3, 2])
def test_special_blocks_bit_exact(bits):
    """Zero / -0 blocks, one-hots, exact-zero ties, saturating and subnormal norms:
    every code and norm must equal the oracle's exactly (these t are exact in float)."""
    xb = _special_blocks()
    nb = xb.shape[0]
    x = torch.from_numpy(xb).reshape(1, 1, nb, 128)
    codes, norms = _gpu_encode(bits, x, nb, 0)
    out = torch.empty((1, 1, nb, 128), dtype=torch.float16, device="cuda")
    tq.tq_decode(bits, codes, norms, 0, out)
    torch.cuda.synchronize()
    oc, on, _ = oracle.encode_blocks(bits, xb)
    gc = codes.cpu().numpy().reshape(nb, -1)
    gn = norms.cpu().numpy().reshape(nb)
    assert np.array_equal(unpack_codes(gc, bits), unpack_codes(oc, bits))
    assert np.array_equal(gn.view(np.uint16), on.view(np.uint16))
    assert float(gn[-3]) == 65504.0
    ref, _ = oracle.decode_blocks(bits, gc, gn)
    check_decode(out.cpu().numpy(), ref, "special")
    assert np.all(out.cpu().numpy().reshape(nb, 128)[:2] == 0)   # zero blocks decode to 0


@pytest.mark.parametrize("bits", [3, 2])
def test_append_leaves_other_rows(bits):
    """Decode-step append: one token per (layer, head) written at row t0; every other
    byte of the cache is unchanged."""
    L, H, Tc, D = 2, 4, 33, 128
    prefill = _rand_kv(21, L, H, Tc - 1, D)
    codes, norms = tq.empty_cache(bits, L, H, Tc, D)
    codes.zero_()
    norms.zero_()
    tq.tq_encode(bits, prefill.cuda(), codes, norms, 0)
    before_c, before_n = codes.clone(), norms.clone()
    tok = _rand_kv(22, L, H, 1, D)
    tq.tq_encode(bits, tok.cuda(), codes, norms, Tc - 1)
    torch.cuda.synchronize()
    assert torch.equal(codes[:, :, :Tc - 1], before_c[:, :, :Tc - 1])
    assert torch.equal(norms[:, :, :Tc - 1], before_n[:, :, :Tc - 1])
    oc, on, dist = oracle.encode_blocks(bits, tok.numpy(), want_dist=True)
    check_codes(bits, codes[:, :, Tc - 1].cpu().numpy().reshape(-1, 16 * bits), oc, dist, "append")
    check_norms(norms[:, :, Tc - 1].cpu().numpy(), on, tok.numpy(), "append")


def _qk_case(bits, B, Hkv, G, Tc, T, D, seed, q_mul=None, scale=None):
    k = _rand_kv(seed, B, Hkv, Tc, D)
    codes, norms = _gpu_encode(bits, k, Tc, 0)
    q = gen.queries(seed + 1, B, Hkv * G, D)
    if q_mul is not None:   # per-head magnitudes, [Hq] factors
        q = (q.double() * torch.as_tensor(q_mul, dtype=torch.float64)[None, :, None]).half()
        assert bool(torch.isfinite(q).all())
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    scores = torch.empty((B, Hkv * G, T), dtype=torch.float32, device="cuda")
    tq.tq_qk_scores(bits, codes, norms, q.cuda(), scale, scores)
    torch.cuda.synchronize()
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    ref = oracle.qk_scores(bits, gc, gn, q.numpy(), scale, T=T)
    khat, _ = oracle.decode(bits, gc, gn, 0, T)                       # [B, Hkv, T, D]
    kn = np.linalg.norm(khat, axis=-1)                                  # [B, Hkv, T]
    qn = np.linalg.norm(q.numpy().astype(np.float64), axis=-1)         # [B, Hq]
    knh = np.repeat(kn, G, axis=1)                                      # head h reads kv h // G
    return check_scores(scores.cpu().numpy(), ref, qn[:, :, None] * abs(scale), knh,
                        f"qk bits={bits} B={B} Hkv={Hkv} G={G} T={T} D={D}")


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("case", [
    (2, 2, 4, 100, 97, 128),     # GQA group 4, ragged T < Tc
    (1, 3, 1, 70, 70, 128),      # no grouping
    (2, 1, 8, 40, 33, 128),      # group 8: one full pass of eight heads
    (1, 1, 12, 40, 40, 128),     # group 12: passes of eight and four heads
    (1, 1, 16, 64, 61, 128),     # group 16: two full passes
    (1, 2, 3, 50, 50, 256),      # odd group, head_dim 256
    (1, 1, 2, 1100, 1100, 384),  # three blocks per row, several token chunks
    (1, 2, 5, 20, 17, 1024),     # eight blocks per row
    (1, 1, 2, 24, 21, 2048),     # sixteen blocks per row (largest head_dim, 96 KB of LDS for turbo2)
    (1, 2, 4, 5000, 4999, 128),  # many token chunks and waves, ragged last group
    (1, 2, 4, 5000, 5000, 128),  # score rows 16-byte aligned: whole 128-row batches, then a ragged one
    (1, 1, 12, 1000, 1000, 128), # whole batches in passes of eight and four heads
    (2, 2, 4, 700, 644, 128),    # whole batches with Tc > T, waves past the last row
    (1, 2, 4, 5000, 5000, 256),  # head_dim 256: whole 64-row batches, then a ragged one
    (1, 2, 4, 5000, 4999, 256),  # head_dim 256, ragged last group
    (1, 1, 12, 1000, 1000, 256), # head_dim 256, passes of eight and four heads
    (2, 2, 4, 700, 644, 256),    # head_dim 256, Tc > T, waves past the last row
])
def test_qk_scores(bits, case):
    B, Hkv, G, Tc, T, D = case
    print(_qk_case(bits, B, Hkv, G, Tc, T, D, seed=31 + D + G))


@pytest.mark.parametrize("bits", [3, 2])
def test_qk_query_magnitudes(bits):
    """Query heads from 1e-4 to 3e3 times N(0, 1) in one call (fp16 subnormals at the
    small end), and a negative scale: every head keeps the 2e-3 relative bound, so the
    per-head fp16 operand scaling holds whatever the query's magnitude."""
    mul = [1e-4, 3e-3, 1.0, 40.0, 3e3, 0.5, 1e-2, 7.0]
    print(_qk_case(bits, 1, 2, 4, 300, 300, 128, seed=77, q_mul=mul))
    print(_qk_case(bits, 1, 1, 3, 64, 64, 256, seed=78, scale=-0.37))


# ---------------------------------------------------------------- decode attention

def _attn_case(bits, B, Hkv, G, Tc, T, seed, q_mul=1.0, scale=None, v_mul=1.0, zero_rows=(), D=128):
    k = _rand_kv(seed, B, Hkv, Tc, D)
    v = _rand_kv(seed + 7, B, Hkv, Tc, D)
    v = (v.double() * v_mul).half()
    for t in zero_rows:
        v[:, :, t] = 0
    kc, kn = _gpu_encode(bits, k, Tc, 0)
    vc, vn = _gpu_encode(bits, v, Tc, 0)
    q = (gen.queries(seed + 1, B, Hkv * G, D).double() * q_mul).half()
    assert bool(torch.isfinite(q).all()) and bool(torch.isfinite(v).all())
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device="cuda")
    tq.tq_attn_decode(bits, kc, kn, vc, vn, q.cuda(), scale, out, T=T)
    torch.cuda.synchronize()
    vcn, vnn = vc.cpu().numpy(), vn.cpu().numpy()
    ref = oracle.attn_decode(bits, kc.cpu().numpy(), kn.cpu().numpy(), vcn, vnn, q.numpy(), scale, T=T)
    vhat = oracle.decode_blocks(bits, vcn[:, :, :T].reshape(-1, 16 * bits), vnn[:, :, :T].reshape(-1))[0]
    vmax = np.repeat(np.abs(vhat).reshape(B, Hkv, -1).max(axis=-1), G, axis=1)
    return check_attn(out.cpu().numpy(), ref, vmax, T, f"attn bits={bits} B={B} Hkv={Hkv} G={G} T={T} D={D}")


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("case", [
    (1, 2, 4, 100, 97),      # GQA group 4, ragged T < Tc
    (2, 1, 8, 40, 33),       # group 8: one full pass
    (1, 1, 12, 300, 300),    # group 12: passes of eight and four heads
    (1, 3, 1, 70, 70),       # no grouping
    (1, 2, 2, 1, 1),         # one row: the output is that row's value
    (1, 2, 4, 5000, 4999),   # many row chunks and waves, ragged last unit
    (3, 2, 4, 2000, 1500),   # several sequences, T well below Tc
    (1, 1, 16, 64, 61),      # group 16: two full passes of eight heads
    (1, 2, 3, 50, 50),       # odd group: one set of four heads, three used
    (2, 2, 5, 300, 257),     # group 5: two sets in one pass, the second with one head
])
def test_attn_decode(bits, case):
    B, Hkv, G, Tc, T = case
    print(_attn_case(bits, B, Hkv, G, Tc, T, seed=41 + G + T % 97))


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("case", [
    (1, 2, 4, 100, 97),      # GQA group 4, ragged T < Tc
    (2, 1, 8, 40, 33),       # group 8: one full pass
    (1, 1, 12, 300, 300),    # group 12: passes of eight and four heads
    (1, 3, 1, 70, 70),       # no grouping
    (1, 2, 2, 1, 1),         # one row: the output is that row's value
    (1, 2, 4, 5000, 4999),   # many row chunks and waves, ragged last unit
    (3, 2, 4, 2000, 1500),   # several sequences, T well below Tc
    (1, 1, 16, 64, 61),      # group 16: two full passes of eight heads
    (1, 2, 3, 50, 50),       # odd group
    (2, 2, 5, 300, 257),     # group 5: two sets in one pass, the second with one head
])
def test_attn_decode_head_dim_256(bits, case):
    """head_dim 256 (two 128-blocks per row, each with its own norm; section
    "実モデルでの数値"): the fused attention against the oracle."""
    B, Hkv, G, Tc, T = case
    print(_attn_case(bits, B, Hkv, G, Tc, T, seed=61 + G + T % 89, D=256))


@pytest.mark.parametrize("bits", [3, 2])
def test_attn_decode_head_dim_256_extremes(bits):
    """head_dim 256 under a peaked softmax, value norms far from the usual and rows of
    zeros in the values that carry the largest weights."""
    print(_attn_case(bits, 1, 2, 4, 600, 600, seed=71, scale=2.0, D=256))
    print(_attn_case(bits, 1, 2, 4, 600, 590, seed=72, v_mul=1e-4, D=256))
    print(_attn_case(bits, 1, 2, 4, 300, 300, seed=73, scale=2.0, zero_rows=range(1, 300, 2), D=256))


@pytest.mark.parametrize("bits", [3, 2])
def test_attn_decode_extremes(bits):
    """A peaked softmax (large scale), a nearly flat one (tiny scale), value norms from
    1e-4 to 30 times the usual and all-zero value rows, also under a softmax whose
    largest weights sit on zero rows (outputs many orders below the values, down to
    about 1e-155 of them): the running maximum and the power-of-two weight scaling
    keep every head within the bound."""
    print(_attn_case(bits, 1, 2, 4, 600, 600, seed=51, scale=2.0))
    print(_attn_case(bits, 1, 2, 4, 600, 600, seed=52, scale=1e-4))
    print(_attn_case(bits, 1, 2, 4, 600, 590, seed=53, v_mul=1e-4))
    print(_attn_case(bits, 1, 2, 4, 600, 600, seed=54, v_mul=30.0, q_mul=3.0))
    print(_attn_case(bits, 1, 2, 4, 300, 300, seed=55, zero_rows=range(0, 300, 3)))
    print(_attn_case(bits, 1, 2, 4, 300, 300, seed=60, scale=0.3, zero_rows=range(1, 300, 2)))
    print(_attn_case(bits, 1, 2, 4, 300, 300, seed=57, scale=2.0, zero_rows=range(1, 300, 2)))


def test_attn_decode_side_stream_without_workspace():
    """tq_attn_decode on a side stream with no workspace given: the binding allocates the
    workspace on that stream, so memory work queued on the default stream right after the
    call (allocations that may reuse freed blocks, and writes into them) cannot overlap
    the kernels' use of it; the result equals the call with a workspace of its own."""
    bits, B, Hkv, G, Tc, T = 3, 2, 2, 4, 3000, 3000
    k = _rand_kv(71, B, Hkv, Tc, 128)
    v = _rand_kv(72, B, Hkv, Tc, 128)
    kc, kn = _gpu_encode(bits, k, Tc, 0)
    vc, vn = _gpu_encode(bits, v, Tc, 0)
    q = gen.queries(73, B, Hkv * G, 128).cuda()
    scale = 1.0 / math.sqrt(128)
    ref = torch.empty((B, Hkv * G, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_attn_workspace_bytes(bits, B, Hkv, Tc, 128, T, Hkv * G),
                     dtype=torch.uint8, device="cuda")
    tq.tq_attn_decode(bits, kc, kn, vc, vn, q, scale, ref, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        out = torch.empty_like(ref)
        side.wait_stream(torch.cuda.current_stream())
        tq.tq_attn_decode(bits, kc, kn, vc, vn, q, scale, out, stream=side)
        for i in range(8):   # default-stream allocations and writes right behind the call
            junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
            junk.fill_(float(rep * 8 + i))
            del junk
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"repetition {rep}"
