"""HIP path vs the CPU oracle at the evaluation workloads' full sizes (GPU).

Every workload runs in the same launch configuration as bench.py (whole
tensors, one call per op), and every element is compared with the oracle: the
whole-cache workloads one K or V layer at a time, the decode step's 16.8M
scores and all its attention outputs at once.  Properties that hold at any size
(finite outputs, untouched rows, round-trip error statistics) are checked too.
"""
import math

import numpy as np
import pytest
import torch

import gen
import kv_cache_quantization_block_amd as tq
import oracle
from _parity import (check_attn, check_codes, check_codes_full, check_decode, check_decode_torch,
                     check_norms, check_scores_torch)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    tq.lib()
    yield
    torch.cuda.empty_cache()


def _tensor(w, name, device=DEV):
    x = torch.empty((w.L, w.H, w.T, w.D), dtype=torch.float16, device=device)
    for l in range(w.L):
        x[l] = gen.kv_layer(w.seed, name, w.spec, l, w.H, w.T, w.D, device=device)
    return x


def _rel_mse_per_block(x, xh):
    """Mean over blocks of ||x_hat - x||^2 / ||x||^2, computed on the GPU in float."""
    a = x.reshape(-1, 128).float()
    b = xh.reshape(-1, 128).float()
    num = ((b - a) ** 2).sum(1)
    den = (a * a).sum(1).clamp_min(1e-30)
    return float((num / den).mean())


def _check_blocks(bits, xb, gc, gn, gx, what):
    """Oracle on a set of whole blocks: codes + norms from x, decode from the GPU's cache."""
    oc, on, dist = oracle.encode_blocks(bits, xb, want_dist=True)
    st = check_codes(bits, gc, oc, dist, what)
    st.update(check_norms(gn, on, xb, what))
    ref, _ = oracle.decode_blocks(bits, gc, gn)
    st.update(check_decode(gx, ref, what))
    return st


@pytest.mark.parametrize("bits", [3, 2])
def test_one_layer_every_element(bits):
    """K and V [8, 32768, 128] (2 x 33.5M values), both types: every code, norm and
    decoded value of the whole layer against the oracle."""
    w = gen.WORKLOADS["one_layer"]
    for name in ("K", "V"):
        x = _tensor(w, name)
        codes, norms = tq.empty_cache(bits, w.L, w.H, w.T, w.D)
        tq.tq_encode(bits, x, codes, norms, 0)
        out = torch.empty_like(x)
        tq.tq_decode(bits, codes, norms, 0, out)
        torch.cuda.synchronize()
        st = _check_blocks(bits, x.cpu().numpy().reshape(-1, 128),
                           codes.cpu().numpy().reshape(-1, 16 * bits), norms.cpu().numpy().reshape(-1),
                           out.cpu().numpy().reshape(-1, 128), f"one_layer {name} turbo{bits}")
        print(name, bits, st)
        del x, codes, norms, out


# ---------------------------------------------------------------- whole caches
#
# The whole-cache workloads run exactly as bench.py times them: K and V of every layer
# as one [2 L, H, T, D] tensor, one encode launch over all of it, one decode launch
# back.  The checks then stream over the cache one K or V layer at a time and compare
# every code, norm and decoded value with the oracle.

def _whole_cache(wname, bits):
    w = gen.WORKLOADS[wname]
    Lx = 2 * w.L
    x = torch.empty((Lx, w.H, w.T, w.D), dtype=torch.float16, device=DEV)
    for i, name in enumerate(("K", "V")):
        for l in range(w.L):
            x[i * w.L + l] = gen.kv_layer(w.seed, name, w.spec, l, w.H, w.T, w.D, device=DEV)
    codes, norms = tq.empty_cache(bits, Lx, w.H, w.T, w.D)
    tq.tq_encode(bits, x, codes, norms, 0)
    y = torch.empty_like(x)
    tq.tq_decode(bits, codes, norms, 0, y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "non-finite decoded values"
    assert bool(torch.isfinite(norms).all()), "non-finite norms"
    return {"w": w, "bits": bits, "x": x, "codes": codes, "norms": norms, "y": y}


def _check_layers(c, layers):
    """Every block of the given K / V layer tensors against the oracle: codes and norms
    from the layer's fp16 input, the decode of the GPU's own codes and norms."""
    bits, w = c["bits"], c["w"]
    total = {"values": 0, "mismatches": 0, "ties": 0, "norm_ulp_diffs": 0,
             "decode_worst_over_tol": 0.0, "decode_max_rel": 0.0}
    for li in layers:
        what = f"{w.name} {'KV'[li // w.L]} layer {li % w.L} turbo{bits}"
        xb = c["x"][li].reshape(-1, 128).cpu().numpy()
        gc = c["codes"][li].reshape(-1, 16 * bits).cpu().numpy()
        gn = c["norms"][li].reshape(-1).cpu().numpy()
        oc, on, dist = oracle.encode_blocks(bits, xb, want_dist=True)
        st = check_codes_full(bits, gc, oc, dist, what)
        del oc, dist
        st.update(check_norms(gn, on, xb, what))
        ref, _ = oracle.decode_blocks(bits, gc, gn)
        st.update(check_decode_torch(c["y"][li], ref, what))
        del ref
        for k in ("values", "mismatches", "ties", "norm_ulp_diffs"):
            total[k] += st[k]
        for k in ("decode_worst_over_tol", "decode_max_rel"):
            total[k] = max(total[k], st[k])
    print(total, flush=True)
    return total


@pytest.fixture(scope="module")
def full_cache_14b():
    c = _whole_cache("full_cache_14b", 3)
    yield c
    c.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_full_cache_14b_turbo3_every_element(full_cache_14b, part):
    """48 layers x 8 kv heads x 32768 x 128, K and V (6.4 GB fp16): turbo3 encode of the
    whole cache in one launch, decode back in one; a quarter of the 96 K / V layers per
    part, every code, norm and decoded value against the oracle."""
    n = 2 * full_cache_14b["w"].L
    _check_layers(full_cache_14b, range(part * n // 4, (part + 1) * n // 4))


def test_full_cache_14b_turbo3_distortion(full_cache_14b):
    """The mean relative round-trip error of all 25M blocks sits at the Gaussian turbo3
    distortion (0.0345 without outliers; the outlier channels lower it)."""
    mse = _rel_mse_per_block(full_cache_14b["x"], full_cache_14b["y"])
    print({"rel_mse": mse})
    assert 0.02 < mse < 0.04


@pytest.fixture(scope="module")
def head_dim_256():
    c = _whole_cache("head_dim_256", 2)
    yield c
    c.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_head_dim_256_turbo2_every_element(head_dim_256, part):
    """32 layers x 4 kv heads x 32768, head_dim 256 (two blocks per vector), Student-t(3)
    outlier channels: turbo2 encode and decode of the whole cache, one launch each; a
    quarter of the 64 K / V layers per part, every element against the oracle."""
    n = 2 * head_dim_256["w"].L
    _check_layers(head_dim_256, range(part * n // 4, (part + 1) * n // 4))


def test_head_dim_256_turbo2_distortion(head_dim_256):
    """Relative round-trip error near the Gaussian turbo2 distortion (0.117)."""
    mse = _rel_mse_per_block(head_dim_256["x"], head_dim_256["y"])
    print({"rel_mse": mse})
    assert 0.05 < mse < 0.13


def test_head_dim_256_read_path_every_element(head_dim_256):
    """The fused read over the same head_dim-256 cache, as bench.py times it: its 32 K
    layers as a batch of 32 sequences (4 kv heads, 16 query heads, GQA 4, all 32768
    rows): every one of the 16.8M q.K scores and every output of the fused attention
    over the K and V layers against the oracle over the same GPU-written caches."""
    c = head_dim_256
    w, bits = c["w"], c["bits"]
    B, Hkv, T, D, G = w.L, w.H, w.T, w.D, 4
    Hq = Hkv * G
    kc, kn = c["codes"][: w.L], c["norms"][: w.L]
    vc, vn = c["codes"][w.L:], c["norms"][w.L:]
    q = gen.queries(w.seed, B, Hq, D, device=DEV)
    scale = 1.0 / math.sqrt(D)
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)
    tq.tq_qk_scores(bits, kc, kn, q, scale, scores)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    tq.tq_attn_decode(bits, kc, kn, vc, vn, q, scale, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(scores).all()) and bool(torch.isfinite(out).all())
    kcn, knn, qn = kc.cpu().numpy(), kn.cpu().numpy(), q.cpu().numpy()
    ref = oracle.qk_scores(bits, kcn, knn, qn, scale)
    # ||k_hat|| per row over both blocks, from the oracle's decode, one layer at a time
    knorm = np.empty((B, Hkv, T))
    for l in range(B):
        xh, _ = oracle.decode_blocks(bits, kcn[l].reshape(-1, 16 * bits), knn[l].reshape(-1))
        knorm[l] = np.sqrt((xh.reshape(Hkv, T, -1) ** 2).sum(axis=-1))
        del xh
    qnorm = scale * np.linalg.norm(qn.astype(np.float64), axis=2)[:, :, None]
    print(check_scores_torch(scores, ref, qnorm, np.repeat(knorm, G, axis=1), "head_dim 256 q.K"))
    del ref, knorm
    vcn, vnn = vc.cpu().numpy(), vn.cpu().numpy()
    aref = oracle.attn_decode(bits, kcn, knn, vcn, vnn, qn, scale)
    vmax = np.empty((B, Hkv))
    for l in range(B):
        xh, _ = oracle.decode_blocks(bits, vcn[l].reshape(-1, 16 * bits), vnn[l].reshape(-1))
        vmax[l] = np.abs(xh.reshape(Hkv, -1)).max(axis=1)
        del xh
    print(check_attn(out.cpu().numpy(), aref, np.repeat(vmax, G, axis=1), T, "head_dim 256 attention"))


# ---------------------------------------------------------------- decode step

@pytest.fixture(scope="module")
def decode_step():
    """Per sequence turbo3 K and V caches [8, 32768, 128] (16 sequences), rows 0..32766
    prefilled by tq_encode, row 32767 appended for K and V (the launches bench.py times),
    queries for 32 heads (GQA 4)."""
    w = gen.WORKLOADS["decode_step"]
    B, Hkv, T, D, Hq = w.L, w.H, w.T, w.D, w.Hq
    bits = 3
    c = {"w": w, "bits": bits, "B": B, "Hkv": Hkv, "T": T, "D": D, "Hq": Hq}
    for name in ("K", "V"):
        x = torch.empty((B, Hkv, T - 1, D), dtype=torch.float16, device=DEV)
        for b in range(B):
            x[b] = gen.kv_layer(w.seed, name, w.spec, b, Hkv, T - 1, D, device=DEV, T_total=T)
        codes, norms = tq.empty_cache(bits, B, Hkv, T, D)
        tq.tq_encode(bits, x, codes, norms, 0)
        del x
        before_c = codes[:, :, : T - 1].clone()
        before_n = norms[:, :, : T - 1].clone()
        tok = torch.empty((B, Hkv, 1, D), dtype=torch.float16, device=DEV)
        for b in range(B):
            tok[b] = gen.kv_layer(w.seed, name, w.spec, b, Hkv, 1, D, device=DEV,
                                  t_offset=T - 1, T_total=T)
        tq.tq_encode(bits, tok, codes, norms, T - 1)
        torch.cuda.synchronize()
        c[name + "_untouched"] = (torch.equal(codes[:, :, : T - 1], before_c) and
                                  torch.equal(norms[:, :, : T - 1], before_n))
        del before_c, before_n
        c[name] = (codes, norms)
        c[name + "_tok"] = tok
    c["q"] = gen.queries(w.seed, B, Hq, D, device=DEV)
    c["scale"] = 1.0 / math.sqrt(D)
    yield c
    c.clear()
    torch.cuda.empty_cache()


def test_decode_step_append(decode_step):
    """The appended row of K and V (256 blocks) against the oracle; the append leaves the
    32767 prefilled rows of every cache untouched."""
    c = decode_step
    T = c["T"]
    for name in ("K", "V"):
        assert c[name + "_untouched"], f"append touched prefilled {name} rows"
        codes, norms = c[name]
        tb = c[name + "_tok"].cpu().numpy().reshape(-1, 128)
        oc, on, dist = oracle.encode_blocks(3, tb, want_dist=True)
        print(check_codes(3, codes[:, :, T - 1].cpu().numpy().reshape(-1, 48), oc, dist, f"append {name}"),
              check_norms(norms[:, :, T - 1].cpu().numpy(), on, tb, f"append {name}"))


def _decoded_norms_and_max(bits, codes, norms):
    """Per cache row: ||k_hat|| and max |k_hat| of the oracle's decode, one sequence at a
    time (codes [B, H, T, 1, 16 bits] numpy)."""
    B, H, T = codes.shape[:3]
    nrm = np.empty((B, H, T))
    amax = np.empty((B, H, T))
    for b in range(B):
        xh, _ = oracle.decode_blocks(bits, codes[b].reshape(-1, 16 * bits), norms[b].reshape(-1))
        nrm[b] = np.linalg.norm(xh, axis=1).reshape(H, T)
        amax[b] = np.abs(xh).max(axis=1).reshape(H, T)
        del xh
    return nrm, amax


def test_decode_step_qk_every_score(decode_step):
    """q.K of 32 query heads over all 32768 rows of the 16 sequences' K caches, one
    launch: every one of the 16.8M scores against the oracle's scores over the same
    GPU-written cache."""
    c = decode_step
    B, Hkv, T, Hq = c["B"], c["Hkv"], c["T"], c["Hq"]
    G = Hq // Hkv
    kc, kn = c["K"]
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)
    tq.tq_qk_scores(3, kc, kn, c["q"], c["scale"], scores)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(scores).all())
    kcn, knn = kc.cpu().numpy(), kn.cpu().numpy()
    qn = c["q"].cpu().numpy()
    ref = oracle.qk_scores(3, kcn, knn, qn, c["scale"])
    knorm, _ = _decoded_norms_and_max(3, kcn, knn)
    qnorm = c["scale"] * np.linalg.norm(qn.astype(np.float64), axis=2)[:, :, None]
    kn_h = np.repeat(knorm, G, axis=1)                      # query head h reads kv head h / G
    print(check_scores_torch(scores, ref, qnorm, kn_h, "decode_step q.K"))


def test_decode_step_attention_every_head(decode_step):
    """The fused decode attention of 32 query heads over the 16 sequences' K and V caches
    (all 32768 rows), one call: every output of all 128 (sequence, kv head) pairs against
    the oracle's attention over the same GPU-written caches."""
    c = decode_step
    B, Hkv, T, D, Hq = c["B"], c["Hkv"], c["T"], c["D"], c["Hq"]
    G = Hq // Hkv
    (kc, kn), (vc, vn) = c["K"], c["V"]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    tq.tq_attn_decode(3, kc, kn, vc, vn, c["q"], c["scale"], out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    vcn, vnn = vc.cpu().numpy(), vn.cpu().numpy()
    ref = oracle.attn_decode(3, kc.cpu().numpy(), kn.cpu().numpy(), vcn, vnn, c["q"].cpu().numpy(),
                             c["scale"])
    _, vabs = _decoded_norms_and_max(3, vcn, vnn)
    vmax = np.repeat(vabs.max(axis=2), G, axis=1)          # [B, Hq]
    print(check_attn(out.cpu().numpy(), ref, vmax, T, "decode_step attention"))
