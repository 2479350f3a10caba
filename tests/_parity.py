"""Comparison rules between the HIP path and the CPU oracle (test helper).

Rules (readings of the tolerances, each applied element by element):
  codes   bit-exact, except values whose oracle t lies within TIE_BAND of a
          decision threshold (both codes are then equally valid); every
          mismatch must be such a tie and the mismatch fraction must not
          exceed MISMATCH_FRAC (at least one mismatch is tolerated in samples
          smaller than 1 / MISMATCH_FRAC values);
  norms   fp16 bit-exact, or one ulp apart where the exact norm lies within
          1e-6 (relative) of the midpoint of the two fp16 values (float32 on
          the GPU vs binary64 in the oracle may round such a norm either way);
  decode  |g - r| <= 1e-3 * max(|r|, 0.01 * rms(block of r)) + 2^-25, r the
          oracle's binary64 decode of the GPU's own codes and norms (2^-25 is
          half the smallest fp16 spacing: the output format's own resolution);
          where r lies beyond the fp16 range (|r| >= 65520, e.g. a turbo2
          one-hot outlier reconstructed at 1.51x) both sides must give the
          same infinity, the IEEE round-to-nearest result;
  scores  |g - r| <= 2e-3 * max(|r|, 0.01 * ||q|| * ||k_hat||), r the oracle's
          scores over the GPU-written cache;
  attention |g - r| <= 2e-3 * max(|r|, 0.01 * rms(r over the head's 128 outputs)), r the
          oracle's binary64 decode attention over the GPU-written K and V caches.
"""
from __future__ import annotations

import numpy as np

TIE_BAND = 1e-5
MISMATCH_FRAC = 1e-6


def unpack_codes(codes, bits: int) -> np.ndarray:
    """u8 [..., 16*bits] → int codes [..., 128] (little-endian bit stream)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    shp = codes.shape[:-1]
    stream = np.unpackbits(codes.reshape(-1, 16 * bits), axis=1, bitorder="little")
    c = (stream.reshape(-1, 128, bits) * (1 << np.arange(bits))).sum(axis=2)
    return c.reshape(*shp, 128)


def check_codes(bits, gpu_codes, ora_codes, ora_dist, what=""):
    g = unpack_codes(gpu_codes, bits).reshape(-1)
    o = unpack_codes(ora_codes, bits).reshape(-1)
    d = np.asarray(ora_dist).reshape(-1)
    assert g.shape == o.shape == d.shape
    bad = g != o
    nbad = int(bad.sum())
    ties = int((d < TIE_BAND).sum())
    if nbad:
        assert np.all(d[bad] < TIE_BAND), \
            f"{what}: {int((d[bad] >= TIE_BAND).sum())} code mismatches outside the tie band"
        assert np.all(np.abs(g[bad] - o[bad]) == 1), f"{what}: mismatch by more than one cell"
    allowed = max(1, int(MISMATCH_FRAC * g.size))
    assert nbad <= allowed, f"{what}: {nbad} tie mismatches in {g.size} values (allowed {allowed})"
    return {"values": int(g.size), "mismatches": nbad, "ties": ties}


def check_norms(gpu_n16, ora_n16, x_blocks, what=""):
    g = np.asarray(gpu_n16, dtype=np.float16).reshape(-1)
    o = np.asarray(ora_n16, dtype=np.float16).reshape(-1)
    diff = g.view(np.uint16) != o.view(np.uint16)
    n = int(diff.sum())
    if n:
        x = np.asarray(x_blocks, dtype=np.float16).reshape(-1, 128)[diff].astype(np.float64)
        exact = np.linalg.norm(x, axis=1)
        gi, oi = g[diff].view(np.uint16).astype(np.int64), o[diff].view(np.uint16).astype(np.int64)
        assert np.all(np.abs(gi - oi) == 1), f"{what}: norm differs by more than one ulp"
        mid = (g[diff].astype(np.float64) + o[diff].astype(np.float64)) / 2
        assert np.all(np.abs(exact - mid) <= 1e-6 * exact), f"{what}: norm ulp diff away from a midpoint"
    return {"norm_ulp_diffs": n}


def check_decode(gpu_x16, ref, what=""):
    g = np.asarray(gpu_x16, dtype=np.float16).astype(np.float64).reshape(-1, 128)
    r = np.asarray(ref, dtype=np.float64).reshape(-1, 128)
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    tol = 1e-3 * np.maximum(np.abs(r), 0.01 * rms) + 2.0 ** -25
    over = np.abs(r) >= 65520.0
    if over.any():
        assert np.array_equal(g[over], np.sign(r[over]) * np.inf), f"{what}: overflow not inf"
        g = np.where(over, r, g)
    err = np.abs(g - r)
    worst = float(np.max(err / tol)) if err.size else 0.0
    assert np.all(err <= tol), f"{what}: decode error {worst:.3f} x tolerance"
    nz = np.abs(r) > 0
    max_rel = float(np.max(err[nz] / np.abs(r[nz]))) if nz.any() else 0.0
    return {"decode_worst_over_tol": worst, "decode_max_rel": max_rel}


def check_scores(gpu, ref, qnorm, knorm, what=""):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    floor = 0.01 * np.asarray(qnorm) * np.asarray(knorm)
    tol = 2e-3 * np.maximum(np.abs(r), floor)
    err = np.abs(g - r)
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    assert np.all(err <= tol), f"{what}: score error {worst:.3f} x tolerance"
    return {"scores_worst_over_tol": worst}


def check_attn(gpu, ref, vmax, T, what=""):
    """Decode attention [B, Hq, D]: 2e-3 of max(|r|, 1% of the head's rms), plus an
    absolute floor T 2^-38 max|v_hat| (vmax [B, Hq], over the head's rows < T).

    The floor bounds what the weights' finite resolution may cost.  The page's own
    attention path dequantises K and V to fp16 and runs Flash Attention, whose P.V
    product takes the softmax weights in fp16: with the largest weight at 1, each
    weight is then off by up to half of fp16's smallest spacing, 2^-25, and the output
    by up to sum_t 2^-25 |v_hat_t| / sum_t p_t <= T 2^-25 max|v_hat|.  The floor here is
    2^13 times tighter than that bound.  It matters only where the output lies many
    orders below the values (a softmax that sits on rows of zeros, say); elsewhere the
    relative term dominates."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    floor = T * 2.0 ** -38 * np.asarray(vmax, dtype=np.float64)[..., None]
    tol = 2e-3 * np.maximum(np.abs(r), 0.01 * rms) + floor
    err = np.abs(g - r)
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    assert np.all(err <= tol), f"{what}: attention error {worst:.3f} x tolerance"
    return {"attn_worst_over_tol": worst}


# ---------------------------------------------------------------- whole tensors
#
# The same rules at the workloads' full sizes, where every element is compared: the
# oracle runs on the host, and the element-wise comparisons of large arrays run in
# torch (float64 on the tensors' device), with the codes compared block by block and
# unpacked only where a block differs.

def check_codes_full(bits, gpu_codes, ora_codes, ora_dist, what=""):
    """Codes of many blocks (u8 [nb, 16*bits] numpy), distances [nb, 128]: the rule of
    check_codes, the allowance taken over all nb * 128 values."""
    gc = np.ascontiguousarray(gpu_codes).reshape(-1, 16 * bits)
    oc = np.ascontiguousarray(ora_codes).reshape(-1, 16 * bits)
    d = np.asarray(ora_dist).reshape(-1, 128)
    nvals = gc.shape[0] * 128
    ties = int(np.count_nonzero(d < TIE_BAND))
    bad_blk = np.nonzero((gc != oc).any(axis=1))[0]
    nbad = 0
    if bad_blk.size:
        g = unpack_codes(gc[bad_blk], bits).reshape(-1)
        o = unpack_codes(oc[bad_blk], bits).reshape(-1)
        db = d[bad_blk].reshape(-1)
        bad = g != o
        nbad = int(bad.sum())
        assert np.all(db[bad] < TIE_BAND), \
            f"{what}: {int((db[bad] >= TIE_BAND).sum())} code mismatches outside the tie band"
        assert np.all(np.abs(g[bad] - o[bad]) == 1), f"{what}: mismatch by more than one cell"
    allowed = max(1, int(MISMATCH_FRAC * nvals))
    assert nbad <= allowed, f"{what}: {nbad} tie mismatches in {nvals} values (allowed {allowed})"
    return {"values": nvals, "mismatches": nbad, "ties": ties}


def check_decode_torch(gpu_x16, ref, what=""):
    """check_decode over a whole tensor: gpu_x16 a torch fp16 tensor [..., 128] (any
    device), ref the oracle's binary64 decode (numpy, same element count)."""
    import torch
    g = gpu_x16.reshape(-1, 128).to(torch.float64)
    r = torch.from_numpy(np.ascontiguousarray(ref).reshape(-1, 128)).to(g.device)
    rms = torch.sqrt(torch.mean(r * r, dim=1, keepdim=True))
    tol = 1e-3 * torch.maximum(r.abs(), 0.01 * rms) + 2.0 ** -25
    over = r.abs() >= 65520.0
    if bool(over.any()):
        assert torch.equal(g[over], torch.sign(r[over]) * float("inf")), f"{what}: overflow not inf"
        g = torch.where(over, r, g)
    err = (g - r).abs()
    worst = float((err / tol).max()) if err.numel() else 0.0
    assert bool((err <= tol).all()), f"{what}: decode error {worst:.3f} x tolerance"
    nz = r.abs() > 0
    max_rel = float((err[nz] / r[nz].abs()).max()) if bool(nz.any()) else 0.0
    return {"decode_worst_over_tol": worst, "decode_max_rel": max_rel}


def check_scores_torch(gpu, ref, qnorm, knorm, what=""):
    """check_scores over a whole score tensor: gpu a torch float32 tensor, ref, qnorm and
    knorm numpy arrays broadcastable to it (float64)."""
    import torch
    g = gpu.to(torch.float64)
    dev = g.device
    r = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float64)).to(dev)
    floor = 0.01 * torch.from_numpy(np.ascontiguousarray(qnorm, dtype=np.float64)).to(dev) * \
        torch.from_numpy(np.ascontiguousarray(knorm, dtype=np.float64)).to(dev)
    tol = 2e-3 * torch.maximum(r.abs(), floor)
    err = (g - r).abs()
    worst = float((err / tol.clamp_min(1e-300)).max()) if err.numel() else 0.0
    assert bool((err <= tol).all()), f"{what}: score error {worst:.3f} x tolerance"
    return {"scores": int(g.numel()), "scores_worst_over_tol": worst}
