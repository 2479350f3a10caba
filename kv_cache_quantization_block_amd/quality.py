"""Synthetic quality of the compressed KV cache against the uncompressed one.

The article reports turbo3 as practically free of quality loss in its long-context
use and turbo2's trade-off as real and model dependent (section "使い方"), with no
numbers; this harness puts numbers beside that on synthetic inputs (no model, no
dataset).  For one decode step of B sequences (Hkv kv heads, G query heads per kv
head, head_dim 128, context T):

  reference   softmax(scale q.K^T) V over the fp16 K and V as given (binary64,
              numpy, on the host: the uncompressed cache);
  compressed  the same step through this library: K and V encoded by tq_encode,
              scores by tq_qk_scores, the attention output by tq_attn_decode
              (all on the GPU, optionally with the randomised rotation H D).

Metrics, per (sequence, query head), then mean and worst over heads:
  rel_l2     ||o - o_ref|| / ||o_ref||   of the attention output;
  cos        <o, o_ref> / (||o|| ||o_ref||);
  score_rel  rms(s - s_ref) / rms(s_ref) of the scaled scores;
  top{k}     |top-k rows of s  intersect  top-k rows of s_ref| / k, k = 1, 8, 32.

Inputs (gen's seeded generators): K and V either as in the decode-step workload
("outliers": three x20 outlier channels per head, per-token log-uniform scale in
[0.5, 4]) or plain N(0, 1) rows ("gaussian", the codec's design point); queries
either N(0, 1) ("random": the outlier channels alone make many of these softmaxes
peaked) or "needle": each head's query points at one random key row of its kv head,
q = 4 sqrt(128) k_j / ||k_j|| + N(0, 1), which puts most of the softmax on row j, as
a retrieval head does.

Run: python -m kv_cache_quantization_block_amd.quality [--T 1024 4096 ...] -- one
JSON line per configuration.
"""
from __future__ import annotations

import argparse
import json
import math

import numpy as np
import torch

import gen
from . import empty_cache, tq_attn_decode, tq_encode, tq_qk_scores

KV_SPECS = {"outliers": gen.KVSpec(n_outliers=3, row_scale=True), "gaussian": gen.KVSpec()}
TOPK = (1, 8, 32)


def make_inputs(seed: int, B: int, Hkv: int, G: int, T: int, queries: str, device="cuda",
                kv: str = "outliers"):
    """(k, v) fp16 [B, Hkv, T, 128] and q fp16 [B, Hkv * G, 128] on `device`."""
    D = 128
    spec = KV_SPECS[kv]
    k = torch.empty((B, Hkv, T, D), dtype=torch.float16, device=device)
    v = torch.empty_like(k)
    for b in range(B):
        k[b] = gen.kv_layer(seed, "K", spec, b, Hkv, T, D, device=device)
        v[b] = gen.kv_layer(seed, "V", spec, b, Hkv, T, D, device=device)
    q = gen.queries(seed, B, Hkv * G, D, device=device)
    if queries == "needle":
        # per head a target row j (counter-based draw), q = 4 sqrt(128) k_j / |k_j| + noise
        u = gen.uniform(gen.stream_key(seed, 7), B * Hkv * G, 0, device)
        j = torch.clamp((u * T).long(), max=T - 1).view(B, Hkv * G)
        g = torch.arange(Hkv * G, device=device) // G
        kj = k[torch.arange(B, device=device)[:, None], g[None, :], j].double()
        kj = kj / kj.norm(dim=-1, keepdim=True)
        q = (4.0 * math.sqrt(D) * kj + q.double()).to(torch.float16)
    elif queries != "random":
        raise ValueError("queries must be 'random' or 'needle'")
    return k, v, q


def reference(k: np.ndarray, v: np.ndarray, q: np.ndarray, scale: float):
    """Uncompressed attention in binary64: (scores [B, Hq, T], out [B, Hq, 128])."""
    B, Hkv, T, D = k.shape
    Hq = q.shape[1]
    G = Hq // Hkv
    kd, vd = k.astype(np.float64), v.astype(np.float64)
    qd = q.astype(np.float64).reshape(B, Hkv, G, D)
    s = scale * np.einsum("bgrd,bgtd->bgrt", qd, kd)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    out = np.einsum("bgrt,bgtd->bgrd", p, vd)
    return s.reshape(B, Hq, T), out.reshape(B, Hq, D)


def metrics(out: np.ndarray, out_ref: np.ndarray, s: np.ndarray, s_ref: np.ndarray) -> dict:
    """The harness's metrics of one configuration (see the module docstring)."""
    o, r = out.astype(np.float64), out_ref.astype(np.float64)
    num = np.linalg.norm(o - r, axis=-1)
    den = np.linalg.norm(r, axis=-1)
    rel = num / np.maximum(den, 1e-300)
    cos = np.sum(o * r, axis=-1) / np.maximum(np.linalg.norm(o, axis=-1) * den, 1e-300)
    sd, sr = s.astype(np.float64), s_ref.astype(np.float64)
    srel = np.sqrt(np.mean((sd - sr) ** 2, axis=-1)) / np.sqrt(np.mean(sr ** 2, axis=-1))
    res = {"rel_l2_mean": float(rel.mean()), "rel_l2_max": float(rel.max()),
           "cos_mean": float(cos.mean()), "cos_min": float(cos.min()),
           "score_rel_mean": float(srel.mean())}
    T = s.shape[-1]
    for kk in TOPK:
        if kk > T:
            continue
        a = np.argpartition(-sd, kk - 1, axis=-1)[..., :kk]
        b = np.argpartition(-sr, kk - 1, axis=-1)[..., :kk]
        hit = np.array([len(np.intersect1d(x, y)) for x, y in zip(a.reshape(-1, kk), b.reshape(-1, kk))])
        res[f"top{kk}_mean"] = float(hit.mean() / kk)
        res[f"top{kk}_min"] = float(hit.min() / kk)
    return res


def compressed(bits: int, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, scale: float,
               signs=None):
    """The library's path: (caches, scores [B, Hq, T] fp32, out [B, Hq, 128] fp32)."""
    B, Hkv, T, D = k.shape
    Hq = q.shape[1]
    kc, kn = empty_cache(bits, B, Hkv, T, D, k.device)
    vc, vn = empty_cache(bits, B, Hkv, T, D, k.device)
    tq_encode(bits, k, kc, kn, 0, signs=signs)
    tq_encode(bits, v, vc, vn, 0, signs=signs)
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device=k.device)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=k.device)
    tq_qk_scores(bits, kc, kn, q, scale, scores, signs=signs)
    tq_attn_decode(bits, kc, kn, vc, vn, q, scale, out, signs=signs)
    torch.cuda.synchronize()
    return (kc, kn, vc, vn), scores, out


def run(bits: int, T: int, queries: str = "random", signs=None, B: int = 2, Hkv: int = 8,
        G: int = 4, seed: int = 11, kv: str = "outliers") -> dict:
    k, v, q = make_inputs(seed, B, Hkv, G, T, queries, kv=kv)
    scale = 1.0 / math.sqrt(128)
    _, s, out = compressed(bits, k, v, q, scale, signs)
    s_ref, out_ref = reference(k.cpu().numpy(), v.cpu().numpy(), q.cpu().numpy(), scale)
    res = {"type": f"turbo{bits}", "rotation": "H" if signs is None else "H D", "T": T,
           "kv": kv, "queries": queries, "sequences": B, "kv_heads": Hkv, "query_heads": Hkv * G}
    res.update(metrics(out.cpu().numpy(), out_ref, s.cpu().numpy(), s_ref))
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--T", type=int, nargs="+", default=[1024, 4096, 16384, 32768])
    ap.add_argument("--seed", type=int, default=11)
    args = ap.parse_args(argv)
    signs = np.where(np.random.default_rng(args.seed).random(128) < 0.5, -1.0, 1.0)
    for kv in ("outliers", "gaussian"):
        for T in args.T:
            for queries in ("random", "needle"):
                for bits in (3, 2):
                    for sg in (None, signs):
                        print(json.dumps(run(bits, T, queries, sg, seed=args.seed, kv=kv)), flush=True)


if __name__ == "__main__":
    main()
