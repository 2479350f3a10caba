"""Benchmark of the turbo3 / turbo2 KV-cache codec hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: one layer of a GQA model's cache, K and V fp16 [8 kv heads, 32768
tokens, 128], N(0,1) with 3 of 128 channels (2%) scaled x20 and a per-token
scale log-uniform on [0.5, 4] (synthetic, seeded; generated on the GPU).

One step runs the whole path once:
  turbo3 encode K, V   turbo2 encode K, V   turbo3 decode K, V   turbo2 decode K, V
  1-token append of K and V (turbo3, row 32767)
  fused q.K scores of 32 query heads (GQA group 4) against the turbo3 K cache.
Each type encodes its own copy of K and V and decodes into its own buffers, so
no op re-reads data another op of the step left in the 256 MB Infinity Cache.

Printed: one JSON line.  value = algorithmic bytes of the step / wall time per
step (GB/s); the dominant kernel's roofline is timed with HIP events on the
launch stream over the same timed steps; cpu_baseline times the CPU oracle on
one full step of the same inputs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "turbo3/turbo2 KV encode+decode GB/s and fraction of HBM peak, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
L, H, T, D = 1, 8, 32768, 128  # one layer
HQ = 32                        # query heads (GQA group 4)
SEED = 2


def codec_bytes(nblocks: int, bits: int) -> int:
    """Algorithmic bytes of encoding or decoding nblocks: fp16 side + packed side."""
    return nblocks * (256 + 16 * bits + 2)


def qk_bytes(B, Hkv, T_, m, Hq, bits) -> int:
    return B * Hkv * T_ * m * (16 * bits + 2) + B * Hq * T_ * 4 + B * Hq * m * 128 * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (default: usable cores, at most 16)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this codec path runs on a single MI355X "
              "(every block is independent; multi-GPU sharding is not part of this build).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gen
    import kv_cache_quantization_block_amd as tq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tq.lib()
    stream = torch.cuda.current_stream()

    w = gen.WORKLOADS["one_layer"]
    m = D // 128
    K = torch.empty((L, H, T, D), dtype=torch.float16, device=dev)
    V = torch.empty_like(K)
    K[0] = gen.kv_layer(w.seed, "K", w.spec, 0, H, T, D, device=dev)
    V[0] = gen.kv_layer(w.seed, "V", w.spec, 0, H, T, D, device=dev)
    q = gen.queries(w.seed, 1, HQ, D, device=dev)
    tok_k = gen.kv_layer(w.seed + 100, "K", w.spec, 0, H, 1, D, device=dev).unsqueeze(0)
    tok_v = gen.kv_layer(w.seed + 100, "V", w.spec, 0, H, 1, D, device=dev).unsqueeze(0)

    bufs = {}
    for bits in (3, 2):
        bufs[bits] = dict(
            K=K.clone(), V=V.clone(),
            cK=tq.empty_cache(bits, L, H, T, D, dev), cV=tq.empty_cache(bits, L, H, T, D, dev),
            oK=torch.empty_like(K), oV=torch.empty_like(K))
    scores = torch.empty((1, HQ, T), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    nblk = L * H * T * m

    ops = []   # (name, bytes, fn)
    for bits in (3, 2):
        b = bufs[bits]
        ops.append((f"encode_turbo{bits}_K", codec_bytes(nblk, bits),
                    lambda b=b, bits=bits: tq.tq_encode(bits, b["K"], *b["cK"], 0)))
        ops.append((f"encode_turbo{bits}_V", codec_bytes(nblk, bits),
                    lambda b=b, bits=bits: tq.tq_encode(bits, b["V"], *b["cV"], 0)))
    for bits in (3, 2):
        b = bufs[bits]
        ops.append((f"decode_turbo{bits}_K", codec_bytes(nblk, bits),
                    lambda b=b, bits=bits: tq.tq_decode(bits, *b["cK"], 0, b["oK"])))
        ops.append((f"decode_turbo{bits}_V", codec_bytes(nblk, bits),
                    lambda b=b, bits=bits: tq.tq_decode(bits, *b["cV"], 0, b["oV"])))
    b3 = bufs[3]
    ops.append(("append_turbo3_K", codec_bytes(L * H * m, 3),
                lambda: tq.tq_encode(3, tok_k, *b3["cK"], T - 1)))
    ops.append(("append_turbo3_V", codec_bytes(L * H * m, 3),
                lambda: tq.tq_encode(3, tok_v, *b3["cV"], T - 1)))
    ops.append(("qk_turbo3", qk_bytes(L, H, T, m, HQ, 3),
                lambda: tq.tq_qk_scores(3, *b3["cK"], q, scale, scores)))
    step_bytes = sum(o[1] for o in ops)

    def step(events=None):
        for i, (_, _, fn) in enumerate(ops):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, wall clock between two device synchronisations
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes * args.steps / elapsed / 1e9

    per_op = {}
    for i, (name, nbytes, _) in enumerate(ops):
        ms = sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)) / args.steps
        per_op[name] = {"us": round(ms * 1e3, 2), "bytes": nbytes,
                        "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    # dominant kernel = the op family with the largest share of the step
    fam = {}
    for name, rec in per_op.items():
        key = name.rsplit("_", 1)[0] if name.endswith(("_K", "_V")) else name
        fam.setdefault(key, []).append(rec)
    dom = max(fam, key=lambda k: sum(r["us"] for r in fam[k]))
    d_us = sum(r["us"] for r in fam[dom]) / len(fam[dom])
    d_bytes = fam[dom][0]["bytes"]
    achieved = d_bytes / (d_us * 1e-6) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None, "bytes_per_launch": d_bytes, "avg_launch_us": round(d_us, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(K, V, q, tok_k, tok_v, scale, step_bytes, args.cpu_threads)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "one_layer: K,V fp16 [8 kv_heads, 32768 tokens, 128]; turbo3+turbo2 "
                               "encode+decode of K and V, 1-token turbo3 append, turbo3 q.K of 32 "
                               "query heads (GQA 4)",
                   "bytes_per_step": step_bytes, "values_per_step_codec": 8 * nblk * 128,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ops": per_op,
    }
    print(json.dumps(out))


def cpu_baseline(K, V, q, tok_k, tok_v, scale, step_bytes, threads):
    """The CPU oracle, untuned, on one full step of the same inputs (host copies)."""
    import numpy as np

    import oracle
    if threads <= 0:
        threads = min(len(os.sched_getaffinity(0)), 16)
    Kn, Vn = K.cpu().numpy(), V.cpu().numpy()
    qn = q.cpu().numpy()
    tk, tv = tok_k.cpu().numpy(), tok_v.cpu().numpy()
    m = D // 128
    t0 = time.perf_counter()
    caches = {}
    for bits in (3, 2):
        for name, x in (("K", Kn), ("V", Vn)):
            c = np.zeros((L, H, T, m, 16 * bits), np.uint8)
            n = np.zeros((L, H, T, m), np.float16)
            oracle.encode(bits, x, c, n, nthreads=threads)
            caches[(bits, name)] = (c, n)
    for bits in (3, 2):
        for name in ("K", "V"):
            oracle.decode(bits, *caches[(bits, name)], 0, T, nthreads=threads)
    oracle.encode(3, tk, *caches[(3, "K")], t0=T - 1, nthreads=threads)
    oracle.encode(3, tv, *caches[(3, "V")], t0=T - 1, nthreads=threads)
    oracle.qk_scores(3, *caches[(3, "K")], qn, scale, nthreads=threads)
    el = time.perf_counter() - t0
    return {"value": round(step_bytes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(el, 2),
            "sample": "one full step of the same workload on host copies of the same inputs"}


if __name__ == "__main__":
    main()
