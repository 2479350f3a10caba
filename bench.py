"""Benchmark of the turbo3 / turbo2 KV-cache codec hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: one layer of a GQA model's cache, K and V fp16 [8 kv heads, 32768
tokens, 128], N(0,1) with 3 of 128 channels (2%) scaled x20 and a per-token
scale log-uniform on [0.5, 4] (synthetic, seeded; generated on the GPU).

K and V are held as one [2, 8, 32768, 128] tensor, so each op below is one launch
covering both.  One step runs the whole path once:
  turbo3 encode of K,V   turbo2 encode of K,V   turbo3 decode   turbo2 decode
  1-token append of K and V (turbo3, row 32767)
  fused q.K scores of 32 query heads (GQA group 4) against the turbo3 K cache.
Each type encodes its own copy of K,V and decodes into its own buffers, so no
op re-reads data another op of the step left in the 256 MB Infinity Cache.

Before the W warm-up steps, whole steps run untimed for 0.2 s ("settle_steps"):
the GPU raises its clocks only after tens of milliseconds of sustained load, and a
short warm-up would time the ramp instead of the steady state.

Printed: one JSON line.  value = algorithmic bytes of the step / wall time per
step (GB/s); the dominant kernel's roofline is timed with HIP events on the
launch stream over the same timed steps; cpu_baseline times the CPU oracle on
whole steps of the same inputs (at least 10 s of CPU work).  Outside the timed
steps and not part of value: "decode_step" times the read path at the decode-step
size (16 sequences, each with turbo3 K and V caches [8 kv heads, 32768 rows, 128]
prefilled by encode: the 1-token append of K and V at row 32767, q.K of 32 query
heads over all rows, and the fused decode attention of the 32 heads over the
compressed K and V); "rotation" times turbo3 encode and decode of the layer with the
randomised rotation H D (seeded signs); "records" times the repack of that turbo3
cache into interleaved 50-byte block records and back; "bandwidth_configs" times
encode and decode of
a whole 14B-shaped turbo3 cache and a head_dim-256 turbo2 cache.
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
COPY_CAL_BYTES = 256 << 20     # bytes read (and written) by one calibration copy
SETTLE_S = 0.2                 # untimed steps before the warm-up (clock ramp-up)


def codec_bytes(nblocks: int, bits: int) -> int:
    """Algorithmic bytes of encoding or decoding nblocks: fp16 side + packed side."""
    return nblocks * (256 + 16 * bits + 2)


def qk_bytes(B, Hkv, T_, m, Hq, bits) -> int:
    return B * Hkv * T_ * m * (16 * bits + 2) + B * Hq * T_ * 4 + B * Hq * m * 128 * 2


def attn_bytes(B, Hkv, T_, Hq, bits) -> int:
    """Algorithmic bytes of a decode attention over T_ rows (head_dim 128): the K and V
    codes and norms once, the fp16 queries and the fp32 outputs."""
    return 2 * B * Hkv * T_ * (16 * bits + 2) + B * Hq * 128 * (2 + 4)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-step", action="store_true",
                    help="skip the decode-step read-path timing")
    ap.add_argument("--decode-step-only", action="store_true",
                    help="run only the decode-step read-path timing and print its figures "
                         "(a short run for profiling the decode attention)")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the full-cache and head_dim-256 bandwidth timings")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (default: usable cores, at most 16)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run three plain 256 MiB device copies (a kernel "
                         "of known traffic for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this codec path runs on a single MI355X "
              "(every block is independent; a cache sharded over GPUs runs this same path on each "
              "GPU's shard, launched by its own process).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gen
    import kv_cache_quantization_block_amd as tq
    import numpy as np

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tq.lib()
    stream = torch.cuda.current_stream()
    if args.decode_step_only:
        print(json.dumps({"decode_step": decode_step(tq, gen, dev, stream)}), flush=True)
        return

    w = gen.WORKLOADS["one_layer"]
    m = D // 128
    # K and V of the layer as one [2, H, T, D] tensor (index 0 = K, 1 = V): every op
    # of the step handles both in a single launch.
    KV = torch.empty((2, H, T, D), dtype=torch.float16, device=dev)
    KV[0] = gen.kv_layer(w.seed, "K", w.spec, 0, H, T, D, device=dev)
    KV[1] = gen.kv_layer(w.seed, "V", w.spec, 0, H, T, D, device=dev)
    q = gen.queries(w.seed, 1, HQ, D, device=dev)
    tok = torch.empty((2, H, 1, D), dtype=torch.float16, device=dev)
    tok[0] = gen.kv_layer(w.seed + 100, "K", w.spec, 0, H, 1, D, device=dev)
    tok[1] = gen.kv_layer(w.seed + 100, "V", w.spec, 0, H, 1, D, device=dev)

    bufs = {}
    for bits in (3, 2):
        bufs[bits] = dict(x=KV.clone(), c=tq.empty_cache(bits, 2, H, T, D, dev),
                          o=torch.empty_like(KV))
    scores = torch.empty((1, HQ, T), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    nblk = 2 * H * T * m          # K and V blocks

    ops = []   # (name, bytes, fn)
    for bits in (3, 2):
        b = bufs[bits]
        ops.append((f"encode_turbo{bits}", codec_bytes(nblk, bits),
                    lambda b=b, bits=bits: tq.tq_encode(bits, b["x"], *b["c"], 0)))
    for bits in (3, 2):
        b = bufs[bits]
        ops.append((f"decode_turbo{bits}", codec_bytes(nblk, bits),
                    lambda b=b, bits=bits: tq.tq_decode(bits, *b["c"], 0, b["o"])))
    c3, n3 = bufs[3]["c"]
    kc, kn = c3[0:1], n3[0:1]     # the K half of the turbo3 cache, [1, H, T, D/128, 48]
    ops.append(("append_turbo3", codec_bytes(2 * H * m, 3),
                lambda: tq.tq_encode(3, tok, c3, n3, T - 1)))
    ops.append(("qk_turbo3", qk_bytes(1, H, T, m, HQ, 3),
                lambda: tq.tq_qk_scores(3, kc, kn, q, scale, scores)))
    step_bytes = sum(o[1] for o in ops)
    op_values = {f"{k}_turbo{bits}": nblk * 128 for k in ("encode", "decode") for bits in (3, 2)}

    def step(dom_i=-1, ev=None):
        for i, (_, _, fn) in enumerate(ops):
            if i == dom_i:   # the launch's own dispatch records start and stop
                tq.tq_time_next_launch(ev[0], ev[1])
            fn()

    # Settle: the GPU ramps its clocks up only after tens of milliseconds of sustained
    # load, so whole steps run untimed for at least SETTLE_S before the W warm-up steps.
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    settle_steps = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-op durations: each op launched back to back REPS times between two events
    reps = 20
    per_op = {}
    for name, nbytes, fn in ops:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        per_op[name] = {"us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        if name in op_values:
            per_op[name]["Gvalues_per_s"] = round(op_values[name] / (us * 1e-6) / 1e9, 2)
    dom = max(per_op, key=lambda k: per_op[k]["us"])   # the dominant kernel of the step
    dom_i = [o[0] for o in ops].index(dom)

    # the randomised rotation H D (seeded signs, not part of the step): turbo3 encode and
    # decode of the same layer through the _rot entry points, timed like the table above
    signs = np.where(np.random.default_rng(w.seed).random(128) < 0.5, -1.0, 1.0)
    b3 = bufs[3]
    rotation = {}
    for name, fn in (("encode_turbo3_rot", lambda: tq.tq_encode(3, b3["x"], *b3["c"], 0, signs=signs)),
                     ("decode_turbo3_rot", lambda: tq.tq_decode(3, *b3["c"], 0, b3["o"], signs=signs))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = codec_bytes(nblk, 3)
        plain = per_op[name[:-4]]["us"]
        rotation[name] = {"us": round(us, 2), "bytes": nbytes,
                          "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "vs_plain": round(us / plain, 3)}

    # interleaved 50-byte records of the same turbo3 cache (not part of the step): both
    # directions read and write 50 bytes per block
    rec = torch.empty(nblk * 50, dtype=torch.uint8, device=dev)
    records = {}
    for name, fn in (("pack_records_turbo3", lambda: tq.tq_pack_records(3, *b3["c"], rec)),
                     ("unpack_records_turbo3", lambda: tq.tq_unpack_records(3, rec, *b3["c"]))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = 2 * nblk * 50
        records[name] = {"us": round(us, 2), "bytes": nbytes,
                         "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del rec
    for _ in range(2):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, wall clock between two device synchronisations; each
    # launch of the dominant kernel records HIP events on its stream from its own
    # dispatch packet (tq_time_next_launch; the events are created by a first record)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(dom_i, ev[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes * args.steps / elapsed / 1e9

    d_bytes = per_op[dom]["bytes"]
    d_us = sum(a.elapsed_time(b) for a, b in ev) * 1e3 / args.steps
    achieved = d_bytes / (d_us * 1e-6) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom), "bytes_per_launch": d_bytes,
                "avg_launch_us": round(d_us, 2)}

    ops_cold = cold_op_times(tq, ops, op_values, dev, stream)   # after the timed steps: it idles the GPU
    dstep = decode_step(tq, gen, dev, stream) if not args.no_decode_step else None
    bw_cfgs = bandwidth_configs(tq, gen, dev, stream) if not args.no_large else None
    copy_ctx = copy_bandwidth(dev, stream)

    if args.copy_calibration:
        src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(KV, q, tok, scale, step_bytes, args.cpu_threads)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "one_layer: K,V fp16 [8 kv_heads, 32768 tokens, 128]; turbo3+turbo2 "
                               "encode+decode of K and V, 1-token turbo3 append, turbo3 q.K of 32 "
                               "query heads (GQA 4)",
                   "bytes_per_step": step_bytes, "values_per_step_codec": 4 * nblk * 128,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ops": per_op,
        "ops_cold": ops_cold,
        "rotation": rotation,
        "records": records,
        "decode_step": dstep,
        "bandwidth_configs": bw_cfgs,
        "copy_context": copy_ctx,
    }
    print(json.dumps(out))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "one_layer_kv_kernels_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "kv_cache_quantization_block_amd", "csrc", f)
                  for f in ("kernels.hip", "internal.h")]


def kernel_code_sha() -> str:
    """First 16 hex digits of the sha256 of the kernels' code (kernels.hip, internal.h):
    comments removed and
    every run of whitespace made one space, so an edit of comments or layout alone does
    not count as a change of the kernels."""
    import hashlib
    import re
    src = "".join(open(f, encoding="utf-8").read() for f in KERNEL_SOURCES)
    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)
    code = tok.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", src)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of op `kernel` (encode_turbo3, decode_turbo3, ...) from the
    committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE scaled by a copy of
    known size), or None when the summary does not cover this op or the kernel source
    changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    for line in open(TRAFFIC_FILE):
        line = line.split("#")[0].strip()
        if ":" in line:
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_code_sha256_16") != kernel_code_sha() or f"{kernel}.fetch_size_kib" not in rec:
        return None
    copy_kib = int(rec["copy_bytes"]) / 1024
    fetch = float(rec[f"{kernel}.fetch_size_kib"]) * copy_kib / float(rec["copy_fetch_size_kib"])
    write = float(rec[f"{kernel}.write_size_kib"]) * copy_kib / float(rec["copy_write_size_kib"])
    return int(round((fetch + write) * 1024))


ISSUE_FILES = {"qk": os.path.join(ROOT, "profiles", "qk_decode_step_counters.txt"),
               "attn": os.path.join(ROOT, "profiles", "attn_partial_decode_step_counters.txt")}


def issue_utilisation(which: str):
    """Issue-port utilisation of the decode-step q.K ("qk") or attention partials
    ("attn") from the committed rocprofv3 counter summary, or None when the kernel
    source changed since it was taken.  Fractions of the kernel's cycles (GRBM_GUI_ACTIVE
    over the 8 XCDs): VALU per SIMD and LDS per CU from SQ_ACTIVE_INST_* (4-cycle units),
    the matrix core per SIMD from SQ_INSTS_MFMA at 16 cycles each."""
    path = ISSUE_FILES[which]
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if ":" in line:
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_code_sha256_16") != kernel_code_sha():
        return None
    cyc = float(rec["GRBM_GUI_ACTIVE"]) / 8
    return {"valu_per_simd": round(float(rec["SQ_ACTIVE_INST_VALU"]) * 4 / 1024 / cyc, 3),
            "lds_per_cu": round(float(rec["SQ_ACTIVE_INST_LDS"]) * 4 / 256 / cyc, 3),
            "mfma_per_simd": round(float(rec["SQ_INSTS_MFMA"]) * 16 / 1024 / cyc, 3),
            "source": os.path.relpath(path, ROOT)}


def decode_step(tq, gen, dev, stream, reps=20):
    """Average times of the decode-step read path: per sequence turbo3 K and V caches
    of [8, 32768, 128] (16 sequences), rows 0..32766 prefilled by tq_encode; the 1-token
    append of K and of V at row 32767 (two launches), q.K of 32 query heads, and the
    fused decode attention of the 32 heads over all 32768 rows (partials + combine)."""
    import torch
    w = gen.WORKLOADS["decode_step"]
    B, Hkv, T_, D_, Hq = w.L, w.H, w.T, w.D, w.Hq
    bits = 3
    kc, kn = tq.empty_cache(bits, B, Hkv, T_, D_, dev)
    vc, vn = tq.empty_cache(bits, B, Hkv, T_, D_, dev)
    for name, c_, n_ in (("K", kc, kn), ("V", vc, vn)):
        for b in range(B):   # prefill one sequence at a time (67 MB of fp16 each)
            xb = gen.kv_layer(w.seed, name, w.spec, b, Hkv, T_ - 1, D_, device=dev, T_total=T_)
            tq.tq_encode(bits, xb.unsqueeze(0), c_[b:b + 1], n_[b:b + 1], 0)
            del xb
    tok = {}
    for name in ("K", "V"):
        t_ = torch.empty((B, Hkv, 1, D_), dtype=torch.float16, device=dev)
        for b in range(B):
            t_[b] = gen.kv_layer(w.seed, name, w.spec, b, Hkv, 1, D_, device=dev,
                                 t_offset=T_ - 1, T_total=T_)
        tok[name] = t_
    q = gen.queries(w.seed, B, Hq, D_, device=dev)
    scores = torch.empty((B, Hq, T_), dtype=torch.float32, device=dev)
    attn = torch.empty((B, Hq, D_), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_attn_workspace_bytes(bits, B, Hkv, T_, D_, T_, Hq), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / math.sqrt(D_)
    ops = [("append_kv", lambda: (tq.tq_encode(bits, tok["K"], kc, kn, T_ - 1),
                                  tq.tq_encode(bits, tok["V"], vc, vn, T_ - 1))),
           ("qk", lambda: tq.tq_qk_scores(bits, kc, kn, q, scale, scores)),
           ("attn", lambda: tq.tq_attn_decode(bits, kc, kn, vc, vn, q, scale, attn, workspace=ws))]
    # each op back to back `reps` times between two events (the queue never drains, so
    # host launch latency stays hidden), after two untimed launches
    med = {}
    for name, fn in ops:
        fn()
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        med[name] = e0.elapsed_time(e1) * 1e3 / reps
    qb = qk_bytes(B, Hkv, T_, 1, Hq, bits)
    ab = attn_bytes(B, Hkv, T_, Hq, bits)
    out = {"workload": f"{B} sequences x {Hkv} kv heads x {T_} rows x {D_}, {Hq} query heads, turbo3",
           "qk_us": round(med["qk"], 2), "qk_bytes": qb,
           "qk_GBps": round(qb / (med["qk"] * 1e-6) / 1e9, 1),
           "qk_frac_of_hbm_peak": round(qb / (med["qk"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "attn_us": round(med["attn"], 2), "attn_bytes": ab,
           "attn_GBps": round(ab / (med["attn"] * 1e-6) / 1e9, 1),
           "attn_frac_of_hbm_peak": round(ab / (med["attn"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "append_kv_us": round(med["append_kv"], 2),
           # below 70 % of HBM peak these two are bound by instruction issue
           "qk_issue": issue_utilisation("qk"), "attn_issue": issue_utilisation("attn")}
    del kc, kn, vc, vn, scores, attn, ws
    torch.cuda.empty_cache()
    return out


def copy_bandwidth(dev, stream, nbytes=512 << 20, reps=10):
    """Context for the roofline: what a plain device-to-device copy of 512 MiB (torch's
    copy kernel, read + write counted) reaches on this GPU, HIP events around `reps`
    back-to-back copies after three untimed ones."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"what": "device-to-device copy, 512 MiB read + 512 MiB written", "us": round(us, 1),
            "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def bandwidth_configs(tq, gen, dev, stream, reps=10):
    """Encode then decode of two whole caches, the sizes where launch ramp and tail
    stop mattering: a 14B-shaped turbo3 cache (48 layers x 8 kv heads x 32768 x 128,
    K and V as one [96, 8, 32768, 128] tensor, 6.4 GB of fp16) and a head_dim-256
    turbo2 cache (32 layers x 4 kv heads x 32768 x 256, K and V, 4.3 GB); the turbo3
    cache also through tq_pack_records / tq_unpack_records (1.26 GB each way).  Average
    of `reps` back-to-back launches per op after ten untimed ones."""
    import torch
    out = {}
    for wname, bits in (("full_cache_14b", 3), ("head_dim_256", 2)):
        w = gen.WORKLOADS[wname]
        Lx = 2 * w.L
        x = torch.empty((Lx, w.H, w.T, w.D), dtype=torch.float16, device=dev)
        for i, name in enumerate(("K", "V")):
            for l in range(w.L):
                x[i * w.L + l] = gen.kv_layer(w.seed, name, w.spec, l, w.H, w.T, w.D, device=dev)
        codes, norms = tq.empty_cache(bits, Lx, w.H, w.T, w.D, dev)
        y = torch.empty_like(x)
        nblk = x.numel() // 128
        res = {"workload": f"{w.L} layers x {w.H} kv heads x {w.T} x {w.D}, K and V, turbo{bits}"}
        ops = [("encode", lambda: tq.tq_encode(bits, x, codes, norms, 0)),
               ("decode", lambda: tq.tq_decode(bits, codes, norms, 0, y))]
        rec = None
        if wname == "full_cache_14b":   # the whole cache through the record layout and back
            rec = torch.empty(nblk * (2 + 16 * bits), dtype=torch.uint8, device=dev)
            ops += [("pack_records", lambda: tq.tq_pack_records(bits, codes, norms, rec)),
                    ("unpack_records", lambda: tq.tq_unpack_records(bits, rec, codes, norms))]
        for op, fn in ops:
            for _ in range(10):   # about 15 ms of load: clocks at their sustained level
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            if op.endswith("records"):
                nb = 2 * nblk * (2 + 16 * bits)
                res[op] = {"us": round(us, 1), "bytes": nb, "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                           "frac_of_hbm_peak": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                continue
            nb = codec_bytes(nblk, bits)
            res[op] = {"us": round(us, 1), "bytes": nb, "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                       "frac_of_hbm_peak": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "Gvalues_per_s": round(nblk * 128 / (us * 1e-6) / 1e9, 1)}
        out[wname] = res
        del x, y, codes, norms, rec
        torch.cuda.empty_cache()
    return out


FLUSH_BYTES = 512 << 20   # twice the 256 MB Infinity Cache


def cold_op_times(tq, ops, op_values, dev, stream, reps=20):
    """Each op of the step timed alone with cold caches: before every one of `reps`
    launches (after three untimed), a 512 MiB buffer is written so that none of the
    op's inputs is left in the Infinity Cache.  The op's kernel records its own start
    and stop from its dispatch (tq_time_next_launch), so neither the buffer write nor
    the host's launch latency on the idle queue is counted.  Median and minimum per
    op, GB/s and values/s at the median, and encode + decode combined (sum of bytes /
    sum of median times)."""
    import torch
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)   # creates the events the hook records on
    e1.record(stream)
    out = {}
    for name, nbytes, fn in ops:
        times = []
        for r in range(3 + reps):
            scratch.fill_(float(r))
            tq.tq_time_next_launch(e0, e1)
            fn()
            torch.cuda.synchronize()
            if r >= 3:
                times.append(e0.elapsed_time(e1) * 1e3)
        times.sort()
        med = times[len(times) // 2]
        out[name] = {"median_us": round(med, 2), "min_us": round(times[0], 2), "bytes": nbytes,
                     "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if name in op_values:
            out[name]["Gvalues_per_s"] = round(op_values[name] / (med * 1e-6) / 1e9, 2)
    del scratch
    codec = [k for k in out if k.startswith(("encode_", "decode_"))]
    nb = sum(out[k]["bytes"] for k in codec)
    us = sum(out[k]["median_us"] for k in codec)
    out["encode_decode_combined"] = {"ops": codec, "bytes": nb, "us": round(us, 2),
                                     "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                                     "frac_of_hbm_peak": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(KV, q, tok, scale, step_bytes, threads):
    """The CPU oracle, untuned, on whole steps of the same inputs (host copies),
    repeated until at least 10 s of CPU work."""
    import numpy as np

    import oracle
    if threads <= 0:
        threads = min(len(os.sched_getaffinity(0)), 16)
    x = KV.cpu().numpy()
    qn = q.cpu().numpy()
    tk = tok.cpu().numpy()
    m = D // 128
    def one_step():
        caches = {}
        for bits in (3, 2):
            c = np.zeros((2, H, T, m, 16 * bits), np.uint8)
            n = np.zeros((2, H, T, m), np.float16)
            oracle.encode(bits, x, c, n, nthreads=threads)
            caches[bits] = (c, n)
        for bits in (3, 2):
            oracle.decode(bits, *caches[bits], 0, T, nthreads=threads)
        oracle.encode(3, tk, *caches[3], t0=T - 1, nthreads=threads)
        c3, n3 = caches[3]
        oracle.qk_scores(3, c3[0:1], n3[0:1], qn, scale, nthreads=threads)

    # whole steps until at least min_seconds of CPU work (a bounded sample)
    min_seconds = 10.0
    t0 = time.perf_counter()
    steps = 0
    while True:
        one_step()
        steps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": round(step_bytes * steps / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(el, 2), "cpu": cpu_model(),
            "Gvalues_per_s_codec": round(4 * x.size * steps / el / 1e9, 4),
            "sample": f"{steps} full steps of the same workload (one layer, K and V) on host "
                      f"copies of the same inputs, repeated until at least {min_seconds:.0f} s"}


if __name__ == "__main__":
    main()
