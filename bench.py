"""Benchmark of the turbo3 / turbo2 KV-cache codec hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Headline workload: the whole KV cache of a 14B-class GQA model at 32,768 tokens of
context (the article's section "実モデルでの数値" quotes a 14B model at that
length): K and V fp16 [48 layers, 8 kv heads, 32768 tokens, 128], N(0,1) with 3 of
128 channels (2%) scaled x20 and a per-token scale log-uniform on [0.5, 4]
(synthetic, seeded, generated on the GPU).  K and V are held as one
[96, 8, 32768, 128] tensor (6.4 GB), so each op below is one launch covering both.

One step: turbo3 encode of the whole cache (25,165,824 blocks), then turbo3 decode
of it back to fp16.  value = algorithmic bytes of the step (306 B per block and op:
256 B of fp16 plus 48 B of codes and a 2-byte norm) / wall time per step, with the
inputs resident in HBM.  Before the W warm-up steps, whole steps run untimed for
0.2 s ("settle_steps"): the GPU raises its clocks only after tens of milliseconds of
sustained load.  Each launch of the two kernels in the timed steps records HIP
events from its own dispatch packet (tq_time_next_launch); the roofline names the
slower of the two, its average duration and its algorithmic GB/s.  cpu_baseline
times the CPU oracle on a bounded sample of the same workload (whole K / V layers of
the same cache, encode then decode).

Printed: one JSON line.  Outside the timed steps and not part of value:
  "read_path_14b"     the 1-token append of K and V into every layer of the same
                      cache and the fused q.K of 32 query heads (GQA 4) over all 48
                      layers' keys (one decode step of the whole model's q.K);
  "records_14b"       the same turbo3 cache into interleaved 50-byte block records
                      and back;
  "head_dim_256"      turbo2 encode and decode of a whole head_dim-256 cache
                      (32 layers x 4 kv heads x 32768 x 256, K and V), and the fused
                      read over it (its K layers as 32 sequences, 16 query heads: q.K
                      and the decode attention over the K and V layers);
  "decode_step"       the read path at the decode-step size (16 sequences, each with
                      turbo3 K and V caches [8, 32768, 128]): the append of K and V, q.K
                      of 32 query heads and the fused decode attention over the
                      compressed K and V;
  "one_layer"         one layer (K and V [8, 32768, 128]) through every op of the
                      codec: turbo3 and turbo2 encode and decode, append, q.K, the
                      randomised rotation and the records, back to back and with a
                      cold Infinity Cache;
  "copy_context"      a plain 512 MiB device copy, the achievable-bandwidth context.
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
HEADLINE = "full_cache_14b"    # 48 x 8 x 32768 x 128, K and V, turbo3
HQ = 32                        # query heads (GQA group 4)
COPY_CAL_BYTES = 256 << 20     # bytes read (and written) by one calibration copy
SETTLE_S = 0.2                 # untimed steps before the warm-up (clock ramp-up)
CPU_MIN_SECONDS = 10.0         # CPU-baseline sample: at least this much oracle time


def codec_bytes(nblocks: int, bits: int) -> int:
    """Algorithmic bytes of encoding or decoding nblocks: fp16 side + packed side."""
    return nblocks * (256 + 16 * bits + 2)


def qk_bytes(B, Hkv, T_, m, Hq, bits) -> int:
    return B * Hkv * T_ * m * (16 * bits + 2) + B * Hq * T_ * 4 + B * Hq * m * 128 * 2


def attn_bytes(B, Hkv, T_, Hq, bits, m=1) -> int:
    """Algorithmic bytes of a decode attention over T_ rows (head_dim 128 m): the K and V
    codes and norms once, the fp16 queries and the fp32 outputs."""
    return 2 * B * Hkv * T_ * m * (16 * bits + 2) + B * Hq * 128 * m * (2 + 4)


def gbs(nbytes: float, us: float) -> float:
    return nbytes / (us * 1e-6) / 1e9


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the timed whole-cache steps (and --copy-calibration): a short run "
                         "for profiling the headline kernels")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip every figure outside the timed steps except the CPU baseline")
    ap.add_argument("--decode-step-only", action="store_true",
                    help="run only the decode-step read-path timing and print its figures "
                         "(a short run for profiling the fused read)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads (default: every core this process may run on)")
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

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tq.lib()
    stream = torch.cuda.current_stream()
    if args.decode_step_only:
        print(json.dumps({"decode_step": decode_step(tq, gen, dev, stream)}), flush=True)
        return

    hl = Headline(tq, gen, dev, stream)
    res = hl.run(args.steps, args.warmup)
    if args.copy_calibration:
        copy_calibration(dev)
    extras = {}
    cpu = None
    if not args.headline_only:
        if not args.no_extras:
            extras["read_path_14b"] = hl.read_path()
            extras["records_14b"] = hl.records()
        if not args.no_cpu_baseline:
            cpu = hl.cpu_baseline(args.cpu_threads)
    hl.free()
    if not args.headline_only and not args.no_extras:
        extras["head_dim_256"] = head_dim_256(tq, gen, dev, stream)
        extras["decode_step"] = decode_step(tq, gen, dev, stream)
        extras["one_layer"] = one_layer(tq, gen, dev, stream)
        extras["copy_context"] = copy_bandwidth(dev, stream)

    out = {
        "metric": METRIC, "value": res["value"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": res["settle_steps"],
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": res["config"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "kernels": res["kernels"],
        **extras,
    }
    print(json.dumps(out), flush=True)


class Headline:
    """The whole 14B-shaped cache, resident on the GPU: fp16 K and V [96, 8, 32768, 128],
    its turbo3 planes and the decoded fp16 output."""

    def __init__(self, tq, gen, dev, stream):
        import torch
        self.tq, self.gen, self.dev, self.stream = tq, gen, dev, stream
        w = gen.WORKLOADS[HEADLINE]
        self.w = w
        self.bits = 3
        self.Lx = 2 * w.L
        self.x = torch.empty((self.Lx, w.H, w.T, w.D), dtype=torch.float16, device=dev)
        for i, name in enumerate(("K", "V")):
            for l in range(w.L):
                self.x[i * w.L + l] = gen.kv_layer(w.seed, name, w.spec, l, w.H, w.T, w.D, device=dev)
        self.codes, self.norms = tq.empty_cache(self.bits, self.Lx, w.H, w.T, w.D, dev)
        self.y = torch.empty_like(self.x)
        self.nblk = self.x.numel() // 128
        self.op_bytes = codec_bytes(self.nblk, self.bits)
        self.ops = [("encode_turbo3", lambda: tq.tq_encode(self.bits, self.x, self.codes, self.norms, 0)),
                    ("decode_turbo3", lambda: tq.tq_decode(self.bits, self.codes, self.norms, 0, self.y))]

    def step(self, ev=None):
        for i, (_, fn) in enumerate(self.ops):
            if ev is not None:   # the launch's own dispatch records its start and stop
                self.tq.tq_time_next_launch(ev[i][0], ev[i][1])
            fn()

    def run(self, steps, warmup):
        import torch
        torch.cuda.synchronize()
        t_settle = time.perf_counter()
        settle_steps = 0
        while time.perf_counter() - t_settle < SETTLE_S:
            self.step()
            settle_steps += 1
            torch.cuda.synchronize()
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        # timed region: K steps, wall clock between two device synchronisations; every
        # launch records HIP events on its stream from its own dispatch packet (the
        # events are created by a first record)
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in self.ops] for _ in range(steps)]
        for per_step in ev:
            for a, b in per_step:
                a.record(self.stream)
                b.record(self.stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(steps):
            self.step(ev[s_])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        step_bytes = len(self.ops) * self.op_bytes
        value = step_bytes * steps / elapsed / 1e9
        kernels = {}
        for i, (name, _) in enumerate(self.ops):
            us = [ev[s_][i][0].elapsed_time(ev[s_][i][1]) * 1e3 for s_ in range(steps)]
            avg = sum(us) / len(us)
            kernels[name] = {"avg_launch_us": round(avg, 2), "min_launch_us": round(min(us), 2),
                             "bytes_per_launch": self.op_bytes,
                             "GBps": round(gbs(self.op_bytes, avg), 1),
                             "frac_of_hbm_peak": round(gbs(self.op_bytes, avg) / HBM_PEAK_GBS, 4),
                             "Gvalues_per_s": round(self.nblk * 128 / (avg * 1e-6) / 1e9, 1),
                             "traffic": measured_traffic(name)}
        dom = max(kernels, key=lambda k: kernels[k]["avg_launch_us"])   # the dominant kernel
        d = kernels[dom]
        roofline = {"kernel": dom, "bound": "hbm", "achieved": d["GBps"], "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": d["frac_of_hbm_peak"], "traffic": d["traffic"],
                    "bytes_per_launch": self.op_bytes, "avg_launch_us": d["avg_launch_us"]}
        w = self.w
        config = {"workload": f"{HEADLINE}: K,V fp16 [{w.L} layers, {w.H} kv_heads, {w.T} tokens, "
                              f"{w.D}] as one [{self.Lx}, {w.H}, {w.T}, {w.D}] tensor; turbo3 encode of "
                              f"the whole cache, then decode back to fp16",
                  "blocks_per_op": self.nblk, "bytes_per_step": step_bytes,
                  "values_per_step": len(self.ops) * self.nblk * 128,
                  "Gvalues_per_s": round(len(self.ops) * self.nblk * 128 * steps / elapsed / 1e9, 1),
                  "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)}
        return {"value": round(value, 1), "ms_per_step": round(elapsed * 1e3 / steps, 4),
                "settle_steps": settle_steps, "roofline": roofline, "kernels": kernels,
                "config": config}

    def read_path(self, reps=10):
        """On the same resident cache: the 1-token append of K and V into row T - 1 of every
        layer (one launch over [96, 8, 1, 128]), and q.K of 32 query heads over the keys of
        all 48 layers (the K half as a batch of 48, one launch: each layer's decode-step
        scores).  Average of `reps` back-to-back launches after 0.2 s of untimed ones."""
        import torch
        tq, gen, w = self.tq, self.gen, self.w
        tok = torch.empty((self.Lx, w.H, 1, w.D), dtype=torch.float16, device=self.dev)
        for i, name in enumerate(("K", "V")):
            for l in range(w.L):
                tok[i * w.L + l] = gen.kv_layer(w.seed + 100, name, w.spec, l, w.H, 1, w.D, device=self.dev)
        q = gen.queries(w.seed, w.L, HQ, w.D, device=self.dev)
        scores = torch.empty((w.L, HQ, w.T), dtype=torch.float32, device=self.dev)
        kc, kn = self.codes[: w.L], self.norms[: w.L]
        scale = 1.0 / math.sqrt(w.D)
        res = {"workload": f"the headline cache: append of one token into row {w.T - 1} of every K and V "
                           f"layer; q.K of {HQ} query heads over the {w.L} layers' keys"}
        for name, nbytes, fn in (
                ("append_kv", codec_bytes(self.Lx * w.H, self.bits),
                 lambda: tq.tq_encode(self.bits, tok, self.codes, self.norms, w.T - 1)),
                ("qk", qk_bytes(w.L, w.H, w.T, 1, HQ, self.bits),
                 lambda: tq.tq_qk_scores(self.bits, kc, kn, q, scale, scores))):
            us = time_back_to_back(fn, self.stream, reps)
            res[name] = {"us": round(us, 2), "bytes": nbytes, "GBps": round(gbs(nbytes, us), 1),
                         "frac_of_hbm_peak": round(gbs(nbytes, us) / HBM_PEAK_GBS, 4)}
            if name == "append_kv":   # a launch-latency-bound call: its kernel alone too
                res[name]["kernel_median_us"] = round(launch_median(tq, fn, reps), 2)
        del tok, q, scores
        return res

    def records(self, reps=10):
        """The same turbo3 cache through tq_pack_records and back (1.26 GB each way)."""
        import torch
        tq = self.tq
        rec = torch.empty(self.nblk * (2 + 16 * self.bits), dtype=torch.uint8, device=self.dev)
        nb = 2 * self.nblk * (2 + 16 * self.bits)
        res = {}
        for name, fn in (("pack", lambda: tq.tq_pack_records(self.bits, self.codes, self.norms, rec)),
                         ("unpack", lambda: tq.tq_unpack_records(self.bits, rec, self.codes, self.norms))):
            us = time_back_to_back(fn, self.stream, reps)
            res[name] = {"us": round(us, 1), "bytes": nb, "GBps": round(gbs(nb, us), 1),
                         "frac_of_hbm_peak": round(gbs(nb, us) / HBM_PEAK_GBS, 4)}
        del rec
        return res

    def cpu_baseline(self, threads):
        """The CPU oracle, untuned, on a bounded sample of the same workload: whole K and V
        layers of the same cache ([8, 32768, 128] each, host copies of the GPU's inputs),
        turbo3 encode then decode, layer after layer until at least CPU_MIN_SECONDS of
        oracle time; only the oracle calls are timed."""
        import numpy as np

        import oracle
        host_cores = len(os.sched_getaffinity(0))
        if threads <= 0:
            threads = host_cores
        w, bits = self.w, self.bits
        m = w.D // 128
        el, nlayers = 0.0, 0
        order = [i * w.L + l for l in range(w.L) for i in (0, 1)]   # K0, V0, K1, V1, ...
        for li in order:
            xl = self.x[li:li + 1].cpu().numpy()
            c = np.zeros((1, w.H, w.T, m, 16 * bits), np.uint8)
            n = np.zeros((1, w.H, w.T, m), np.float16)
            t0 = time.perf_counter()
            oracle.encode(bits, xl, c, n, nthreads=threads)
            oracle.decode(bits, c, n, 0, w.T, nthreads=threads)
            el += time.perf_counter() - t0
            nlayers += 1
            del xl, c, n
            if el >= CPU_MIN_SECONDS:
                break
        nblk = nlayers * w.H * w.T * m
        nbytes = 2 * codec_bytes(nblk, bits)
        return {"value": round(nbytes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
                "host_cores": host_cores, "cpus_online": os.cpu_count(),
                "kind": "oracle", "seconds": round(el, 2), "cpu": cpu_model(),
                "Gvalues_per_s": round(2 * nblk * 128 / el / 1e9, 4),
                "sample": f"{nlayers} of the {self.Lx} K/V layer tensors [{w.H}, {w.T}, {w.D}] of the "
                          f"same cache (host copies of the same inputs), turbo3 encode then decode, "
                          f"until at least {CPU_MIN_SECONDS:.0f} s of oracle time"}

    def free(self):
        import torch
        del self.x, self.y, self.codes, self.norms, self.ops
        torch.cuda.empty_cache()


def time_back_to_back(fn, stream, reps, settle_s=SETTLE_S):
    """Average microseconds of `reps` back-to-back calls between two events (the queue
    never drains, so host launch latency stays hidden), after `settle_s` seconds of the
    same calls untimed: as for the headline steps, the clocks settle under the call's own
    sustained load first (launched right after a different kind of load, a kernel's first
    milliseconds run at the clocks the power manager set for that load)."""
    import torch
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t_settle >= settle_s:
            break
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def launch_median(tq, fn, reps):
    """Median microseconds of one kernel launch measured by the launch itself (the events
    recorded from its dispatch packet, tq_time_next_launch), over `reps` launches issued
    back to back after two untimed: the kernel's own duration, without the host's launch
    latency.  fn must launch exactly one kernel."""
    import statistics
    import torch
    fn()
    fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:   # torch creates an event's HIP event at its first record
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for e0, e1 in ev:
        tq.tq_time_next_launch(e0, e1)
        fn()
    torch.cuda.synchronize()
    return statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)


def copy_calibration(dev):
    """Three plain 256 MiB device copies: a kernel of known traffic for scaling the
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "full_cache_14b_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "kv_cache_quantization_block_amd", "csrc", f)
                  for f in ("kernels.hip", "internal.h")]


def kernel_code_sha() -> str:
    """First 16 hex digits of the sha256 of the kernels' code (kernels.hip, internal.h):
    comments removed and every run of whitespace made one space, so an edit of comments
    or layout alone does not count as a change of the kernels."""
    import hashlib
    import re
    src = "".join(open(f, encoding="utf-8").read() for f in KERNEL_SOURCES)
    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)
    code = tok.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", src)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()[:16]


def read_summary(path: str) -> dict:
    """key: value lines of a committed profile summary (# starts a comment)."""
    rec = {}
    if not os.path.exists(path):
        return rec
    for line in open(path):
        line = line.split("#")[0].strip()
        if ":" in line:
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    return rec


def measured_traffic(kernel: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch of op `kernel` (encode_turbo3, decode_turbo3) at the headline
    size from the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE scaled by
    a copy of known size), or None when the summary does not cover this op or the kernel
    source changed since it was taken."""
    rec = read_summary(path)
    if rec.get("kernel_code_sha256_16") != kernel_code_sha() or f"{kernel}.fetch_size_kib" not in rec:
        return None
    copy_kib = int(rec["copy_bytes"]) / 1024
    fetch = float(rec[f"{kernel}.fetch_size_kib"]) * copy_kib / float(rec["copy_fetch_size_kib"])
    write = float(rec[f"{kernel}.write_size_kib"]) * copy_kib / float(rec["copy_write_size_kib"])
    return int(round((fetch + write) * 1024))


ISSUE_FILES = {"qk": os.path.join(PROFILES, "qk_decode_step_counters.txt"),
               "attn": os.path.join(PROFILES, "attn_partial_decode_step_counters.txt")}


def issue_utilisation(which: str):
    """Issue-port utilisation of the decode-step q.K ("qk") or attention partials
    ("attn") from the committed rocprofv3 counter summary, or None when the kernel
    source changed since it was taken.  Fractions of the kernel's cycles (GRBM_GUI_ACTIVE
    over the 8 XCDs): VALU per SIMD and LDS per CU from SQ_ACTIVE_INST_* (4-cycle units),
    the matrix core per SIMD from SQ_INSTS_MFMA at 16 cycles each."""
    rec = read_summary(ISSUE_FILES[which])
    if not rec or rec.get("kernel_code_sha256_16") != kernel_code_sha():
        return None
    cyc = float(rec["GRBM_GUI_ACTIVE"]) / 8
    return {"valu_per_simd": round(float(rec["SQ_ACTIVE_INST_VALU"]) * 4 / 1024 / cyc, 3),
            "lds_per_cu": round(float(rec["SQ_ACTIVE_INST_LDS"]) * 4 / 256 / cyc, 3),
            "mfma_per_simd": round(float(rec["SQ_INSTS_MFMA"]) * 16 / 1024 / cyc, 3),
            "source": os.path.relpath(ISSUE_FILES[which], ROOT)}


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
    med = {name: time_back_to_back(fn, stream, reps) for name, fn in ops}
    qb = qk_bytes(B, Hkv, T_, 1, Hq, bits)
    ab = attn_bytes(B, Hkv, T_, Hq, bits)
    out = {"workload": f"{B} sequences x {Hkv} kv heads x {T_} rows x {D_}, {Hq} query heads, turbo3",
           "qk_us": round(med["qk"], 2), "qk_bytes": qb,
           "qk_GBps": round(gbs(qb, med["qk"]), 1),
           "qk_frac_of_hbm_peak": round(gbs(qb, med["qk"]) / HBM_PEAK_GBS, 4),
           "attn_us": round(med["attn"], 2), "attn_bytes": ab,
           "attn_GBps": round(gbs(ab, med["attn"]), 1),
           "attn_frac_of_hbm_peak": round(gbs(ab, med["attn"]) / HBM_PEAK_GBS, 4),
           "append_kv_us": round(med["append_kv"], 2),
           # the K append's own kernel duration (128 blocks), without host launch latency
           "append_kernel_us": round(launch_median(
               tq, lambda: tq.tq_encode(bits, tok["K"], kc, kn, T_ - 1), reps), 2),
           # issue-port utilisation from the committed counters (what binds a kernel
           # that runs below the HBM roofline)
           "qk_issue": issue_utilisation("qk"), "attn_issue": issue_utilisation("attn")}
    del kc, kn, vc, vn, scores, attn, ws
    torch.cuda.empty_cache()
    return out


def head_dim_256(tq, gen, dev, stream, reps=10):
    """turbo2 encode then decode of a whole head_dim-256 cache (32 layers x 4 kv heads x
    32768 x 256, K and V as one [64, 4, 32768, 256] tensor, 4.3 GB of fp16), average of
    `reps` back-to-back launches per op after 0.2 s of untimed ones; then the fused read over
    the same cache: its 32 K layers as a batch of 32 sequences (16 query heads, GQA 4),
    q.K over all 32768 rows and the decode attention over the K and V layers."""
    import torch
    w = gen.WORKLOADS["head_dim_256"]
    bits = 2
    Lx = 2 * w.L
    x = torch.empty((Lx, w.H, w.T, w.D), dtype=torch.float16, device=dev)
    for i, name in enumerate(("K", "V")):
        for l in range(w.L):
            x[i * w.L + l] = gen.kv_layer(w.seed, name, w.spec, l, w.H, w.T, w.D, device=dev)
    codes, norms = tq.empty_cache(bits, Lx, w.H, w.T, w.D, dev)
    y = torch.empty_like(x)
    nblk = x.numel() // 128
    nb = codec_bytes(nblk, bits)
    res = {"workload": f"{w.L} layers x {w.H} kv heads x {w.T} x {w.D}, K and V, turbo{bits}"}
    for op, fn in (("encode", lambda: tq.tq_encode(bits, x, codes, norms, 0)),
                   ("decode", lambda: tq.tq_decode(bits, codes, norms, 0, y))):
        for _ in range(8):   # clocks at their sustained level
            fn()
        us = time_back_to_back(fn, stream, reps)
        res[op] = {"us": round(us, 1), "bytes": nb, "GBps": round(gbs(nb, us), 1),
                   "frac_of_hbm_peak": round(gbs(nb, us) / HBM_PEAK_GBS, 4),
                   "Gvalues_per_s": round(nblk * 128 / (us * 1e-6) / 1e9, 1)}
    del x, y
    B, Hkv, T_, D_, Hq = w.L, w.H, w.T, w.D, 4 * w.H
    m = D_ // 128
    kc, kn, vc, vn = codes[: w.L], norms[: w.L], codes[w.L:], norms[w.L:]
    q = gen.queries(w.seed, B, Hq, D_, device=dev)
    scores = torch.empty((B, Hq, T_), dtype=torch.float32, device=dev)
    attn = torch.empty((B, Hq, D_), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_attn_workspace_bytes(bits, B, Hkv, T_, D_, T_, Hq), dtype=torch.uint8,
                     device=dev)
    scale = 1.0 / math.sqrt(D_)
    for name, nbytes, fn in (
            ("qk", qk_bytes(B, Hkv, T_, m, Hq, bits),
             lambda: tq.tq_qk_scores(bits, kc, kn, q, scale, scores)),
            ("attn", attn_bytes(B, Hkv, T_, Hq, bits, m),
             lambda: tq.tq_attn_decode(bits, kc, kn, vc, vn, q, scale, attn, workspace=ws))):
        us = time_back_to_back(fn, stream, reps)
        res[name] = {"workload": f"the {B} K layers as {B} sequences x {Hkv} kv heads x {T_} rows x "
                                 f"{D_}, {Hq} query heads" + (", V layers as values" if name == "attn" else ""),
                     "us": round(us, 2), "bytes": nbytes, "GBps": round(gbs(nbytes, us), 1),
                     "frac_of_hbm_peak": round(gbs(nbytes, us) / HBM_PEAK_GBS, 4)}
    del codes, norms, q, scores, attn, ws
    torch.cuda.empty_cache()
    return res


FLUSH_BYTES = 512 << 20   # twice the 256 MB Infinity Cache


def one_layer(tq, gen, dev, stream, reps=20):
    """One layer, K and V [8, 32768, 128] as one [2, 8, 32768, 128] tensor, through every
    op of the codec: turbo3 and turbo2 encode and decode (each type its own copy of the
    inputs and outputs), the 1-token append of K and V, q.K of 32 query heads, the
    randomised rotation H D (seeded signs) and the interleaved records.  Each op `reps`
    times back to back ("ops"), and alone with a cold Infinity Cache ("ops_cold": before
    each of `reps` launches a 512 MiB buffer is written; the op's kernel records its own
    start and stop from its dispatch, tq_time_next_launch).  At this size every launch
    is about 30 us, so ramp and tail weigh more than on whole caches."""
    import numpy as np
    import torch
    w = gen.WORKLOADS["one_layer"]
    H, T, D = w.H, w.T, w.D
    m = D // 128
    KV = torch.empty((2, H, T, D), dtype=torch.float16, device=dev)
    KV[0] = gen.kv_layer(w.seed, "K", w.spec, 0, H, T, D, device=dev)
    KV[1] = gen.kv_layer(w.seed, "V", w.spec, 0, H, T, D, device=dev)
    q = gen.queries(w.seed, 1, HQ, D, device=dev)
    tok = torch.empty((2, H, 1, D), dtype=torch.float16, device=dev)
    tok[0] = gen.kv_layer(w.seed + 100, "K", w.spec, 0, H, 1, D, device=dev)
    tok[1] = gen.kv_layer(w.seed + 100, "V", w.spec, 0, H, 1, D, device=dev)
    bufs = {bits: dict(x=KV.clone(), c=tq.empty_cache(bits, 2, H, T, D, dev), o=torch.empty_like(KV))
            for bits in (3, 2)}
    scores = torch.empty((1, HQ, T), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    nblk = 2 * H * T * m
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
    ops.append(("append_turbo3", codec_bytes(2 * H * m, 3), lambda: tq.tq_encode(3, tok, c3, n3, T - 1)))
    ops.append(("qk_turbo3", qk_bytes(1, H, T, m, HQ, 3),
                lambda: tq.tq_qk_scores(3, c3[0:1], n3[0:1], q, scale, scores)))
    # the signs as the library's four words, converted once (as a serving loop would)
    signs = tq.sign_words(np.where(np.random.default_rng(w.seed).random(128) < 0.5, -1.0, 1.0))
    b3 = bufs[3]
    rec = torch.empty(nblk * 50, dtype=torch.uint8, device=dev)
    extra_ops = [
        ("encode_turbo3_rot", codec_bytes(nblk, 3), lambda: tq.tq_encode(3, b3["x"], *b3["c"], 0, signs=signs)),
        ("decode_turbo3_rot", codec_bytes(nblk, 3), lambda: tq.tq_decode(3, *b3["c"], 0, b3["o"], signs=signs)),
        ("pack_records_turbo3", 2 * nblk * 50, lambda: tq.tq_pack_records(3, *b3["c"], rec)),
        ("unpack_records_turbo3", 2 * nblk * 50, lambda: tq.tq_unpack_records(3, rec, *b3["c"]))]
    # settle the clocks with whole passes over the ops
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _, _, fn in ops:
            fn()
        torch.cuda.synchronize()
    per_op = {}
    for name, nbytes, fn in ops + extra_ops:
        us = time_back_to_back(fn, stream, reps)
        per_op[name] = {"us": round(us, 2), "bytes": nbytes, "GBps": round(gbs(nbytes, us), 1),
                        "frac_of_hbm_peak": round(gbs(nbytes, us) / HBM_PEAK_GBS, 4)}
    # cold Infinity Cache: every op alone after a 512 MiB buffer write
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)   # creates the events the hook records on
    e1.record(stream)
    cold = {}
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
        cold[name] = {"median_us": round(med, 2), "min_us": round(times[0], 2), "bytes": nbytes,
                      "GBps": round(gbs(nbytes, med), 1),
                      "frac_of_hbm_peak": round(gbs(nbytes, med) / HBM_PEAK_GBS, 4)}
    codec = [k for k in cold if k.startswith(("encode_", "decode_"))]
    nb = sum(cold[k]["bytes"] for k in codec)
    us = sum(cold[k]["median_us"] for k in codec)
    cold["encode_decode_combined"] = {"ops": codec, "bytes": nb, "us": round(us, 2),
                                      "GBps": round(gbs(nb, us), 1),
                                      "frac_of_hbm_peak": round(gbs(nb, us) / HBM_PEAK_GBS, 4)}
    del scratch, KV, bufs, rec, scores
    torch.cuda.empty_cache()
    return {"workload": "K,V fp16 [8 kv_heads, 32768 tokens, 128] as one [2, 8, 32768, 128] tensor",
            "ops": per_op, "ops_cold": cold}


def copy_bandwidth(dev, stream, nbytes=512 << 20, reps=10):
    """Context for the roofline: what a plain device-to-device copy of 512 MiB (torch's
    copy kernel, read + write counted) reaches on this GPU, HIP events around `reps`
    back-to-back copies after 0.2 s of untimed ones."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    us = time_back_to_back(lambda: dst.copy_(src), stream, reps)
    g = 2 * nbytes / (us * 1e-6) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"what": "device-to-device copy, 512 MiB read + 512 MiB written", "us": round(us, 1),
            "GBps": round(g, 1), "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
