"""The calls of test_gpu_launch_shapes, as one function that the test runs both in
its own process and in a child process whose environment shapes the codec grids
differently.  Run as a script it prints one JSON object: the sha256 of every output
buffer, keyed by case.

Cases: turbo3 and turbo2; a cache that holds exactly the encoded rows and one that
holds them at rows [50, 50 + T) of a longer cache (the sentinel bytes around them
must survive); for each, the plain encode and decode and the randomised-rotation
encode and decode.  T = 8195 rows of 2 x 8 heads x 128 values: 131,120 blocks, 4,098
tiles of 32 blocks, the last one ragged.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

L, H, T, D = 2, 8, 8195, 128
LAYOUTS = {"contiguous": (T, 0), "offset": (T + 105, 50)}   # (Tc, t0)
SENT_CODE, SENT_NORM = 0xA5, 7.0


def signs():
    import numpy as np
    return np.where(np.random.default_rng(77).random(128) < 0.5, -1.0, 1.0)


def run_all() -> dict:
    import torch

    import gen
    import kv_cache_quantization_block_amd as tq

    x = gen.kv_tensor(61, "K", gen.KVSpec(n_outliers=3, row_scale=True), L, H, T, D).cuda()
    d = signs()
    out = {}
    for bits in (3, 2):
        for lay, (Tc, t0) in LAYOUTS.items():
            for rot in (False, True):
                s = d if rot else None
                codes, norms = tq.empty_cache(bits, L, H, Tc, D)
                codes.fill_(SENT_CODE)
                norms.fill_(SENT_NORM)
                tq.tq_encode(bits, x, codes, norms, t0, signs=s)
                y = torch.empty((L, H, T, D), dtype=torch.float16, device="cuda")
                tq.tq_decode(bits, codes, norms, t0, y, signs=s)
                torch.cuda.synchronize()
                key = f"turbo{bits}/{lay}/{'rot' if rot else 'plain'}"
                for name, t in (("codes", codes), ("norms", norms), ("decoded", y)):
                    out[f"{key}/{name}"] = hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()
    return out


if __name__ == "__main__":
    print(json.dumps(run_all()), flush=True)
