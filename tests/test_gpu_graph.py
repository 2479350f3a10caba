"""The entry points under HIP graph capture (GPU): an append + q.K + decode attention
+ record repack step captured once into a graph (torch.cuda.CUDAGraph, which records
through hipStreamBeginCapture on the capturing stream) and replayed several times,
with eager work of the program between replays; every replay must reproduce the eager
results exactly.  None of these calls allocates or issues a memset, so all of them
record as plain kernel nodes."""
import math

import pytest
import torch

import gen
import kv_cache_quantization_block_amd as tq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    tq.lib()


@pytest.mark.parametrize("bits", [3, 2])
def test_decode_step_graph_replays_match_eager(bits):
    B, Hkv, G, Tc, D = 2, 4, 4, 1000, 128
    T = Tc - 1
    spec = gen.KVSpec(n_outliers=3, row_scale=True)
    k = gen.kv_tensor(61, "K", spec, B, Hkv, Tc, D).cuda()
    v = gen.kv_tensor(61, "V", spec, B, Hkv, Tc, D).cuda()
    q = gen.queries(62, B, Hkv * G, D).cuda()
    kc, kn = tq.empty_cache(bits, B, Hkv, Tc, D)
    vc, vn = tq.empty_cache(bits, B, Hkv, Tc, D)
    tq.tq_encode(bits, k[:, :, :T].contiguous(), kc, kn, 0)
    tq.tq_encode(bits, v[:, :, :T].contiguous(), vc, vn, 0)
    k_tok, v_tok = k[:, :, T:].contiguous(), v[:, :, T:].contiguous()
    scale = 1.0 / math.sqrt(D)
    scores = torch.empty((B, Hkv * G, Tc), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_attn_workspace_bytes(bits, B, Hkv, Tc, D, Tc, Hkv * G), dtype=torch.uint8,
                     device="cuda")
    rec = torch.empty(kn.numel() * (2 + 16 * bits), dtype=torch.uint8, device="cuda")
    caches = (kc, kn, vc, vn)
    snap = [t.clone() for t in caches]

    def step():
        tq.tq_encode(bits, k_tok, kc, kn, T)
        tq.tq_encode(bits, v_tok, vc, vn, T)
        tq.tq_qk_scores(bits, kc, kn, q, scale, scores)
        tq.tq_attn_decode(bits, kc, kn, vc, vn, q, scale, out, workspace=ws)
        tq.tq_pack_records(bits, kc, kn, rec)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (scores, out, rec, kc, kn, vc, vn)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):   # warm up on the capture stream
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        # eager work of the program between replays: clobber every output and
        # restore the caches' prefilled rows
        for t in (scores, out, rec):
            t.fill_(0)
        for t, s0 in zip(caches, snap):
            t.copy_(s0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (scores, out, rec, kc, kn, vc, vn)
        for name, a, b in zip(("scores", "out", "records", "k codes", "k norms", "v codes", "v norms"),
                              got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r}: {name} differs"
