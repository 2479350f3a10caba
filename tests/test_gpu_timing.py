"""The timing hook on the GPU: the next launch records its own dispatch on the
caller's events, and only that launch."""
import pytest
import torch

import gen
import kv_cache_quantization_block_amd as tq

pytestmark = pytest.mark.gpu


def test_time_next_launch_times_one_decode():
    x = gen.kv_tensor(3, "K", gen.KVSpec(), 2, 8, 4096, 128).cuda()
    codes, norms = tq.empty_cache(3, 2, 8, 4096, 128)
    tq.tq_encode(3, x, codes, norms)
    out = torch.empty_like(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    tq.tq_time_next_launch(e0, e1)
    tq.tq_decode(3, codes, norms, 0, out)
    torch.cuda.synchronize()
    t1 = e0.elapsed_time(e1)
    # 65,536 blocks: about 20 MB, a few microseconds to some tens at any clock
    assert 1e-4 < t1 < 5.0, t1
    # the hook cleared itself: further launches leave the events as they were
    for _ in range(3):
        tq.tq_decode(3, codes, norms, 0, out)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == t1
    # and the decode it timed is the one that produced the output
    ref = torch.empty_like(x)
    tq.tq_decode(3, codes, norms, 0, ref)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
