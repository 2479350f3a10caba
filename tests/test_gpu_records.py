"""Interleaved block records on the GPU vs the oracle's byte copies (GPU): pack and
unpack are bit-exact for ragged block counts (one wave tile, several, a ragged last
tile, one block), for a sub-range given by offset pointers, and round trip the
planes of a real encoded cache."""
import numpy as np
import pytest
import torch

import gen
import kv_cache_quantization_block_amd as tq
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    tq.lib()


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("nb", [1, 7, 63, 64, 65, 200, 1000, 4099])
def test_pack_unpack_bit_exact(bits, nb):
    rng = np.random.default_rng(nb * 10 + bits)
    cb = 16 * bits
    codes = rng.integers(0, 256, (nb, cb), dtype=np.uint8)
    norms = rng.integers(0, 1 << 16, nb, dtype=np.uint64).astype(np.uint16).view(np.float16)
    ref = oracle.pack_records(bits, codes, norms)
    # sentinel bytes after the records: nothing past nb records may be written
    rec = torch.full((nb * (cb + 2) + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    gc, gn = torch.from_numpy(codes).cuda(), torch.from_numpy(norms.copy()).cuda()
    tq.tq_pack_records(bits, gc, gn, rec[: nb * (cb + 2)])
    c2 = torch.full((nb, cb), 0x5A, dtype=torch.uint8, device="cuda")
    n2 = torch.full((nb,), 3.0, dtype=torch.float16, device="cuda")
    tq.tq_unpack_records(bits, rec[: nb * (cb + 2)], c2, n2)
    torch.cuda.synchronize()
    r = rec.cpu().numpy()
    assert np.array_equal(r[: nb * (cb + 2)].reshape(nb, cb + 2), ref)
    assert np.all(r[nb * (cb + 2):] == 0xA5)
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(n2.cpu().numpy().view(np.uint16), norms.view(np.uint16))


@pytest.mark.parametrize("bits", [3, 2])
def test_sub_range_and_cache_round_trip(bits):
    """A cache encoded by tq_encode: records of blocks [72, 72 + 300) through offset
    pointers equal the oracle's records of that range; unpacking all records of the
    cache restores both planes exactly."""
    x = gen.kv_tensor(3, "K", gen.KVSpec(n_outliers=3, row_scale=True), 2, 4, 97, 128)
    codes, norms = tq.empty_cache(bits, 2, 4, 97, 128)
    tq.tq_encode(bits, x.cuda(), codes, norms, 0)
    nb = norms.numel()
    cb = 16 * bits
    cf, nf = codes.view(nb, cb), norms.view(nb)
    b0, n = 72, 300
    rec = torch.empty(n * (cb + 2), dtype=torch.uint8, device="cuda")
    tq.tq_pack_records(bits, cf[b0:b0 + n], nf[b0:b0 + n], rec)
    allrec = torch.empty(nb * (cb + 2), dtype=torch.uint8, device="cuda")
    tq.tq_pack_records(bits, cf, nf, allrec)
    c2, n2 = torch.empty_like(cf), torch.empty_like(nf)
    tq.tq_unpack_records(bits, allrec, c2, n2)
    torch.cuda.synchronize()
    ref = oracle.pack_records(bits, cf.cpu().numpy()[b0:b0 + n], nf.cpu().numpy()[b0:b0 + n])
    assert np.array_equal(rec.cpu().numpy().reshape(n, cb + 2), ref)
    assert torch.equal(c2, cf) and torch.equal(n2.view(torch.int16), nf.view(torch.int16))
