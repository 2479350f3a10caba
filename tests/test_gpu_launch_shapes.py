"""Launch shapes (GPU): the codec's results do not depend on how its grid is shaped.

encode_kernel and decode_kernel take their 32-block tiles either one per wave (the
one-shot grid) or several per wave (a grid capped at some workgroups per compute
unit; the encoder then stores one tile while it loads the next).  All of them use
the one-shot grid by default (the randomised-rotation encode in its build without
the tile loop), and the capped grid only when TQ_ENCODE_GROUPS_PER_CU,
TQ_ENCODE_ROT_GROUPS_PER_CU or TQ_DECODE_GROUPS_PER_CU ask for it, or past 2^22
workgroups.  So:
- in this process, the rotation encode (one tile per wave) is checked against the
  oracle in full;
- a child process whose environment caps the plain grids at one workgroup per CU
  (four tiles per wave) and the rotation encode at two (most waves take two tiles)
  repeats the plain and rotation calls; every output buffer must match this
  process's bit for bit (each block's arithmetic is the same whichever wave does it).
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import _launch_shape_child as child
import gen
import kv_cache_quantization_block_amd as tq
import oracle
from _parity import check_codes, check_decode, check_norms

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    tq.lib()


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("layout", ["contiguous", "offset"])
def test_rot_encode_one_tile_per_wave(bits, layout):
    """4,098 tiles, one per wave, the last one ragged."""
    L, H, T, D = child.L, child.H, child.T, child.D
    Tc, t0 = child.LAYOUTS[layout]
    d = child.signs()
    x = gen.kv_tensor(61, "K", gen.KVSpec(n_outliers=3, row_scale=True), L, H, T, D)
    codes, norms = tq.empty_cache(bits, L, H, Tc, D)
    codes.fill_(child.SENT_CODE)
    norms.fill_(child.SENT_NORM)
    tq.tq_encode(bits, x.cuda(), codes, norms, t0, signs=d)
    y = torch.empty((L, H, T, D), dtype=torch.float16, device="cuda")
    tq.tq_decode(bits, codes, norms, t0, y, signs=d)
    torch.cuda.synchronize()
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    xn = x.numpy()
    oc = np.full(gc.shape, child.SENT_CODE, np.uint8)
    on = np.full(gn.shape, child.SENT_NORM, np.float16)
    dist = oracle.encode(bits, xn, oc, on, t0=t0, want_dist=True, signs=d)
    rows = slice(t0, t0 + T)
    what = f"rot encode, one tile per wave, {layout}"
    st = check_codes(bits, gc[:, :, rows], oc[:, :, rows], dist.reshape(L, H, T, D // 128, 128), what)
    st.update(check_norms(gn[:, :, rows], on[:, :, rows], xn, what))
    assert np.all(gc[:, :, :t0] == child.SENT_CODE) and np.all(gc[:, :, t0 + T:] == child.SENT_CODE)
    assert np.all(gn[:, :, :t0] == child.SENT_NORM) and np.all(gn[:, :, t0 + T:] == child.SENT_NORM)
    ref, _ = oracle.decode(bits, gc, gn, t0, T, signs=d)
    st.update(check_decode(y.cpu().numpy(), ref, what))
    print(st)


def test_other_grid_shapes_give_the_same_bytes():
    here = child.run_all()
    env = dict(os.environ, TQ_ENCODE_GROUPS_PER_CU="1", TQ_DECODE_GROUPS_PER_CU="1",
               TQ_ENCODE_ROT_GROUPS_PER_CU="2")
    print("child: plain grids at one group per CU, rotation encode at two", flush=True)
    r = subprocess.run([sys.executable, os.path.join(HERE, "_launch_shape_child.py")], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    there = json.loads(r.stdout.strip().splitlines()[-1])
    assert there.keys() == here.keys()
    differ = [k for k in here if here[k] != there[k]]
    assert not differ, f"outputs that depend on the grid shape: {differ}"
