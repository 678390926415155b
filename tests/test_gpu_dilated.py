"""GPU parity of the dilated window (swa_prefill_dilated), through the C ABI,
against the fp64 oracle.

* Small and ragged shapes, both modes, dilations 2 to 9 (also larger than the
  sequence, so some residue classes are empty), windows shorter and longer
  than a tile, GQA, d in {32, 64, 128}, bf16 and fp32, element by element.
* dilation 1 gives bit-for-bit the output of swa_prefill.
* The Longformer workload of the page's example (symmetric W=512, dilation
  2, B=4, T=4096, 12 heads, d=64), in the launch configuration the benchmark
  times, on sampled rows of every sequence.
"""

import math

import numpy as np
import pytest

import oracle
import swa_inputs as si
from helpers import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sliding_window_attention_swa_amd as m
    m.load()
    return m


DILATED_SMALL = [
    # (mode, T, W, dil, B, Hq, Hkv, d)
    (0, 300, 8, 2, 1, 2, 1, 64),
    (1, 300, 8, 2, 2, 4, 2, 64),
    (0, 257, 64, 2, 1, 4, 1, 128),     # one class one row longer than the other
    (1, 1000, 33, 3, 1, 2, 2, 32),
    (0, 5, 3, 7, 2, 2, 1, 64),         # dilation above T: empty classes
    (1, 5, 4, 7, 1, 2, 2, 128),
    (0, 700, 100, 5, 1, 6, 3, 64),
    (1, 700, 100, 5, 1, 2, 1, 32),
    (0, 390, 200, 3, 2, 2, 2, 128),
    (1, 129, 1, 9, 1, 2, 1, 64),       # W = 1 symmetric: self only
    (0, 520, 512, 2, 1, 2, 1, 64),     # window wider than a class
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,T,W,dil,B,Hq,Hkv,d", DILATED_SMALL)
def test_dilated_small(swa, dtype, mode, T, W, dil, B, Hq, Hkv, d):
    print("dilated", dtype, dict(mode=mode, T=T, W=W, dil=dil, B=B, Hq=Hq, Hkv=Hkv, d=d), flush=True)
    q, k, v = si.prefill_inputs(7, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, dtype=dtype)
    scale = 1 / math.sqrt(d)
    out = swa.prefill_dilated(to_device(q), to_device(k), to_device(v), W, dil, mode=mode)
    torch.cuda.synchronize()
    ref = oracle.attention_dilated_dense(q.values, k.values, v.values, W, mode, scale, dil)
    assert_parity(to_f64(out), ref, dtype, "dilated")


@pytest.mark.parametrize("mode,W", [(0, 40), (1, 40), (0, 20)])
def test_dilation_one_is_prefill_bit_for_bit(swa, mode, W):
    q, k, v = (to_device(t) for t in si.prefill_inputs(7, B=1, Hq=4, Hkv=2, T=333, d=64))
    a = swa.prefill(q, k, v, W, mode=mode)
    b = swa.prefill_dilated(q, k, v, W, 1, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_longformer_dilated_sampled(swa):
    """B=4, T=4096, symmetric W=512 at dilation 2, 12 heads, d=64: sampled
    rows (both residue classes, both sequence ends) vs the oracle; every
    output finite."""
    cfg = si.WORKLOADS[7]
    q, k, v = si.prefill_inputs(7)
    out = swa.prefill_dilated(to_device(q), to_device(k), to_device(v), cfg["W"], cfg["dilation"],
                              mode=cfg["mode"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    got = to_f64(out)
    rows = [0, 1, 2, 511, 512, 513, 1000, 2047, 2048, 4094, 4095]
    scale = 1 / math.sqrt(cfg["d"])
    for b in range(cfg["B"]):
        for h in (0, 7, 11):
            ref = oracle.attention_dilated_rows(q.values, k.values, v.values, cfg["W"], cfg["mode"],
                                                scale, cfg["dilation"], b, h, rows)
            assert_parity(got[b, h, rows], ref, "bf16", "longformer dilated b=%d h=%d" % (b, h))
