"""GPU parity of the dilated window plus global tokens
(swa_prefill_dilated_global, through the C ABI) against the fp64 oracle:
small shapes in bf16 and fp32 (causal and symmetric, dilations 2 to 5,
global tokens inside and outside the rows' dilated windows, ragged residue
classes, grouped heads, batches) and the Longformer shapes with the rows
sampled."""

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


SMALL = [
    # (mode, T, W, dil, gpos, B, Hq, Hkv, d)
    (1, 300, 16, 2, [0, 1, 150], 1, 2, 1, 64),
    (0, 300, 16, 2, [0, 7, 299], 1, 4, 2, 64),
    (1, 257, 9, 3, [0, 3, 6, 100, 255, 256], 2, 2, 2, 128),
    (0, 511, 40, 3, list(range(0, 511, 7)), 1, 2, 1, 32),   # 73 global keys: two global tiles
    (1, 700, 33, 5, [5, 10, 350, 699], 1, 6, 3, 64),
    (0, 129, 300, 2, [64], 2, 2, 1, 128),                     # window longer than each class
    (1, 64, 1, 4, [0, 63], 1, 2, 1, 64),                      # W = 1: self plus globals
    (1, 37, 5, 40, [0, 36], 1, 2, 1, 64),                     # dilation > T: one-row classes
    (0, 50, 9, 49, [3, 49], 1, 4, 2, 128),                    # dilation T - 1
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,T,W,dil,gpos,B,Hq,Hkv,d", SMALL)
def test_dilated_global_small(swa, dtype, mode, T, W, dil, gpos, B, Hq, Hkv, d):
    print("dilated global", dtype, dict(mode=mode, T=T, W=W, dil=dil, G=len(gpos), B=B, Hq=Hq,
                                        Hkv=Hkv, d=d), flush=True)
    gpos = np.array(gpos, dtype=np.int32)
    q, k, v = si.prefill_inputs(9, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, dtype=dtype)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), W,
                             torch.from_numpy(gpos).cuda(), mode=mode, dilation=dil)
    torch.cuda.synchronize()
    ref = oracle.attention_global_dense(q.values, k.values, v.values, W, mode, 1 / math.sqrt(d),
                                        gpos, dil)
    assert_parity(to_f64(out), ref, dtype, "dilated global")


def test_no_global_is_dilated_and_dilation_one_is_global(swa):
    q, k, v = (to_device(t) for t in si.prefill_inputs(9, B=1, Hq=4, Hkv=2, T=333, d=64))
    none = torch.zeros(0, dtype=torch.int32, device="cuda")
    a = swa.prefill_dilated(q, k, v, 40, 3, mode=1)
    b = swa.prefill_global(q, k, v, 40, none, mode=1, dilation=3)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    g = torch.tensor([0, 100, 332], dtype=torch.int32, device="cuda")
    c = swa.prefill_global(q, k, v, 40, g, mode=0)
    e = swa.prefill_global(q, k, v, 40, g, mode=0, dilation=1)
    torch.cuda.synchronize()
    assert torch.equal(c, e)


def test_longformer_dilated_global_sampled(swa):
    """B=4, T=4096, symmetric W=512 at dilation 2, 12 heads, d=64, global
    tokens 0..7: the global rows and sampled rows of both residue classes."""
    cfg = si.WORKLOADS[9]
    q, k, v = si.prefill_inputs(9)
    gpos = np.array(cfg["global_pos"], dtype=np.int32)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), cfg["W"],
                             torch.from_numpy(gpos).cuda(), mode=cfg["mode"],
                             dilation=cfg["dilation"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    got = to_f64(out)
    rows = list(gpos) + [8, 9, 255, 256, 513, 514, 515, 1000, 2047, 2048, 4094, 4095]
    scale = 1 / math.sqrt(cfg["d"])
    for b in range(cfg["B"]):
        for h in (0, 11):
            ref = oracle.attention_global_rows(q.values, k.values, v.values, cfg["W"], cfg["mode"],
                                               scale, gpos, b, h, rows, cfg["dilation"])
            assert_parity(got[b, h, rows], ref, "bf16", "longformer dilated global b=%d h=%d" % (b, h))
