"""GPU parity of decode with attention sinks (swa_decode_sinks) and of the
per-layer local/global alternation, through the C ABI, against the fp64
oracle.

* Decode with sinks: rings with random contents, sinks inside and before
  the window, wrapped rings, inactive sequences, GQA, bf16 and fp32.
* Serving with sinks: the prompt's prefill with the first S tokens global
  (causal), its K/V appended to the ring and its first S rows kept as sinks,
  then generated tokens decoded with sinks: every output equals the oracle's
  row of the whole sequence under the window-or-sink mask.
* Local/global alternation (Gemma 3: five windowed layers per global one):
  a windowed layer keeps a W-slot ring, a global layer a ring as long as the
  context (W >= T is full causal attention); each layer's prefill and decode
  match the oracle with its own W.
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


SINK_SMALL = [
    # (B, Hq, Hkv, W, d, S, pos)
    (3, 4, 1, 37, 64, 4, [0, 5, 36]),          # sinks inside the window
    (2, 8, 2, 100, 128, 4, [250, 99]),         # before the window / just covered
    (4, 8, 1, 64, 32, 1, [-1, 0, 63, 640]),
    (2, 6, 3, 300, 64, 16, [1000, 150]),
    (1, 32, 8, 4096, 128, 4, [20000]),
    (2, 2, 2, 8, 64, 12, [30, 10]),            # more sinks than window slots
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,W,d,S,pos", SINK_SMALL)
def test_decode_sinks_small(swa, dtype, B, Hq, Hkv, W, d, S, pos):
    print("decode_sinks", dtype, dict(B=B, Hq=Hq, Hkv=Hkv, W=W, d=d, S=S, pos=pos), flush=True)
    q = si.normal(131, (B, Hq, d), dtype)
    kr, vr = si.normal(132, (B, Hkv, W, d), dtype), si.normal(133, (B, Hkv, W, d), dtype)
    ks, vs = si.normal(134, (B, Hkv, S, d), dtype), si.normal(135, (B, Hkv, S, d), dtype)
    pos = np.array(pos, dtype=np.int32)
    out = swa.decode_sinks(to_device(q), to_device(kr), to_device(vr), to_device(ks), to_device(vs),
                           torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = oracle.decode_sinks(q.values, kr.values, vr.values, ks.values, vs.values, pos,
                              1 / math.sqrt(d))
    assert_parity(got, ref, dtype, "decode_sinks")
    for b in np.flatnonzero(pos < 0):
        assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_streaming_with_sinks(swa, dtype):
    """Prompt of 300 tokens (causal W=48, 4 sinks) prefilled, then 200 more
    tokens generated one at a time with sinks beside the 48-slot ring."""
    B, Hq, Hkv, W, d, S, P, T = 2, 8, 2, 48, 64, 4, 300, 500
    q, k, v = si.prefill_inputs(2, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, dtype=dtype)
    sinks = np.arange(S, dtype=np.int32)
    ref = oracle.attention_global_dense(q.values, k.values, v.values, W, si.CAUSAL,
                                        1 / math.sqrt(d), sinks)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    pre = swa.prefill_global(qd[:, :, :P].contiguous(), kd[:, :, :P].contiguous(),
                             vd[:, :, :P].contiguous(), W, torch.from_numpy(sinks).cuda(), mode=0)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kr = torch.zeros((B, Hkv, W, d), dtype=tdt, device="cuda")
    vr = torch.zeros_like(kr)
    swa.cache_append_chunk(kr, vr, torch.zeros(B, dtype=torch.int32, device="cuda"),
                           kd[:, :, :P].contiguous(), vd[:, :, :P].contiguous())
    ks, vs = kd[:, :, :S].contiguous(), vd[:, :, :S].contiguous()
    outs = []
    for p in range(P, T):
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        swa.cache_append(kr, vr, pos, kd[:, :, p].contiguous(), vd[:, :, p].contiguous())
        outs.append(swa.decode_sinks(qd[:, :, p].contiguous(), kr, vr, ks, vs, pos))
    torch.cuda.synchronize()
    assert_parity(to_f64(pre), ref[:, :, :P], dtype, "prompt with sinks")
    assert_parity(np.stack([to_f64(o) for o in outs], axis=2), ref[:, :, P:], dtype,
                  "generation with sinks")


def test_local_and_global_layers(swa):
    """A windowed layer (W=64, 64-slot ring) and a global layer (ring as long
    as the 400-token context) over the same token stream: prefill of a
    256-token prompt, then decode of the rest, each layer against the oracle
    with its own window."""
    B, Hq, Hkv, d, P, T = 1, 8, 2, 128, 256, 400
    layers = [("local", 64), ("global", T)]
    q, k, v = si.prefill_inputs(3, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    for name, W in layers:
        ref = oracle.attention_banded(q.values, k.values, v.values, W, si.CAUSAL, 1 / math.sqrt(d))
        pre = swa.prefill(qd[:, :, :P].contiguous(), kd[:, :, :P].contiguous(),
                          vd[:, :, :P].contiguous(), W)
        kr = torch.zeros((B, Hkv, W, d), dtype=torch.bfloat16, device="cuda")
        vr = torch.zeros_like(kr)
        swa.cache_append_chunk(kr, vr, torch.zeros(B, dtype=torch.int32, device="cuda"),
                               kd[:, :, :P].contiguous(), vd[:, :, :P].contiguous())
        outs = []
        for p in range(P, T):
            pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
            swa.cache_append(kr, vr, pos, kd[:, :, p].contiguous(), vd[:, :, p].contiguous())
            outs.append(swa.decode(qd[:, :, p].contiguous(), kr, vr, pos))
        torch.cuda.synchronize()
        assert_parity(to_f64(pre), ref[:, :, :P], "bf16", "%s prefill" % name)
        assert_parity(np.stack([to_f64(o) for o in outs], axis=2), ref[:, :, P:], "bf16",
                      "%s decode" % name)
