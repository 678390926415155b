"""GPU parity at the size and position limits, through the C ABI, against the
fp64 oracle.

* A 2^20-token causal prefill (W=4096, d=64): sampled rows at the start, on
  tile and block boundaries and at the very end.
* 2^20 tokens with global tokens: global rows over every key (8192 key
  splits merged) and the rows beside them.
* Positions near 2^31 - 1: ring append, decode, multi-token append and a
  chunked prefill whose chunk ends at position 2^31 - 2; decode with sinks far
  into the sequence.
"""

import math

import numpy as np
import pytest

import oracle
import swa_inputs as si
from helpers import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

P_MAX = 2**31 - 2  # a position whose successor still fits int32


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sliding_window_attention_swa_amd as m
    m.load()
    return m


def test_million_token_prefill_sampled(swa):
    T, W, d = 2**20, 4096, 64
    print("prefill T=%d W=%d d=%d" % (T, W, d), flush=True)
    q, k, v = si.prefill_inputs(3, B=1, Hq=2, Hkv=1, T=T, d=d)
    out = swa.prefill(to_device(q), to_device(k), to_device(v), W)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 127, 128, 4095, 4096, 4097, T // 2 + 5, T - 129, T - 128,
                     T - 2, T - 1])
    for h in range(2):
        ref = oracle.attention_rows(q.values, k.values, v.values, W, 0, 1 / math.sqrt(d), 0, h, rows)
        got = out[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        assert_parity(got, ref, "bf16", "T=2^20 head %d" % h)


def test_million_token_global_rows(swa):
    """2^20 tokens, symmetric W=512, d=64, global tokens at the start, the
    middle and the end: each global row attends to all 2^20 keys (8192 key
    splits of the matrix-core rows pass, merged), and rows next to them see
    their window plus the global keys."""
    T, W, d = 2**20, 512, 64
    gpos = np.array([0, 1000, 2**19, T - 1], dtype=np.int32)
    print("global rows T=%d W=%d d=%d G=%d" % (T, W, d, len(gpos)), flush=True)
    q, k, v = si.prefill_inputs(9, B=1, Hq=2, Hkv=1, T=T, d=d)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), W,
                             torch.from_numpy(gpos).cuda(), mode=si.SYMMETRIC)
    torch.cuda.synchronize()
    rows = np.array(list(gpos) + [1, 999, 1001, 2**19 + 300, T - 2], dtype=np.int64)
    for h in range(2):
        ref = oracle.attention_global_rows(q.values, k.values, v.values, W, si.SYMMETRIC,
                                           1 / math.sqrt(d), gpos, 0, h, rows)
        got = out[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        assert_parity(got, ref, "bf16", "T=2^20 global rows head %d" % h)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_near_the_largest_position(swa, dtype):
    B, Hq, Hkv, W, d = 4, 8, 2, 300, 64
    pos = np.array([P_MAX, P_MAX - 4097, W - 1, 0], dtype=np.int32)
    q = si.normal(141, (B, Hq, d), dtype)
    kr, vr = si.normal(142, (B, Hkv, W, d), dtype), si.normal(143, (B, Hkv, W, d), dtype)
    out = swa.decode(to_device(q), to_device(kr), to_device(vr), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ref = oracle.decode(q.values, kr.values, vr.values, pos, 1 / math.sqrt(d))
    assert_parity(to_f64(out), ref, dtype, "decode at large positions")


def test_append_near_the_largest_position(swa):
    B, Hkv, W, n, d = 2, 2, 37, 50, 64
    pos = np.array([P_MAX - n + 1, 2**30], dtype=np.int32)  # chunk 0 ends at P_MAX
    k, v = si.normal(144, (B, Hkv, n, d), "bf16"), si.normal(145, (B, Hkv, n, d), "bf16")
    kr0, vr0 = si.normal(146, (B, Hkv, W, d), "bf16"), si.normal(147, (B, Hkv, W, d), "bf16")
    kr, vr = to_device(kr0), to_device(vr0)
    swa.cache_append_chunk(kr, vr, torch.from_numpy(pos).cuda(), to_device(k), to_device(v))
    one = torch.from_numpy(pos + n).cuda()  # one more token after each chunk: 2^31 - 1 for sequence 0
    k1, v1 = si.normal(148, (B, Hkv, d), "bf16"), si.normal(149, (B, Hkv, d), "bf16")
    swa.cache_append(kr, vr, one, to_device(k1), to_device(v1))
    torch.cuda.synchronize()
    want_k, want_v = kr0.bits.copy(), vr0.bits.copy()
    oracle.ring_append_chunk(want_k, want_v, pos, k.bits, v.bits)
    oracle.ring_append(want_k, want_v, one.cpu().numpy(), k1.bits, v1.bits)
    assert np.array_equal(kr.cpu().view(torch.int16).numpy(), want_k.view(np.int16))
    assert np.array_equal(vr.cpu().view(torch.int16).numpy(), want_v.view(np.int16))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_prefill_ending_at_the_largest_position(swa, dtype):
    B, Hq, Hkv, n, W, d = 2, 4, 2, 200, 300, 64
    pos = np.array([P_MAX - n + 1, 2**30 + 3], dtype=np.int32)
    q, k, v, kr, vr, _ = si.chunk_inputs(6, B=B, Hq=Hq, Hkv=Hkv, n=n, W=W, d=d, dtype=dtype)
    out = swa.prefill_chunk(to_device(q), to_device(k), to_device(v), to_device(kr), to_device(vr),
                            torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk(q.values, k.values, v.values, kr.values, vr.values, pos, W,
                               1 / math.sqrt(d))
    assert_parity(to_f64(out), ref, dtype, "chunk ending at P_MAX")


def test_decode_sinks_far_into_the_sequence(swa):
    B, Hq, Hkv, W, d, S = 2, 8, 2, 128, 128, 4
    pos = np.array([P_MAX, 10**9], dtype=np.int32)
    q = si.normal(150, (B, Hq, d), "bf16")
    kr, vr = si.normal(151, (B, Hkv, W, d), "bf16"), si.normal(152, (B, Hkv, W, d), "bf16")
    ks, vs = si.normal(153, (B, Hkv, S, d), "bf16"), si.normal(154, (B, Hkv, S, d), "bf16")
    out = swa.decode_sinks(to_device(q), to_device(kr), to_device(vr), to_device(ks), to_device(vs),
                           torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ref = oracle.decode_sinks(q.values, kr.values, vr.values, ks.values, vs.values, pos,
                              1 / math.sqrt(d))
    assert_parity(to_f64(out), ref, "bf16", "decode with sinks far into the sequence")
