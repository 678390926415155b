"""GPU parity of the ring cache (swa_cache_append) and of swa_decode, through
the C ABI, against the fp64 oracle.

* Ring indexing is bit-exact: after appends of positions 0..P (several wraps)
  slot s holds the row of the latest position p <= P with p = s (mod W);
  slots never written keep their fill; negative positions write nothing.
* Decode equals windowed prefill: the oracle's prefill row p of the linear
  sequence (not the ring) is the reference for the decode of position p.
* The full-size Mistral-7B decode (B=64, W=4096 ring, positions drawn from
  [4096, 32768)) is checked on every output.
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


def tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("W,d", [(5, 64), (4, 32), (64, 128), (1, 64)])
def test_ring_append_bit_exact(swa, dtype, W, d):
    print("ring", dtype, W, d, flush=True)
    B, Hkv, P = 3, 2, 3 * W + 2
    seq = si.normal(41, (P + 1, B, Hkv, d), dtype)
    seqd = to_device(seq)
    fill = -7.0
    kr = torch.full((B, Hkv, W, d), fill, dtype=tdtype(dtype), device="cuda")
    vr = torch.full((B, Hkv, W, d), fill, dtype=tdtype(dtype), device="cuda")
    for p in range(P + 1):
        # sequence 2 starts late (negative positions write nothing)
        pos = torch.tensor([p, p, p - 4], dtype=torch.int32, device="cuda")
        swa.cache_append(kr, vr, pos, seqd[p].contiguous(), (seqd[p] * 2).contiguous())
    torch.cuda.synchronize()
    for b, last in [(0, P), (1, P), (2, P - 4)]:
        for s in range(W):
            writers = [p for p in range(0, last + 1) if p % W == s]
            if not writers:
                assert torch.all(kr[b, :, s] == fill) and torch.all(vr[b, :, s] == fill)
                continue
            src = max(writers) + (4 if b == 2 else 0)
            assert torch.equal(kr[b, :, s], seqd[src, b]), (b, s)
            assert torch.equal(vr[b, :, s], seqd[src, b] * 2), (b, s)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [4, 16])
def test_toy_decode_every_position(swa, dtype, W):
    """16-token sequence, d=64: append then decode at every position 0..15;
    each output equals the oracle's windowed-prefill row of the linear
    sequence.  W=4 wraps the ring three times."""
    T, d = 16, 64
    q, k, v = si.prefill_inputs(1, dtype=dtype)
    scale = 1 / math.sqrt(d)
    ref = oracle.attention_dense(q.values, k.values, v.values, W, si.CAUSAL, scale)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    kr = torch.zeros((1, 1, W, d), dtype=tdtype(dtype), device="cuda")
    vr = torch.zeros_like(kr)
    for p in range(T):
        pos = torch.tensor([p], dtype=torch.int32, device="cuda")
        swa.cache_append(kr, vr, pos, kd[:, :, p].contiguous(), vd[:, :, p].contiguous())
        out = swa.decode(qd[:, :, p].contiguous(), kr, vr, pos)
        torch.cuda.synchronize()
        assert_parity(to_f64(out)[:, :, :], ref[:, :, p], dtype, "decode p=%d W=%d" % (p, W))


DECODE_SMALL = [
    # (B, Hq, Hkv, W, d, pos list)
    (3, 4, 1, 37, 64, [0, 5, 36]),
    (2, 8, 2, 100, 128, [250, 99]),
    (4, 8, 1, 64, 32, [-1, 0, 63, 64]),
    (2, 6, 3, 300, 64, [1000, 150]),
    (2, 16, 2, 129, 128, [128, 1000]),
    (1, 2, 2, 4096, 128, [5000]),
    (5, 1, 1, 1, 32, [0, 3, 7, -5, 2]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,W,d,pos", DECODE_SMALL)
def test_decode_small(swa, dtype, B, Hq, Hkv, W, d, pos):
    print("decode", dtype, dict(B=B, Hq=Hq, Hkv=Hkv, W=W, d=d, pos=pos), flush=True)
    q = si.normal(51, (B, Hq, d), dtype)
    kr = si.normal(52, (B, Hkv, W, d), dtype)
    vr = si.normal(53, (B, Hkv, W, d), dtype)
    pos = np.array(pos, dtype=np.int32)
    scale = 1 / math.sqrt(d)
    out = swa.decode(to_device(q), to_device(kr), to_device(vr),
                     torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = oracle.decode(q.values, kr.values, vr.values, pos, scale)
    assert_parity(got, ref, dtype, "decode")
    for b in np.flatnonzero(pos < 0):
        assert np.all(got[b] == 0.0)


def test_decode_equals_prefill_rows_gqa(swa):
    """Fill a ring by appending a whole sequence (GQA 8/2, W=48, T=200) and
    decode every position: each output equals the oracle's prefill row."""
    B, Hq, Hkv, T, W, d = 2, 8, 2, 200, 48, 64
    q, k, v = si.prefill_inputs(2, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d)
    scale = 1 / math.sqrt(d)
    ref = oracle.attention_banded(q.values, k.values, v.values, W, si.CAUSAL, scale)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    kr = torch.zeros((B, Hkv, W, d), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    outs = []
    for p in range(T):
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        swa.cache_append(kr, vr, pos, kd[:, :, p].contiguous(), vd[:, :, p].contiguous())
        outs.append(swa.decode(qd[:, :, p].contiguous(), kr, vr, pos))
    torch.cuda.synchronize()
    got = np.stack([to_f64(o) for o in outs], axis=2)  # [B, Hq, T, d]
    assert_parity(got, ref, "bf16", "decode vs prefill rows")


def test_mistral_decode_full(swa):
    """B=64, 32/8 heads, d=128, W=4096 full rings, positions in [4096, 32768).
    One split per (sequence, head) fills the GPU here, so the call needs and
    gets no workspace (a null pointer reaches the C ABI)."""
    cfg = si.WORKLOADS[4]
    assert swa.decode_workspace_bytes(cfg["B"], cfg["Hq"], cfg["W"], cfg["d"]) == 0
    q, kr, vr, pos = si.decode_inputs(4)
    out = swa.decode(to_device(q), to_device(kr), to_device(vr), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ref = oracle.decode(q.values, kr.values, vr.values, pos, 1 / math.sqrt(cfg["d"]))
    assert_parity(to_f64(out), ref, "bf16", "Mistral decode")


def test_decode_deterministic(swa):
    q, kr, vr, pos = si.decode_inputs(4, B=8)
    args = (to_device(q), to_device(kr), to_device(vr), torch.from_numpy(pos).cuda())
    a = swa.decode(*args)
    b = swa.decode(*args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_workspace_reused_across_calls_and_shapes(swa):
    """One workspace serves consecutive calls of different sizes: every
    partial the merge reads is written by the same call, so nothing from an
    earlier call is read and the workspace needs no clearing."""
    ws = swa.decode_workspace(8, 32, 4096, 128)
    for B, W in [(8, 4096), (3, 1000), (8, 4096), (1, 64)]:
        q, kr, vr, pos = si.decode_inputs(4, B=B, W=W, pos_lo=W // 2, pos_hi=3 * W)
        args = (to_device(q), to_device(kr), to_device(vr), torch.from_numpy(pos).cuda())
        reused = swa.decode(*args, workspace=ws)
        fresh = swa.decode(*args)
        torch.cuda.synchronize()
        assert torch.equal(reused, fresh), (B, W)
        ref = oracle.decode(q.values, kr.values, vr.values, pos, 1 / math.sqrt(128))
        assert_parity(to_f64(reused), ref, "bf16", "reused workspace B=%d W=%d" % (B, W))


def test_decode_checks_out_before_launch(swa):
    """A caller-supplied `out` of the wrong shape, or on another device, is
    refused by the binding before anything is launched (the C ABI sees only
    pointers)."""
    q, kr, vr, pos = si.decode_inputs(4, B=2, W=256, pos_lo=300, pos_hi=900)
    args = (to_device(q), to_device(kr), to_device(vr), torch.from_numpy(pos).cuda())
    small = torch.empty((2, 31, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="shape"):
        swa.decode(*args, out=small)
    host = torch.empty((2, 32, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        swa.decode(*args, out=host)
    ks = torch.zeros((2, 8, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="shape"):
        swa.decode_sinks(args[0], args[1], args[2], ks, ks.clone(), args[3], out=small)
