"""GPU parity of chunked prefill into an existing ring (swa_prefill_chunk) and
of the multi-token append (swa_cache_append_chunk), through the C ABI,
against the fp64 oracle.

* Multi-token append is bit-exact against n single appends in order, also
  when the chunk is longer than the ring (only its last W tokens remain) and
  for negative positions (nothing written).
* A chunk at positions [p, p+n) with random ring contents (NaN in the slots
  no earlier position wrote) matches the oracle's chunk rows, over ragged chunk lengths, windows shorter and longer
  than a tile, p = 0, p < W - 1 (partly filled ring), wrapped rings, GQA,
  d in {32, 64, 128}, bf16 and fp32, negative positions (zero rows).
* Serving flow: a sequence fed in uneven chunks (prefill the chunk, then
  append it) gives the oracle's causal-prefill rows of the whole sequence,
  and a decode after the last chunk gives its last row.
* The Mistral-7B chunk workload (4 sequences, 2048-token chunks, full
  W=4096 rings), in the launch configuration the benchmark times, is checked
  on sampled rows.
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


APPEND_CASES = [
    # (B, Hkv, W, n, d, pos)
    (2, 2, 8, 3, 64, [0, 6]),
    (3, 1, 5, 13, 32, [2, 0, 11]),     # chunk longer than the ring
    (2, 3, 64, 64, 128, [64, 7]),      # exactly one ring of tokens
    (2, 2, 1, 4, 64, [3, 0]),          # W = 1
    (4, 2, 37, 50, 64, [-1, 100, 36, -7]),
    (1, 8, 4096, 2048, 128, [12000]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hkv,W,n,d,pos", APPEND_CASES)
def test_append_chunk_bit_exact(swa, dtype, B, Hkv, W, n, d, pos):
    print("append_chunk", dtype, dict(B=B, Hkv=Hkv, W=W, n=n, d=d, pos=pos), flush=True)
    k = si.normal(81, (B, Hkv, n, d), dtype)
    v = si.normal(82, (B, Hkv, n, d), dtype)
    kr0 = si.normal(83, (B, Hkv, W, d), dtype)
    vr0 = si.normal(84, (B, Hkv, W, d), dtype)
    kr, vr = to_device(kr0), to_device(vr0)
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    swa.cache_append_chunk(kr, vr, posd, to_device(k), to_device(v))
    torch.cuda.synchronize()
    want_k, want_v = kr0.bits.copy(), vr0.bits.copy()
    oracle.ring_append_chunk(want_k, want_v, np.array(pos), k.bits, v.bits)
    tint, nint = (torch.int16, np.int16) if dtype == "bf16" else (torch.int32, np.int32)
    got_k, got_v = kr.cpu().view(tint).numpy(), vr.cpu().view(tint).numpy()
    want_k, want_v = want_k.view(nint), want_v.view(nint)
    assert np.array_equal(got_k, want_k)
    assert np.array_equal(got_v, want_v)


def poison_unwritten(t, pos, W):
    """NaN in every ring slot that no earlier position wrote (slots >= p of a
    sequence with p < W; the whole ring of an inactive sequence): the kernel
    must never read them."""
    vals, bits = t.values.copy(), t.bits.copy()
    for b, p in enumerate(pos):
        first = max(int(p), 0)
        if first < W:
            vals[b, :, first:] = np.nan
            bits[b, :, first:] = 0x7FC0 if t.dtype == si.BF16 else np.nan
    return si.Tensor(vals, bits, t.dtype)


CHUNK_SMALL = [
    # (B, Hq, Hkv, n, W, d, pos)
    (2, 4, 2, 100, 37, 64, [0, 5]),           # p = 0; p < W - 1; chunk > window
    (2, 8, 2, 256, 64, 128, [64, 1000]),      # tile-aligned, wrapped ring
    (3, 4, 1, 129, 129, 32, [128, 129, 7]),   # ragged tails on both sides
    (1, 2, 2, 300, 4096, 128, [5000]),        # long window: ring tiles dominate
    (4, 8, 1, 65, 33, 64, [-1, 0, 31, 32]),   # inactive sequence; short window
    (2, 6, 3, 200, 1, 64, [0, 10]),           # W = 1: every row sees itself only
    (1, 4, 2, 1, 16, 128, [20]),              # one-token chunk (a decode step)
    (2, 4, 2, 384, 200, 32, [3, 10000]),
    (1, 4, 4, 130, 300, 64, [64]),            # ring partly filled, p on a tile edge
    (2, 2, 1, 70, 2, 128, [1, 2]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,n,W,d,pos", CHUNK_SMALL)
def test_prefill_chunk_small(swa, dtype, B, Hq, Hkv, n, W, d, pos):
    print("prefill_chunk", dtype, dict(B=B, Hq=Hq, Hkv=Hkv, n=n, W=W, d=d, pos=pos), flush=True)
    q, k, v, kr, vr, _ = si.chunk_inputs(6, B=B, Hq=Hq, Hkv=Hkv, n=n, W=W, d=d, dtype=dtype)
    pos = np.array(pos, dtype=np.int32)
    kr, vr = poison_unwritten(kr, pos, W), poison_unwritten(vr, pos, W)
    scale = 1 / math.sqrt(d)
    out = swa.prefill_chunk(to_device(q), to_device(k), to_device(v), to_device(kr),
                            to_device(vr), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = oracle.prefill_chunk(q.values, k.values, v.values, kr.values, vr.values, pos, W, scale)
    assert_parity(got, ref, dtype, "prefill_chunk")
    for b in np.flatnonzero(pos < 0):
        assert np.all(got[b] == 0.0)


def test_prefill_chunk_f32_many_tiles(swa):
    """fp32 chunks on the matrix cores over many ring and chunk tiles: a
    2000-slot ring, 600-token chunks at positions far past one ring turn and
    just after the start, every row against the oracle (unwritten slots
    poisoned)."""
    B, Hq, Hkv, n, W, d = 2, 4, 2, 600, 2000, 128
    q, k, v, kr, vr, _ = si.chunk_inputs(6, B=B, Hq=Hq, Hkv=Hkv, n=n, W=W, d=d, dtype="f32")
    pos = np.array([5000, 300], dtype=np.int32)
    kr, vr = poison_unwritten(kr, pos, W), poison_unwritten(vr, pos, W)
    out = swa.prefill_chunk(to_device(q), to_device(k), to_device(v), to_device(kr),
                            to_device(vr), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk(q.values, k.values, v.values, kr.values, vr.values, pos, W,
                               1 / math.sqrt(d))
    assert_parity(to_f64(out), ref, "f32", "fp32 chunk over many tiles")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_serving_equals_prefill(swa, dtype):
    """Feed a T=700 sequence (GQA 8/2, d=64, W=96) in uneven chunks: each
    chunk is attended against the ring, then appended.  The outputs are the
    oracle's causal-prefill rows of the whole sequence; a decode of the last
    position after the last chunk gives the last row."""
    B, Hq, Hkv, T, W, d = 2, 8, 2, 700, 96, 64
    q, k, v = si.prefill_inputs(2, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, dtype=dtype)
    scale = 1 / math.sqrt(d)
    ref = oracle.attention_banded(q.values, k.values, v.values, W, si.CAUSAL, scale)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kr = torch.zeros((B, Hkv, W, d), dtype=tdt, device="cuda")
    vr = torch.zeros_like(kr)
    outs, p = [], 0
    for n in [1, 50, 128, 200, 33, 288]:
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        qc = qd[:, :, p:p + n].contiguous()
        kc, vc = kd[:, :, p:p + n].contiguous(), vd[:, :, p:p + n].contiguous()
        outs.append(swa.prefill_chunk(qc, kc, vc, kr, vr, pos))
        swa.cache_append_chunk(kr, vr, pos, kc, vc)
        p += n
    assert p == T
    last = swa.decode(qd[:, :, T - 1].contiguous(), kr, vr,
                      torch.full((B,), T - 1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got = np.concatenate([to_f64(o) for o in outs], axis=2)
    assert_parity(got, ref, dtype, "chunked serving vs prefill rows")
    assert_parity(to_f64(last), ref[:, :, T - 1], dtype, "decode after chunks")


def test_prefill_chunk_large_scores_force_rescaling(swa):
    """Scores of sigma ~ 3 sqrt(d) make the running maximum grow inside the
    ring part and again inside the chunk part."""
    B, Hq, Hkv, n, W, d = 1, 4, 2, 256, 300, 128
    q, k, v, kr, vr, _ = si.chunk_inputs(6, B=B, Hq=Hq, Hkv=Hkv, n=n, W=W, d=d)
    bits = si.bf16_bits(q.values * 3.0)  # rounded to bf16 again
    q3 = si.Tensor(si.bf16_to_f32(bits), bits, si.BF16)
    pos = np.array([1000], dtype=np.int32)
    out = swa.prefill_chunk(to_device(q3), to_device(k), to_device(v), to_device(kr),
                            to_device(vr), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk(q3.values, k.values, v.values, kr.values, vr.values, pos, W,
                               1 / math.sqrt(d))
    assert_parity(to_f64(out), ref, "bf16", "prefill_chunk large scores")


def test_mistral_chunk_sampled(swa):
    """B=4, 32/8 heads, d=128, 2048-token chunks, full W=4096 rings, chunk
    positions in [4096, 32768): sampled rows of every sequence vs the oracle;
    every output finite."""
    cfg = si.WORKLOADS[6]
    q, k, v, kr, vr, pos = si.chunk_inputs(6)
    print("mistral chunk", cfg["name"], pos.tolist(), flush=True)
    out = swa.prefill_chunk(to_device(q), to_device(k), to_device(v), to_device(kr),
                            to_device(vr), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    n = cfg["n"]
    rows = [0, 1, 63, 64, 127, 128, 1000, 2047]
    heads = [(b, h) for b in range(cfg["B"]) for h in (0, 5, 31)]
    ref = oracle.prefill_chunk(q.values, k.values, v.values, kr.values, vr.values, pos, cfg["W"],
                               1 / math.sqrt(cfg["d"]), heads=heads, rows=rows)
    got = to_f64(out)
    assert rows[-1] == n - 1
    for b, h in heads:
        assert_parity(got[b, h, rows], ref[b, h, rows], "bf16", "mistral chunk b=%d h=%d" % (b, h))
