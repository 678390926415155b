"""GPU parity of the window plus global tokens (swa_prefill_global), through
the C ABI, against the fp64 oracle.

* Small and ragged shapes, both modes, 1 to 100 global tokens (one, exactly
  one and more than one 64-key global tile), global tokens inside and outside
  each other's windows and at both ends of the sequence, windows shorter and
  longer than a tile, GQA, d in {32, 64, 128}, bf16 and fp32.
* Causal global tokens at the first positions (attention sinks).
* Global positions outside [0, T) are ignored; G = 0 is swa_prefill bit for bit.
* The Longformer workload with 8 global tokens ([CLS] and question tokens),
  in the launch configuration the benchmark times, on sampled rows.
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


def positions(T, G, seed):
    """G distinct sorted positions in [0, T), always including 0 and T-1."""
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(1, T - 1), size=max(0, G - 2), replace=False)
    return np.unique(np.concatenate([[0, T - 1], inner])).astype(np.int32)[:G] if G >= 2 \
        else np.array([T // 2], dtype=np.int32)


GLOBAL_SMALL = [
    # (mode, T, W, G, B, Hq, Hkv, d)
    (1, 300, 16, 1, 1, 2, 1, 64),
    (0, 300, 16, 1, 1, 4, 2, 64),
    (1, 300, 16, 5, 2, 2, 2, 128),
    (0, 257, 64, 5, 1, 4, 1, 128),
    (1, 700, 33, 64, 1, 2, 1, 32),     # exactly one global tile
    (0, 700, 100, 65, 1, 6, 3, 64),    # one key into a second tile
    (1, 1000, 129, 100, 1, 2, 2, 64),
    (0, 129, 300, 7, 2, 2, 1, 32),     # window longer than the sequence
    (1, 64, 1, 3, 1, 2, 1, 128),       # W = 1
    (0, 1500, 200, 20, 1, 32, 8, 128), # 80 (row, head) pairs per KV head, 6 key splits
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,T,W,G,B,Hq,Hkv,d", GLOBAL_SMALL)
def test_global_small(swa, dtype, mode, T, W, G, B, Hq, Hkv, d):
    gpos = positions(T, G, 7 + G)
    print("global", dtype, dict(mode=mode, T=T, W=W, G=G, B=B, Hq=Hq, Hkv=Hkv, d=d), flush=True)
    q, k, v = si.prefill_inputs(8, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, dtype=dtype)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), W,
                             torch.from_numpy(gpos).cuda(), mode=mode)
    torch.cuda.synchronize()
    ref = oracle.attention_global_dense(q.values, k.values, v.values, W, mode, 1 / math.sqrt(d), gpos)
    assert_parity(to_f64(out), ref, dtype, "global")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_sinks(swa, dtype):
    """Causal window W=64 with the first 4 tokens global (attention sinks)."""
    T, W, d = 600, 64, 128
    gpos = np.arange(4, dtype=np.int32)
    q, k, v = si.prefill_inputs(8, B=1, Hq=8, Hkv=2, T=T, d=d, dtype=dtype)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), W,
                             torch.from_numpy(gpos).cuda(), mode=0)
    torch.cuda.synchronize()
    ref = oracle.attention_global_dense(q.values, k.values, v.values, W, 0, 1 / math.sqrt(d), gpos)
    assert_parity(to_f64(out), ref, dtype, "sinks")


def test_positions_outside_the_sequence_are_ignored(swa):
    T, W, d = 200, 20, 64
    q, k, v = si.prefill_inputs(8, B=1, Hq=2, Hkv=1, T=T, d=d)
    gpos = np.array([-5, 3, 150, T, T + 7], dtype=np.int32)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), W,
                             torch.from_numpy(gpos).cuda(), mode=1)
    torch.cuda.synchronize()
    ref = oracle.attention_global_dense(q.values, k.values, v.values, W, 1, 1 / math.sqrt(d), [3, 150])
    assert_parity(to_f64(out), ref, "bf16", "global with out-of-range positions")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", [0, 1])
def test_every_token_global_is_full_attention(swa, dtype, mode):
    """All T positions global: every row is a global row, i.e. full attention
    (causal or bidirectional), whatever the window."""
    T, W, d = 200, 8, 64
    q, k, v = si.prefill_inputs(8, B=1, Hq=4, Hkv=2, T=T, d=d, dtype=dtype)
    gpos = np.arange(T, dtype=np.int32)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), W,
                             torch.from_numpy(gpos).cuda(), mode=mode)
    torch.cuda.synchronize()
    ref = oracle.attention_banded(q.values, k.values, v.values, T if mode == 0 else 2 * T, mode,
                                  1 / math.sqrt(d))
    assert_parity(to_f64(out), ref, dtype, "every token global")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_global_is_prefill_bit_for_bit(swa, dtype):
    q, k, v = (to_device(t) for t in si.prefill_inputs(8, B=1, Hq=4, Hkv=2, T=333, d=64, dtype=dtype))
    a = swa.prefill(q, k, v, 40, mode=1)
    b = swa.prefill_global(q, k, v, 40, torch.zeros(0, dtype=torch.int32, device="cuda"), mode=1)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(a.view(bits), b.view(bits))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_longformer_global_sampled(swa, dtype):
    """B=4, T=4096, symmetric W=512, 12 heads, d=64, global tokens 0..7:
    the global rows and sampled other rows of every sequence vs the oracle
    (bf16, the workload's type; and the same shapes in fp32)."""
    cfg = si.WORKLOADS[8]
    q, k, v = si.prefill_inputs(8, dtype=dtype)
    gpos = np.array(cfg["global_pos"], dtype=np.int32)
    out = swa.prefill_global(to_device(q), to_device(k), to_device(v), cfg["W"],
                             torch.from_numpy(gpos).cuda(), mode=cfg["mode"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    got = to_f64(out)
    rows = list(gpos) + [8, 9, 255, 256, 263, 264, 265, 1000, 2048, 4095]
    scale = 1 / math.sqrt(cfg["d"])
    for b in range(cfg["B"]):
        for h in (0, 11):
            ref = oracle.attention_global_rows(q.values, k.values, v.values, cfg["W"], cfg["mode"],
                                               scale, gpos, b, h, rows)
            assert_parity(got[b, h, rows], ref, dtype, "longformer global b=%d h=%d" % (b, h))
