"""GPU test of swa_decode_noalloc (the decode entry point that allocates
nothing: its split partials live in the library's per-GPU scratch array),
through the C ABI, against swa_decode with a caller-owned workspace and
against the fp64 oracle.  Two calls in a row, the second smaller, so the
second reads nothing the first left behind; ring sizes that split the ring,
so the scratch is really used."""

import math

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


CASES = [
    # (B, Hq, Hkv, W, d, dtype, pos range): the first splits the ring into 64
    # chunks (532 KB of partials), the second into 16 (17 KB)
    (2, 8, 2, 4096, 128, "bf16", (5000, 9000)),
    (1, 4, 1, 1000, 64, "bf16", (300, 2500)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_decode_twice(swa, dtype):
    for B, Hq, Hkv, W, d, _, (lo, hi) in CASES:
        print("noalloc", dtype, B, Hq, Hkv, W, d, flush=True)
        assert swa.decode_workspace_bytes(B, Hq, W, d) > 0  # the scratch is used
        q, kr, vr, pos = si.decode_inputs(4, B=B, Hq=Hq, Hkv=Hkv, W=W, d=d, pos_lo=lo,
                                          pos_hi=hi, dtype=dtype)
        args = (to_device(q), to_device(kr), to_device(vr), torch.from_numpy(pos).cuda())
        out = torch.full_like(args[0], float("nan"))
        got = swa.decode_noalloc(*args, out=out)
        want = swa.decode(*args)
        torch.cuda.synchronize()
        # same kernels, same order of arithmetic: identical bits
        assert torch.equal(got, want), (B, W, d, dtype)
        ref = oracle.decode(q.values, kr.values, vr.values, pos, 1 / math.sqrt(d))
        assert_parity(to_f64(got), ref, dtype, "noalloc B=%d W=%d d=%d" % (B, W, d))


def test_noalloc_one_split_needs_no_scratch(swa):
    """The Mistral-7B decode shape (64 x 32 heads) takes one split per head:
    the output is written directly, no scratch involved."""
    c = si.WORKLOADS[4]
    assert swa.decode_workspace_bytes(c["B"], c["Hq"], c["W"], c["d"]) == 0
    q, kr, vr, pos = si.decode_inputs(4, B=8)
    args = (to_device(q), to_device(kr), to_device(vr), torch.from_numpy(pos).cuda())
    got = swa.decode_noalloc(*args)
    want = swa.decode(*args)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
