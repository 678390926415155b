"""GPU checks of the calibration kernels (swa_calib_*), through the C ABI.

The streaming read is checked exactly: each lane's XOR equals the XOR of the
16-byte vectors it is assigned (workgroup w reads the w-th contiguous chunk,
lane t every 256th vector of it from the t-th), computed on the host, for
sizes with ragged chunks and tails.  The matrix-core loop is checked for
finite, repeatable sums (its FLOP count is fixed by construction).  The
vector chains are checked against a host recurrence: the FMA chain in float64
(the chain contracts, so one rounding per step keeps it within 1e-5), the
exp2 chain against float64 exp2 within the instruction's accuracy."""

import numpy as np
import pytest

import swa_inputs as si

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sliding_window_attention_swa_amd as m
    m.load()
    return m


def expected_read(words, n_wg):
    """words: uint32 [n16, 4]; returns uint32 [n_wg * 256]."""
    n16 = words.shape[0]
    vec = np.bitwise_xor.reduce(words, axis=1)
    per_wg = -(-n16 // n_wg)
    out = np.zeros(n_wg * 256, dtype=np.uint32)
    for w in range(n_wg):
        lo, hi = w * per_wg, min((w + 1) * per_wg, n16)
        for t in range(256):
            sel = vec[lo + t:hi:256] if lo + t < hi else vec[:0]
            out[w * 256 + t] = np.bitwise_xor.reduce(sel) if sel.size else 0
    return out


@pytest.mark.parametrize("n16,n_wg", [(1, 1), (256 * 8, 1), (256 * 8 + 17, 3), (100000, 7),
                                      (4096 * 9 + 5, 16)])
def test_stream_read_reads_every_vector_once(swa, n16, n_wg):
    print("stream read n16=%d n_wg=%d" % (n16, n_wg), flush=True)
    rng = np.random.default_rng(n16 + n_wg)
    words = rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((n_wg * 256,), -1, dtype=torch.int32, device="cuda")
    assert swa.calib_stream_read(src, sink, n_wg) == n16 * 16
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_read(words, n_wg))


def test_mfma_loop_is_finite_and_repeatable(swa):
    ops = si.to_torch(si.normal(99, (32768,), "bf16"), torch.device("cuda:0"))
    n_wg, iters = 64, 20
    a = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    assert swa.calib_mfma(ops, a, n_wg, iters) == n_wg * 4 * iters * 16 * 32768
    swa.calib_mfma(ops, b, n_wg, iters)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)
    assert a.abs().sum() > 0


@pytest.mark.parametrize("op", [0, 1])
def test_vector_chains_follow_their_recurrence(swa, op):
    n_wg, iters = 4, 37
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    assert swa.calib_vector(op, sink, n_wg, iters) == n_wg * 4 * iters * 16
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64)
    # lane t (of its workgroup) starts chain j at -1e-3 * ((t + 16 j) mod 1024)
    t = np.arange(256)
    x = np.stack([-1e-3 * ((t + 16 * j) % 1024) for j in range(16)]).astype(np.float32).astype(np.float64)
    for _ in range(iters):
        x = x * 0.999 + 0.001 if op == 0 else -np.exp2(x)
    want = np.tile(x.sum(axis=0), n_wg)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) < 1e-4
