"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This module holds no attention arithmetic: it draws random numbers, rounds
them to the storage dtype, and describes the workloads' shapes.  Both the HIP
library (through the Python binding) and the fp64 oracle consume exactly the
bits produced here.

Recipe: ``numpy.random.default_rng(seed).standard_normal(shape, float32)``,
then round-to-nearest-even to bfloat16 for bf16 workloads.  Seeds are
``1000 * workload + role`` with role Q=0, K=1, V=2, positions=3, and for
chunked prefill ring K=4, ring V=5.
"""

import numpy as np

ROLE_Q, ROLE_K, ROLE_V, ROLE_POS, ROLE_K_RING, ROLE_V_RING = 0, 1, 2, 3, 4, 5

F32 = "f32"
BF16 = "bf16"

CAUSAL = 0
SYMMETRIC = 1

# The five workloads.  Shapes follow the model families the pages name:
# a 16-token toy window (Ultralytics mask example), TinyMistral-248M
# (12 layers, hidden 1024, GQA 32/8, sliding_window 32 -> head_dim 32),
# Mistral 7B (W=4096, GQA 32/8, head_dim 128) for prefill and decode, and
# Longformer (symmetric W=512, 12 heads, head_dim 64).
WORKLOADS = {
    1: dict(name="toy causal T=16 W=4 d=64 fp32", kind="prefill", B=1, Hq=1, Hkv=1,
            T=16, W=4, d=64, dtype=F32, mode=CAUSAL),
    2: dict(name="TinyMistral-248M causal prefill", kind="prefill", B=8, Hq=32, Hkv=8,
            T=2048, W=32, d=32, dtype=BF16, mode=CAUSAL),
    3: dict(name="Mistral-7B causal prefill", kind="prefill", B=1, Hq=32, Hkv=8,
            T=16384, W=4096, d=128, dtype=BF16, mode=CAUSAL),
    4: dict(name="Mistral-7B ring-cache decode", kind="decode", B=64, Hq=32, Hkv=8,
            W=4096, d=128, dtype=BF16, mode=CAUSAL, pos_lo=4096, pos_hi=32768),
    5: dict(name="Longformer symmetric prefill", kind="prefill", B=4, Hq=12, Hkv=12,
            T=4096, W=512, d=64, dtype=BF16, mode=SYMMETRIC),
    # the dilated Longformer window of aivaro section 4.2 (W=512, dilation 2)
    7: dict(name="Longformer dilated symmetric prefill", kind="prefill", B=4, Hq=12, Hkv=12,
            T=4096, W=512, d=64, dtype=BF16, mode=SYMMETRIC, dilation=2),
    # Longformer with global attention (aivaro section 4.3: usually 1 to 10
    # global tokens): [CLS] at position 0 and seven question tokens after it
    8: dict(name="Longformer symmetric prefill + 8 global tokens", kind="prefill", B=4, Hq=12,
            Hkv=12, T=4096, W=512, d=64, dtype=BF16, mode=SYMMETRIC,
            global_pos=[0, 1, 2, 3, 4, 5, 6, 7]),
    # both together, as Longformer combines them (aivaro sections 4.2, 4.3)
    9: dict(name="Longformer dilated symmetric prefill + 8 global tokens", kind="prefill", B=4,
            Hq=12, Hkv=12, T=4096, W=512, d=64, dtype=BF16, mode=SYMMETRIC, dilation=2,
            global_pos=[0, 1, 2, 3, 4, 5, 6, 7]),
    # serving-style chunked prefill: 4 sequences, each continuing with a
    # 2048-token chunk after at least W tokens are already in its ring
    6: dict(name="Mistral-7B chunked prefill", kind="chunk", B=4, Hq=32, Hkv=8, n=2048,
            W=4096, d=128, dtype=BF16, mode=CAUSAL, pos_lo=4096, pos_hi=32768),
}


def seed_for(workload, role):
    return 1000 * int(workload) + int(role)


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs are finite normal draws, so no
    NaN/Inf handling is needed (and none is attempted).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    lsb += 0x7FFF
    lsb += u  # no wrap-around: finite values stay below 0xFF800000 + 0x8000
    lsb >>= 16
    return lsb.astype(np.uint16)


def bf16_to_f32(bits):
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """A synthetic array in its storage dtype.

    ``values`` is float32 and holds exactly the numbers the storage bits
    encode; ``bits`` is the raw storage (uint16 for bf16, float32 for f32).
    """

    def __init__(self, values, bits, dtype):
        self.values = values
        self.bits = bits
        self.dtype = dtype

    @property
    def shape(self):
        return self.values.shape


def normal(seed, shape, dtype):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if dtype == F32:
        return Tensor(x, x, F32)
    if dtype == BF16:
        bits = bf16_bits(x)
        return Tensor(bf16_to_f32(bits), bits, BF16)
    raise ValueError("unknown dtype %r" % (dtype,))


def positions(seed, n, lo, hi):
    """n int32 positions uniform in [lo, hi)."""
    return np.random.default_rng(seed).integers(lo, hi, size=n).astype(np.int32)


def prefill_inputs(workload, B=None, Hq=None, Hkv=None, T=None, d=None, dtype=None):
    """Q, K, V for a prefill workload (overrides allow shrunken variants)."""
    cfg = WORKLOADS[workload]
    B = cfg["B"] if B is None else B
    Hq = cfg["Hq"] if Hq is None else Hq
    Hkv = cfg["Hkv"] if Hkv is None else Hkv
    T = cfg["T"] if T is None else T
    d = cfg["d"] if d is None else d
    dtype = cfg["dtype"] if dtype is None else dtype
    q = normal(seed_for(workload, ROLE_Q), (B, Hq, T, d), dtype)
    k = normal(seed_for(workload, ROLE_K), (B, Hkv, T, d), dtype)
    v = normal(seed_for(workload, ROLE_V), (B, Hkv, T, d), dtype)
    return q, k, v


def decode_inputs(workload=4, B=None, Hq=None, Hkv=None, W=None, d=None, dtype=None,
                  pos_lo=None, pos_hi=None):
    """Query rows, full rings and positions for a decode workload.

    Every slot of the ring is filled (positions are all >= W), which is what
    a ring looks like after at least W appends.
    """
    cfg = WORKLOADS[workload]
    B = cfg["B"] if B is None else B
    Hq = cfg["Hq"] if Hq is None else Hq
    Hkv = cfg["Hkv"] if Hkv is None else Hkv
    W = cfg["W"] if W is None else W
    d = cfg["d"] if d is None else d
    dtype = cfg["dtype"] if dtype is None else dtype
    lo = cfg.get("pos_lo", W) if pos_lo is None else pos_lo
    hi = cfg.get("pos_hi", 8 * W) if pos_hi is None else pos_hi
    q = normal(seed_for(workload, ROLE_Q), (B, Hq, d), dtype)
    k_ring = normal(seed_for(workload, ROLE_K), (B, Hkv, W, d), dtype)
    v_ring = normal(seed_for(workload, ROLE_V), (B, Hkv, W, d), dtype)
    pos = positions(seed_for(workload, ROLE_POS), B, lo, hi)
    return q, k_ring, v_ring, pos


def chunk_inputs(workload=6, B=None, Hq=None, Hkv=None, n=None, W=None, d=None, dtype=None,
                 pos_lo=None, pos_hi=None):
    """Chunk queries/keys/values, rings and chunk start positions for a
    chunked-prefill workload.  Every ring slot is filled with a random row
    (positions >= W by default), which is what a ring holds after at least W
    appends."""
    cfg = WORKLOADS[workload]
    B = cfg["B"] if B is None else B
    Hq = cfg["Hq"] if Hq is None else Hq
    Hkv = cfg["Hkv"] if Hkv is None else Hkv
    n = cfg["n"] if n is None else n
    W = cfg["W"] if W is None else W
    d = cfg["d"] if d is None else d
    dtype = cfg["dtype"] if dtype is None else dtype
    lo = cfg.get("pos_lo", W) if pos_lo is None else pos_lo
    hi = cfg.get("pos_hi", 8 * W) if pos_hi is None else pos_hi
    q = normal(seed_for(workload, ROLE_Q), (B, Hq, n, d), dtype)
    k = normal(seed_for(workload, ROLE_K), (B, Hkv, n, d), dtype)
    v = normal(seed_for(workload, ROLE_V), (B, Hkv, n, d), dtype)
    k_ring = normal(seed_for(workload, ROLE_K_RING), (B, Hkv, W, d), dtype)
    v_ring = normal(seed_for(workload, ROLE_V_RING), (B, Hkv, W, d), dtype)
    pos = positions(seed_for(workload, ROLE_POS), B, lo, hi)
    return q, k, v, k_ring, v_ring, pos


def to_torch(t, device="cuda"):
    """Tensor -> torch tensor on `device` holding exactly the same bits."""
    import torch
    if t.dtype == BF16:
        host = torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(np.ascontiguousarray(t.bits, dtype=np.float32))
    return host.to(device)
