"""Shared test helpers: device transfer of the seeded inputs and the parity
bars.

Parity bars (fixed for this method): fp32 results within max-abs 1e-5 of the
fp64 oracle; bf16 results within max-abs 2e-2 and relative L2 error 5e-3;
ring-cache contents bit-exact.
"""

import numpy as np

FP32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def to_device(t, device="cuda"):
    """swa_inputs.Tensor -> torch tensor holding exactly the same bits."""
    import swa_inputs
    return swa_inputs.to_torch(t, device)


def to_f64(x):
    """torch tensor (any float dtype, any device) -> float64 numpy."""
    import torch
    return x.detach().to("cpu", torch.float64).numpy()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel_l2


def cosine(got, ref):
    """Cosine similarity of the flattened outputs (logged, not gated)."""
    a = np.asarray(got, dtype=np.float64).ravel()
    b = np.asarray(ref, dtype=np.float64).ravel()
    den = float(np.linalg.norm(a) * np.linalg.norm(b))
    return float(a @ b / den) if den > 0 else 1.0


def assert_parity(got, ref, dtype, what=""):
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    max_abs, rel_l2 = errors(got, ref)
    print("%s: max-abs %.3g rel-L2 %.3g cosine %.9f" % (what, max_abs, rel_l2, cosine(got, ref)))
    if dtype == "f32":
        assert max_abs <= FP32_MAX_ABS, "%s: max-abs %.3g > %.1g" % (what, max_abs, FP32_MAX_ABS)
    else:
        assert max_abs <= BF16_MAX_ABS and rel_l2 <= BF16_REL_L2, \
            "%s: max-abs %.3g (bar %.0e), rel-L2 %.3g (bar %.0e)" % (what, max_abs, BF16_MAX_ABS,
                                                                  rel_l2, BF16_REL_L2)
    return max_abs, rel_l2
