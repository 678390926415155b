"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself alone: each check ties it to a
value a page prints (tests/golden/), a closed form, a library routine that
computes a special case (torch's scaled_dot_product_attention in float64 on
the CPU), or brute force.  The mutation tests at the end plant plausible
mistakes in copies of oracle routines and show that a pin catches each one.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import swa_ref

CAUSAL, SYMMETRIC = oracle.CAUSAL, oracle.SYMMETRIC


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa(q, k, v, scale, mask=None, is_causal=False):
    """torch's own attention in float64 on the CPU (GQA by repeat-interleave)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    am = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=am, is_causal=is_causal,
                                       scale=scale, enable_gqa=q.shape[1] != k.shape[1])
    return o.numpy()


def torch_band(T, W, mode):
    """Band mask from torch's triangle routines (no offset arithmetic)."""
    ones = torch.ones(T, T, dtype=torch.bool)
    if mode == CAUSAL:
        return ones.tril(0).triu(-(W - 1)).numpy()
    h = W // 2
    return ones.tril(h).triu(-h).numpy()


# ---------------------------------------------------------------- page values

def test_page_score_counts(golden):
    g = golden("mask_counts_t16_w4.txt")
    T, W = g["seq_len"], g["window"]
    assert oracle.scores_per_layer(T, W, CAUSAL) == g["scores_window"]
    # full causal attention is the window with W >= T
    assert oracle.scores_per_layer(T, T, CAUSAL) == g["scores_full_causal"]
    assert oracle.scores_per_layer(T, 10 * T, CAUSAL) == g["scores_full_causal"]


def test_page_stacked_reach(golden):
    g = golden("mask_counts_t16_w4.txt")
    T, W = g["seq_len"], g["window"]
    assert oracle.stacked_reach(T, W, len(g["reach"])) == g["reach"]


def test_reach_closed_form_and_upper_bound(golden):
    # brute force boolean mask powers agree with 1 + L(W-1) while the reach
    # stays inside the sequence, and never exceed the L*W bound
    for T, W, L in [(64, 5, 6), (100, 8, 9), (40, 2, 12), (33, 1, 4)]:
        got = oracle.stacked_reach(T, W, L)
        for layer, r in enumerate(got, start=1):
            assert r == min(T, 1 + layer * (W - 1))
            assert r <= layer * W
    g = golden("receptive_field_mistral.txt")
    L, W = g["layers"], g["window"]
    assert L * W == g["upper_bound"]
    assert 1 + L * (W - 1) <= g["upper_bound"]


def test_band_sum_closed_forms():
    # causal: sum_i min(i+1, W) = W(W+1)/2 + (T-W)W for T >= W
    for T, W in [(2048, 32), (16384, 4096), (16, 4), (37, 5)]:
        want = W * (W + 1) // 2 + (T - W) * W
        got = sum(oracle.band(i, T, W, CAUSAL)[1] - oracle.band(i, T, W, CAUSAL)[0] + 1
                  for i in range(T))
        assert got == want
        if T <= 4096:
            assert oracle.scores_per_layer(T, W, CAUSAL) == want
    # symmetric with h = W//2 and T >= 2h+1: T(2h+1) - h(h+1)
    for T, W in [(4096, 512), (50, 7), (50, 8)]:
        h = W // 2
        want = T * (2 * h + 1) - h * (h + 1)
        got = sum(oracle.band(i, T, W, SYMMETRIC)[1] - oracle.band(i, T, W, SYMMETRIC)[0] + 1
                  for i in range(T))
        assert got == want
        assert oracle.scores_per_layer(T, W, SYMMETRIC) == want
    # the in-window work of the three full-size prefill workloads
    assert 32 * 65 == 2080 and (32 * 33 // 2 + (2048 - 32) * 32) == 65040
    assert 4096 * 4097 // 2 + (16384 - 4096) * 4096 == 58722304


def test_band_matches_mask_rows():
    for mode, W in [(CAUSAL, 5), (SYMMETRIC, 5), (SYMMETRIC, 6), (CAUSAL, 1)]:
        T = 23
        M = oracle.window_mask(T, W, mode)
        for i in range(T):
            lo, hi = oracle.band(i, T, W, mode)
            idx = np.flatnonzero(M[i])
            assert idx[0] == lo and idx[-1] == hi and len(idx) == hi - lo + 1
            assert all(oracle.allowed(i, j, T, W, mode) == bool(M[i, j]) for j in range(T))
            assert not any(oracle.allowed(i, j, T, W, mode) for j in (-2, -1, T, T + 1))


# --------------------------------------------------- special cases vs library

@pytest.mark.parametrize("T,d,Hq,Hkv", [(16, 64, 1, 1), (40, 8, 4, 2), (33, 16, 6, 3)])
def test_full_window_equals_library_causal(T, d, Hq, Hkv):
    q, k, v = rand((2, Hq, T, d), 1), rand((2, Hkv, T, d), 2), rand((2, Hkv, T, d), 3)
    scale = 1 / math.sqrt(d)
    want = sdpa(q, k, v, scale, is_causal=True)
    for W in (T, T + 1, 3 * T):
        np.testing.assert_allclose(oracle.attention_dense(q, k, v, W, CAUSAL, scale), want,
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(oracle.attention_banded(q, k, v, W, CAUSAL, scale, block=8),
                                   want, rtol=0, atol=1e-12)


def test_wide_symmetric_equals_library_bidirectional():
    T, d = 21, 8
    q, k, v = rand((1, 4, T, d), 4), rand((1, 2, T, d), 5), rand((1, 2, T, d), 6)
    want = sdpa(q, k, v, 0.3)
    for W in (2 * (T - 1), 2 * T + 1, 100):
        np.testing.assert_allclose(oracle.attention_dense(q, k, v, W, SYMMETRIC, 0.3), want,
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode,W", [(CAUSAL, 4), (CAUSAL, 7), (SYMMETRIC, 6), (SYMMETRIC, 7),
                                    (CAUSAL, 1), (SYMMETRIC, 1)])
def test_window_equals_library_with_triangle_mask(mode, W):
    T, d = 29, 16
    q, k, v = rand((2, 8, T, d), 7), rand((2, 2, T, d), 8), rand((2, 2, T, d), 9)
    want = sdpa(q, k, v, 0.25, mask=torch_band(T, W, mode))
    for got in (oracle.attention_dense(q, k, v, W, mode, 0.25),
                oracle.attention_banded(q, k, v, W, mode, 0.25, block=8)):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_window_one_is_identity():
    # one key per row: softmax weight exactly 1, so O = V bit for bit
    q, k, v = rand((2, 4, 19, 8), 10), rand((2, 2, 19, 8), 11), rand((2, 2, 19, 8), 12)
    o = oracle.attention_dense(q, k, v, 1, CAUSAL, 0.5)
    assert np.array_equal(o, np.repeat(v, 2, axis=1))
    o = oracle.attention_dense(q, k, v, 1, SYMMETRIC, 0.5)  # floor(1/2) = 0: self only
    assert np.array_equal(o, np.repeat(v, 2, axis=1))


def test_constant_values_give_constant_output():
    T, d = 30, 8
    q, k = rand((1, 2, T, d), 13), rand((1, 1, T, d), 14)
    c = rand((d,), 15)
    v = np.broadcast_to(c, (1, 1, T, d)).copy()
    for mode, W in [(CAUSAL, 6), (SYMMETRIC, 9)]:
        o = oracle.attention_dense(q, k, v, W, mode, 0.4)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


# --------------------------------------------------------------- brute force

@pytest.mark.parametrize("mode,W,T,Hq,Hkv,d", [
    (CAUSAL, 4, 16, 1, 1, 8), (CAUSAL, 16, 16, 2, 1, 4), (CAUSAL, 3, 11, 4, 2, 5),
    (SYMMETRIC, 4, 12, 2, 2, 6), (SYMMETRIC, 5, 9, 3, 1, 3), (SYMMETRIC, 30, 7, 1, 1, 4),
])
def test_three_forms_agree(mode, W, T, Hq, Hkv, d):
    q, k, v = rand((2, Hq, T, d), 16), rand((2, Hkv, T, d), 17), rand((2, Hkv, T, d), 18)
    loop = oracle.attention_loop(q, k, v, W, mode, 0.7)
    dense = oracle.attention_dense(q, k, v, W, mode, 0.7)
    banded = oracle.attention_banded(q, k, v, W, mode, 0.7, block=3)
    np.testing.assert_allclose(dense, loop, rtol=0, atol=1e-12)
    np.testing.assert_allclose(banded, loop, rtol=0, atol=1e-12)
    for b in range(2):
        for h in range(Hq):
            rows = oracle.attention_rows(q, k, v, W, mode, 0.7, b, h, list(range(T)))
            np.testing.assert_allclose(rows, loop[b, h], rtol=0, atol=1e-12)


def test_locality_outside_window_is_ignored():
    T, d, W = 40, 8, 6
    q, k, v = rand((1, 1, T, d), 19), rand((1, 1, T, d), 20), rand((1, 1, T, d), 21)
    base = oracle.attention_dense(q, k, v, W, CAUSAL, 0.5)
    i = 25
    k2, v2 = k.copy(), v.copy()
    out_of_window = [j for j in range(T) if not oracle.allowed(i, j, T, W, CAUSAL)]
    k2[0, 0, out_of_window] += 100.0
    v2[0, 0, out_of_window] -= 50.0
    pert = oracle.attention_dense(q, k2, v2, W, CAUSAL, 0.5)
    assert np.array_equal(pert[0, 0, i], base[0, 0, i])
    assert not np.array_equal(pert[0, 0, i + 1], base[0, 0, i + 1])


# ---------------------------------------------------------- ring and decode

def ring_last_writer_holds(append_impl, W=5, P=17, B=2, Hkv=2, d=3):
    """After appending positions 0..P, slot s holds the row of the latest
    position p <= P with p = s (mod W); slots never written keep the fill."""
    rng = np.random.default_rng(22)
    seq_k = rng.standard_normal((P + 1, B, Hkv, d))
    seq_v = rng.standard_normal((P + 1, B, Hkv, d))
    kr = np.full((B, Hkv, W, d), -7.0)
    vr = np.full((B, Hkv, W, d), -7.0)
    for p in range(P + 1):
        append_impl(kr, vr, np.full(B, p), seq_k[p], seq_v[p])
    for s in range(W):
        writers = [p for p in range(P + 1) if p % W == s]
        if not writers:
            if not (np.all(kr[:, :, s] == -7.0) and np.all(vr[:, :, s] == -7.0)):
                return False
            continue
        p = max(writers)
        if not (np.array_equal(kr[:, :, s], seq_k[p]) and np.array_equal(vr[:, :, s], seq_v[p])):
            return False
    return True


def test_ring_last_writer():
    assert ring_last_writer_holds(oracle.ring_append)
    assert ring_last_writer_holds(oracle.ring_append, W=4, P=2)  # ring never fills
    assert ring_last_writer_holds(oracle.ring_append, W=1, P=6)


def test_ring_memory_is_constant(golden):
    g = golden("kv_ring_memory.txt")
    # the ring holds W slots whatever the position; a full cache holds every token
    assert g["tokens"] // g["window"] == g["ratio"]
    W = g["check_window"]
    rows_at = lambda n: min(n, W)
    assert rows_at(g["check_from"]) == rows_at(g["check_to"]) == W


@pytest.mark.parametrize("W,Hq,Hkv,mode_T", [(4, 1, 1, 16), (16, 1, 1, 16), (3, 4, 2, 13)])
def test_decode_equals_prefill_row(W, Hq, Hkv, mode_T):
    T, d, B = mode_T, 8, 2
    q, k, v = rand((B, Hq, T, d), 23), rand((B, Hkv, T, d), 24), rand((B, Hkv, T, d), 25)
    scale = 1 / math.sqrt(d)
    pre = sdpa(q, k, v, scale, mask=torch_band(T, W, CAUSAL))  # library, not the oracle
    kr = np.full((B, Hkv, W, d), np.nan)
    vr = np.full((B, Hkv, W, d), np.nan)
    for p in range(T):
        oracle.ring_append(kr, vr, np.full(B, p), k[:, :, p], v[:, :, p])
        got = oracle.decode(q[:, :, p], kr, vr, np.full(B, p), scale)
        np.testing.assert_allclose(got, pre[:, :, p], rtol=0, atol=1e-12)


def test_decode_mixed_positions_and_empty_sequence():
    B, Hq, Hkv, W, d = 3, 2, 1, 4, 5
    rng = np.random.default_rng(26)
    q = rng.standard_normal((B, Hq, d))
    kr, vr = rng.standard_normal((B, Hkv, W, d)), rng.standard_normal((B, Hkv, W, d))
    pos = np.array([-1, 1, 9])
    out = oracle.decode(q, kr, vr, pos, 0.5)
    assert np.all(out[0] == 0.0)
    # position 1 sees slots 0 and 1 only; position 9 sees all four slots
    for b, slots in [(1, [0, 1]), (2, [0, 1, 2, 3])]:
        for h in range(Hq):
            s = 0.5 * kr[b, 0, slots] @ q[b, h]
            w = np.exp(s - s.max())
            want = (w / w.sum()) @ vr[b, 0, slots]
            np.testing.assert_allclose(out[b, h], want, rtol=0, atol=1e-13)


# ----------------------------------------------- planted mistakes are caught

def test_mutant_window_off_by_one_is_caught(monkeypatch, golden):
    g = golden("mask_counts_t16_w4.txt")

    def wide_mask(T, W, mode):
        pos = np.arange(T)
        off = pos[:, None] - pos[None, :]
        return (off >= 0) & (off <= W)  # one key too many

    monkeypatch.setattr(swa_ref, "window_mask", wide_mask)
    assert oracle.scores_per_layer(g["seq_len"], g["window"], CAUSAL) != g["scores_window"]
    assert swa_ref.stacked_reach(g["seq_len"], g["window"], 4) != g["reach"]


def test_mutant_window_without_self_is_caught(monkeypatch, golden):
    g = golden("mask_counts_t16_w4.txt")

    def shifted_mask(T, W, mode):
        pos = np.arange(T)
        off = pos[:, None] - pos[None, :]
        return (off > 0) & (off <= W)

    monkeypatch.setattr(swa_ref, "window_mask", shifted_mask)
    assert oracle.scores_per_layer(g["seq_len"], g["window"], CAUSAL) != g["scores_window"]


def test_mutant_gqa_mapping_is_caught(monkeypatch):
    T, d = 12, 4
    q, k, v = rand((1, 4, T, d), 27), rand((1, 2, T, d), 28), rand((1, 2, T, d), 29)
    want = sdpa(q, k, v, 0.5, mask=torch_band(T, 3, CAUSAL))
    monkeypatch.setattr(swa_ref, "kv_head", lambda h, Hq, Hkv: h % Hkv)  # interleaved groups
    got = swa_ref.attention_dense(q, k, v, 3, CAUSAL, 0.5)
    assert np.abs(got - want).max() > 1e-3


def test_mutant_swapped_operands_and_missing_scale_are_caught():
    T, d = 12, 4
    q, k, v = rand((1, 1, T, d), 30), rand((1, 1, T, d), 31), rand((1, 1, T, d), 32)
    want = sdpa(q, k, v, 0.5, mask=torch_band(T, 3, CAUSAL))
    assert np.abs(oracle.attention_dense(k, q, v, 3, CAUSAL, 0.5) - want).max() > 1e-3
    assert np.abs(oracle.attention_dense(q, k, v, 3, CAUSAL, 1.0) - want).max() > 1e-3


def test_mutant_ring_slot_is_caught():
    def shifted_append(k_ring, v_ring, pos, k_new, v_new):
        W = k_ring.shape[2]
        for b, p in enumerate(pos):
            k_ring[b, :, (p + 1) % W] = k_new[b]
            v_ring[b, :, (p + 1) % W] = v_new[b]

    assert not ring_last_writer_holds(shifted_append)


def test_mutant_symmetric_as_causal_is_caught():
    T, d, W = 15, 4, 6
    q, k, v = rand((1, 1, T, d), 33), rand((1, 1, T, d), 34), rand((1, 1, T, d), 35)
    want = sdpa(q, k, v, 0.5, mask=torch_band(T, W, SYMMETRIC))
    assert np.abs(oracle.attention_dense(q, k, v, W, CAUSAL, 0.5) - want).max() > 1e-3


# ------------------------------------------------ chunked prefill into a ring

@pytest.mark.parametrize("W,p,n", [(4, 0, 16), (4, 5, 7), (4, 9, 3), (6, 2, 11), (1, 7, 5),
                                   (16, 3, 13), (5, 10, 1), (3, 12, 4)])
def test_chunk_equals_prefill_rows(W, p, n):
    """A chunk at positions [p, p+n) after the ring took positions [0, p) (in
    two chunks) gives the library's masked-softmax rows p..p+n-1 of the whole
    sequence."""
    B, Hq, Hkv, d = 2, 4, 2, 8
    T = p + n
    q, k, v = rand((B, Hq, T, d), 60), rand((B, Hkv, T, d), 61), rand((B, Hkv, T, d), 62)
    scale = 1 / math.sqrt(d)
    want = sdpa(q, k, v, scale, mask=torch_band(T, W, CAUSAL))[:, :, p:]  # library, not the oracle
    kr = np.full((B, Hkv, W, d), np.nan)
    vr = np.full((B, Hkv, W, d), np.nan)
    cut = p // 2
    oracle.ring_append_chunk(kr, vr, np.zeros(B, dtype=int), k[:, :, :cut], v[:, :, :cut])
    oracle.ring_append_chunk(kr, vr, np.full(B, cut), k[:, :, cut:p], v[:, :, cut:p])
    got = oracle.prefill_chunk(q[:, :, p:], k[:, :, p:], v[:, :, p:], kr, vr, np.full(B, p), W, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_chunk_of_one_token_equals_decode():
    B, Hq, Hkv, W, d = 3, 4, 2, 5, 6
    rng = np.random.default_rng(63)
    q = rng.standard_normal((B, Hq, 1, d))
    k1, v1 = rng.standard_normal((B, Hkv, 1, d)), rng.standard_normal((B, Hkv, 1, d))
    kr, vr = rng.standard_normal((B, Hkv, W, d)), rng.standard_normal((B, Hkv, W, d))
    pos = np.array([0, 3, 11])
    got = oracle.prefill_chunk(q, k1, v1, kr, vr, pos, W, 0.7)
    oracle.ring_append(kr, vr, pos, k1[:, :, 0], v1[:, :, 0])
    want = oracle.decode(q[:, :, 0], kr, vr, pos, 0.7)
    np.testing.assert_allclose(got[:, :, 0], want, rtol=0, atol=1e-13)


def test_chunk_negative_position_gives_zeros_and_writes_nothing():
    rng = np.random.default_rng(64)
    q = rng.standard_normal((2, 2, 3, 4))
    k, v = rng.standard_normal((2, 1, 3, 4)), rng.standard_normal((2, 1, 3, 4))
    kr, vr = rng.standard_normal((2, 1, 5, 4)), rng.standard_normal((2, 1, 5, 4))
    out = oracle.prefill_chunk(q, k, v, kr, vr, np.array([-1, 2]), 5, 0.5)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out[1]))
    kr0, vr0 = kr.copy(), vr.copy()
    oracle.ring_append_chunk(kr, vr, np.array([-3, 2]), k, v)
    assert np.array_equal(kr[0], kr0[0]) and np.array_equal(vr[0], vr0[0])
    assert not np.array_equal(kr[1], kr0[1])


@pytest.mark.parametrize("W,p,n", [(5, 0, 3), (5, 3, 4), (5, 7, 12), (1, 4, 3), (8, 13, 8),
                                   (6, 2, 6)])
def test_append_chunk_closed_form(W, p, n):
    """Slot s ends up holding chunk token i* = n-1 - ((p+n-1-s) mod W) (the
    last token whose position is s mod W) when i* >= 0; the other slots keep
    their previous contents."""
    B, Hkv, d = 2, 3, 4
    rng = np.random.default_rng(65)
    k, v = rng.standard_normal((B, Hkv, n, d)), rng.standard_normal((B, Hkv, n, d))
    kr, vr = np.full((B, Hkv, W, d), -9.0), np.full((B, Hkv, W, d), -9.0)
    oracle.ring_append_chunk(kr, vr, np.full(B, p), k, v)
    for s in range(W):
        i_star = n - 1 - ((p + n - 1 - s) % W)
        if i_star >= 0:
            assert np.array_equal(kr[:, :, s], k[:, :, i_star]), s
            assert np.array_equal(vr[:, :, s], v[:, :, i_star]), s
        else:
            assert np.all(kr[:, :, s] == -9.0) and np.all(vr[:, :, s] == -9.0), s


def test_mutant_chunk_appended_before_it_is_read_is_caught():
    """Reading the ring after the chunk was written into it (the wrong order)
    loses keys the early rows of the chunk need."""
    B, Hq, Hkv, d, W, p, n = 1, 2, 1, 8, 4, 9, 3
    T = p + n
    q, k, v = rand((B, Hq, T, d), 66), rand((B, Hkv, T, d), 67), rand((B, Hkv, T, d), 68)
    want = sdpa(q, k, v, 0.5, mask=torch_band(T, W, CAUSAL))[:, :, p:]
    kr, vr = np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, W, d))
    oracle.ring_append_chunk(kr, vr, np.zeros(B, dtype=int), k, v)  # positions 0..T-1, too far
    got = oracle.prefill_chunk(q[:, :, p:], k[:, :, p:], v[:, :, p:], kr, vr, np.full(B, p), W, 0.5)
    assert np.abs(got - want).max() > 1e-3


def test_mutant_chunk_ring_slot_is_caught():
    """A ring filled one slot off (position p' in slot (p'+1) mod W) gives
    different chunk rows."""
    B, Hq, Hkv, d, W, p, n = 1, 2, 1, 8, 4, 9, 3
    T = p + n
    q, k, v = rand((B, Hq, T, d), 69), rand((B, Hkv, T, d), 70), rand((B, Hkv, T, d), 71)
    want = sdpa(q, k, v, 0.5, mask=torch_band(T, W, CAUSAL))[:, :, p:]
    kr, vr = np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, W, d))
    for t in range(p):
        kr[:, :, (t + 1) % W] = k[:, :, t]
        vr[:, :, (t + 1) % W] = v[:, :, t]
    got = oracle.prefill_chunk(q[:, :, p:], k[:, :, p:], v[:, :, p:], kr, vr, np.full(B, p), W, 0.5)
    assert np.abs(got - want).max() > 1e-3


# ------------------------------------------------------ dilated sliding window

def test_page_dilation_example(golden):
    """An interior row of the symmetric window W=512 at dilation 2 has 256 keys
    on each side and spans 1024 positions (aivaro section 4.2)."""
    g = golden("dilation_longformer.txt")
    W, dil = g["window"], g["dilation"]
    T = 2 * dil * W + 1
    i = T // 2
    row = oracle.dilated_mask(T, W, SYMMETRIC, dil)[i]
    keys = np.flatnonzero(row)
    assert int((keys < i).sum()) == g["keys_each_side"] == int((keys > i).sum())
    assert int(keys.max() - keys.min()) == g["span"]


def test_mutant_dilation_as_subsampled_window_is_caught(golden):
    """The other reading (every d-th key of the undilated window) gives 128
    keys a side over 512 positions and fails the page's example."""
    g = golden("dilation_longformer.txt")
    W, dil = g["window"], g["dilation"]
    T = 2 * dil * W + 1
    i = T // 2
    row = oracle.window_mask(T, W, SYMMETRIC)[i] & ((i - np.arange(T)) % dil == 0)
    keys = np.flatnonzero(row)
    assert int((keys < i).sum()) != g["keys_each_side"]
    assert int(keys.max() - keys.min()) != g["span"]


@pytest.mark.parametrize("mode,T,W,dil", [(CAUSAL, 23, 4, 2), (CAUSAL, 31, 5, 3),
                                          (SYMMETRIC, 29, 6, 2), (SYMMETRIC, 26, 5, 4),
                                          (CAUSAL, 17, 3, 7), (SYMMETRIC, 12, 16, 3)])
def test_dilated_equals_plain_window_on_strided_subsequences(mode, T, W, dil):
    """Key j is visible from query i only when i = j (mod d), and then through
    the plain window on the offset / d: dilated attention over the sequence is
    plain windowed attention (pinned above) over each of the d subsequences
    r, r+d, r+2d, ..."""
    B, Hq, Hkv, d = 2, 4, 2, 8
    q, k, v = rand((B, Hq, T, d), 90), rand((B, Hkv, T, d), 91), rand((B, Hkv, T, d), 92)
    got = oracle.attention_dilated_dense(q, k, v, W, mode, 0.4, dil)
    for r in range(dil):
        sub = oracle.attention_dense(q[:, :, r::dil], k[:, :, r::dil], v[:, :, r::dil], W, mode, 0.4)
        np.testing.assert_allclose(got[:, :, r::dil], sub, rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,W,dil", [(40, 4, 3), (64, 16, 2), (10, 20, 5)])
def test_dilated_causal_key_counts(T, W, dil):
    """Causal row i has min(W, i // d + 1) keys."""
    rows = oracle.dilated_mask(T, W, CAUSAL, dil).sum(axis=1)
    assert rows.tolist() == [min(W, i // dil + 1) for i in range(T)]


def test_dilation_one_is_the_plain_window():
    for mode in (CAUSAL, SYMMETRIC):
        assert np.array_equal(oracle.dilated_mask(21, 6, mode, 1), oracle.window_mask(21, 6, mode))
    q, k, v = rand((1, 2, 19, 8), 93), rand((1, 1, 19, 8), 94), rand((1, 1, 19, 8), 95)
    want = sdpa(q, k, v, 0.3, mask=torch_band(19, 5, CAUSAL))  # library
    np.testing.assert_allclose(oracle.attention_dilated_dense(q, k, v, 5, CAUSAL, 0.3, 1), want,
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_dilated_rows_agree_with_dense(mode):
    T, W, dil = 37, 6, 3
    q, k, v = rand((1, 4, T, 8), 96), rand((1, 2, T, 8), 97), rand((1, 2, T, 8), 98)
    dense = oracle.attention_dilated_dense(q, k, v, W, mode, 0.5, dil)
    rows = [0, 1, 2, 5, 17, 35, 36]
    for h in range(4):
        got = oracle.attention_dilated_rows(q, k, v, W, mode, 0.5, dil, 0, h, rows)
        np.testing.assert_allclose(got, dense[0, h, rows], rtol=0, atol=1e-12)


# ------------------------------------------------------- global tokens

@pytest.mark.parametrize("T,W,Hq,Hkv", [(20, 4, 2, 1), (33, 7, 4, 2)])
def test_all_global_is_full_attention(T, W, Hq, Hkv):
    """Every token global: the library's full attention (bidirectional, or
    causal in the causal mode)."""
    d = 8
    q, k, v = rand((1, Hq, T, d), 100), rand((1, Hkv, T, d), 101), rand((1, Hkv, T, d), 102)
    allg = np.arange(T)
    got = oracle.attention_global_dense(q, k, v, W, SYMMETRIC, 0.3, allg)
    np.testing.assert_allclose(got, sdpa(q, k, v, 0.3), rtol=0, atol=1e-12)
    got = oracle.attention_global_dense(q, k, v, W, CAUSAL, 0.3, allg)
    np.testing.assert_allclose(got, sdpa(q, k, v, 0.3, is_causal=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_no_global_is_the_window(mode):
    T, d = 25, 8
    q, k, v = rand((1, 2, T, d), 103), rand((1, 1, T, d), 104), rand((1, 1, T, d), 105)
    want = sdpa(q, k, v, 0.4, mask=torch_band(T, 6, mode))  # library
    got = oracle.attention_global_dense(q, k, v, 6, mode, 0.4, [])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode,T,W,gpos", [(SYMMETRIC, 40, 6, [0]), (SYMMETRIC, 40, 6, [0, 17, 39]),
                                           (CAUSAL, 40, 5, [0, 1, 2]), (CAUSAL, 31, 4, [3, 20])])
def test_global_pair_count_closed_form(mode, T, W, gpos):
    """|window U rows(G) U cols(G)| by inclusion-exclusion: the window, plus
    each global row and column (T each, or its causal part), minus what the
    window already holds, minus the doubly counted (global, global) pairs."""
    win = oracle.window_mask(T, W, mode)
    g = np.zeros(T, dtype=bool)
    g[gpos] = True
    if mode == SYMMETRIC:
        rows_cols = 2 * len(gpos) * T - len(gpos) ** 2
        overlap = int(win[g, :].sum() + win[:, g].sum() - win[np.ix_(g, g)].sum())
    else:
        # causal: row i of a global token adds keys 0..i, column j adds queries j..T-1
        rows_cols = sum(i + 1 for i in gpos) + sum(T - j for j in gpos) \
            - sum(1 for a in gpos for b in gpos if b <= a)
        overlap = int(win[g, :].sum() + win[:, g].sum() - win[np.ix_(g, g)].sum())
    want = int(win.sum()) + rows_cols - overlap
    assert int(oracle.global_mask(T, W, mode, gpos).sum()) == want


def test_global_cost_is_linear_per_token():
    """Each global token adds at most 2T - 1 pairs (its row and column): the
    O(n) extra work per global token of aivaro section 4.3."""
    T, W = 300, 32
    base = int(oracle.window_mask(T, W, SYMMETRIC).sum())
    for G in (1, 5, 10):
        gpos = list(range(0, T, T // G))[:G]
        extra = int(oracle.global_mask(T, W, SYMMETRIC, gpos).sum()) - base
        assert extra <= G * (2 * T - 1)


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_global_rows_agree_with_dense(mode):
    T, W = 45, 6
    gpos = [0, 9, 10, 44]
    q, k, v = rand((1, 4, T, 8), 106), rand((1, 2, T, 8), 107), rand((1, 2, T, 8), 108)
    dense = oracle.attention_global_dense(q, k, v, W, mode, 0.5, gpos)
    rows = [0, 1, 5, 9, 10, 11, 20, 43, 44]
    for h in range(4):
        got = oracle.attention_global_rows(q, k, v, W, mode, 0.5, gpos, 0, h, rows)
        np.testing.assert_allclose(got, dense[0, h, rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_global_token_row_is_full_attention(mode):
    """A global token's own row attends to every key (every earlier key in
    the causal mode): the library's full-attention row."""
    T, gpos = 30, [4, 21]
    q, k, v = rand((1, 2, T, 8), 112), rand((1, 2, T, 8), 113), rand((1, 2, T, 8), 114)
    got = oracle.attention_global_dense(q, k, v, 3, mode, 0.6, gpos)
    full = sdpa(q, k, v, 0.6, is_causal=mode == CAUSAL)
    np.testing.assert_allclose(got[:, :, gpos], full[:, :, gpos], rtol=0, atol=1e-12)


def test_mutant_global_columns_only_is_caught():
    """Forgetting the global rows (tokens attend to the global token, but it
    does not attend to everything) fails the global-row pin."""
    T, g = 20, 5
    q, k, v = rand((1, 1, T, 8), 109), rand((1, 1, T, 8), 110), rand((1, 1, T, 8), 111)
    M = oracle.window_mask(T, 4, SYMMETRIC).copy()
    M[:, g] = True
    S = 0.3 * (q[0, 0] @ k[0, 0].T) + np.where(M, 0.0, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    wrong = (P / P.sum(axis=1, keepdims=True)) @ v[0, 0]
    full = sdpa(q, k, v, 0.3)[0, 0]
    assert np.abs(wrong[g] - full[g]).max() > 1e-3


# ------------------------------------------ dilated window plus global tokens

def brute_dilated_global(T, W, mode, dil, gpos):
    """Pair by pair: key j is in query i's dilated window (i - j a multiple of
    dil whose quotient lies in the plain window), or i or j is a global
    position (j <= i when causal)."""
    g = set(gpos)
    M = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            win = False
            if (i - j) % dil == 0:
                m = (i - j) // dil
                win = 0 <= m <= W - 1 if mode == CAUSAL else -(W // 2) <= m <= W // 2
            M[i, j] = win or ((i in g or j in g) and (mode != CAUSAL or j <= i))
    return M


@pytest.mark.parametrize("T,W,mode,dil,gpos", [
    (12, 3, CAUSAL, 2, [0]), (12, 3, SYMMETRIC, 2, [5]), (17, 4, CAUSAL, 3, [0, 1, 16]),
    (17, 5, SYMMETRIC, 3, [2, 9]), (9, 1, CAUSAL, 2, [4]), (20, 6, SYMMETRIC, 4, [0, 10, 19]),
    (7, 10, CAUSAL, 2, [3]), (11, 2, SYMMETRIC, 5, []),
])
def test_dilated_global_mask_by_brute_force(T, W, mode, dil, gpos):
    assert np.array_equal(oracle.global_mask(T, W, mode, gpos, dil),
                          brute_dilated_global(T, W, mode, dil, gpos))


def test_dilated_global_pair_counts_by_hand():
    """T = 8, W = 2, dilation 2.  Causal, global position 0: row i sees i and
    i - 2 (14 pairs); key 0 adds rows 1, 3, 4, 5, 6, 7 (row 2 already sees it
    through its window, row 0 is the global row and sees only key 0): 20.
    Symmetric, global position 3: row i sees i and i +- 2 inside [0, 8)
    (2+2+3+3+3+3+2+2 = 20); row 3 sees the 5 keys 0, 2, 4, 6, 7 beyond its
    window and column 3 adds rows 0, 2, 4, 6, 7 (rows 1 and 5 have it): 30."""
    assert int(oracle.global_mask(8, 2, CAUSAL, [0], 2).sum()) == 20
    assert int(oracle.global_mask(8, 2, SYMMETRIC, [3], 2).sum()) == 30


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_dilated_global_reduces_to_its_parts(mode):
    T, W = 40, 5
    assert np.array_equal(oracle.global_mask(T, W, mode, [], 3), oracle.dilated_mask(T, W, mode, 3))
    assert np.array_equal(oracle.global_mask(T, W, mode, [2, 30], 1),
                          oracle.global_mask(T, W, mode, [2, 30]))


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_dilated_global_rows_agree_with_dense(mode):
    T, W, dil = 45, 6, 3
    gpos = [0, 9, 10, 44]
    q, k, v = rand((1, 4, T, 8), 115), rand((1, 2, T, 8), 116), rand((1, 2, T, 8), 117)
    dense = oracle.attention_global_dense(q, k, v, W, mode, 0.5, gpos, dil)
    rows = [0, 1, 3, 5, 9, 10, 11, 12, 20, 43, 44]
    for h in range(4):
        got = oracle.attention_global_rows(q, k, v, W, mode, 0.5, gpos, 0, h, rows, dil)
        np.testing.assert_allclose(got, dense[0, h, rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_dilated_global_token_row_is_full_attention(mode):
    T, gpos = 30, [4, 21]
    q, k, v = rand((1, 2, T, 8), 118), rand((1, 2, T, 8), 119), rand((1, 2, T, 8), 120)
    got = oracle.attention_global_dense(q, k, v, 3, mode, 0.6, gpos, 4)
    full = sdpa(q, k, v, 0.6, is_causal=mode == CAUSAL)
    np.testing.assert_allclose(got[:, :, gpos], full[:, :, gpos], rtol=0, atol=1e-12)


def test_mutant_plain_window_exclusion_is_caught():
    """Excluding a global key from a row when it lies in the row's plain
    (undilated) span rather than on its dilated grid would drop keys the row
    must see: the brute-force mask tells them apart."""
    T, W, dil, gpos = 12, 3, 2, [5]
    wrong = oracle.dilated_mask(T, W, SYMMETRIC, dil).copy()
    for i in range(T):
        if abs(i - 5) > W // 2:  # outside the plain span: the (wrong) rule adds the column
            wrong[i, 5] = True
    wrong[5, :] = True
    assert not np.array_equal(wrong, brute_dilated_global(T, W, SYMMETRIC, dil, gpos))


# ------------------------------------------------------ attention sinks

@pytest.mark.parametrize("W,S,T", [(4, 2, 16), (5, 4, 30), (8, 8, 20), (3, 1, 9), (6, 9, 25)])
def test_decode_with_sinks_equals_library_masked_row(W, S, T):
    """Filling the ring and the sink slots from a sequence and decoding every
    position gives the library's attention row p with the mask 'window of p
    or one of the first S positions' (built with torch's triangle routines)."""
    B, Hq, Hkv, d = 2, 4, 2, 8
    q, k, v = rand((B, Hq, T, d), 120), rand((B, Hkv, T, d), 121), rand((B, Hkv, T, d), 122)
    mask = torch_band(T, W, CAUSAL)
    first_cols = torch.ones(T, T, dtype=torch.bool).tril(0)
    first_cols[:, S:] = False
    want = sdpa(q, k, v, 0.5, mask=mask | first_cols.numpy())  # library
    kr, vr = np.full((B, Hkv, W, d), np.nan), np.full((B, Hkv, W, d), np.nan)
    ks, vs = k[:, :, :S].copy(), v[:, :, :S].copy()
    for p in range(T):
        oracle.ring_append(kr, vr, np.full(B, p), k[:, :, p], v[:, :, p])
        got = oracle.decode_sinks(q[:, :, p], kr, vr, ks, vs, np.full(B, p), 0.5)
        np.testing.assert_allclose(got, want[:, :, p], rtol=0, atol=1e-12)


def test_decode_with_no_sinks_is_decode():
    rng = np.random.default_rng(123)
    q = rng.standard_normal((3, 4, 6))
    kr, vr = rng.standard_normal((3, 2, 5, 6)), rng.standard_normal((3, 2, 5, 6))
    empty = np.zeros((3, 2, 0, 6))
    pos = np.array([-1, 2, 17])
    np.testing.assert_allclose(oracle.decode_sinks(q, kr, vr, empty, empty, pos, 0.3),
                               oracle.decode(q, kr, vr, pos, 0.3), rtol=0, atol=1e-13)


def test_mutant_sinks_counted_twice_is_caught():
    """Reading the sinks in addition to a window that already holds them
    double-counts them and fails the library pin."""
    W, S, T, d = 6, 3, 8, 8
    q, k, v = rand((1, 1, T, d), 124), rand((1, 1, T, d), 125), rand((1, 1, T, d), 126)
    p = 4  # the window [0, 4] holds all three sinks
    keys = np.concatenate([np.arange(S), np.arange(0, p + 1)])
    sc = 0.5 * (k[0, 0, keys] @ q[0, 0, p])
    e = np.exp(sc - sc.max())
    wrong = (e / e.sum()) @ v[0, 0, keys]
    want = sdpa(q, k, v, 0.5, mask=torch_band(T, W, CAUSAL))[0, 0, p]
    assert np.abs(wrong - want).max() > 1e-3
