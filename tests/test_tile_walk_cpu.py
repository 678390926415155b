"""CPU check of the bf16 prefill kernels' index arithmetic.

tests/tile_walk.cpp is built with the host compiler from the same header the
kernels use for their tile ranges, tile classification, masks and load
addresses (sliding_window_attention_swa_amd/csrc/swa_tile_math.h).  It replays
the kernels' loops over workgroups, waves, lanes and tiles and reports any
load outside its buffer resource, any counted key whose LDS row holds other
data (a clamped row), any key counted twice, and per query row the set of
keys it counts.  Here every row's set is compared with the fp64 oracle's
mask for that row: the plain causal and symmetric windows, the dilated
windows (dilation above T included), the chunk continuing a ring, the window
plus global tokens (also dilated), the short-window kernel, the global-row
kernel and the fp32 matrix-core kernel.  No GPU is involved.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sliding_window_attention_swa_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "tile_walk.cpp")

CAUSAL, SYMMETRIC = 0, 1


@pytest.fixture(scope="module")
def walker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("walk") / "tile_walk")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", exe],
                   check=True)
    return exe


def run(walker, lines):
    """Feed shape lines to the walker; one result dict per shape."""
    out = subprocess.run([walker], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         check=True).stdout
    results, cur = [], {"rows": {}, "problems": []}
    for line in out.splitlines():
        tok = line.split()
        if tok[0] == "END":
            results.append(cur)
            cur = {"rows": {}, "problems": []}
        elif tok[0] == "R":
            cur["rows"][int(tok[1])] = tuple(int(x) for x in tok[2:])
        else:
            cur["problems"].append(line)
    assert len(results) == len(lines)
    return results


def signature(keys):
    keys = np.asarray(keys, dtype=np.int64)
    return (len(keys), int(keys.sum()), int((keys * keys).sum()))


def expect_rows(mask, rows=None):
    rows = range(mask.shape[0]) if rows is None else rows
    return {i: signature(np.nonzero(mask[i])[0]) for i in rows}


def check(res, want, what):
    assert not res["problems"], (what, res["problems"][:5])
    got = res["rows"]
    missing = sorted(set(want) - set(got))
    assert not missing, (what, "rows without keys", missing[:5])
    for i, sig in want.items():
        assert got[i] == sig, (what, "row", i, "counts", got[i], "want", sig)


T_LIST = [1, 5, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 257, 300, 513]
W_LIST = [1, 2, 3, 16, 31, 32, 33, 34, 63, 64, 65, 100, 128, 129, 255, 256, 257, 512, 1000]


def plain_shapes():
    rng = np.random.default_rng(7)
    shapes = []
    for T in T_LIST:
        for W in W_LIST:
            for mode in (CAUSAL, SYMMETRIC):
                shapes.append((mode, T, W, int(rng.choice([32, 64, 128]))))
    return shapes


def test_plain_windows_tiled(walker):
    """Causal and symmetric windows through the tiled kernel: every row counts
    exactly its window, loads stay inside their tiles."""
    shapes = plain_shapes()
    res = run(walker, ["tiled %d %d %d 1 0 %d 0" % (m, T, W, D) for m, T, W, D in shapes])
    for (m, T, W, D), r in zip(shapes, res):
        check(r, expect_rows(oracle.window_mask(T, W, m)), ("tiled", m, T, W, D))


def test_symmetric_block_classes_every_alignment(walker):
    """Symmetric edge tiles skip, take whole or mask each 32-key block: half
    windows of every residue mod 32 (and both parities of W), sequence ends
    inside and at block boundaries."""
    shapes = [(T, W) for T in (96, 129, 300) for W in range(2, 140)]
    res = run(walker, ["tiled 1 %d %d 1 0 64 0" % (T, W) for T, W in shapes])
    for (T, W), r in zip(shapes, res):
        check(r, expect_rows(oracle.window_mask(T, W, SYMMETRIC)), ("sym blocks", T, W))


def test_short_window_kernel(walker):
    """The short-window kernel (causal W <= 33, symmetric W/2 <= 16; any W
    is walked): each row's 64-key block holds its whole window."""
    shapes = [(m, T, W, D) for (m, T, W, D) in plain_shapes()
              if (m == CAUSAL and W <= 33) or (m == SYMMETRIC and W // 2 <= 16)]
    assert len(shapes) > 40
    res = run(walker, ["short %d %d %d %d" % (m, T, W, D) for m, T, W, D in shapes])
    for (m, T, W, D), r in zip(shapes, res):
        check(r, expect_rows(oracle.window_mask(T, W, m)), ("short", m, T, W, D))


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_dilated_windows(walker, mode):
    """Residue-class workgroups of the dilated modes (3, 4), dilations 2-9
    and above T: each row counts its dilated window, strided loads stay
    inside the class rows."""
    shapes = []
    for T in (1, 7, 64, 129, 300, 513):
        for W in (1, 4, 33, 65, 128, 300):
            for dil in (2, 3, 5, 9, T + 3):
                shapes.append((T, W, dil, 64 if (T + W + dil) % 2 else 128))
    kmode = 3 if mode == CAUSAL else 4
    res = run(walker, ["tiled %d %d %d %d 0 %d 0" % (kmode, T, W, dil, D) for T, W, dil, D in shapes])
    for (T, W, dil, D), r in zip(shapes, res):
        check(r, expect_rows(oracle.dilated_mask(T, W, mode, dil)), ("dilated", mode, T, W, dil))


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_fp32_matrix_core_kernel(walker, mode):
    """The fp32 matrix-core kernel (4-byte rows, plain and dilated windows,
    edge tiles masked by the direct test): each row counts exactly its
    window, loads stay inside their tiles and class rows."""
    shapes = [(T, W, 1, D) for (m, T, W, D) in plain_shapes() if m == mode]
    for T in (1, 64, 129, 300, 513):
        for W in (1, 33, 65, 300):
            for dil in (2, 5, T + 3):
                shapes.append((T, W, dil, 32 if (T + W) % 3 == 0 else (64 if (T + W) % 3 == 1 else 128)))
    res = run(walker, ["tiledf32 %d %d %d %d 0 %d 0" % (mode, T, W, dil, D) for T, W, dil, D in shapes])
    for (T, W, dil, D), r in zip(shapes, res):
        want = oracle.window_mask(T, W, mode) if dil == 1 else oracle.dilated_mask(T, W, mode, dil)
        check(r, expect_rows(want), ("fp32", mode, T, W, dil, D))


def chunk_window(n, W, p):
    """Rows of a chunk at position p: position p + i sees [max(0, p+i-W+1), p+i]."""
    want = {}
    for i in range(n):
        P = p + i
        want[P] = signature(np.arange(max(0, P - W + 1), P + 1))
    return want


def test_chunk_continuing_a_ring(walker):
    """Chunked prefill (mode 2): ring tiles for the positions before the chunk
    (slot = position mod W), chunk tiles after; rows before position 0 are
    never counted; ring reads stay inside the W slots."""
    shapes = []
    for n in (1, 5, 64, 65, 128, 200, 300):
        for W in (1, 3, 32, 64, 65, 100, 256, 513):
            for p in (0, 1, 7, W - 1, W, W + 5, 3 * W + 17, 1000):
                if p >= 0:
                    shapes.append((n, W, p, 128 if (n + W) % 2 else 64))
    res = run(walker, ["tiled 2 %d %d 1 %d %d 0" % (n, W, p, D) for n, W, p, D in shapes])
    for (n, W, p, D), r in zip(shapes, res):
        check(r, chunk_window(n, W, p), ("chunk", n, W, p))
    # the fp32 matrix-core kernel's chunk mode (4-byte rows, direct masks)
    res = run(walker, ["tiledf32 2 %d %d 1 %d %d 0" % (n, W, p, D) for n, W, p, D in shapes])
    for (n, W, p, D), r in zip(shapes, res):
        check(r, chunk_window(n, W, p), ("chunk fp32", n, W, p))


GLOBALS = [[0], [0, 1, 2, 3, 4, 5, 6, 7], [3, 40, 41, 200], [10, 77, 150, 299, 500],
           list(range(0, 300, 4)), [-5, 2, 9, 10_000]]


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
@pytest.mark.parametrize("dil", [1, 2, 3])
def test_window_plus_global_tokens(walker, mode, dil):
    """Modes 5-8: after the window tiles, the gathered global key tiles; a
    global key is counted once (not again when already in the window), never
    after the row when causal, positions outside [0, T) ignored.  Non-global
    rows are compared here; the global rows come from the global-row pass."""
    shapes = []
    for T in (1, 64, 129, 300, 513):
        for W in (4, 33, 65, 200):
            for g in GLOBALS:
                shapes.append((T, W, g))
    kmode = (5 if mode == CAUSAL else 6) if dil == 1 else (7 if mode == CAUSAL else 8)
    lines = ["tiled %d %d %d %d 0 64 %d %s" % (kmode, T, W, dil, len(g), " ".join(map(str, g)))
             for T, W, g in shapes]
    # the bf16 kernel (d = 64), then the fp32 matrix-core kernel (4-byte rows)
    fmode = 5 if mode == CAUSAL else 6
    lines += ["tiledf32 %d %d %d %d 0 %d %d %s" % (fmode, T, W, dil, 32 if T % 2 else 128, len(g),
                                                  " ".join(map(str, g))) for T, W, g in shapes]
    res = run(walker, lines)
    for (T, W, g), r in zip(shapes + shapes, res):
        valid = sorted(p for p in g if 0 <= p < T)
        mask = oracle.global_mask(T, W, mode, valid, dil)
        rows = [i for i in range(T) if i not in set(valid)]
        check({"rows": {i: r["rows"][i] for i in rows if i in r["rows"]},
               "problems": r["problems"]}, expect_rows(mask, rows), ("global", mode, dil, T, W, g))


@pytest.mark.parametrize("mode", [CAUSAL, SYMMETRIC])
def test_global_row_units(walker, mode):
    """The global-row pass: split-K over 128-key chunks, each global row counts
    every key (every earlier key when causal), loads clamped inside the
    sequence."""
    shapes = [(T, g) for T in (1, 100, 128, 129, 513, 1000) for g in GLOBALS]
    lines = ["grows %d %d 128 %d %s" % (mode, T, len(g), " ".join(map(str, g))) for T, g in shapes]
    res = run(walker, lines)
    for (T, g), r in zip(shapes, res):
        valid = sorted(p for p in g if 0 <= p < T)
        if not valid:
            assert not r["problems"] and not r["rows"]
            continue
        mask = oracle.global_mask(T, 4, mode, valid)
        check(r, expect_rows(mask, valid), ("grows", mode, T, g))


def test_walker_catches_a_wrong_window(walker):
    """The comparison has teeth: the walk of W is not the oracle's W + 1."""
    r = run(walker, ["tiled 0 300 100 1 0 128 0"])[0]
    with pytest.raises(AssertionError):
        check(r, expect_rows(oracle.window_mask(300, 101, CAUSAL)), "planted")
