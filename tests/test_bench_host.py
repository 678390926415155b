"""CPU tests of bench.py's host logic: the work counts its figures divide by
(in-window pairs, FLOPs, algorithmic bytes) against the oracle's masks and
brute force, the traffic read-back guard, and the one-GPU refusal."""

import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import swa_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("T,W", [(16, 4), (16, 16), (50, 7), (7, 50), (1, 1)])
def test_causal_pairs_are_the_mask_count(T, W):
    assert bench.band_pairs_causal(T, W) == int(oracle.window_mask(T, W, oracle.CAUSAL).sum())
    assert bench.band_pairs(T, W, 0) == bench.band_pairs_causal(T, W)


@pytest.mark.parametrize("T,W,mode,dil", [(50, 7, 1, 1), (53, 8, 1, 2), (40, 100, 1, 3),
                                          (50, 7, 0, 3), (61, 5, 0, 4), (9, 4, 1, 11)])
def test_band_pairs_are_the_mask_count(T, W, mode, dil):
    assert bench.band_pairs(T, W, mode, dil) == int(oracle.dilated_mask(T, W, mode, dil).sum())


@pytest.mark.parametrize("T,W,mode,gpos", [(50, 7, 1, [0]), (50, 7, 0, [0, 3, 49]),
                                           (61, 9, 1, list(range(0, 61, 5))), (40, 100, 0, [10, 20]),
                                           (33, 1, 0, [32]), (33, 4, 1, [])])
def test_global_pairs_are_the_mask_count(T, W, mode, gpos):
    assert bench.global_pairs(T, W, mode, gpos) == int(oracle.global_mask(T, W, mode, gpos).sum())


@pytest.mark.parametrize("T,W,mode,gpos,dil", [(50, 7, 1, [0], 2), (50, 7, 0, [0, 3, 49], 3),
                                               (61, 9, 1, list(range(0, 61, 5)), 4),
                                               (40, 100, 0, [10, 20], 2), (33, 1, 0, [32], 5),
                                               (33, 4, 1, [], 3), (8, 2, 1, [3], 2)])
def test_dilated_global_pairs_are_the_mask_count(T, W, mode, gpos, dil):
    assert bench.global_pairs(T, W, mode, gpos, dil) == int(
        oracle.global_mask(T, W, mode, gpos, dil).sum())


def test_prefill_and_decode_work_of_the_workloads():
    flops, bytes_ = bench.prefill_work()
    assert flops == 962106228736  # 4 * 128 * 58,722,304 pairs * 32 heads
    assert bytes_ == 335544320    # Q, K, V, O in bf16
    pos = np.array([4096, 5000, 10, 0], dtype=np.int32)
    flops, kv, qo = bench.decode_work(pos)
    rows = 4096 + 4096 + 11 + 1
    c = si.WORKLOADS[4]
    assert kv == rows * c["Hkv"] * c["d"] * 4
    assert flops == 4 * c["d"] * rows * c["Hq"]


def test_chunk_work_by_brute_force():
    c = dict(si.WORKLOADS[6], B=3, n=9, W=5, d=8, Hq=4, Hkv=2)
    pos = np.array([0, 2, 40])
    flops, bytes_ = bench.chunk_work(c, pos)
    keys = 0
    ring_rows = 0
    for p in pos:
        for i in range(c["n"]):
            P = p + i
            keys += len(range(max(0, P - c["W"] + 1), P + 1))
        ring_rows += len(range(max(0, p - c["W"] + 1), p))  # ring positions some row reads
    assert flops == 4 * c["d"] * keys * c["Hq"]
    assert bytes_ == 2 * c["d"] * (c["B"] * c["n"] * (2 * c["Hq"] + 2 * c["Hkv"])
                                   + 2 * c["Hkv"] * ring_rows)


def test_traffic_is_null_for_another_source(tmp_path, monkeypatch):
    f = tmp_path / "t.md"
    f.write_text("traffic_bytes_per_launch: 123\ntraffic_kernel_sha256: %s\n"
                 % bench.source_hash(bench.PREFILL_SOURCE))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic("", bench.PREFILL_SOURCE) == 123
    f.write_text("traffic_bytes_per_launch: 123\ntraffic_kernel_sha256: 00\n")
    assert bench.read_traffic("", bench.PREFILL_SOURCE) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_summary_arithmetic(tmp_path, capsys):
    """A synthetic prefill dispatch of 1 ms at 1.8 GHz on every XCD, with the
    matrix cores busy half of the SIMD cycles and exactly the in-window FLOPs
    issued."""
    flops, _ = bench.prefill_work()
    cycles = 1.8e9 * 1e-3
    rows = [("GRBM_GUI_ACTIVE", cycles * bench.N_XCD),
            ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cycles * bench.N_SIMD),
            ("SQ_INSTS_VALU_MFMA_MOPS_BF16", flops / 512)]
    f = tmp_path / "c.csv"
    with open(f, "w") as fh:
        fh.write('"Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
        for name, val in rows:
            fh.write('"swa::prefill_bf16_kernel<128, 0>","%s",%r,1000000,2000000\n' % (name, val))
    assert bench.summarize_counters([str(f)]) == 0
    out = capsys.readouterr().out
    assert "clock 1800 MHz" in out
    assert "MFMA busy: 50.0%" in out
    assert "1.000 x the in-window FLOPs" in out


def test_small_traffic_summary(tmp_path, capsys):
    """Counters that read exactly the algorithmic bytes (with FETCH_SIZE
    reading half the bytes, as the calibration copy shows) are reported as
    such."""
    rows = [("__amd_rocclr_copyBuffer", "FETCH_SIZE", bench.COPY_BYTES / 2048),
            ("__amd_rocclr_copyBuffer", "WRITE_SIZE", bench.COPY_BYTES / 1024)]
    for wl, pat in bench.SMALL_TRAFFIC:
        c = si.WORKLOADS[wl]
        rd = 2 * c["T"] * c["d"] * c["B"] * (c["Hq"] + 2 * c["Hkv"])
        wr = 2 * c["T"] * c["d"] * c["B"] * c["Hq"]
        rows += [("swa::%s<...>" % pat, "FETCH_SIZE", rd / 2048), ("swa::%s<...>" % pat, "WRITE_SIZE", wr / 1024)]
    f = tmp_path / "c.csv"
    with open(f, "w") as fh:
        fh.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for n, ctr, v in rows:
            fh.write('"%s","%s",%r\n' % (n, ctr, v))
    assert bench.summarize_pmc_small([str(f)]) == 0
    out = capsys.readouterr().out.splitlines()
    assert len(out) == len(bench.SMALL_TRAFFIC)
    for line in out:
        nums = [int(x) for x in line.replace("(", " ").replace(")", " ").replace(",", " ").split() if x.isdigit()]
        assert nums[0] == nums[1] and nums[2] == nums[3], line


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    d = tmp_path / "sliding_window_attention_swa_amd" / "csrc"
    d.mkdir(parents=True)
    f = d / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f.write_text("int a = 1;  // one\n/* block\n comment */ int b = a + 2;\n")
    h0 = bench.source_hash(("k.hip",))
    f.write_text("int a = 1;  // another comment\n\nint b = a + 2;  /* x */\n")
    assert bench.source_hash(("k.hip",)) == h0
    f.write_text("int a = 1;\nint b = a + 3;\n")
    assert bench.source_hash(("k.hip",)) != h0


def test_source_hash_covers_every_file(tmp_path, monkeypatch):
    """The prefill's figures are tied to the kernel and its index header."""
    d = tmp_path / "sliding_window_attention_swa_amd" / "csrc"
    d.mkdir(parents=True)
    (d / "k.hip").write_text("int a = 1;\n")
    (d / "h.h").write_text("int b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash(("k.hip", "h.h"))
    (d / "h.h").write_text("int b = 3;\n")
    assert bench.source_hash(("k.hip", "h.h")) != h0
    assert "swa_tile_math.h" in bench.PREFILL_SOURCE


def test_kernel_trace_summary_drops_the_warmups(tmp_path, capsys):
    """Three warm-up dispatches of 2000 us, then timed ones of 1000 and
    1010 us: only the timed ones are averaged."""
    f = tmp_path / "run_kernel_trace.csv"
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    for us in (2000, 2000, 2000, 1000, 1010):
        rows.append('"void swa::prefill_bf16_kernel<128, 0>(args)",%d,%d' % (t, t + us * 1000))
        rows.append('"append_kernel(args)",%d,%d' % (t + 3_000_000, t + 3_004_000))
        t += 10_000_000
    f.write_text("\n".join(rows) + "\n")
    assert bench.summarize_kernel_trace([str(f)], 3) == 0
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if "prefill_bf16_kernel" in l][0]
    cells = [c.strip() for c in line.split("|")]
    assert cells[2] == "2" and cells[3] == "1005.0" and cells[5] == "1010.0"


def test_config_counter_summary_counts_a_repeated_counter_once(tmp_path, capsys):
    """GRBM_GUI_ACTIVE in each of three passes: the clock comes from one of
    them (2.0 GHz over a 50 us dispatch), and only the first dispatch of the
    prefill kernel in a file is read."""
    cycles = 2.0e9 * 50e-6
    paths = []
    for i, extra in enumerate(("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA")):
        f = tmp_path / ("p%d.csv" % i)
        lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"]
        for disp, scale in ((7, 1.0), (8, 5.0)):
            lines.append("%d,prefill_bf16_kernel<64>(x),GRBM_GUI_ACTIVE,%f,0,50000"
                         % (disp, scale * cycles * bench.N_XCD))
            lines.append("%d,prefill_bf16_kernel<64>(x),%s,%f,0,50000" % (disp, extra, 100.0 * (i + 1) * scale))
        f.write_text("\n".join(lines) + "\n")
        paths.append(str(f))
    assert bench.summarize_config_counters(paths, 5) == 0
    out = capsys.readouterr().out
    assert "clock 2000 MHz" in out
    assert "VALU instructions per MFMA 0.67" in out


def test_short_names_of_mangled_kernels():
    """Kernel traces may leave this library's kernels mangled (anonymous
    namespace, bf16 template arguments)."""
    f = bench.short_kernel_name
    assert f("_ZN3swa12_GLOBAL__N_119prefill_bf16_kernelILi128ELi0EEEvPKDF16bS3_S3_PDF16bii") == \
        "prefill_bf16_kernel<128, 0>"
    assert f("_ZN3swa12_GLOBAL__N_119decode_split_kernelIDF16bLi128ELi4ELi0EEEvPKT_S4_") == \
        "decode_split_kernel<bf16, 128, 4, 0>"
    assert f("swa::(anonymous namespace)::append_kernel(HIP_vector_type<unsigned int, 4u>*, int)") == \
        "append_kernel"
    assert f("void at::native::fill_kernel<16>(int)") == "fill_kernel<16>"
