"""The GPU tests, smoke() and bench.py read the library sources, the tests,
the oracle, the input generator and the committed traffic summary: none of
them may be matched by a pattern of .gpurunignore (tar patterns: "./x"
anchors at the top, other patterns match at any depth)."""

import fnmatch
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

NEEDED = [
    "bench.py", "__graft_entry__.py", "swa_inputs.py", "pytest.ini",
    "profiles/prefill_mistral7b_traffic.md",
    "sliding_window_attention_swa_amd/__init__.py", "sliding_window_attention_swa_amd/build.py",
    "sliding_window_attention_swa_amd/csrc/swa_prefill_bf16.hip",
    "sliding_window_attention_swa_amd/csrc/swa_ring.hip", "include/swa.h",
    "oracle/swa_ref.py", "tests/conftest.py", "tests/helpers.py", "tests/test_gpu_prefill.py",
]


def excluded(path, patterns):
    parts = path.split("/")
    for pat in patterns:
        if pat.startswith("./"):
            p = pat[2:].rstrip("/")
            if path == p or path.startswith(p + "/"):
                return True
        elif any(fnmatch.fnmatch(parts[i], pat) or fnmatch.fnmatch("/".join(parts[i:]), pat)
                 for i in range(len(parts))):
            return True
    return False


def test_gpu_runs_get_every_file_they_read():
    f = os.path.join(ROOT, ".gpurunignore")
    patterns = [l.strip() for l in open(f) if l.strip() and not l.startswith("#")] \
        if os.path.exists(f) else []
    for path in NEEDED:
        assert os.path.exists(os.path.join(ROOT, path)), path
        assert not excluded(path, patterns), path


def test_the_check_sees_an_exclusion():
    assert excluded("profiles/prefill_mistral7b_traffic.md", ["./profiles"])
    assert excluded("tests/x.log", ["*.log"])
    assert not excluded("bench.py", ["./profiles", "*.log"])
