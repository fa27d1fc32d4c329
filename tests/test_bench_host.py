"""bench.py's host-side logic, on the CPU: the refusal of more than one GPU
(before anything touches a GPU), the kernel-source hash that ties the
committed HBM counters to the code they were taken on (comments and
whitespace do not change it, code does), and the reading of that profile
only for its own source."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr and not r.stdout.strip()


def _hash_of(tmp_path, text):
    d = tmp_path / "loss_scaling_fp8_amd" / "csrc"
    d.mkdir(parents=True, exist_ok=True)
    (d / "k.hip").write_text(text)
    old = bench.ROOT
    bench.ROOT = str(tmp_path)
    try:
        return bench.kernel_source_hash(["k.hip"])
    finally:
        bench.ROOT = old


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    base = _hash_of(tmp_path, "int f(int x) {\n    return x + 1;  // one more\n}\n")
    assert _hash_of(tmp_path, "/* a header */\nint f(int x) {\n  return x + 1;\n}\n") == base
    assert _hash_of(tmp_path, "int f(int x) {\n    return x + 2;\n}\n") != base


def test_committed_counters_are_read_only_for_their_own_source():
    """The committed counter profile carries the hash of the code it was
    taken on: bench.py reports its traffic for that hash and none for any
    other (a changed kernel reports null until its counters are re-taken)."""
    stored = [l.split("=", 1)[1].strip() for l in open(bench.PMC_FILE)
              if l.startswith("source_sha256_16")]
    assert len(stored) == 1 and len(stored[0]) == 16
    traffic = bench.pmc_traffic(stored[0])
    assert traffic is not None and traffic > 48181567488     # above the algorithmic bytes
    assert bench.pmc_traffic("0" * 16) is None


def test_ceiling_patterns_agree_with_the_streaming_library():
    """Every pattern bench.py names has its byte counts, and the streaming
    library accepts exactly those pattern numbers: its argument checks
    (pattern, unroll, layout, policy, whole units, 16-byte alignment) return
    -1 before any HIP call, and an empty stream returns 0, so this runs
    without a GPU."""
    import ctypes
    if not os.path.exists(bench.CEIL_LIB):
        import pytest
        pytest.skip("libgsceil.so is not built")
    L = ctypes.CDLL(bench.CEIL_LIB)
    L.gsc_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_void_p]
    L.gsc_stream.restype = ctypes.c_int
    assert sorted(bench.CEIL_PATTERNS.values()) == list(range(6))
    for p in bench.CEIL_PATTERNS.values():
        assert p in bench.CEIL_SRC_BYTES and p in bench.CEIL_DST_BYTES
        assert L.gsc_stream(p, None, None, 0, 1, 0, 0, 0, 0, None) == 0       # nothing to do
    unit = {0: 16, 1: 16, 2: 4, 3: 16, 4: 4, 5: 8}
    for p, u in unit.items():
        assert L.gsc_stream(p, None, None, u + 1, 1, 0, 0, 0, 0, None) == -1  # not whole units
        assert L.gsc_stream(p, 8, None, u, 1, 0, 0, 0, 0, None) == -1        # misaligned source
    assert L.gsc_stream(6, None, None, 0, 1, 0, 0, 0, 0, None) == -1
    assert L.gsc_stream(5, None, None, 8, 3, 0, 0, 0, 0, None) == -1          # unroll 3
    assert L.gsc_stream(5, None, None, 8, 1, 2, 0, 0, 0, None) == -1          # layout 2
    assert L.gsc_stream(5, None, None, 8, 1, 0, 0, 3, 0, None) == -1          # policy 3
    # the byte counts of one pass over n elements
    n = 1 << 20
    moved = {p: bench.CEIL_SRC_BYTES[p](n) + bench.CEIL_DST_BYTES[p](n)
             for p in bench.CEIL_PATTERNS.values()}
    assert moved == {0: n, 1: n, 2: 6 * n, 3: 3 * n, 4: 5 * n, 5: 3 * n}
