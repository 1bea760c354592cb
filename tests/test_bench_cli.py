"""Host-side behaviour of the benchmark script (no GPU needed): it refuses
more than one GPU with a message and a non-zero status before touching a
device, and its source digest (which invalidates the stored HBM-traffic
figures when a library source changes) follows every library source's code
and ignores its comments and blank lines."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _digest_with(tmp_path, monkeypatch, name, extra):
    """The digest with `extra` appended to library source `name` (read
    through a patched open(), the files themselves untouched)."""
    real_open = open

    def patched(path, *a, **k):
        if os.path.basename(str(path)) == name:
            with real_open(path, *a, **k) as f:
                data = f.read()
            alt = tmp_path / name
            alt.write_text(data + extra)
            return real_open(alt, *a, **k)
        return real_open(path, *a, **k)

    monkeypatch.setattr("builtins.open", patched)
    try:
        return bench.kernel_source_digest()
    finally:
        monkeypatch.setattr("builtins.open", real_open)


def test_source_digest_tracks_every_library_source(tmp_path, monkeypatch):
    d0 = bench.kernel_source_digest()
    assert len(d0) == 16 and d0 == bench.kernel_source_digest()
    csrc = os.path.join(ROOT, "mixture_experts_grouped_top_amd", "csrc")
    sources = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    assert {"gmm.hip", "fp8.hip", "permute.hip", "common.h"} <= set(sources)
    for name in sources:
        assert _digest_with(tmp_path, monkeypatch, name, "\nstatic int digest_probe;\n") != d0, name
    # comments and blank lines do not count
    assert _digest_with(tmp_path, monkeypatch, "gmm.hip", "\n// a comment\n\n") == d0
