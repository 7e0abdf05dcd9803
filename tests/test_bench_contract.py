"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message and exit status 2, before any GPU work; the kernel-source hash
that ties recorded counters to the source ignores comments."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_kernel_source_hash_ignores_comments():
    sys.path.insert(0, ROOT)
    import bench
    src = {rel: open(os.path.join(ROOT, rel)).read() for rel in bench.KERNEL_SOURCES}
    h0 = bench.kernel_source_hash(lambda rel: src[rel])
    assert bench.kernel_source_hash() == h0
    commented = {rel: "// a note\n\n" + text.replace("{\n", "{  // brace\n", 1) for rel, text in src.items()}
    assert bench.kernel_source_hash(lambda rel: commented[rel]) == h0
    changed = dict(src)
    first = bench.KERNEL_SOURCES[0]
    changed[first] = src[first].replace("kWaves = 4", "kWaves = 8")
    assert changed[first] != src[first]
    assert bench.kernel_source_hash(lambda rel: changed[rel]) != h0
