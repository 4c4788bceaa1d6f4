"""bench.py's contract checks that need no GPU: more than one GPU is refused with a message on
stdout and exit status 2, before torch or the library is touched."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_kernel_digest_ignores_comments_and_layout():
    """The traffic summaries are tied to the code of the kernel sources: comments and
    whitespace do not change the digest, code does."""
    sys.path.insert(0, ROOT)
    from exact_io_aware_42_amd.profiling import strip_comments
    a = "int f(int x) { // add one\n  return x + 1; /* done */ }\n"
    b = "int f(int x)\n{\n    return x + 1;\n}"
    c = "int f(int x) { return x + 2; }"
    assert strip_comments(a) == strip_comments(b) != strip_comments(c)
    assert strip_comments('const char* s = "// kept";') == 'const char* s = "// kept";'


def test_committed_traffic_summaries_match_the_sources():
    """Every committed traffic summary was taken on the current kernel code (else the
    benchmark line reports traffic as null)."""
    sys.path.insert(0, ROOT)
    import glob
    import re
    from exact_io_aware_42_amd.profiling import kernel_source_digest
    files = glob.glob(os.path.join(ROOT, "profiles", "traffic_*.txt"))
    assert files
    for f in files:
        s = open(f).read()
        k = re.search(r"# HBM traffic of (\S+) on workload", s).group(1)
        assert f"kernel_source_digest: {kernel_source_digest(k)}" in s, f
