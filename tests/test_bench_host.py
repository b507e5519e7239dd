"""Host-side pieces of bench.py (no GPU): the one-GPU guard and the code hash
that keys the stored HBM traffic summary to the kernel source."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_code_hash_ignores_comments_and_whitespace(tmp_path):
    src = 'int f(int x) {\n    // twice\n    return 2 * x; /* no carry */\n}\nconst char *s = "a // b";\n'
    a = tmp_path / "a.hip"
    a.write_text(src)
    h = bench._code_sha256(str(a))
    a.write_text(src.replace("// twice", "// two times x").replace("    return", "\n\treturn"))
    assert bench._code_sha256(str(a)) == h
    a.write_text(src.replace("2 * x", "3 * x"))                 # code
    assert bench._code_sha256(str(a)) != h
    a.write_text(src.replace('"a // b"', '"a // c"'))           # a string literal is code
    assert bench._code_sha256(str(a)) != h


def test_stored_traffic_matches_the_kernel_source():
    # the committed counter summary was taken on the current kernel code
    assert bench.stored_traffic() is not None
