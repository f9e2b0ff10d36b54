"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message and a non-zero exit, before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2",
                        "--steps", "1", "--warmup", "0"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_code_digest_ignores_comments_not_code(tmp_path):
    """The traffic figure is keyed to the attention code: a comment or layout
    edit keeps the digest, a change to the code or to a string literal does not."""
    import bench
    a = tmp_path / "a.hip"
    a.write_text('int f(int x) {  // one\n  return x + 1; /* two\n lines */ }\nconst char* s = "a//b";\n')
    b = tmp_path / "b.hip"
    b.write_text('int f(int x) {\n\n  return x + 1;   }  // other words\nconst char* s = "a//b";\n')
    c = tmp_path / "c.hip"
    c.write_text('int f(int x) { return x + 2; }\nconst char* s = "a//b";\n')
    d = tmp_path / "d.hip"
    d.write_text('int f(int x) { return x + 1; }\nconst char* s = "a/*b";\n')
    assert bench.code_digest(a) == bench.code_digest(b)
    assert bench.code_digest(a) != bench.code_digest(c)
    assert bench.code_digest(a) != bench.code_digest(d)
