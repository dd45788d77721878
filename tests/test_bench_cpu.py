"""bench.py's contract checks that need no GPU: more than one GPU is refused
with a message (the path runs on one GPU's share), and a machine without a
GPU gets an error, not a number."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_is_an_error():
    import pytest
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert r.stdout.strip() == ""


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_code_of_drops_comments_only():
    """The sources digest is taken over the code with comments removed: line
    and block comments go, string and character literals that contain
    comment markers stay, blank lines are skipped."""
    code_of = _bench().code_of
    src = ('int a = 1;  // one\n'
           '/* a block\n   comment */ int b = 2;\n'
           '\n'
           'const char* u = "http://x/*y*/";\n'
           "char c = '/'; char d = '\\'';\n"
           'int e = 4 / 2; // */ stays a comment\n')
    assert code_of(src) == ('int a = 1;\n'
                            '  int b = 2;\n'
                            'const char* u = "http://x/*y*/";\n'
                            "char c = '/'; char d = '\\'';\n"
                            'int e = 4 / 2;')


def test_sources_digest_ignores_comments_not_code():
    bench = _bench()
    files = {p: open(os.path.join(ROOT, p), encoding="utf-8").read() for p in bench.CAST_SOURCES}
    base = bench.sources_digest(read=files.__getitem__)
    assert base == bench.sources_digest()
    first = bench.CAST_SOURCES[0]
    commented = dict(files)
    commented[first] = "// a new comment\n" + files[first].replace("\n", "  /* note */\n", 1)
    assert bench.sources_digest(read=commented.__getitem__) == base
    changed = dict(files)
    changed[first] = files[first] + "\nstatic int extra_symbol;\n"
    assert bench.sources_digest(read=changed.__getitem__) != base
