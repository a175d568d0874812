"""bench.py host logic without a GPU: the one-GPU contract and the hash that
keeps recorded HBM traffic tied to the kernel code it was measured on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and r.stdout == ""
    assert "one GPU" in r.stderr


def test_code_hash_ignores_comments_but_not_code():
    src = "int a = 1; // note\n/* block\n comment */\nint b = 2;\n\n"
    same = "int a = 1;\n\n// other note\nint b = 2; /* x */\n"
    other = "int a = 1;\nint b = 3;\n"
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(other)

