"""The product path has no fallback (CPU only).

* Without the built library the first call raises, naming the build step.
* Importing and using the package never imports the oracle: nothing under
  chunked_kl_loss_row_amd/ names it.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_raises():
    code = (
        "import sys\n"
        "from chunked_kl_loss_row_amd import binding as B\n"
        "B.LIB_PATH = '/nonexistent/libkdchunk.so'\n"
        "B._lib = None\n"
        "try:\n"
        "    B.kd_chunked_workspace_size(B.problem(10, 8, 100, 4, 4))\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(3)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "build" in r.stdout and "no fallback" in r.stdout


def test_package_never_imports_the_oracle():
    code = (
        "import sys\n"
        "import chunked_kl_loss_row_amd.loss, chunked_kl_loss_row_amd.binding, chunked_kl_loss_row_amd.inputs\n"
        "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "[]"
    pkg = os.path.join(ROOT, "chunked_kl_loss_row_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
