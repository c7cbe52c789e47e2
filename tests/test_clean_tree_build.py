"""A clean copy of the tracked sources (no built library) imports the package,
reports the missing library loudly on first use, and builds it with
__graft_entry__.build(), which also compiles the C oracle (CPU only: hipcc
cross-compiles for gfx950 here)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ("__graft_entry__.py", "include", "draft_token_verification_row_amd", "synth", "oracle")


def _copy_sources(dst):
    for name in SOURCES:
        src = os.path.join(ROOT, name)
        if os.path.isdir(src):
            shutil.copytree(src, os.path.join(dst, name),
                            ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "*.o", "__pycache__"))
        else:
            shutil.copy2(src, dst)


def _run(code, cwd):
    return subprocess.run([sys.executable, "-c", code], cwd=cwd, capture_output=True, text=True,
                          timeout=600)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_build_from_a_tree_without_the_library(tmp_path):
    _copy_sources(tmp_path)
    so = tmp_path / "draft_token_verification_row_amd" / "libspecverify.so"
    assert not so.exists()
    r = _run("import draft_token_verification_row_amd as sv\n"
             "try:\n"
             "    sv.spec_verify_workspace_bytes(1, 1, 10)\n"
             "except sv.LibraryMissingError as e:\n"
             "    print('missing:', e)\n"
             "else:\n"
             "    raise SystemExit('no error without the library')\n", tmp_path)
    assert r.returncode == 0 and "missing:" in r.stdout, r.stdout + r.stderr
    r = _run("import __graft_entry__ as g; g.build()\n"
             "import draft_token_verification_row_amd as sv\n"
             "print('bytes', sv.spec_verify_workspace_bytes(4, 8, 1000))\n", tmp_path)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert so.exists()
    assert (tmp_path / "oracle" / "liboracle_verify.so").exists()     # the C oracle, built too
    assert "bytes " in r.stdout and int(r.stdout.split("bytes ")[-1]) > 0
