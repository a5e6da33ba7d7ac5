"""The C ABI from plain C: a C99 program (tests/c/abi_from_c.c) includes include/pa.h, links the
built library and calls its host-only entry points (no GPU involved).  Checks that the header is
valid C (no C++ types or overloads leak into it) and that the exported symbols link by name."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def libdir():
    from paged_kv_cache_gqa_amd import build
    if build.is_stale():
        build.build()
    return os.path.dirname(build.LIB_PATH)


def test_header_compiles_as_c99_and_links(libdir, tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_from_c"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", libdir, "-lpa_mi355x",
           f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("done"), r.stdout + r.stderr
