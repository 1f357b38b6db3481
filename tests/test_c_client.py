"""The C ABI from a plain C program (CPU only): tests/c_client/stream_walk.c is compiled by the
system C compiler against include/swattn.h and linked with libswattn.so -- no Python binding,
no torch types -- and walks 1000 chunks of a metadata-only cache against the closed form of the
bounded cache ("Vidu S2 vs PixVerse R2" blog, section "Choice 3: bounded memory")."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "streaming_block_causal_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_client_walks_a_stream(tmp_path):
    exe = tmp_path / "stream_walk"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-O1", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_client", "stream_walk.c"), "-L", PKG, "-lswattn",
                    f"-Wl,-rpath,{PKG}", "-o", str(exe)], check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(x for x in ("/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")) if x)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "1000 chunks ok" in r.stdout
