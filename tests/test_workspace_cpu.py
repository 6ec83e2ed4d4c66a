"""CPU checks of the library's scratch-buffer bookkeeping (no GPU).

csrc/workspace.h holds the rules of the split-K and asymmetric-path
workspaces with the allocator as a template parameter; tests/workspace_check.cpp
drives it with a tracking stand-in allocator: two host threads growing one
stream's slot (every buffer handed out stays allocated and is not touched by
the other thread while a call holds it), growth retiring rather than freeing,
no allocation during a stream capture, separate buffers per device / stream /
slot, and nested acquisition by one thread.  Built with g++ twice: plain, and
under ThreadSanitizer where the toolchain has it.
"""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "workspace_check.cpp")


def _build_and_run(tmp_path, extra):
    exe = str(tmp_path / "workspace_check")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-pthread", *extra, "-o", exe, SRC],
                       capture_output=True, text=True)
    if r.returncode != 0:
        return None, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    return r, None


def test_workspace_bookkeeping(tmp_path):
    r, err = _build_and_run(tmp_path, [])
    assert r is not None, err
    assert r.returncode == 0, r.stdout + r.stderr


def test_workspace_bookkeeping_thread_sanitizer(tmp_path):
    r, err = _build_and_run(tmp_path, ["-fsanitize=thread"])
    if r is None:
        pytest.skip(f"g++ cannot build with -fsanitize=thread here: {err[:200]}")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr
