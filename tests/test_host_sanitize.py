"""The library's host-side validation and planning code (``plan.cpp``: tree
checks, ancestor sets, the re-root plan, the attention tiling) built on its
own with g++ and the address and undefined-behaviour sanitizers, then driven
by ``host_plan_fuzz.cpp`` with randomised valid and corrupted requests. The
driver hands the library heap blocks of exactly the size a call may touch,
so an access past them is reported; valid requests must be accepted with
outputs that satisfy the plan's invariants, corrupted ones refused. A
planted off-by-one in the parent check (reading one entry past the array)
and a dropped ascending-survivor check are both caught by it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "tree_masked_attention_attn_amd", "csrc")


def test_plan_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / "host_plan_fuzz")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(HERE, "host_plan_fuzz.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", exe]
    b = subprocess.run(build, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    # the driver must exercise the accepting paths, not only refusals
    words = r.stdout.split()
    counts = [int(words[i - 1]) for i, w in enumerate(words) if w in ("ancestor", "re-root", "attention")]
    assert len(counts) == 3 and min(counts) > 1000, r.stdout
