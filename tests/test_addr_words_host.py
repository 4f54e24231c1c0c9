"""The address join behind every buffer resource, checked on the host.

The HIP kernels read their tiles through buffer resources whose 64-bit base
address is assembled from two words returned by readfirstlane as int.
Widening the low word straight to 64 bits sign-extends it into the high word
whenever its bit 31 is set, which points the resource at the wrong memory
(a GPU memory fault).  f16wm::join_words is the one place that joins the
words; this test compiles it for the host and checks addresses whose low word
has bit 31 set and clear.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "f16_weight_matrix_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "helpers", "join_words_check.cpp")


def test_join_words_keeps_the_high_word(tmp_path):
    exe = str(tmp_path / "join_words_check")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, SRC, "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 8 and not any("WRONG" in line for line in lines)
    # the case that faulted: low word 0x80000000 under a non-zero high word
    assert "00007fff80000000 -> 00007fff80000000" in r.stdout


def test_buffer_resources_use_join_words():
    """Every buffer resource is built by buffer_rsrc, which joins the address
    words through join_words (no other 64-bit join of readfirstlane words)."""
    txt = open(os.path.join(CSRC, "buffer_rsrc.h")).read()
    assert "join_words(lo, hi)" in txt
    for name in os.listdir(CSRC):
        if name.endswith((".hip", ".h")) and name not in ("buffer_rsrc.h", "addr_words.h"):
            body = open(os.path.join(CSRC, name)).read()
            assert "__builtin_amdgcn_make_buffer_rsrc" not in body, name
