"""Host logic of bench.py that needs no GPU: the code-only source hash that
decides whether a stored traffic summary still applies to the kernels."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_layout():
    a = 'int a = 1;  // one\n/* two\n lines */ float b = 2.0f;\n'
    b = 'int a = 1;\nfloat b = 2.0f;'
    assert bench.code_only(a) == bench.code_only(b)


def test_code_only_keeps_literals_and_code():
    # comment markers inside literals are code, not comments
    s = 'asm("s_nop 0 // x" ::: "memory"); char c = \'/\'; const char* u = "/* y */";'
    assert bench.code_only(s) == s
    # a change of code changes the text the hash covers
    assert bench.code_only("x = a * b;") != bench.code_only("x = a + b;")


def test_source_hash_is_stable_and_per_phase():
    h1 = bench.source_hash("bwd_main")
    assert h1 == bench.source_hash("bwd_main") and len(h1) == 16
    assert h1 != bench.source_hash("proj_gemm")
