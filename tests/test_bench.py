"""Host logic of bench.py that decides whether stored counter figures apply."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _sources():
    out = {}
    for f in bench.KERNEL_SOURCES:
        with open(os.path.join(ROOT, "chunked_top_kl_head_amd", "csrc", f), encoding="utf-8") as fh:
            out[f] = fh.read()
    return out


def test_code_only_drops_comments_and_keeps_literals():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "// not a comment"; char c = \'/\';\n'
    assert bench._code_only(src) == 'int a = 1; const char* s = "// not a comment"; char c = \'/\';'


def test_source_hash_ignores_comments_but_not_code():
    src = _sources()
    h = bench.kernel_source_hash(src)
    assert h == bench.kernel_source_hash()
    f = "kd_gemm_dtl.hpp"
    commented = dict(src)
    commented[f] = "// an added comment line\n" + src[f].replace("\n", "   \n", 3)
    assert bench.kernel_source_hash(commented) == h
    changed = dict(src)
    changed[f] = src[f].replace("constexpr int kDtlBK = 64;", "constexpr int kDtlBK = 32;")
    assert changed[f] != src[f]
    assert bench.kernel_source_hash(changed) != h
