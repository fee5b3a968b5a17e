"""Host-side checks of bench.py helpers (no GPU)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* note */\n}\n"
    b = "// header comment\nint f(int x) {\n\n  return 2 * x;\n}"
    assert bench._code_only(a) == bench._code_only(b) == "int f(int x) { return 2 * x; }"
    assert bench._code_only("return 3 * x;") != bench._code_only("return 2 * x;")


def test_gradient_digest_is_stable_hex():
    d1, d2 = bench.grad_source_digest(), bench.grad_source_digest()
    assert d1 == d2 and len(d1) == 64 and int(d1, 16) >= 0
