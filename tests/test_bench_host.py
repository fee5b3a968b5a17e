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


def test_flop_counts_match_hand_computed_values():
    # algorithmic FLOPs per config (update per inner step, apply, Newton-Schulz per step),
    # against values worked out by hand from 12 d m per token, 6 d m per query and
    # 5 (4 r^2 c + 2 r^3) per matrix and optimiser step (five Newton-Schulz iterations)
    from test_weight_layers_amd.configs import CONFIGS
    c5a = CONFIGS["c5a"]
    g, a, ns, conv = bench.flops(c5a, 1_374_000, 1_374_000)
    assert abs(2 * g / 1e9 - 17_289) < 1 and abs(a / 1e9 - 4_322) < 1 and abs(ns / 1e9 - 10.07) < 0.01
    assert abs(conv / 1e9 - 25.3) < 0.1
    c2 = CONFIGS["c2"]
    g, a, ns, _ = bench.flops(c2, 8_192, 16_384)
    assert abs(g / 1e9 - 57.98) < 0.01 and abs(a / 1e9 - 57.98) < 0.01 and abs(ns / 1e9 - 40.77) < 0.01
    c4z = CONFIGS["c4z"]
    assert bench.gate_flops(c4z, 1_118_436) == 2.0 * 1_118_436 * 1024 ** 2


def test_per_call_stats_median_and_p90():
    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t
    marks = []
    for s, (u, a) in enumerate([(3.0, 1.0), (5.0, 2.0), (4.0, 1.5)]):
        t = 100.0 * s
        marks += [("start", Ev(t)), ("update", Ev(t + u)), ("apply", Ev(t + u + a))]
    st = bench.per_call_stats(marks)
    assert st["update"]["median"] == 4.0 and st["apply"]["median"] == 1.5
    assert st["step"]["median"] == 5.5 and st["step"]["n"] == 3


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_traffic_figure_only_for_the_profiled_kernel():
    assert bench.measured_traffic(128) is None
