"""The C-ABI library loads, exports every symbol the header declares, and its
host-side argument checks and workspace queries work without a GPU.

The argument-error tests pass made-up addresses that every check rejects before
any launch.  They run only where no GPU is visible: on a machine with a GPU a
regressed check would launch kernels on those addresses.
"""
import ctypes
import os
import re

import pytest
import torch

from test_weight_layers_amd import ttt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ttt.LIB_PATH):
        pytest.fail("libttt.so is not built; run __graft_entry__.build()")
    return ttt.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ttt.EXPORTS)


# torch.cuda.device_count() counts devices without initialising the HIP runtime
cpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                              reason="passes made-up device addresses; CPU-only by design")


def _ws(lib, fn, *args):
    out = ctypes.c_size_t()
    st = getattr(lib, fn)(*args, ctypes.byref(out))
    return st, out.value


def test_workspace_queries(lib):
    st, b = _ws(lib, "ttt_update_workspace_bytes", 4, 256, 512, 1374000, ttt.TTT_BF16)
    assert st == 0 and b > 3 * 4 * 256 * 512 * 4
    st, b0 = _ws(lib, "ttt_update_workspace_bytes", 1, 64, 128, 0, ttt.TTT_F32)
    assert st == 0 and b0 > 0
    st, a = _ws(lib, "ttt_apply_workspace_bytes", 4, 256, 512, 1000, ttt.TTT_BF16)
    assert st == 0 and a >= 3 * 4 * 256 * 512 * 2
    st, a = _ws(lib, "ttt_apply_workspace_bytes", 1, 64, 128, 1000, ttt.TTT_F32)
    assert st == 0 and a == 0
    st, s = _ws(lib, "ttt_stream_workspace_bytes", 4, 256, 512, 43968, ttt.TTT_BF16)
    assert st == 0 and s > 0


@pytest.mark.parametrize("d", [64, 192, 320, 384, 640, 960, 1024])
def test_workspace_query_accepts_every_multiple_of_64(lib, d):
    for dt in (ttt.TTT_BF16, ttt.TTT_F32):
        st, b = _ws(lib, "ttt_update_workspace_bytes", 2, d, 128, 5000, dt)
        assert st == 0 and b >= 3 * 2 * d * 128 * 4
        st, _ = _ws(lib, "ttt_apply_workspace_bytes", 2, d, 128, 5000, dt)
        assert st == 0


@pytest.mark.parametrize("args,code", [
    ((4, 100, 512, 10, ttt.TTT_BF16), -2),     # d unsupported
    ((4, 1088, 512, 10, ttt.TTT_BF16), -2),    # d above 1024
    ((4, 0, 512, 10, ttt.TTT_BF16), -2),       # d zero
    ((4, 256, 500, 10, ttt.TTT_BF16), -2),     # m not a multiple of 64
    ((0, 256, 512, 10, ttt.TTT_BF16), -1),     # heads
    ((4, 256, 512, -1, ttt.TTT_BF16), -1),     # n < 0
    ((4, 256, 512, 10, 7), -2),                # dtype
])
def test_workspace_query_rejects_bad_shapes(lib, args, code):
    st, _ = _ws(lib, "ttt_update_workspace_bytes", *args)
    assert st == code
    assert len(lib.ttt_last_error()) > 0


@cpu_only
def test_update_argument_errors_return_before_any_launch(lib):
    # null weights
    st = lib.ttt_update(1, 64, 128, None, None, None, None, None, None, None, None, 64, None, 0, 10, 0.01, 1,
                        ttt.TTT_F32, None, None, None, 0, None)
    assert st == -1
    fake = 1 << 20   # never dereferenced: every check below fails first
    # steps < 1
    st = lib.ttt_update(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, fake, fake, 64, fake, 0,
                        10, 0.01, 0, ttt.TTT_F32, None, None, fake, 1 << 30, None)
    assert st == -1 and b"steps" in lib.ttt_last_error()
    # ld too small
    st = lib.ttt_update(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, fake, fake, 32, fake, 0,
                        10, 0.01, 1, ttt.TTT_F32, None, None, fake, 1 << 30, None)
    assert st == -1 and b"ld" in lib.ttt_last_error()
    # workspace too small
    st = lib.ttt_update(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, fake, fake, 64, fake, 0,
                        10, 0.01, 1, ttt.TTT_F32, None, None, fake, 16, None)
    assert st == -3
    # overlapping (but not identical) output weights
    st = lib.ttt_update(1, 64, 128, fake, fake * 2, fake * 3, fake + 64, fake * 5, fake * 6, fake, fake, 64, fake,
                        0, 10, 0.01, 1, ttt.TTT_F32, None, None, fake, 1 << 30, None)
    assert st == -1 and b"overlap" in lib.ttt_last_error()


@cpu_only
def test_apply_and_conv_argument_errors(lib):
    fake = 1 << 20
    st = lib.ttt_apply(1, 64, 128, fake, fake, fake, fake, 64, fake + 16, 64, 10, ttt.TTT_F32, None, 0, None)
    assert st == -1 and b"overlap" in lib.ttt_last_error()
    st = lib.ttt_apply(1, 64, 128, fake, fake, fake, fake + 8, 64, fake * 8, 64, 10, ttt.TTT_F32, None, 0, None)
    assert st == -1 and b"aligned" in lib.ttt_last_error()
    st = lib.ttt_apply(1, 64, 128, fake, fake, fake, fake, 64, fake * 8, 64, 10, ttt.TTT_BF16, None, 0, None)
    assert st == -3
    st = lib.ttt_shortconv2d(fake, fake * 8, 1024, fake, 2, 1374, 4, 37, 37, 1024, ttt.TTT_BF16, None)
    assert st == -1 and b"tokens_per_frame" in lib.ttt_last_error()
    st = lib.ttt_shortconv2d(fake, fake * 8, 1024, fake, 2, 1374, 5, 37, 37, 1020, ttt.TTT_BF16, None)
    assert st == -2
    st = lib.ttt_set_option(9, 1)
    assert st == -1


@cpu_only
def test_update_ex_stream_ex_and_gate_argument_errors(lib):
    fake = 1 << 20   # never dereferenced: every check below fails first
    # unknown flag bits
    st = lib.ttt_update_ex(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, fake, fake, 64, fake,
                           0, 10, 0.01, 1, ttt.TTT_F32, 6, None, None, fake, 1 << 30, None)
    assert st == -1 and b"flag" in lib.ttt_last_error()
    st = lib.ttt_stream_ex(1, 64, 128, fake, fake * 2, fake * 3, fake, fake, 64, fake, 0, fake, 64, fake * 8, 64, 10,
                           5, 0.01, 1, ttt.TTT_F32, 2, fake, 1 << 30, None)
    assert st == -1 and b"flag" in lib.ttt_last_error()
    # gate: channels not a multiple of 64, bad eps, overlap, misaligned W_g
    st = lib.ttt_output_gate(96, fake, 96, fake * 4, fake * 8, 1e-6, fake * 16, 96, 10, ttt.TTT_BF16, None)
    assert st == -2
    st = lib.ttt_output_gate(64, fake, 64, fake * 4, fake * 8, -1.0, fake * 16, 64, 10, ttt.TTT_BF16, None)
    assert st == -1 and b"eps" in lib.ttt_last_error()
    st = lib.ttt_output_gate(64, fake, 64, fake * 4, fake * 8, 1e-6, fake + 64, 64, 10, ttt.TTT_BF16, None)
    assert st == -1 and b"overlap" in lib.ttt_last_error()
    st = lib.ttt_output_gate(64, fake, 64, fake * 4 + 2, fake * 8, 1e-6, fake * 16, 64, 10, ttt.TTT_BF16, None)
    assert st == -1 and b"wg" in lib.ttt_last_error()
    st = lib.ttt_output_gate(64, fake, 32, fake * 4, fake * 8, 1e-6, fake * 16, 64, 10, ttt.TTT_BF16, None)
    assert st == -1
    # n = 0 launches nothing and succeeds
    assert lib.ttt_output_gate(64, None, 64, None, None, 1e-6, None, 64, 0, ttt.TTT_BF16, None) == 0


@cpu_only
def test_update_host_argument_errors(lib):
    fake = 1 << 20
    st, nb = _ws(lib, "ttt_update_host_workspace_bytes", 4, 256, 512, 4096, 1024, ttt.TTT_BF16)
    assert st == 0 and nb > 2 * 4096 * 1024 * 2 * 2          # two staging slots of K and V at least
    st, _ = _ws(lib, "ttt_update_host_workspace_bytes", 4, 256, 512, 0, 1024, ttt.TTT_BF16)
    assert st == -1
    # batch < 1, null host rows, unaligned rows: rejected before any copy or launch
    st = lib.ttt_update_host(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, fake, fake, 64,
                             fake, 0, 10, 0, 0.01, 1, ttt.TTT_F32, 0, None, None, fake, 1 << 30, None)
    assert st == -1 and b"batch" in lib.ttt_last_error()
    st = lib.ttt_update_host(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, None, fake, 64,
                             fake, 0, 10, 5, 0.01, 1, ttt.TTT_F32, 0, None, None, fake, 1 << 30, None)
    assert st == -1 and b"null" in lib.ttt_last_error()
    st = lib.ttt_update_host(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, fake, fake, 66,
                             fake, 0, 10, 5, 0.01, 1, ttt.TTT_BF16, 0, None, None, fake, 1 << 30, None)
    assert st == -1 and b"aligned" in lib.ttt_last_error()
    st = lib.ttt_update_host(1, 64, 128, fake, fake * 2, fake * 3, fake * 4, fake * 5, fake * 6, fake, fake, 64,
                             fake, 0, 10, 5, 0.01, 1, ttt.TTT_F32, 0, None, None, fake, 16, None)
    assert st == -3


def test_mfma_rate_probe_argument_errors(lib):
    flop = ctypes.c_double()
    assert lib.ttt_mfma_rate_probe(0, None, ctypes.byref(flop)) == -1
    assert b"iters" in lib.ttt_last_error()
    assert lib.ttt_mfma_rate_probe(16, None, None) == -1
