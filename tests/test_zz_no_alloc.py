"""The allocation-free update entry point against the workspace one.

ttt_update_noalloc runs the same plan and kernels as ttt_update_ex in a
library-owned device array, so its results must be bit-identical to the
workspace path on the same inputs.  Two calls in a row, the second with fewer
tokens (and a different shape), check that the array's left-over contents from
the first call do not leak into the second.  Oversized plans are refused
before anything runs.
"""
import pytest
import torch

from helpers import cfg_like
from test_weight_layers_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_weight_layers_amd import ttt
    ttt.load()
    ttt.set_option(ttt.OPT_FORCE_GENERAL, 0)
    ttt.set_option(ttt.OPT_SPLITS, 0)
    ttt.set_option(ttt.OPT_NS_UNFUSED, 0)


def _pair(cfg, n, steps, norm):
    from test_weight_layers_amd import ttt
    H, d, m = cfg.heads, cfg.d, cfg.m
    print(f"no-alloc case {cfg.name} H={H} d={d} m={m} n={n} steps={steps} norm={norm}", flush=True)
    dv = synth.to_device(synth.make_inputs(cfg, n=n, nq_extra=0), "cuda")
    w = (dv.w1, dv.w3, dv.w2)
    mat = H * m * d
    g_ref, ns_ref = torch.empty(3 * mat, device="cuda"), torch.empty(3 * mat, device="cuda")
    w_ref = ttt.update(w, dv.k, dv.v, dv.eta, cfg.lr, steps, grad_out=g_ref, ns_out=ns_ref, norm_preserve=norm)
    g, ns = torch.full_like(g_ref, float("nan")), torch.full_like(ns_ref, float("nan"))
    out = tuple(torch.full_like(x, float("nan")) for x in w)
    w_na = ttt.update_noalloc(w, dv.k, dv.v, dv.eta, cfg.lr, steps, out=out, grad_out=g, ns_out=ns,
                              norm_preserve=norm)
    torch.cuda.synchronize()
    assert torch.equal(g, g_ref) and torch.equal(ns, ns_ref)
    for a, b in zip(w_na, w_ref):
        assert torch.equal(a, b)


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 4 heads of 256/512, two steps, 50,000 tokens (the fast kernels and the
    # pacing counters in the scratch); second: a smaller input of another shape
    _pair(cfg_like("c4", heads=4), 50000, 2, False)
    _pair(cfg_like("c4", heads=2, d=128, m=256), 3001, 1, True)


def test_noalloc_in_place_and_fp32():
    from test_weight_layers_amd import ttt
    cfg = cfg_like("c1")
    dv = synth.to_device(synth.make_inputs(cfg), "cuda")
    w = (dv.w1, dv.w3, dv.w2)
    ref = ttt.update(w, dv.k, dv.v, dv.eta, cfg.lr, 1)
    w_in = tuple(x.clone() for x in w)
    ttt.update_noalloc(w_in, dv.k, dv.v, dv.eta, cfg.lr, 1, out=w_in)
    torch.cuda.synchronize()
    for a, b in zip(w_in, ref):
        assert torch.equal(a, b)


def test_noalloc_refuses_a_plan_larger_than_its_array():
    from test_weight_layers_amd import ttt
    limit = ttt.noalloc_scratch_bytes()
    assert limit == 128 << 20
    # the wide-head path's intermediates grow with n: 1 x 1024/2048 at 200,000 tokens
    H, d, m, n = 1, 1024, 2048, 200000
    assert ttt.update_workspace_bytes(H, d, m, n, torch.bfloat16) > limit
    w = tuple(torch.zeros(s, device="cuda") for s in ((H, m, d), (H, m, d), (H, d, m)))
    k = torch.zeros((n, H * d), dtype=torch.bfloat16, device="cuda")
    eta = torch.zeros((H, n), device="cuda")
    with pytest.raises(ttt.TTTError, match="scratch"):
        ttt.update_noalloc(w, k, k, eta, 0.01, 1)
