"""GPU parity: the HIP library against the fp64 CPU oracle on the same seeded inputs.

Gate (relative Frobenius error per head and per matrix, on G, NS(G), W^ and O
separately): 1e-4 when tokens are fp32, 2e-2 when tokens are bf16 (the oracle
then runs on the same bf16-rounded inputs, upcast).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, cfg_like, gpu_layer, oracle_layer, parity_report
from test_weight_layers_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from test_weight_layers_amd import ttt
    ttt.load()          # raises if the library is missing: no fallback
    ttt.set_option(ttt.OPT_FORCE_GENERAL, 0)
    ttt.set_option(ttt.OPT_SPLITS, 0)
    yield
    ttt.set_option(ttt.OPT_FORCE_GENERAL, 0)
    ttt.set_option(ttt.OPT_SPLITS, 0)


def _check(cfg, n=None, nq_extra=None, steps=None, lr=None, general=False, splits=0, unfused=False):
    from test_weight_layers_amd import ttt
    inp = synth.make_inputs(cfg, n=n, nq_extra=nq_extra)
    ttt.set_option(ttt.OPT_FORCE_GENERAL, 1 if general else 0)
    ttt.set_option(ttt.OPT_SPLITS, splits)
    ttt.set_option(ttt.OPT_NS_UNFUSED, 1 if unfused else 0)
    try:
        got = gpu_layer(inp, steps=steps, lr=lr)
    finally:
        ttt.set_option(ttt.OPT_FORCE_GENERAL, 0)
        ttt.set_option(ttt.OPT_SPLITS, 0)
        ttt.set_option(ttt.OPT_NS_UNFUSED, 0)
    ref = oracle_layer(inp, steps=steps, lr=lr)
    rep = parity_report(got, ref, cfg.heads, cfg.d)
    worst = max(rep, key=rep.get)
    print(f"{cfg.name} n={inp.k.shape[0]} nq={inp.q.shape[0]} general={general} worst {worst}={rep[worst]:.3e}")
    tol = TOL[cfg.dtype]
    bad = {k: v for k, v in rep.items() if not v <= tol}
    assert not bad, bad
    return got, ref, rep


def test_c1_tiny_fp32_full():
    from test_weight_layers_amd.configs import CONFIGS
    _check(CONFIGS["c1"])


def test_c1_tiny_in_bf16_mode():
    _check(cfg_like("c1", dtype="bf16"))


@pytest.mark.parametrize("general", [False, True])
def test_vggt_heads_ragged_tokens(general):
    # 4 heads x 256, hidden 512; 1000 tokens = 31 blocks of 32 + 8, Nq with a ragged tail
    _check(cfg_like("c4", norm_v=False), n=1000, nq_extra=77, general=general)


def test_vggt_heads_fp32_general():
    _check(cfg_like("c4", dtype="f32"), n=700, nq_extra=5)


@pytest.mark.parametrize("d,m", [(64, 128), (128, 256), (64, 512)])
def test_other_fast_widths(d, m):
    _check(cfg_like("c4", heads=2, d=d, m=m), n=777, nq_extra=3)


@pytest.mark.parametrize("d,m", [(256, 64), (256, 192), (256, 320), (256, 448), (128, 192), (64, 320)])
def test_fast_kernels_hidden_sizes(d, m):
    # hidden sizes whose 32-unit chunk count (2, 6, 10, 14) leaves the apply kernel's
    # three-stage pipeline ending in each of its stages, and odd hidden-tile counts
    # for the gradient kernel's block map
    _check(cfg_like("c4", heads=2, d=d, m=m), n=500, nq_extra=41)


def test_tttlrm_width_768():
    # the tttLRM head (d = m = 768): the wide-head kernels (big_* in bigd.hip)
    from test_weight_layers_amd.configs import CONFIGS
    _check(CONFIGS["c2"], n=1500, nq_extra=300)


def test_zipmap_single_head_1024_2048():
    # the ZipMap layer's own shape (one head, d = 1024, m = 2048, state 6 d^2): the
    # wide-head kernels (bigd.hip), the 1024 x 2048 Newton-Schulz products, a ragged
    # token tail; the full-size workload is checked in test_gpu_fullsize.py
    from test_weight_layers_amd.configs import CONFIGS
    _check(CONFIGS["zipmap1h"], n=1500, nq_extra=77)


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("shape", [(2, 512, 512, 1000, 77), (2, 768, 256, 333, 5), (1, 1024, 512, 70, 300),
                                   (1, 512, 1024, 333, 7)])
def test_wide_heads(shape, general):
    # the two-kernel wide-head path (d >= 512) and the general kernels, both against
    # the oracle: ragged token tails, fewer tokens than one 256-row tile, Nq > N
    H, d, m, n, extra = shape
    _check(cfg_like("c4", heads=H, d=d, m=m), n=n, nq_extra=extra, general=general)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,m", [(192, 128), (320, 256), (384, 512), (640, 192), (512, 320)])
def test_every_multiple_of_64_width(d, m, dtype):
    # head widths outside the fast and wide sets (and a wide d with m % 256 != 0) run
    # the general kernels with d taken at run time
    _check(cfg_like("c4", heads=2, d=d, m=m, dtype=dtype), n=333, nq_extra=17)


def test_two_inner_steps_with_conv():
    cfg = cfg_like("c3", frames=2)
    _check(cfg, steps=2)


@pytest.mark.parametrize("n,splits", [(1, 0), (31, 0), (33, 0), (64, 1), (95, 2), (2000, 60)])
def test_fast_gradient_few_blocks_per_split(n, splits):
    # The fast gradient kernel stages K/V two 32-token blocks ahead; splits of one or
    # two blocks (and splits with none, when n is tiny) take its short pipeline paths.
    _check(cfg_like("c4", heads=2), n=n, nq_extra=3, splits=splits)


def test_many_splits_and_single_split_agree():
    cfg = cfg_like("c4", heads=1)
    g1, _, _ = _check(cfg, n=4000, splits=1)
    g2, _, _ = _check(cfg, n=4000, splits=37)
    for j in range(3):
        assert np.max(np.abs(g1["G"][j] - g2["G"][j])) <= 1e-3 * np.max(np.abs(g1["G"][j]))


@pytest.mark.parametrize("case", ["c1-fp32", "vggt-2step", "d64-m128", "d768"])
def test_fused_and_unfused_optimiser_step(case):
    # the folded optimiser step (split sum, Newton-Schulz with the Frobenius scale
    # folded into its first products, the step in the last product's epilogue: 16
    # launches) against the unfolded sequence of separate kernels: both against the
    # oracle, and against each other
    from test_weight_layers_amd.configs import CONFIGS
    cfg, kw = {"c1-fp32": (CONFIGS["c1"], dict(steps=2)),
               "vggt-2step": (cfg_like("c4", heads=2), dict(n=1500, nq_extra=0, steps=2)),
               "d64-m128": (cfg_like("c4", heads=3, d=64, m=128), dict(n=900, nq_extra=0)),
               "d768": (CONFIGS["c2"], dict(n=1000, nq_extra=0))}[case]
    a, _, _ = _check(cfg, **kw)
    b, _, _ = _check(cfg, unfused=True, **kw)
    tol = 1e-5 if cfg.dtype == "f32" else 1e-3
    for key in ("G", "NS", "W"):
        for j in range(3):
            x, y = np.asarray(a[key][j], np.float64), np.asarray(b[key][j], np.float64)
            assert np.linalg.norm(x - y) <= tol * np.linalg.norm(y), (key, j)


def test_lr_zero_is_bit_exact_and_n_zero_leaves_w():
    from test_weight_layers_amd import ttt
    cfg = cfg_like("c4", heads=2)
    inp = synth.to_device(synth.make_inputs(cfg, n=300, nq_extra=0), "cuda")
    w = (inp.w1, inp.w3, inp.w2)
    out = ttt.update(w, inp.k, inp.v, inp.eta, 0.0, 1)
    for a, b in zip(out, w):
        assert torch.equal(a, b)
    g = torch.full((3 * 2 * 512 * 256,), 7.0, device="cuda")
    ns = torch.full_like(g, 7.0)
    out = ttt.update(w, inp.k[:0], inp.v[:0], inp.eta[:, :0], 0.01, 1, grad_out=g, ns_out=ns)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g) == 0 and torch.count_nonzero(ns) == 0
    for a, b in zip(out, w):
        assert torch.equal(a, b)


def test_in_place_update_and_determinism():
    from test_weight_layers_amd import ttt
    cfg = cfg_like("c4", heads=2)
    inp = synth.to_device(synth.make_inputs(cfg, n=2000, nq_extra=0), "cuda")
    w = (inp.w1, inp.w3, inp.w2)
    a = ttt.update(w, inp.k, inp.v, inp.eta, 0.01, 2)
    b = ttt.update(w, inp.k, inp.v, inp.eta, 0.01, 2)
    wc = tuple(x.clone() for x in w)
    ttt.update(wc, inp.k, inp.v, inp.eta, 0.01, 2, out=wc)
    for x, y, z in zip(a, b, wc):
        assert torch.equal(x, y) and torch.equal(x, z)
    # two single steps equal one two-step call
    s1 = ttt.update(w, inp.k, inp.v, inp.eta, 0.01, 1)
    s2 = ttt.update(s1, inp.k, inp.v, inp.eta, 0.01, 1)
    for x, y in zip(a, s2):
        assert torch.equal(x, y)


def test_shared_eta_across_heads():
    from test_weight_layers_amd import ttt
    cfg = cfg_like("c4", heads=2)
    inp = synth.make_inputs(cfg, n=500, nq_extra=0)
    e1 = inp.eta[0].clone()
    inp_shared = synth.LayerInputs(cfg, inp.w1, inp.w3, inp.w2, None, inp.k, inp.v, inp.q, e1.expand(2, -1))
    ref = oracle_layer(inp_shared)
    d = synth.to_device(inp, "cuda")
    w_hat = ttt.update((d.w1, d.w3, d.w2), d.k, d.v, e1.cuda(), cfg.lr, 1)
    for j in range(3):
        got = w_hat[j].double().cpu().numpy()
        for h in range(2):
            den = np.linalg.norm(ref["W"][j][h] - synth.as_f64((inp.w1, inp.w3, inp.w2)[j][h]))
            err = np.linalg.norm(got[h] - ref["W"][j][h])
            assert err <= 2e-2 * den


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shortconv2d_against_oracle(dtype):
    from test_weight_layers_amd import ttt
    cfg = cfg_like("c3", frames=3, dtype=dtype)
    inp = synth.make_inputs(cfg)
    geo = dict(frames=3, tokens_per_frame=cfg.tokens_per_frame, n_special=cfg.n_special,
               grid_h=cfg.grid_h, grid_w=cfg.grid_w)
    got = ttt.shortconv2d(inp.v.cuda(), inp.wconv.cuda(), **geo)
    torch.cuda.synchronize()
    ref = oracle.shortconv2d(synth.as_f64(inp.v), synth.as_f64(inp.wconv), **geo)
    g = got.double().cpu().numpy()
    if dtype == "f32":
        np.testing.assert_allclose(g, ref, rtol=1e-5, atol=1e-6)
    else:   # one bf16 rounding of the fp32 sum
        np.testing.assert_allclose(g, ref, rtol=2 ** -8, atol=1e-6)
    # special tokens are copied bit for bit
    sp = np.concatenate([np.arange(f * cfg.tokens_per_frame, f * cfg.tokens_per_frame + cfg.n_special)
                         for f in range(3)])
    assert torch.equal(got[sp].cpu(), inp.v[sp])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid_h,grid_w,n_special,channels", [
    (1, 1, 0, 64), (3, 2, 2, 128), (5, 7, 1, 192), (2, 63, 3, 64), (4, 64, 1, 64), (3, 5, 2, 72)])
def test_shortconv2d_grids(dtype, grid_h, grid_w, n_special, channels):
    # edge geometries: one-row and one-column grids, no special tokens, odd widths,
    # wide grids, and channel counts that are not a multiple of 64
    from test_weight_layers_amd import ttt
    frames, tpf = 3, n_special + grid_h * grid_w
    rng = np.random.default_rng(7 + grid_w)
    v = torch.from_numpy(rng.standard_normal((frames * tpf, channels)).astype(np.float32))
    v = v.to(torch.bfloat16) if dtype == "bf16" else v
    wconv = torch.from_numpy((0.1 * rng.standard_normal((channels, 3, 3))).astype(np.float32))
    geo = dict(frames=frames, tokens_per_frame=tpf, n_special=n_special, grid_h=grid_h, grid_w=grid_w)
    got = ttt.shortconv2d(v.cuda(), wconv.cuda(), **geo)
    torch.cuda.synchronize()
    ref = oracle.shortconv2d(synth.as_f64(v), synth.as_f64(wconv), **geo)
    g = got.double().cpu().numpy()
    if dtype == "f32":
        np.testing.assert_allclose(g, ref, rtol=1e-5, atol=1e-6)
    else:
        np.testing.assert_allclose(g, ref, rtol=2 ** -8, atol=1e-6)
    sp = np.concatenate([np.arange(f * tpf, f * tpf + n_special) for f in range(frames)]).astype(np.int64)
    assert torch.equal(got[sp].cpu(), v[sp])


@pytest.mark.parametrize("kind", ["bf16-fast", "f32", "bf16-d768"])
def test_stream_against_oracle(kind):
    # the stream carries each chunk's operand copies to the next chunk; covered for
    # the shared-layout case (bf16, d <= 256), fp32, and the general apply (d = 768)
    from test_weight_layers_amd import ttt
    cfg = {"bf16-fast": cfg_like("c4", heads=2, d=256, m=512),
           "f32": cfg_like("c4", heads=2, d=128, m=256, dtype="f32"),
           "bf16-d768": cfg_like("c2", heads=1)}[kind]
    tol = TOL[cfg.dtype]
    n, chunk = 1000, 300
    inp = synth.make_inputs(cfg, n=n, nq_extra=0)
    d = synth.to_device(inp, "cuda")
    w = tuple(x.clone() for x in (d.w1, d.w3, d.w2))
    o = ttt.stream(w, d.k, d.v, d.eta, d.q, cfg.lr, 1, chunk)
    torch.cuda.synchronize()
    f = lambda t: synth.as_f64(t)
    o_ref, w_ref = oracle.stream(f(inp.w1), f(inp.w3), f(inp.w2), f(inp.k), f(inp.v), f(inp.eta), f(inp.q),
                                 cfg.lr, 1, chunk)
    from helpers import rel
    assert rel(o.double().cpu().numpy(), o_ref) <= tol
    for j in range(3):
        for h in range(cfg.heads):
            dw_ref = w_ref[j][h] - f((inp.w1, inp.w3, inp.w2)[j][h])
            dw = w[j][h].double().cpu().numpy() - f((inp.w1, inp.w3, inp.w2)[j][h])
            assert rel(dw, dw_ref) <= tol


@pytest.mark.parametrize("norm,n,chunk,steps", [(False, 20000, 4096, 1), (True, 20000, 4096, 1),
                                               (False, 8193, 4096, 1), (False, 9000, 4096, 2)])
def test_stream_bit_equals_sequential_calls(norm, n, chunk, steps):
    # with the fast apply, the stream runs each chunk's apply on a second stream beside
    # its first optimiser step; the result must be that of apply-then-update
    # per chunk bit for bit (repeated, with a ragged last chunk and a one-token one, so
    # that a missing wait between the two streams would show)
    from test_weight_layers_amd import ttt
    cfg = cfg_like("c4", heads=4, d=256, m=512)
    inp = synth.make_inputs(cfg, n=n, nq_extra=0)
    d = synth.to_device(inp, "cuda")
    w_seq = tuple(x.clone() for x in (d.w1, d.w3, d.w2))
    o_seq = torch.empty_like(d.q)
    for t0 in range(0, n, chunk):
        t1 = min(n, t0 + chunk)
        ttt.apply(w_seq, d.q[t0:t1], out=o_seq[t0:t1])
        ttt.update(w_seq, d.k[t0:t1], d.v[t0:t1], d.eta[:, t0:t1], cfg.lr, steps, out=w_seq, norm_preserve=norm)
    torch.cuda.synchronize()
    for rep in range(3):
        w = tuple(x.clone() for x in (d.w1, d.w3, d.w2))
        o = ttt.stream(w, d.k, d.v, d.eta, d.q, cfg.lr, steps, chunk, norm_preserve=norm)
        torch.cuda.synchronize()
        assert torch.equal(o, o_seq), rep
        for a, b in zip(w, w_seq):
            assert torch.equal(a, b), rep


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gradient_token_order_and_shard_additivity(dtype):
    # one gradient sees every token in any order (ZipMap 关键设计 1; Scal3R 方案1), and it
    # is a sum over token shards (Scal3R 方案2: the multi-GPU all-reduce, here emulated by
    # shards summed on one device): both hold up to the fp32 order of the sum
    from test_weight_layers_amd import ttt
    cfg = cfg_like("c4", heads=2, d=128, m=256, dtype=dtype)
    n = 3000
    inp = synth.to_device(synth.make_inputs(cfg, n=n, nq_extra=0), "cuda")
    H, d, m = cfg.heads, cfg.d, cfg.m
    w = (inp.w1, inp.w3, inp.w2)
    mat = 3 * H * m * d
    g_full = torch.empty(mat, device="cuda")
    ttt.update(w, inp.k, inp.v, inp.eta, 0.0, 1, grad_out=g_full)
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3)).cuda()
    g_perm = torch.empty_like(g_full)
    ttt.update(w, inp.k[perm].contiguous(), inp.v[perm].contiguous(), inp.eta[:, perm].contiguous(), 0.0, 1,
               grad_out=g_perm)
    g_sum = torch.zeros_like(g_full)
    for t0, t1 in ((0, 1000), (1000, 1777), (1777, 3000)):
        g_s = torch.empty_like(g_full)
        ttt.update(w, inp.k[t0:t1], inp.v[t0:t1], inp.eta[:, t0:t1].contiguous(), 0.0, 1, grad_out=g_s)
        g_sum += g_s
    torch.cuda.synchronize()
    ref = g_full.double()
    tol = 1e-5 if dtype == "f32" else 1e-4
    for got in (g_perm, g_sum):
        err = float((got.double() - ref).norm() / ref.norm())
        assert err <= tol, err
