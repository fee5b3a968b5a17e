// C ABI of libttt.so (declared in include/ttt.h): argument checks, workspace
// planning and the launch sequences of the LaCT layer.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "ttt.h"
#include "kernels.h"

using namespace ttt;

// Scratch of ttt_update_noalloc: one copy per device, held by the loaded code object
// until the process ends.  Host code never uses this name as an address: it takes the
// device address from hipGetSymbolAddress (scratch_base below).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_err;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

// ----------------------------------------------------------------- options
int64_t g_force_general = 0;   // 1: use the general kernels even where a fast one exists
int64_t g_splits = 0;          // >0: fixed number of token splits for the gradient
int64_t g_ns_unfused = 0;      // 1: normalisation, step and casts as kernels of their own

// ----------------------------------------------------------------- timing
struct Pending {
  int kind;
  hipEvent_t e0, e1;
};
std::mutex g_prof_mu;
bool g_prof = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free_events;
double g_ms[TTT_K_COUNT];
int64_t g_count[TTT_K_COUNT];

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Set for the duration of an allocation-free call: no timing events are created or
// recorded in it, whatever ttt_profile_enable says.
thread_local bool t_no_events = false;

template <class F>
int run(int kind, const char *what, hipStream_t s, F &&f) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool prof = g_prof && !t_no_events;
  if (prof) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    e0 = take_event();
    e1 = take_event();
    if (e0) hipEventRecord(e0, s);
  }
  const hipError_t err = f();
  if (prof && e0 && e1) {
    hipEventRecord(e1, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_pending.push_back({kind, e0, e1});
  }
  if (err != hipSuccess) return fail(TTT_EHIP, "%s: %s", what, hipGetErrorString(err));
  return TTT_OK;
}

// ----------------------------------------------------------------- checks
// Every head width that is a multiple of the 64-wide tile, up to 1024.  d in {64, 128,
// 256} (bf16) runs the fused fast kernels, bf16 d in {512, 768, 1024} with m % 256 == 0
// the wide-head kernels, everything else the general kernels.
bool d_supported(int d) { return d >= 64 && d <= 1024 && d % 64 == 0; }

int check_shape(int heads, int d, int m, int dtype) {
  if (heads < 1) return fail(TTT_EINVAL, "heads must be >= 1 (got %d)", heads);
  if (dtype != TTT_F32 && dtype != TTT_BF16) return fail(TTT_EUNSUPPORTED, "unknown dtype %d", dtype);
  if (!d_supported(d)) return fail(TTT_EUNSUPPORTED, "d=%d is not a multiple of 64 in [64, 1024]", d);
  if (m < 64 || m % 64 != 0) return fail(TTT_EUNSUPPORTED, "m=%d must be a positive multiple of 64", m);
  return TTT_OK;
}

size_t esize(int dtype) { return dtype == TTT_BF16 ? 2 : 4; }

int check_rows(const void *p, int64_t ld, int heads, int d, int dtype, const char *name) {
  if (!p) return fail(TTT_EINVAL, "%s is null", name);
  if (ld < (int64_t)heads * d) return fail(TTT_EINVAL, "ld of %s (%lld) < heads*d (%d)", name, (long long)ld, heads * d);
  if (((uintptr_t)p) % 16 != 0 || (ld * (int64_t)esize(dtype)) % 16 != 0)
    return fail(TTT_EINVAL, "%s rows must be 16-byte aligned", name);
  return TTT_OK;
}

// The gradient kernels index tokens and the rows of one 32-token block with 32-bit
// integers: n must leave room for a whole block, and 32 rows must span < 2 GiB.
constexpr int64_t kMaxTokens = 2147483647LL - 64;
int check_token_limits(int64_t n, int64_t ld, int dtype, const char *name) {
  if (n > kMaxTokens) return fail(TTT_EUNSUPPORTED, "n=%lld exceeds %lld tokens per call", (long long)n,
                                  (long long)kMaxTokens);
  if (n > 0 && ld * (int64_t)esize(dtype) * 32 >= 2147483648LL)
    return fail(TTT_EUNSUPPORTED, "row stride of %s too large (32 rows must span < 2 GiB)", name);
  return TTT_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
  return x < y + nb && y < x + na;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ----------------------------------------------------------------- update plan
struct UpdatePlan {
  int H, d, m, r, c;
  bool bf16, fast, xcd, big;
  int dchunks, splits, grid;
  int64_t n, nblk, n_pad;
  size_t off_wop, off_part, off_g, off_sumsq, off_x0, off_x1, off_xt0, off_xt1, off_a, off_b, off_sync, off_wsq;
  size_t off_inter, total;
};

UpdatePlan plan_update(int H, int d, int m, int64_t n, int dtype) {
  UpdatePlan p{};
  p.H = H, p.d = d, p.m = m, p.n = n;
  p.r = d < m ? d : m;
  p.c = d < m ? m : d;
  p.bf16 = dtype == TTT_BF16;
  p.fast = !g_force_general && grad_fast_supported(d, p.bf16);
  p.big = !g_force_general && !p.fast && big_supported(d, m, p.bf16);
  p.dchunks = p.fast || p.big ? 1 : d / grad_general_dc(d, p.bf16);
  p.nblk = (n + kTokBlock - 1) / kTokBlock;
  const int mtiles = m / kHidTile;
  const int64_t per_split = (int64_t)H * mtiles * p.dchunks;
  const int64_t target = p.fast ? 256 : 1024;     // one fast workgroup fills a CU
  int64_t s = (target + per_split - 1) / per_split;
  if (g_splits > 0) s = g_splits;
  if (p.nblk > 0 && s > p.nblk) s = p.nblk;
  if (s < 1) s = 1;
  p.splits = (int)s;
  p.grid = (int)(per_split * s);
  if (p.big) {
    // Wide heads: the two contraction kernels split the tokens into S ranges, each
    // writing a full fp32 partial of G (3 H d m floats) that the optimiser step sums.
    // More ranges fill more CUs but add partial traffic; S minimises a simple cost:
    // the launches' rounds of 256 workgroups times one workgroup's blocks (~1 us per
    // 32-token block), plus writing and reading the partials at ~4 TB/s.
    p.n_pad = big_pad_tokens(n);
    const int64_t blocks = p.n_pad / 32;
    const int64_t t0 = (int64_t)H * big_contract_tiles(d, m, 0), t1 = (int64_t)H * big_contract_tiles(d, m, 1);
    const double part_bytes = 3.0 * H * d * m * 4.0;
    int64_t sb = 1;
    double best = 0.0;
    for (int64_t sc = 1; sc <= 64 && sc <= (blocks > 0 ? blocks : 1); ++sc) {
      const int64_t rounds = (t0 * sc + 255) / 256 + (t1 * sc + 255) / 256;
      const double cost = (double)rounds * (double)((blocks + sc - 1) / sc) * 1000.0 + 2.0 * sc * part_bytes / 4000.0;
      if (sc == 1 || cost < best) best = cost, sb = sc;
    }
    if (g_splits > 0) sb = g_splits;
    if (blocks > 0 && sb > blocks) sb = blocks;
    p.splits = (int)(sb < 1 ? 1 : sb);
    p.grid = 0;
  }
  p.xcd = p.fast && p.grid % 8 == 0 && (p.grid / 8) % mtiles == 0;
  const size_t mat = (size_t)H * d * m;
  size_t off = 0;
  p.off_wop = off;
  off = align256(off + (p.bf16 ? 3 * mat * 2 : mat * 4));
  p.off_part = off;
  off = align256(off + (size_t)p.splits * 3 * mat * 4);
  p.off_g = off;
  off = align256(off + 3 * mat * 4);
  p.off_sumsq = off;
  off = align256(off + 3 * mat / 4096 * 4);
  p.off_x0 = off;
  off = align256(off + 3 * mat * 4);
  p.off_x1 = off;
  off = align256(off + 3 * mat * 4);
  p.off_xt0 = off;
  off = align256(off + 3 * mat * 4);
  p.off_xt1 = off;
  off = align256(off + 3 * mat * 4);
  p.off_a = off;
  off = align256(off + (size_t)3 * H * p.r * p.r * 4);
  p.off_b = off;
  off = align256(off + (size_t)3 * H * p.r * p.r * 4);
  p.off_sync = off;
  off = align256(off + (size_t)H * p.splits * 4);
  p.off_wsq = off;                                   // norm-preserving step: 2 x [3H][d*m/4096]
  off = align256(off + 2 * (3 * mat / 4096) * 4);
  p.off_inter = off;                                 // wide heads: dZ1 | dZ3 | H', [H][n_pad][m] bf16
  if (p.big) off = align256(off + 3 * (size_t)H * p.n_pad * m * 2);
  p.total = off;
  return p;
}

bool apply_big(int d, int m, int dtype) {
  return dtype == TTT_BF16 && !g_force_general && !apply_fast_supported(d, true) && big_supported(d, m, true);
}

// bf16: the operand copies (3 H d m); wide heads also the hidden activations
// H [H][nq_pad][m] of the two-kernel apply
size_t apply_ws(int H, int d, int m, int64_t nq, int dtype) {
  if (dtype != TTT_BF16) return 0;
  size_t b = align256((size_t)3 * H * d * m * 2);
  if (apply_big(d, m, dtype)) b += align256((size_t)H * big_pad_tokens(nq) * m * 2);
  return b;
}

struct W3 {
  const float *w1, *w3, *w2;
};
struct W3o {
  float *w1, *w3, *w2;
};

// Muon's quintic Newton-Schulz coefficients and the Frobenius-norm guard.
constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f;
constexpr int kNsIters = 5;
constexpr float kNsEps = 1e-7f;

// Operand copies of `src` at the start of the workspace (bf16 W1, W3, W2^T; fp32
// mode only W2^T), cast unless `ready`.  Returns the pointers the gradient reads.
struct GradOps {
  const void *w1, *w3, *w2t;
};
int prepare_operands(const UpdatePlan &P, W3 src, bool ready, char *ws, hipStream_t s, GradOps *ops) {
  const size_t mat = (size_t)P.H * P.d * P.m;
  void *const wop = ws + P.off_wop;
  if (P.bf16) {
    __bf16 *b = static_cast<__bf16 *>(wop);
    if (!ready) {
      const int st = run(TTT_K_CAST, "cast", s, [&] {
        return launch_cast(src.w1, src.w3, src.w2, b, b + mat, b + 2 * mat, nullptr, P.H, P.d, P.m, true, s);
      });
      if (st) return st;
    }
    *ops = GradOps{b, b + mat, b + 2 * mat};
  } else {
    float *w2t = static_cast<float *>(wop);
    if (!ready) {
      const int st = run(TTT_K_CAST, "cast", s, [&] {
        return launch_cast(src.w1, src.w3, src.w2, nullptr, nullptr, w2t, nullptr, P.H, P.d, P.m, false, s);
      });
      if (st) return st;
    }
    *ops = GradOps{src.w1, src.w3, w2t};
  }
  return TTT_OK;
}

// Split partials of G over the plan's P.n tokens (k, v, eta) into `part`
// ([P.splits][3][H][m d]).  The plan's workspace holds the pacing counters and
// the wide-head intermediates.
int gradient_pass(const UpdatePlan &P, const GradOps &ops, const void *k, const void *v, int64_t ld,
                  const float *eta, int64_t eta_hs, float *part, char *ws, hipStream_t s) {
  const size_t mat = (size_t)P.H * P.d * P.m;
  if (P.big) {
    BigFwdParams fp{};
    fp.k = k, fp.v = v, fp.ld = ld, fp.eta = eta, fp.eta_hs = eta_hs;
    fp.w1 = ops.w1, fp.w3 = ops.w3, fp.w2t = ops.w2t, fp.out = ws + P.off_inter;
    fp.n = P.n, fp.n_pad = P.n_pad, fp.heads = P.H, fp.d = P.d, fp.m = P.m;
    BigCtrParams cp{};
    cp.k = k, cp.v = v, cp.ld = ld, cp.inter = ws + P.off_inter, cp.part = part;
    cp.n = P.n, cp.n_pad = P.n_pad, cp.heads = P.H, cp.d = P.d, cp.m = P.m, cp.splits = P.splits;
    return run(TTT_K_GRAD, "gradient", s, [&] {
      if (P.n == 0)
        return launch_zero_u32(reinterpret_cast<unsigned *>(part), (int)(3 * mat * (size_t)P.splits), s);
      const hipError_t e = launch_big_fwd(fp, s);
      return e != hipSuccess ? e : launch_big_contract(cp, s);
    });
  }
  GradParams gp{};
  gp.k = k, gp.v = v, gp.ld = ld, gp.eta = eta, gp.eta_hs = eta_hs;
  gp.w1 = ops.w1, gp.w3 = ops.w3, gp.w2t = ops.w2t;
  gp.part = part, gp.n = P.n, gp.nblk = P.nblk;
  gp.heads = P.H, gp.d = P.d, gp.m = P.m, gp.splits = P.splits, gp.dchunks = P.dchunks, gp.xcd_map = P.xcd;
  // the hidden tiles of a token range keep pace through these counters (see the kernel)
  if (P.fast && P.xcd) gp.group_sync = reinterpret_cast<unsigned *>(ws + P.off_sync);
  return run(TTT_K_GRAD, "gradient", s, [&] {
    if (gp.group_sync) {
      const hipError_t e = launch_zero_u32(gp.group_sync, P.H * P.splits, s);
      if (e != hipSuccess) return e;
    }
    return launch_grad(gp, P.d, P.bf16, P.fast, P.grid, s);
  });
}

// One optimiser step from the split partials `part` ([splits][3][H][m d]):
// G = their fixed-order sum, W_out = W_src - lr NS(G) (or the norm-preserving
// form).  write_ops: the folded path leaves the operand copies of W_out at the
// start of the workspace.  grad_out / ns_out: optional copies of G and NS(G).
int optimiser_step(const UpdatePlan &P, W3 src, W3o out, const float *part, int splits, float lr, bool write_ops,
                   float *grad_out, float *ns_out, bool norm, char *ws, hipStream_t s,
                   hipEvent_t before_write = nullptr) {
  const size_t mat = (size_t)P.H * P.d * P.m;
  void *const wop = ws + P.off_wop;
  float *g = reinterpret_cast<float *>(ws + P.off_g);
  float *sumsq = reinterpret_cast<float *>(ws + P.off_sumsq);
  float *x0 = reinterpret_cast<float *>(ws + P.off_x0);
  float *x1 = reinterpret_cast<float *>(ws + P.off_x1);
  float *am = reinterpret_cast<float *>(ws + P.off_a);
  float *bm = reinterpret_cast<float *>(ws + P.off_b);
  float *wsq = reinterpret_cast<float *>(ws + P.off_wsq);
  const int slots = P.d * P.m / 4096;
  const NsShape sh{P.H, P.d, P.m};
  int st;
  if (!g_ns_unfused) {
    NsStepParams np{};
    np.part = part, np.splits = splits, np.per_split = (int64_t)3 * mat;
    np.grad_out = grad_out, np.ns_out = ns_out;
    np.sumsq = sumsq;
    np.x[0] = x0, np.x[1] = x1;
    np.xt[0] = reinterpret_cast<float *>(ws + P.off_xt0), np.xt[1] = reinterpret_cast<float *>(ws + P.off_xt1);
    np.am = am, np.bm = bm;
    np.w1 = src.w1, np.w3 = src.w3, np.w2 = src.w2;
    np.w1o = out.w1, np.w3o = out.w3, np.w2o = out.w2;
    if (write_ops) {
      if (P.bf16) {
        __bf16 *b = static_cast<__bf16 *>(wop);
        np.op1v = b, np.op3v = b + mat, np.op2tv = b + 2 * mat;
      } else {
        np.op2tv = wop;
      }
    }
    np.lr = lr, np.eps = kNsEps, np.a_coef = kNsA, np.b_coef = kNsB, np.c_coef = kNsC;
    np.iters = kNsIters, np.heads = P.H, np.d = P.d, np.m = P.m, np.r = P.r, np.c = P.c;
    np.norm_preserve = norm, np.wsq = wsq;
    st = run(TTT_K_NS, "newton_schulz", s, [&] { return launch_ns_optimiser(np, P.bf16, s, before_write); });
    if (st) return st;
    if (norm) {
      st = run(TTT_K_NS, "norm_rescale", s, [&] {
        return launch_norm_rescale(out.w1, out.w3, out.w2, wsq, slots, np.op1v, np.op3v, np.op2tv, P.H, P.d, P.m,
                                   P.bf16, s);
      });
      if (st) return st;
    }
    return TTT_OK;
  }
  if (before_write) {   // this path rewrites W_out early: wait before anything
    const hipError_t e = hipStreamWaitEvent(s, before_write, 0);
    if (e != hipSuccess) return fail(TTT_EHIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
  }
  st = run(TTT_K_REDUCE, "reduce", s, [&] {
    return launch_reduce(part, splits, (int64_t)3 * mat, g, grad_out, sumsq, s);
  });
  if (st) return st;
  st = run(TTT_K_NS, "ns_normalize", s, [&] { return launch_ns_normalize(g, sumsq, x0, sh, kNsEps, s); });
  if (st) return st;
  float *x = x0, *xn = x1;
  const int B = 3 * P.H;
  const int64_t srr = (int64_t)P.r * P.r, src_ = (int64_t)P.r * P.c;
  for (int it = 0; it < kNsIters; ++it) {
    GemmBatch g1{x, x, nullptr, am, P.r, P.r, P.c, P.c, P.c, 0, P.r, 1, src_, src_, 0, srr, 1.0f, 0.0f, B};
    GemmBatch g2{am, am, am, bm, P.r, P.r, P.r, P.r, P.r, P.r, P.r, 1, srr, srr, srr, srr, kNsC, kNsB, B};
    GemmBatch g3{bm, x, x, xn, P.r, P.c, P.r, P.r, P.c, P.c, P.c, 0, srr, src_, src_, src_, 1.0f, kNsA, B};
    st = run(TTT_K_NS, "ns_gemm", s, [&] { return launch_gemm_f32(g1, s); });
    if (st) return st;
    st = run(TTT_K_NS, "ns_gemm", s, [&] { return launch_gemm_f32(g2, s); });
    if (st) return st;
    st = run(TTT_K_NS, "ns_gemm", s, [&] { return launch_gemm_f32(g3, s); });
    if (st) return st;
    float *tmp = x;
    x = xn;
    xn = tmp;
  }
  if (norm) {
    st = run(TTT_K_NS, "weight_sumsq", s, [&] { return launch_weight_sumsq(src.w1, src.w3, src.w2, wsq, P.H, P.d,
                                                                            P.m, s); });
    if (st) return st;
  }
  st = run(TTT_K_NS, "ns_step", s, [&] {
    return launch_ns_step(x, src.w1, src.w3, src.w2, out.w1, out.w3, out.w2, ns_out, lr, sh, s);
  });
  if (st) return st;
  if (norm) {
    st = run(TTT_K_NS, "weight_sumsq", s, [&] {
      return launch_weight_sumsq(out.w1, out.w3, out.w2, wsq + 3 * P.H * slots, P.H, P.d, P.m, s);
    });
    if (st) return st;
    st = run(TTT_K_NS, "norm_rescale", s, [&] {
      return launch_norm_rescale(out.w1, out.w3, out.w2, wsq, slots, nullptr, nullptr, nullptr, P.H, P.d, P.m,
                                 P.bf16, s);
    });
    if (st) return st;
  }
  return TTT_OK;
}

// ops_ready: the operand copies of `in` are already at the start of the workspace
// (written by the previous call's last step or by an apply cast of the same layout).
// keep_ops: the last step leaves the operand copies of `out` there.
// norm: the norm-preserving step (W^ = ||W|| (W - lr NS) / ||W - lr NS|| per matrix).
int do_update(const UpdatePlan &P, W3 in, W3o out, const void *k, const void *v, int64_t ld, const float *eta,
              int64_t eta_hs, float lr, int steps, float *grad_out, float *ns_out, char *ws, hipStream_t s,
              bool norm, bool ops_ready = false, bool keep_ops = false) {
  const bool fused = !g_ns_unfused;
  float *part = reinterpret_cast<float *>(ws + P.off_part);
  int st;
  for (int t = 0; t < steps; ++t) {
    const W3 src = t == 0 ? in : W3{out.w1, out.w3, out.w2};
    const bool last = t == steps - 1;
    // the folded step writes the next step's copies
    GradOps ops{};
    if ((st = prepare_operands(P, src, t == 0 ? ops_ready : fused, ws, s, &ops))) return st;
    if ((st = gradient_pass(P, ops, k, v, ld, eta, eta_hs, part, ws, s))) return st;
    if ((st = optimiser_step(P, src, out, part, P.splits, lr, !last || keep_ops, last ? grad_out : nullptr,
                             last ? ns_out : nullptr, norm, ws, s)))
      return st;
  }
  return TTT_OK;
}

// The workspace starts with the operand copies in the update's layout when the
// fast bf16 kernel runs (W1, W3, W2^T as [H][m][d]); ops_ready skips their cast.
bool apply_shares_update_ops(int d, int dtype) {
  return dtype == TTT_BF16 && !g_force_general && apply_fast_supported(d, true);
}

int do_apply(int H, int d, int m, W3 w, const void *q, int64_t ldq, void *o, int64_t ldo, int64_t nq, int dtype,
             char *ws, hipStream_t s, bool ops_ready = false) {
  if (nq == 0) return TTT_OK;
  const bool bf16 = dtype == TTT_BF16;
  const bool fast = !g_force_general && apply_fast_supported(d, bf16);
  if (apply_big(d, m, dtype)) {
    const size_t mat = (size_t)H * d * m;
    __bf16 *b = reinterpret_cast<__bf16 *>(ws);
    const int st = run(TTT_K_CAST, "cast", s, [&] {
      return launch_cast(w.w1, w.w3, w.w2, b, b + mat, nullptr, b + 2 * mat, H, d, m, true, s);
    });
    if (st) return st;
    BigApplyParams bp{};
    bp.q = q, bp.ldq = ldq, bp.o = o, bp.ldo = ldo, bp.w1 = b, bp.w3 = b + mat, bp.w2 = b + 2 * mat;
    bp.hbuf = ws + align256(3 * mat * 2);
    bp.nq = nq, bp.nq_pad = big_pad_tokens(nq), bp.heads = H, bp.d = d, bp.m = m;
    return run(TTT_K_APPLY, "apply", s, [&] { return launch_big_apply(bp, s); });
  }
  ApplyParams ap{};
  ap.q = q, ap.ldq = ldq, ap.o = o, ap.ldo = ldo, ap.nq = nq, ap.heads = H, ap.d = d, ap.m = m;
  ap.dchunks = fast ? 1 : d / apply_general_dc(d, bf16);
  if (bf16) {
    // the fast kernel reads W2 transposed ([H][m][d]), the general one as stored
    const size_t mat = (size_t)H * d * m;
    __bf16 *b = reinterpret_cast<__bf16 *>(ws);
    if (!(ops_ready && fast)) {
      const int st = run(TTT_K_CAST, "cast", s, [&] {
        return launch_cast(w.w1, w.w3, w.w2, b, b + mat, fast ? b + 2 * mat : nullptr, fast ? nullptr : b + 2 * mat,
                           H, d, m, true, s);
      });
      if (st) return st;
    }
    ap.w1 = b, ap.w3 = b + mat, ap.w2 = b + 2 * mat, ap.w2t = b + 2 * mat;
  } else {
    ap.w1 = w.w1, ap.w3 = w.w3, ap.w2 = w.w2;
  }
  return run(TTT_K_APPLY, "apply", s, [&] { return launch_apply(ap, d, bf16, fast, s); });
}

int check_ws(void *ws, size_t have, size_t need) {
  if (need == 0) return TTT_OK;
  if (!ws) return fail(TTT_EWORKSPACE, "workspace is null (need %zu bytes)", need);
  if (((uintptr_t)ws) % 256 != 0) return fail(TTT_EINVAL, "workspace must be 256-byte aligned");
  if (have < need) return fail(TTT_EWORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  return TTT_OK;
}

int check_weights(const float *w1, const float *w3, const float *w2) {
  if (!w1 || !w3 || !w2) return fail(TTT_EINVAL, "fast-weight pointer is null");
  return TTT_OK;
}

}  // namespace

extern "C" {

const char *ttt_last_error(void) { return g_err.c_str(); }

int ttt_update_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t n, int32_t dtype, size_t *bytes) {
  int st = check_shape(heads, d, m, dtype);
  if (st) return st;
  if (n < 0) return fail(TTT_EINVAL, "n must be >= 0");
  if (!bytes) return fail(TTT_EINVAL, "bytes is null");
  *bytes = plan_update(heads, d, m, n, dtype).total;
  return TTT_OK;
}

int ttt_apply_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t nq, int32_t dtype, size_t *bytes) {
  int st = check_shape(heads, d, m, dtype);
  if (st) return st;
  if (nq < 0) return fail(TTT_EINVAL, "nq must be >= 0");
  if (!bytes) return fail(TTT_EINVAL, "bytes is null");
  *bytes = apply_ws(heads, d, m, nq, dtype);
  return TTT_OK;
}

int ttt_stream_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t chunk, int32_t dtype, size_t *bytes) {
  int st = check_shape(heads, d, m, dtype);
  if (st) return st;
  if (chunk < 1) return fail(TTT_EINVAL, "chunk must be >= 1");
  if (!bytes) return fail(TTT_EINVAL, "bytes is null");
  const size_t a = plan_update(heads, d, m, chunk, dtype).total, b = apply_ws(heads, d, m, chunk, dtype);
  *bytes = a > b ? a : b;
  return TTT_OK;
}

// Checks shared by the update entry points: shapes, flags, weight pointers and
// their aliasing, n, steps, lr.
int check_update_args(int32_t heads, int32_t d, int32_t m, const float *w1, const float *w3, const float *w2,
                      float *w1_out, float *w3_out, float *w2_out, int64_t n, float lr, int32_t steps, int32_t dtype,
                      uint32_t flags) {
  int st = check_shape(heads, d, m, dtype);
  if (st) return st;
  if (flags & ~uint32_t(TTT_NORM_PRESERVE)) return fail(TTT_EINVAL, "unknown flag bits 0x%x", flags);
  if ((st = check_weights(w1, w3, w2))) return st;
  if (!w1_out || !w3_out || !w2_out) return fail(TTT_EINVAL, "output fast-weight pointer is null");
  const size_t wb = (size_t)heads * d * m * 4;
  const float *ins[3] = {w1, w3, w2};
  float *outs[3] = {w1_out, w3_out, w2_out};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      if (overlap(ins[i], wb, outs[j], wb) && !(i == j && ins[i] == outs[j]))
        return fail(TTT_EINVAL, "output weights must equal their input or not overlap any input");
  if (n < 0) return fail(TTT_EINVAL, "n must be >= 0");
  if (steps < 1) return fail(TTT_EINVAL, "steps must be >= 1");
  if (!std::isfinite(lr)) return fail(TTT_EINVAL, "lr must be finite");
  return TTT_OK;
}

int ttt_update_ex(int32_t heads, int32_t d, int32_t m, const float *w1, const float *w3, const float *w2,
                  float *w1_out, float *w3_out, float *w2_out, const void *k, const void *v, int64_t ld_kv,
                  const float *eta, int64_t eta_head_stride, int64_t n, float lr, int32_t steps, int32_t dtype,
                  uint32_t flags, float *grad_out, float *ns_out, void *workspace, size_t workspace_bytes,
                  void *stream) {
  int st = check_update_args(heads, d, m, w1, w3, w2, w1_out, w3_out, w2_out, n, lr, steps, dtype, flags);
  if (st) return st;
  if ((st = check_token_limits(n, ld_kv, dtype, "k/v"))) return st;
  if (n > 0) {
    if ((st = check_rows(k, ld_kv, heads, d, dtype, "k"))) return st;
    if ((st = check_rows(v, ld_kv, heads, d, dtype, "v"))) return st;
    if (!eta) return fail(TTT_EINVAL, "eta is null");
    if (eta_head_stride < 0) return fail(TTT_EINVAL, "eta_head_stride must be >= 0");
  }
  const UpdatePlan P = plan_update(heads, d, m, n, dtype);
  if ((st = check_ws(workspace, workspace_bytes, P.total))) return st;
  return do_update(P, W3{w1, w3, w2}, W3o{w1_out, w3_out, w2_out}, k, v, ld_kv, eta, eta_head_stride, lr, steps,
                   grad_out, ns_out, static_cast<char *>(workspace), static_cast<hipStream_t>(stream),
                   (flags & TTT_NORM_PRESERVE) != 0);
}

// ------------------------------------------------------- allocation-free update
// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept: each device holds its own copy at its own address.
static int scratch_base(char **out) {
  static std::mutex mu;
  static void *base[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TTT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TTT_EUNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(TTT_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    base[dev] = ptr;
  }
  *out = static_cast<char *>(base[dev]);
  return TTT_OK;
}

int ttt_update_noalloc(int32_t heads, int32_t d, int32_t m, const float *w1, const float *w3, const float *w2,
                       float *w1_out, float *w3_out, float *w2_out, const void *k, const void *v, int64_t ld_kv,
                       const float *eta, int64_t eta_head_stride, int64_t n, float lr, int32_t steps,
                       int32_t dtype, uint32_t flags, float *grad_out, float *ns_out, void *stream) {
  int st = check_update_args(heads, d, m, w1, w3, w2, w1_out, w3_out, w2_out, n, lr, steps, dtype, flags);
  if (st) return st;
  if ((st = check_token_limits(n, ld_kv, dtype, "k/v"))) return st;
  if (n > 0) {
    if ((st = check_rows(k, ld_kv, heads, d, dtype, "k"))) return st;
    if ((st = check_rows(v, ld_kv, heads, d, dtype, "v"))) return st;
    if (!eta) return fail(TTT_EINVAL, "eta is null");
    if (eta_head_stride < 0) return fail(TTT_EINVAL, "eta_head_stride must be >= 0");
  }
  const UpdatePlan P = plan_update(heads, d, m, n, dtype);
  if (P.total > kNoAllocScratchBytes)
    return fail(TTT_EWORKSPACE, "this update needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                P.total, kNoAllocScratchBytes);
  char *ws = nullptr;
  if ((st = scratch_base(&ws))) return st;
  t_no_events = true;
  st = do_update(P, W3{w1, w3, w2}, W3o{w1_out, w3_out, w2_out}, k, v, ld_kv, eta, eta_head_stride, lr, steps,
                 grad_out, ns_out, ws, static_cast<hipStream_t>(stream), (flags & TTT_NORM_PRESERVE) != 0);
  t_no_events = false;
  return st;
}

int ttt_noalloc_scratch_bytes(size_t *bytes) {
  if (!bytes) return fail(TTT_EINVAL, "bytes is null");
  *bytes = kNoAllocScratchBytes;
  return TTT_OK;
}

// ------------------------------------------------------- out-of-core update
// One copy stream per device (default priority, created on first use, kept for
// the life of the process): host -> device copies of the next batch run on it
// while the gradient of the current one runs on the caller's stream.
static int copy_stream(hipStream_t *out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TTT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TTT_EUNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) {
    e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking);
    if (e != hipSuccess) return fail(TTT_EHIP, "hipStreamCreateWithFlags: %s", hipGetErrorString(e));
  }
  *out = streams[dev];
  return TTT_OK;
}

// One side stream per device (default priority, created on first use, kept for the
// life of the process): a stream's apply of chunk c runs on it while the caller's
// stream runs chunk c's optimiser step (both read only the weights of chunk c).
static int side_stream(hipStream_t *out) {
  static std::mutex mu;
  static hipStream_t streams[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TTT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TTT_EUNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) {
    e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking);
    if (e != hipSuccess) return fail(TTT_EHIP, "hipStreamCreateWithFlags: %s", hipGetErrorString(e));
  }
  *out = streams[dev];
  return TTT_OK;
}

// Workspace of ttt_update_host: the update plan of one batch, the running G, and
// two staging slots (K rows, V rows, the batch's rates).
struct HostPlan {
  UpdatePlan P;
  size_t off_gacc, off_slot[2], slot_k, slot_e, total;
};
HostPlan plan_host(int H, int d, int m, int64_t batch, int64_t ld, int dtype) {
  HostPlan h{};
  h.P = plan_update(H, d, m, batch, dtype);
  size_t off = h.P.total;
  h.off_gacc = off;
  off = align256(off + (size_t)3 * H * d * m * 4);
  h.slot_k = align256((size_t)batch * ld * esize(dtype));
  h.slot_e = align256((size_t)H * batch * 4);
  for (int i = 0; i < 2; ++i) {
    h.off_slot[i] = off;
    off += 2 * h.slot_k + h.slot_e;
  }
  h.total = off;
  return h;
}

int ttt_update_host_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t batch, int64_t ld_kv,
                                    int32_t dtype, size_t *bytes) {
  int st = check_shape(heads, d, m, dtype);
  if (st) return st;
  if (batch < 1) return fail(TTT_EINVAL, "batch must be >= 1");
  if (ld_kv < (int64_t)heads * d) return fail(TTT_EINVAL, "ld_kv < heads*d");
  if (!bytes) return fail(TTT_EINVAL, "bytes is null");
  *bytes = plan_host(heads, d, m, batch, ld_kv, dtype).total;
  return TTT_OK;
}

int ttt_update_host(int32_t heads, int32_t d, int32_t m, const float *w1, const float *w3, const float *w2,
                    float *w1_out, float *w3_out, float *w2_out, const void *k, const void *v, int64_t ld_kv,
                    const float *eta, int64_t eta_head_stride, int64_t n, int64_t batch, float lr, int32_t steps,
                    int32_t dtype, uint32_t flags, float *grad_out, float *ns_out, void *workspace,
                    size_t workspace_bytes, void *stream) {
  int st = check_update_args(heads, d, m, w1, w3, w2, w1_out, w3_out, w2_out, n, lr, steps, dtype, flags);
  if (st) return st;
  if (batch < 1) return fail(TTT_EINVAL, "batch must be >= 1");
  if ((st = check_token_limits(batch, ld_kv, dtype, "k/v"))) return st;
  if (ld_kv < (int64_t)heads * d) return fail(TTT_EINVAL, "ld_kv (%lld) < heads*d", (long long)ld_kv);
  if ((ld_kv * (int64_t)esize(dtype)) % 16 != 0) return fail(TTT_EINVAL, "k/v rows must be 16-byte aligned");
  if (n > 0 && (!k || !v || !eta)) return fail(TTT_EINVAL, "k, v or eta is null");
  if (eta_head_stride < 0) return fail(TTT_EINVAL, "eta_head_stride must be >= 0");
  const HostPlan HP = plan_host(heads, d, m, batch, ld_kv, dtype);
  if ((st = check_ws(workspace, workspace_bytes, HP.total))) return st;
  char *ws = static_cast<char *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool norm = (flags & TTT_NORM_PRESERVE) != 0;
  if (n == 0)   // G = 0: the in-core path with no tokens
    return do_update(plan_update(heads, d, m, 0, dtype), W3{w1, w3, w2}, W3o{w1_out, w3_out, w2_out}, nullptr,
                     nullptr, ld_kv, nullptr, 0, lr, steps, grad_out, ns_out, ws, s, norm);
  hipStream_t cs;
  if ((st = copy_stream(&cs))) return st;
  hipEvent_t ev[5] = {};     // ready[2], free[2], start
  for (int i = 0; i < 5; ++i) {
    const hipError_t e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      for (int j = 0; j < i; ++j) hipEventDestroy(ev[j]);
      return fail(TTT_EHIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
    }
  }
  auto hip_ok = [&](hipError_t e, const char *what) -> int {
    if (e == hipSuccess) return TTT_OK;
    return fail(TTT_EHIP, "%s: %s", what, hipGetErrorString(e));
  };
  const size_t es = esize(dtype);
  const size_t mat = (size_t)heads * d * m;
  float *gacc = reinterpret_cast<float *>(ws + HP.off_gacc);
  const int erows = eta_head_stride == 0 ? 1 : heads;
  // the copies start after the caller's earlier work on `stream` (which may still
  // read this workspace)
  st = hip_ok(hipEventRecord(ev[4], s), "hipEventRecord");
  if (!st) st = hip_ok(hipStreamWaitEvent(cs, ev[4], 0), "hipStreamWaitEvent");
  int64_t cnt = 0;
  for (int t = 0; t < steps && !st; ++t) {
    const W3 src = t == 0 ? W3{w1, w3, w2} : W3{w1_out, w3_out, w2_out};
    const bool last = t == steps - 1;
    GradOps ops{};
    if ((st = prepare_operands(HP.P, src, t > 0 && !g_ns_unfused, ws, s, &ops))) break;
    for (int64_t t0 = 0; t0 < n && !st; t0 += batch, ++cnt) {
      const int64_t len = n - t0 < batch ? n - t0 : batch;
      const int slot = (int)(cnt & 1);
      char *sk = ws + HP.off_slot[slot], *sv = sk + HP.slot_k;
      float *se = reinterpret_cast<float *>(sv + HP.slot_k);
      // copy stream: slot free (its previous batch consumed), then K, V, eta
      if (cnt >= 2 && (st = hip_ok(hipStreamWaitEvent(cs, ev[2 + slot], 0), "hipStreamWaitEvent"))) break;
      const size_t rows_b = (size_t)len * ld_kv * es;
      if ((st = hip_ok(hipMemcpyAsync(sk, static_cast<const char *>(k) + t0 * ld_kv * es, rows_b,
                                      hipMemcpyHostToDevice, cs), "hipMemcpyAsync(k)")))
        break;
      if ((st = hip_ok(hipMemcpyAsync(sv, static_cast<const char *>(v) + t0 * ld_kv * es, rows_b,
                                      hipMemcpyHostToDevice, cs), "hipMemcpyAsync(v)")))
        break;
      if (erows == 1 || eta_head_stride >= len) {
        const size_t spitch = (size_t)(erows > 1 ? eta_head_stride : len) * 4;
        st = hip_ok(hipMemcpy2DAsync(se, (size_t)len * 4, eta + t0, spitch, (size_t)len * 4, erows,
                                     hipMemcpyHostToDevice, cs), "hipMemcpy2DAsync(eta)");
      } else {           // head rows closer than the batch: one copy per head
        for (int hh = 0; hh < erows && !st; ++hh)
          st = hip_ok(hipMemcpyAsync(se + (size_t)hh * len, eta + hh * eta_head_stride + t0, (size_t)len * 4,
                                     hipMemcpyHostToDevice, cs), "hipMemcpyAsync(eta)");
      }
      if (st) break;
      if ((st = hip_ok(hipEventRecord(ev[slot], cs), "hipEventRecord"))) break;
      // compute stream: gradient of the batch, added to the running G
      if ((st = hip_ok(hipStreamWaitEvent(s, ev[slot], 0), "hipStreamWaitEvent"))) break;
      const UpdatePlan Pb = plan_update(heads, d, m, len, dtype);
      float *part = reinterpret_cast<float *>(ws + Pb.off_part);
      if ((st = gradient_pass(Pb, ops, sk, sv, ld_kv, se, erows > 1 ? len : 0, part, ws, s))) break;
      st = run(TTT_K_REDUCE, "accumulate", s, [&] {
        return launch_accumulate(gacc, part, Pb.splits, (int64_t)3 * mat, t0 == 0, s);
      });
      if (st) break;
      st = hip_ok(hipEventRecord(ev[2 + slot], s), "hipEventRecord");
    }
    if (st) break;
    st = optimiser_step(HP.P, src, W3o{w1_out, w3_out, w2_out}, gacc, 1, lr, !last, last ? grad_out : nullptr,
                        last ? ns_out : nullptr, norm, ws, s);
  }
  for (int i = 0; i < 5; ++i) hipEventDestroy(ev[i]);   // released once their work completes
  return st;
}

int ttt_update(int32_t heads, int32_t d, int32_t m, const float *w1, const float *w3, const float *w2, float *w1_out,
               float *w3_out, float *w2_out, const void *k, const void *v, int64_t ld_kv, const float *eta,
               int64_t eta_head_stride, int64_t n, float lr, int32_t steps, int32_t dtype, float *grad_out,
               float *ns_out, void *workspace, size_t workspace_bytes, void *stream) {
  return ttt_update_ex(heads, d, m, w1, w3, w2, w1_out, w3_out, w2_out, k, v, ld_kv, eta, eta_head_stride, n, lr,
                       steps, dtype, 0u, grad_out, ns_out, workspace, workspace_bytes, stream);
}

int ttt_apply(int32_t heads, int32_t d, int32_t m, const float *w1, const float *w3, const float *w2, const void *q,
              int64_t ld_q, void *o, int64_t ld_o, int64_t nq, int32_t dtype, void *workspace,
              size_t workspace_bytes, void *stream) {
  int st = check_shape(heads, d, m, dtype);
  if (st) return st;
  if ((st = check_weights(w1, w3, w2))) return st;
  if (nq < 0) return fail(TTT_EINVAL, "nq must be >= 0");
  if (nq > 0) {
    if ((st = check_rows(q, ld_q, heads, d, dtype, "q"))) return st;
    if ((st = check_rows(o, ld_o, heads, d, dtype, "o"))) return st;
    if (overlap(q, (size_t)nq * ld_q * esize(dtype), o, (size_t)nq * ld_o * esize(dtype)))
      return fail(TTT_EINVAL, "q and o must not overlap");
  }
  if ((st = check_ws(workspace, workspace_bytes, apply_ws(heads, d, m, nq, dtype)))) return st;
  return do_apply(heads, d, m, W3{w1, w3, w2}, q, ld_q, o, ld_o, nq, dtype, static_cast<char *>(workspace),
                  static_cast<hipStream_t>(stream));
}

int ttt_shortconv2d(const void *v, void *v_out, int64_t ld, const float *wconv, int32_t frames,
                    int32_t tokens_per_frame, int32_t n_special, int32_t grid_h, int32_t grid_w, int32_t channels,
                    int32_t dtype, void *stream) {
  if (dtype != TTT_F32 && dtype != TTT_BF16) return fail(TTT_EUNSUPPORTED, "unknown dtype %d", dtype);
  if (frames < 0 || n_special < 0 || grid_h < 1 || grid_w < 1 || channels < 8)
    return fail(TTT_EINVAL, "bad conv geometry");
  if (tokens_per_frame != n_special + grid_h * grid_w)
    return fail(TTT_EINVAL, "tokens_per_frame (%d) != n_special + grid_h*grid_w (%d)", tokens_per_frame,
                n_special + grid_h * grid_w);
  if (channels % 8 != 0) return fail(TTT_EUNSUPPORTED, "channels must be a multiple of 8");
  if (frames == 0) return TTT_OK;
  if (!wconv) return fail(TTT_EINVAL, "wconv is null");
  int st;
  if ((st = check_rows(v, ld, 1, channels, dtype, "v"))) return st;
  if ((st = check_rows(v_out, ld, 1, channels, dtype, "v_out"))) return st;
  const size_t bytes = (size_t)frames * tokens_per_frame * ld * esize(dtype);
  if (overlap(v, bytes, v_out, bytes)) return fail(TTT_EINVAL, "v and v_out must not overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return run(TTT_K_CONV, "shortconv2d", s, [&] {
    return launch_conv(v, v_out, ld, wconv, frames, tokens_per_frame, n_special, grid_h, grid_w, channels,
                       dtype == TTT_BF16, s);
  });
}

int ttt_output_gate(int32_t channels, const void *o_in, int64_t ld_in, const void *wg, const float *gamma,
                    float eps, void *o_out, int64_t ld_out, int64_t n, int32_t dtype, void *stream) {
  if (dtype != TTT_F32 && dtype != TTT_BF16) return fail(TTT_EUNSUPPORTED, "unknown dtype %d", dtype);
  if (channels < 64 || channels % 64 != 0) return fail(TTT_EUNSUPPORTED, "channels must be a positive multiple of 64");
  if (n < 0) return fail(TTT_EINVAL, "n must be >= 0");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(TTT_EINVAL, "eps must be finite and >= 0");
  if (n == 0) return TTT_OK;
  int st;
  if ((st = check_rows(o_in, ld_in, 1, channels, dtype, "o_in"))) return st;
  if ((st = check_rows(o_out, ld_out, 1, channels, dtype, "o_out"))) return st;
  if (!wg || reinterpret_cast<uintptr_t>(wg) % 16 != 0) return fail(TTT_EINVAL, "wg is null or not 16-byte aligned");
  if (!gamma || reinterpret_cast<uintptr_t>(gamma) % 16 != 0)
    return fail(TTT_EINVAL, "gamma is null or not 16-byte aligned");
  const size_t es = esize(dtype);
  // the kernel addresses a 256-row tile of o_in and of W_g through 32-bit offsets
  if ((uint64_t)256 * ld_in * es >= (1ull << 32) || (uint64_t)256 * channels * es >= (1ull << 32))
    return fail(TTT_EUNSUPPORTED, "256 rows of o_in or W_g must span < 4 GiB");
  const size_t in_b = (size_t)n * ld_in * es, out_b = (size_t)n * ld_out * es, wg_b = (size_t)channels * channels * es;
  if (overlap(o_in, in_b, o_out, out_b)) return fail(TTT_EINVAL, "o_in and o_out must not overlap");
  if (overlap(wg, wg_b, o_out, out_b)) return fail(TTT_EINVAL, "wg and o_out must not overlap");
  GateParams gp{};
  gp.o_in = o_in, gp.ld_in = ld_in, gp.wg = wg, gp.gamma = gamma, gp.eps = eps;
  gp.o_out = o_out, gp.ld_out = ld_out, gp.n = n, gp.channels = channels, gp.tiles_n = gate_tiles(n);
  const int64_t blocks = (gp.tiles_n * ((channels + 127) / 128) + 7) / 8 * 8;
  if (blocks > 0x7fffffffLL) return fail(TTT_EUNSUPPORTED, "n too large for one launch");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return run(TTT_K_GATE, "output_gate", s, [&] { return launch_gate(gp, dtype == TTT_BF16, s); });
}

}  // extern "C"

namespace {
// The stream with the fast apply kernel (bf16, d <= 256): chunk c's first gradient runs
// on the caller's stream, then its apply on the side stream alongside the first
// optimiser step.  Both read only W_c: the apply the shared operand copies, which that
// step's last product overwrites, so that product waits for the apply.  The next
// chunk's apply waits for its gradient to be issued after all of chunk c's steps.  The
// results are those of apply-then-update per chunk, bit for bit (same kernels, same
// inputs); the side stream joins the caller's through the last chunk's first step.
int stream_overlapped(int heads, int d, int m, W3o w, const char *k, const char *v, int64_t ld_kv, const float *eta,
                      int64_t eta_hs, const char *q, int64_t ld_q, char *o, int64_t ld_o, int64_t n, int64_t chunk,
                      float lr, int steps, bool norm, char *ws, hipStream_t s) {
  hipStream_t s2 = nullptr;
  int st = side_stream(&s2);
  if (st) return st;
  hipEvent_t ready = nullptr, applied = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&applied, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (ready) hipEventDestroy(ready);
    return fail(TTT_EHIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
  }
  const size_t es = 2;
  for (int64_t t0 = 0; t0 < n && !st; t0 += chunk) {
    const int64_t len = n - t0 < chunk ? n - t0 : chunk;
    const UpdatePlan P = plan_update(heads, d, m, len, TTT_BF16);
    float *part = reinterpret_cast<float *>(ws + P.off_part);
    for (int t = 0; t < steps && !st; ++t) {
      GradOps ops{};
      // the operand copies: cast for the stream's first step, left by the previous step after it
      if ((st = prepare_operands(P, W3{w.w1, w.w3, w.w2}, t0 != 0 || t != 0, ws, s, &ops))) break;
      if ((st = gradient_pass(P, ops, k + t0 * ld_kv * es, v + t0 * ld_kv * es, ld_kv, eta + t0, eta_hs, part, ws,
                              s)))
        break;
      if (t == 0) {
        if ((e = hipEventRecord(ready, s)) != hipSuccess || (e = hipStreamWaitEvent(s2, ready, 0)) != hipSuccess) {
          st = fail(TTT_EHIP, "stream event: %s", hipGetErrorString(e));
          break;
        }
        if ((st = do_apply(heads, d, m, W3{w.w1, w.w3, w.w2}, q + t0 * ld_q * es, ld_q, o + t0 * ld_o * es, ld_o,
                           len, TTT_BF16, ws, s2, true)))
          break;
        if ((e = hipEventRecord(applied, s2)) != hipSuccess) {
          st = fail(TTT_EHIP, "stream event: %s", hipGetErrorString(e));
          break;
        }
      }
      st = optimiser_step(P, W3{w.w1, w.w3, w.w2}, w, part, P.splits, lr, true, nullptr, nullptr, norm, ws, s,
                          t == 0 ? applied : nullptr);
    }
  }
  if (st) hipStreamWaitEvent(s, applied, 0);   // an error: still join what was issued
  hipEventDestroy(ready);
  hipEventDestroy(applied);
  return st;
}
}  // namespace

extern "C" {

int ttt_stream_ex(int32_t heads, int32_t d, int32_t m, float *w1, float *w3, float *w2, const void *k,
                  const void *v, int64_t ld_kv, const float *eta, int64_t eta_head_stride, const void *q, int64_t ld_q,
                  void *o, int64_t ld_o, int64_t n, int64_t chunk, float lr, int32_t steps, int32_t dtype,
                  uint32_t flags, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_shape(heads, d, m, dtype);
  if (st) return st;
  if (flags & ~uint32_t(TTT_NORM_PRESERVE)) return fail(TTT_EINVAL, "unknown flag bits 0x%x", flags);
  if ((st = check_weights(w1, w3, w2))) return st;
  if (n < 0 || chunk < 1 || steps < 1) return fail(TTT_EINVAL, "need n >= 0, chunk >= 1, steps >= 1");
  if (!std::isfinite(lr)) return fail(TTT_EINVAL, "lr must be finite");
  if (n == 0) return TTT_OK;
  if ((st = check_token_limits(chunk < n ? chunk : n, ld_kv, dtype, "k/v"))) return st;
  if ((st = check_rows(k, ld_kv, heads, d, dtype, "k"))) return st;
  if ((st = check_rows(v, ld_kv, heads, d, dtype, "v"))) return st;
  if ((st = check_rows(q, ld_q, heads, d, dtype, "q"))) return st;
  if ((st = check_rows(o, ld_o, heads, d, dtype, "o"))) return st;
  if (!eta || eta_head_stride < 0) return fail(TTT_EINVAL, "eta is null or has a negative head stride");
  size_t need = 0;
  ttt_stream_workspace_bytes(heads, d, m, chunk, dtype, &need);
  if ((st = check_ws(workspace, workspace_bytes, need))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  const size_t es = esize(dtype);
  // With the folded optimiser step, each chunk's last step leaves the operand copies
  // of the new weights at the start of the workspace, where the next chunk's apply
  // (when its layout is the same) and gradient read them: one cast per stream.
  const bool carry = !g_ns_unfused;
  const bool shared = carry && apply_shares_update_ops(d, dtype);
  if (shared && dtype == TTT_BF16 && !g_force_general && apply_fast_supported(d, true))
    return stream_overlapped(heads, d, m, W3o{w1, w3, w2}, static_cast<const char *>(k), static_cast<const char *>(v),
                             ld_kv, eta, eta_head_stride, static_cast<const char *>(q), ld_q, static_cast<char *>(o),
                             ld_o, n, chunk, lr, steps, (flags & TTT_NORM_PRESERVE) != 0, ws, s);
  for (int64_t t0 = 0; t0 < n; t0 += chunk) {
    const int64_t len = n - t0 < chunk ? n - t0 : chunk;
    const bool first = t0 == 0;
    st = do_apply(heads, d, m, W3{w1, w3, w2}, static_cast<const char *>(q) + t0 * ld_q * es, ld_q,
                  static_cast<char *>(o) + t0 * ld_o * es, ld_o, len, dtype, ws, s, shared && !first);
    if (st) return st;
    const UpdatePlan P = plan_update(heads, d, m, len, dtype);
    // the apply just cast W into the update's operand layout (shared), or the previous
    // chunk's step left them (fp32 keeps only W2^T there, which apply never touches)
    const bool ready = shared || (carry && dtype == TTT_F32 && !first);
    st = do_update(P, W3{w1, w3, w2}, W3o{w1, w3, w2}, static_cast<const char *>(k) + t0 * ld_kv * es,
                   static_cast<const char *>(v) + t0 * ld_kv * es, ld_kv, eta + t0, eta_head_stride, lr, steps,
                   nullptr, nullptr, ws, s, (flags & TTT_NORM_PRESERVE) != 0, ready, carry);
    if (st) return st;
  }
  return TTT_OK;
}

int ttt_stream(int32_t heads, int32_t d, int32_t m, float *w1, float *w3, float *w2, const void *k, const void *v,
               int64_t ld_kv, const float *eta, int64_t eta_head_stride, const void *q, int64_t ld_q, void *o,
               int64_t ld_o, int64_t n, int64_t chunk, float lr, int32_t steps, int32_t dtype, void *workspace,
               size_t workspace_bytes, void *stream) {
  return ttt_stream_ex(heads, d, m, w1, w3, w2, k, v, ld_kv, eta, eta_head_stride, q, ld_q, o, ld_o, n, chunk, lr,
                       steps, dtype, 0u, workspace, workspace_bytes, stream);
}

int ttt_set_option(int32_t option, int64_t value) {
  switch (option) {
    case TTT_OPT_FORCE_GENERAL: g_force_general = value != 0; return TTT_OK;
    case TTT_OPT_SPLITS:
      if (value < 0) return fail(TTT_EINVAL, "splits must be >= 0");
      g_splits = value;
      return TTT_OK;
    case TTT_OPT_NS_UNFUSED: g_ns_unfused = value != 0; return TTT_OK;
  }
  return fail(TTT_EINVAL, "unknown option %d", option);
}

int ttt_mfma_rate_probe(int32_t iters, void *stream, double *flop) {
  if (iters < 1 || !flop) return fail(TTT_EINVAL, "iters must be >= 1 and flop non-null");
  const hipError_t e = launch_mfma_probe(iters, static_cast<hipStream_t>(stream), flop);
  if (e != hipSuccess) return fail(TTT_EHIP, "mfma_probe: %s", hipGetErrorString(e));
  return TTT_OK;
}

int ttt_profile_enable(int32_t on) {
  g_prof = on != 0;
  return TTT_OK;
}

int ttt_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto &p : g_pending) {
    hipEventSynchronize(p.e1);
    g_free_events.push_back(p.e0);
    g_free_events.push_back(p.e1);
  }
  g_pending.clear();
  for (int i = 0; i < TTT_K_COUNT; ++i) g_ms[i] = 0.0, g_count[i] = 0;
  return TTT_OK;
}

int ttt_profile_read(int32_t kind, double *total_ms, int64_t *launches) {
  if (kind < 0 || kind >= TTT_K_COUNT || !total_ms || !launches) return fail(TTT_EINVAL, "bad profile query");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto &p : g_pending) {
    hipError_t e = hipEventSynchronize(p.e1);
    if (e != hipSuccess) return fail(TTT_EHIP, "profile: %s", hipGetErrorString(e));
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, p.e0, p.e1);
    if (e != hipSuccess) return fail(TTT_EHIP, "profile: %s", hipGetErrorString(e));
    g_ms[p.kind] += ms;
    g_count[p.kind] += 1;
    g_free_events.push_back(p.e0);
    g_free_events.push_back(p.e1);
  }
  g_pending.clear();
  *total_ms = g_ms[kind];
  *launches = g_count[kind];
  return TTT_OK;
}

}  // extern "C"
