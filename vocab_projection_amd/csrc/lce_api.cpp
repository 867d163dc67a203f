// lce_api.cpp - the C ABI of include/lce.h: argument checks, the strip-width
// policy, the workspace carve and the strip loop.  Every call only enqueues
// kernels on the caller's stream; nothing here waits for the device or
// allocates device memory.
#include "lce.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "lce_kernels.h"

namespace {

constexpr int64_t kStripTile = 256;  // vocabulary tile of the strip kernels
constexpr int64_t kPartRows = 128;   // vocabulary rows per forward partial
constexpr size_t kHeader = 256;
constexpr int64_t kMaxHidden = 1LL << 20;
constexpr int64_t kMaxStrip = 1LL << 21;

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

struct Plan {
  int64_t N, H, V, Vs, ldg;
  int dtype, reduction;
  int32_t ignore_index;
  size_t elt;
  size_t off_m, off_s, off_zt, off_strip, total;
  int64_t fwd_chunk;  // widest vocabulary range one forward fold can take (>= Vs)
};

bool problem_ok(const lce_problem_t* p) {
  if (!p) return false;
  if (p->n_tokens < 1 || p->hidden < 1 || p->vocab < 1) return false;
  if (p->strip < 0 || p->strip > p->vocab) return false;
  if (p->dtype != LCE_F32 && p->dtype != LCE_BF16) return false;
  if (p->reduction != LCE_MEAN && p->reduction != LCE_SUM) return false;
  if (p->reserved != 0) return false;
  // The kernels address one tile with byte offsets below 2^31: at most 256
  // rows of H elements or of a strip row of round_up(Vs, 256) elements, at
  // most 4 bytes each.  H <= 2^20 and Vs <= 2^21 keep 256 * 4 * max(H, Vs)
  // within 2^31.
  if (p->n_tokens > (1LL << 31) || p->hidden > kMaxHidden || p->vocab > (1LL << 31)) return false;
  if (p->strip > kMaxStrip) return false;
  return true;
}

size_t elt_of(int dtype) { return dtype == LCE_BF16 ? 2 : 4; }

// Workspace: a 256-byte control block, then one strip region of
// round_up(N, 16) x ldg elements.  The backward keeps its gradient strip G there; the forward keeps
// the running per-token state (max, sum, target logit; each column padded to
// 256 bytes) at the region's end and its per-block partials [blocks, N] of
// (max, sum) before it.  The region is the larger of the two needs; the
// forward's is smaller except for a handful of tokens.  A partial takes 8
// bytes per 128 vocabulary rows, against 128 x elt bytes of G, so the
// region holds the partials of about 32 (bf16) or 64 (f32) strips beside the
// state: lce_forward folds that many strips per launch.
size_t state_col_bytes(int64_t n) { return (size_t)round_up(4 * n, 256); }

size_t partial_bytes(int64_t n, int64_t ldg) { return (size_t)n * (size_t)(ldg / kPartRows) * 8; }

size_t bytes_for_strip(int64_t n, int64_t vs, size_t elt) {
  const int64_t ldg = round_up(vs, kStripTile);
  // backward G strip: whole 16-token bands (bf16 strips are kept in blocks of 16 rows)
  const size_t g = (size_t)round_up(n, 16) * (size_t)ldg * elt;
  const size_t fwd = partial_bytes(n, ldg) + 3 * state_col_bytes(n);      // forward use
  return kHeader + (g > fwd ? g : fwd);
}

// Widest strip (a multiple of the 256-row tile, at most V rounded up and at
// most 2^21, then clamped to V) whose whole workspace - the larger of the
// backward's gradient strip and the forward's partials plus running state,
// and the header - fits in `budget`; -1 if not even one tile's does.
// bytes_for_strip grows with the strip, so the widest fit is found by
// bisection over the tile count.
int64_t pick_strip(const lce_problem_t* p, size_t budget) {
  const size_t elt = elt_of(p->dtype);
  const int64_t n = p->n_tokens;
  int64_t hi = round_up(p->vocab, kStripTile);
  if (hi > kMaxStrip) hi = kMaxStrip;
  int64_t lo_t = 0, hi_t = hi / kStripTile;  // widest fitting tile count in [lo_t, hi_t]
  while (lo_t < hi_t) {
    const int64_t mid = (lo_t + hi_t + 1) / 2;
    if (bytes_for_strip(n, mid * kStripTile, elt) <= budget)
      lo_t = mid;
    else
      hi_t = mid - 1;
  }
  if (lo_t == 0) return -1;
  const int64_t vs = lo_t * kStripTile;
  return vs > p->vocab ? p->vocab : vs;
}

lce_status_t make_plan(const lce_problem_t* p, Plan* pl) {
  if (!problem_ok(p)) return LCE_ERR_INVALID_VALUE;
  const size_t elt = elt_of(p->dtype);
  if ((p->hidden * (int64_t)elt) % 16 != 0) return LCE_ERR_UNSUPPORTED;
  pl->N = p->n_tokens;
  pl->H = p->hidden;
  pl->V = p->vocab;
  if (p->strip) {
    pl->Vs = p->strip;
  } else {
    // the default budget, or one tile when not even that fits it
    const int64_t vs = pick_strip(p, LCE_DEFAULT_BUDGET);
    pl->Vs = vs > 0 ? vs : (p->vocab < kStripTile ? p->vocab : kStripTile);
  }
  pl->ldg = round_up(pl->Vs, kStripTile);
  pl->dtype = p->dtype;
  pl->reduction = p->reduction;
  pl->ignore_index = p->ignore_index;
  pl->elt = elt;
  const size_t col = state_col_bytes(pl->N);
  pl->total = bytes_for_strip(pl->N, pl->Vs, elt);
  pl->off_strip = kHeader;
  pl->off_zt = pl->total - col;
  pl->off_s = pl->off_zt - col;
  pl->off_m = pl->off_s - col;
  // partial blocks that fit before the state; at least ldg / 128 by construction
  const int64_t blocks = (int64_t)((pl->off_m - pl->off_strip) / ((size_t)pl->N * 8));
  int64_t chunk = blocks * kPartRows;
  if (chunk > kMaxStrip) chunk = kMaxStrip;  // same tile-offset bound as one strip
  pl->fwd_chunk = chunk > pl->Vs ? chunk : pl->Vs;
  return LCE_OK;
}

bool aligned(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

lce_status_t check_ws(const Plan& pl, void* ws, size_t ws_bytes) {
  if (!ws || !aligned(ws)) return LCE_ERR_WORKSPACE;
  if (ws_bytes < pl.total) return LCE_ERR_WORKSPACE;
  return LCE_OK;
}

lce_status_t launched(hipError_t e) { return e == hipSuccess ? LCE_OK : LCE_ERR_LAUNCH; }

struct Carve {
  lce::Control* ctrl;
  float *m, *s, *zt;
  char* strip;
};

Carve carve(const Plan& pl, void* ws) {
  char* b = static_cast<char*>(ws);
  return Carve{reinterpret_cast<lce::Control*>(b), reinterpret_cast<float*>(b + pl.off_m),
               reinterpret_cast<float*>(b + pl.off_s), reinterpret_cast<float*>(b + pl.off_zt),
               b + pl.off_strip};
}

// A fold's vocabulary rows: at most max_len of them (the strip for the
// backward, the forward's partials capacity for the forward), inside [0, V).
lce_status_t check_strip(const Plan& pl, const void* weight_strip, int64_t v_begin,
                         int64_t v_len, int64_t max_len) {
  if (!weight_strip || !aligned(weight_strip)) return LCE_ERR_INVALID_VALUE;
  if (v_len < 1 || v_len > max_len || v_begin < 0 || v_begin > pl.V - v_len)
    return LCE_ERR_INVALID_VALUE;
  return LCE_OK;
}

template <typename T>
lce_status_t fold_fwd(const Plan& pl, const void* hidden, const void* weight_strip,
                      int64_t v_begin, int64_t v_len, const int32_t* targets, void* ws,
                      unsigned steps, hipStream_t st) {
  Carve c = carve(pl, ws);
  lce::StripArgs<T> a{};
  a.hidden = static_cast<const T*>(hidden);
  a.weight_strip = static_cast<const T*>(weight_strip);
  a.targets = targets;
  a.N = pl.N;
  a.H = pl.H;
  a.v_begin = v_begin;
  a.v_len = v_len;
  a.ignore_index = pl.ignore_index;
  a.partials = reinterpret_cast<float2*>(c.strip);
  a.z_target = c.zt;
  if (steps & LCE_STEP_STRIP) {
    lce_status_t s = launched(lce::launch_strip_lse<T>(a, st));
    if (s != LCE_OK) return s;
  }
  if (steps & LCE_STEP_MERGE) {
    const int64_t nblk = (v_len + kPartRows - 1) / kPartRows;
    return launched(lce::launch_fold(a.partials, nblk, c.m, c.s, pl.N, st));
  }
  return LCE_OK;
}

template <typename T>
lce_status_t fold_bwd(const Plan& pl, const void* hidden, const void* weight_strip,
                      int64_t v_begin, int64_t v_len, const int32_t* targets, const float* lse,
                      float* d_hidden, int accumulate, float* d_weight_strip, void* ws,
                      unsigned steps, hipStream_t st) {
  Carve c = carve(pl, ws);
  lce::StripArgs<T> a{};
  a.hidden = static_cast<const T*>(hidden);
  a.weight_strip = static_cast<const T*>(weight_strip);
  a.targets = targets;
  a.N = pl.N;
  a.H = pl.H;
  a.v_begin = v_begin;
  a.v_len = v_len;
  a.ignore_index = pl.ignore_index;
  a.lse = lse;
  a.ctrl = c.ctrl;
  a.g_strip = reinterpret_cast<T*>(c.strip);
  a.ldg = pl.ldg;
  lce_status_t s = LCE_OK;
  if (steps & LCE_STEP_GRAD) {
    if ((s = launched(lce::launch_strip_grad<T>(a, st))) != LCE_OK) return s;
  }
  const int acc_dh = (accumulate & LCE_ACC_DHIDDEN) != 0;
  const int acc_dw = (accumulate & LCE_ACC_DWEIGHT) != 0;
  if ((steps & LCE_STEP_DHIDDEN) && (steps & LCE_STEP_DWEIGHT)) {
    return launched(lce::launch_dh_dw<T>(a.g_strip, pl.ldg, a.weight_strip, a.hidden, v_len, pl.N,
                                         pl.H, d_hidden, acc_dh, d_weight_strip, acc_dw, st));
  }
  if (steps & LCE_STEP_DHIDDEN) {
    s = launched(lce::launch_dh<T>(a.g_strip, pl.ldg, a.weight_strip, v_len, pl.N, pl.H, d_hidden,
                                   acc_dh, st));
    if (s != LCE_OK) return s;
  }
  if (steps & LCE_STEP_DWEIGHT) {
    s = launched(lce::launch_dw<T>(a.g_strip, pl.ldg, a.hidden, v_len, pl.N, pl.H,
                                   d_weight_strip, acc_dw, st));
  }
  return s;
}

// ---- The backward without a strip buffer ----
constexpr int64_t kFusedBlocks = 256;  // blocks a fused sweep aims for (one per compute unit)

struct FusedSweep {
  int64_t C, R, tok_per_r, voc_per_c;
  int do_dh, do_dw;
  int64_t blocks() const { return C * R; }
};

struct FusedPlan {
  FusedSweep sweep[2];
  int n_sweeps;
  size_t off_g, off_parts, total;
};

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Groups of `tiles` tiles so that `groups` <= want: (groups, tiles per group).
void split_groups(int64_t tiles, int64_t want, int64_t* groups, int64_t* per) {
  if (want < 1) want = 1;
  *per = cdiv64(tiles, want < tiles ? want : tiles);
  *groups = cdiv64(tiles, *per);
}

size_t sweep_partials(const Plan& pl, const FusedSweep& sw) {
  size_t b = 0;
  if (sw.do_dh && sw.C > 1) b += (size_t)sw.C * pl.N * pl.H * 4;
  if (sw.do_dw && sw.R > 1) b += (size_t)sw.R * pl.V * pl.H * 4;
  return b;
}

lce_status_t make_fused_plan(const Plan& pl, int mode, FusedPlan* fp) {
  const int64_t tt = cdiv64(pl.N, kStripTile), vt = cdiv64(pl.V, kStripTile);
  if (mode == LCE_FUSED_ONE_SWEEP) {
    // one sweep over all pairs, both outputs: the token x vocabulary grid of
    // groups with the least partial memory among those that fill the device
    FusedSweep best{};
    size_t best_bytes = (size_t)-1;
    const int64_t need = tt * vt < kFusedBlocks ? tt * vt : kFusedBlocks;
    for (int64_t r_want = 1; r_want <= (tt < kFusedBlocks ? tt : kFusedBlocks); ++r_want) {
      FusedSweep sw{};
      sw.do_dh = sw.do_dw = 1;
      split_groups(tt, r_want, &sw.R, &sw.tok_per_r);
      split_groups(vt, cdiv64(kFusedBlocks, sw.R), &sw.C, &sw.voc_per_c);
      if (sw.blocks() < need && sw.R * sw.C < tt * vt) continue;
      const size_t b = sweep_partials(pl, sw);
      if (b < best_bytes) { best_bytes = b; best = sw; }
    }
    fp->sweep[0] = best;
    fp->n_sweeps = 1;
  } else if (mode == LCE_FUSED_TWO_SWEEPS) {
    // sweep 1: dH, a block per token group (vocabulary split only if there
    // are too few token tiles); sweep 2: dW, a block per vocabulary group
    FusedSweep a{}, b{};
    a.do_dh = 1;
    split_groups(tt, kFusedBlocks, &a.R, &a.tok_per_r);
    split_groups(vt, kFusedBlocks / a.R, &a.C, &a.voc_per_c);
    b.do_dw = 1;
    split_groups(vt, kFusedBlocks, &b.C, &b.voc_per_c);
    split_groups(tt, kFusedBlocks / b.C, &b.R, &b.tok_per_r);
    fp->sweep[0] = a;
    fp->sweep[1] = b;
    fp->n_sweeps = 2;
  } else {
    return LCE_ERR_INVALID_VALUE;
  }
  int64_t blocks = 0;
  size_t parts = 0;
  for (int k = 0; k < fp->n_sweeps; ++k) {
    if (fp->sweep[k].blocks() > blocks) blocks = fp->sweep[k].blocks();
    const size_t b = sweep_partials(pl, fp->sweep[k]);
    if (b > parts) parts = b;
  }
  fp->off_g = kHeader;
  fp->off_parts = fp->off_g + (size_t)round_up((int64_t)blocks * kStripTile * kStripTile * pl.elt, 256);
  fp->total = fp->off_parts + parts;
  return LCE_OK;
}

template <typename T>
lce_status_t fused_backward(const Plan& pl, const FusedPlan& fp, const void* hidden,
                            const void* weight, const int32_t* targets, const float* lse,
                            float* d_hidden, float* d_weight, void* ws, hipStream_t st) {
  char* b = static_cast<char*>(ws);
  float* parts = reinterpret_cast<float*>(b + fp.off_parts);
  for (int k = 0; k < fp.n_sweeps; ++k) {
    const FusedSweep& sw = fp.sweep[k];
    lce::FusedLaunch<T> L{};
    L.hidden = static_cast<const T*>(hidden);
    L.weight = static_cast<const T*>(weight);
    L.targets = targets;
    L.lse = lse;
    L.ctrl = reinterpret_cast<const lce::Control*>(b);
    L.N = pl.N; L.H = pl.H; L.V = pl.V;
    L.ignore_index = pl.ignore_index;
    L.g_scratch = reinterpret_cast<T*>(b + fp.off_g);
    L.C = sw.C; L.R = sw.R; L.tok_per_r = sw.tok_per_r; L.voc_per_c = sw.voc_per_c;
    L.do_dh = sw.do_dh; L.do_dw = sw.do_dw;
    const bool dh_parts = sw.do_dh && sw.C > 1, dw_parts = sw.do_dw && sw.R > 1;
    L.dh_dst = dh_parts ? parts : d_hidden;
    L.dw_dst = dw_parts ? parts + (dh_parts ? (size_t)sw.C * pl.N * pl.H : 0) : d_weight;
    lce_status_t s = launched(lce::launch_fused_bwd<T>(L, st));
    if (s != LCE_OK) return s;
    if (dh_parts && (s = launched(lce::launch_sum_parts(L.dh_dst, sw.C, pl.N * pl.H, d_hidden,
                                                        st))) != LCE_OK)
      return s;
    if (dw_parts && (s = launched(lce::launch_sum_parts(L.dw_dst, sw.R, pl.V * pl.H, d_weight,
                                                        st))) != LCE_OK)
      return s;
  }
  return LCE_OK;
}

}  // namespace

extern "C" {

const char* lce_status_string(lce_status_t s) {
  switch (s) {
    case LCE_OK: return "LCE_OK";
    case LCE_ERR_INVALID_VALUE: return "LCE_ERR_INVALID_VALUE";
    case LCE_ERR_UNSUPPORTED: return "LCE_ERR_UNSUPPORTED";
    case LCE_ERR_WORKSPACE: return "LCE_ERR_WORKSPACE";
    case LCE_ERR_LAUNCH: return "LCE_ERR_LAUNCH";
  }
  return "LCE_ERR_UNKNOWN";
}

int64_t lce_pick_strip(const lce_problem_t* p, size_t budget_bytes) {
  if (!problem_ok(p)) return -1;
  return pick_strip(p, budget_bytes);
}

int64_t lce_forward_fold_max(const lce_problem_t* p) {
  Plan pl;
  if (make_plan(p, &pl) != LCE_OK) return -1;
  return pl.fwd_chunk < pl.V ? pl.fwd_chunk : pl.V;
}

int lce_backward_fold_gemm_launches(const lce_problem_t* p, int64_t v_len) {
  Plan pl;
  if (make_plan(p, &pl) != LCE_OK || v_len < 1 || v_len > pl.Vs) return -1;
  const int64_t split = pl.dtype == LCE_BF16 ? lce::dh_dw_split<__bf16>(v_len, pl.N, pl.H)
                                             : lce::dh_dw_split<float>(v_len, pl.N, pl.H);
  return split > 0 ? 1 : 2;
}

size_t lce_workspace_bytes(const lce_problem_t* p) {
  Plan pl;
  if (make_plan(p, &pl) != LCE_OK) return 0;
  return pl.total;
}

lce_status_t lce_forward_begin(const lce_problem_t* p, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  Carve c = carve(pl, ws);
  return launched(lce::launch_state_init(c.m, c.s, c.zt, pl.N, stream));
}

lce_status_t lce_forward_fold(const lce_problem_t* p, const void* hidden,
                              const void* weight_strip, int64_t v_begin, int64_t v_len,
                              const int32_t* targets, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  return lce_forward_fold_steps(p, hidden, weight_strip, v_begin, v_len, targets, ws, ws_bytes,
                                LCE_STEP_STRIP | LCE_STEP_MERGE, stream);
}

lce_status_t lce_forward_fold_steps(const lce_problem_t* p, const void* hidden,
                                    const void* weight_strip, int64_t v_begin, int64_t v_len,
                                    const int32_t* targets, void* ws, size_t ws_bytes,
                                    unsigned steps, hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!hidden || !aligned(hidden) || !targets) return LCE_ERR_INVALID_VALUE;
  if ((s = check_strip(pl, weight_strip, v_begin, v_len, pl.fwd_chunk)) != LCE_OK) return s;
  if (steps & ~(unsigned)(LCE_STEP_STRIP | LCE_STEP_MERGE)) return LCE_ERR_INVALID_VALUE;
  return pl.dtype == LCE_BF16
             ? fold_fwd<__bf16>(pl, hidden, weight_strip, v_begin, v_len, targets, ws, steps,
                                stream)
             : fold_fwd<float>(pl, hidden, weight_strip, v_begin, v_len, targets, ws, steps,
                               stream);
}

lce_status_t lce_forward_end(const lce_problem_t* p, const int32_t* targets, float* loss,
                             float* lse, float* row_loss, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!targets || !loss || !lse) return LCE_ERR_INVALID_VALUE;
  Carve c = carve(pl, ws);
  return launched(lce::launch_finalize(c.m, c.s, c.zt, targets, pl.N, pl.ignore_index,
                                       pl.reduction, lse, row_loss, loss, stream));
}

lce_status_t lce_forward(const lce_problem_t* p, const void* hidden, const void* weight,
                         const int32_t* targets, float* loss, float* lse, float* row_loss,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!hidden || !weight || !targets || !loss || !lse) return LCE_ERR_INVALID_VALUE;
  if (!aligned(hidden) || !aligned(weight)) return LCE_ERR_INVALID_VALUE;
  if ((s = lce_forward_begin(p, ws, ws_bytes, stream)) != LCE_OK) return s;
  // Folds as wide as the workspace's partials allow (several strips each):
  // fewer, fuller launches; the same kernels as lce_forward_fold.
  const char* w = static_cast<const char*>(weight);
  const unsigned all = LCE_STEP_STRIP | LCE_STEP_MERGE;
  for (int64_t v0 = 0; v0 < pl.V; v0 += pl.fwd_chunk) {
    const int64_t len = pl.V - v0 < pl.fwd_chunk ? pl.V - v0 : pl.fwd_chunk;
    const void* w_rows = w + (size_t)v0 * pl.H * pl.elt;
    s = pl.dtype == LCE_BF16
            ? fold_fwd<__bf16>(pl, hidden, w_rows, v0, len, targets, ws, all, stream)
            : fold_fwd<float>(pl, hidden, w_rows, v0, len, targets, ws, all, stream);
    if (s != LCE_OK) return s;
  }
  return lce_forward_end(p, targets, loss, lse, row_loss, ws, ws_bytes, stream);
}

lce_status_t lce_forward_state(const lce_problem_t* p, float* state, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!state) return LCE_ERR_INVALID_VALUE;
  Carve c = carve(pl, ws);
  return launched(lce::launch_state_export(c.m, c.s, c.zt, state, pl.N, stream));
}

lce_status_t lce_forward_merge_state(const lce_problem_t* p, const float* state, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!state) return LCE_ERR_INVALID_VALUE;
  Carve c = carve(pl, ws);
  return launched(lce::launch_state_merge(state, c.m, c.s, c.zt, pl.N, stream));
}

lce_status_t lce_backward_begin(const lce_problem_t* p, const int32_t* targets,
                                const float* grad_out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!targets || !grad_out) return LCE_ERR_INVALID_VALUE;
  Carve c = carve(pl, ws);
  return launched(lce::launch_grad_scale(targets, pl.N, pl.ignore_index, pl.reduction, grad_out,
                                         c.ctrl, stream));
}

lce_status_t lce_backward_fold(const lce_problem_t* p, const void* hidden,
                               const void* weight_strip, int64_t v_begin, int64_t v_len,
                               const int32_t* targets, const float* lse, float* d_hidden,
                               int accumulate, float* d_weight_strip, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  return lce_backward_fold_steps(p, hidden, weight_strip, v_begin, v_len, targets, lse, d_hidden,
                                 accumulate, d_weight_strip, ws, ws_bytes, LCE_STEP_ALL, stream);
}

lce_status_t lce_backward_fold_steps(const lce_problem_t* p, const void* hidden,
                                     const void* weight_strip, int64_t v_begin, int64_t v_len,
                                     const int32_t* targets, const float* lse, float* d_hidden,
                                     int accumulate, float* d_weight_strip, void* ws,
                                     size_t ws_bytes, unsigned steps, hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!hidden || !aligned(hidden) || !targets || !lse || !d_hidden || !d_weight_strip)
    return LCE_ERR_INVALID_VALUE;
  if (!aligned(d_hidden) || !aligned(d_weight_strip)) return LCE_ERR_INVALID_VALUE;
  if ((s = check_strip(pl, weight_strip, v_begin, v_len, pl.Vs)) != LCE_OK) return s;
  if (steps & ~(unsigned)LCE_STEP_ALL) return LCE_ERR_INVALID_VALUE;
  if (accumulate & ~(LCE_ACC_DHIDDEN | LCE_ACC_DWEIGHT)) return LCE_ERR_INVALID_VALUE;
  return pl.dtype == LCE_BF16
             ? fold_bwd<__bf16>(pl, hidden, weight_strip, v_begin, v_len, targets, lse, d_hidden,
                                accumulate, d_weight_strip, ws, steps, stream)
             : fold_bwd<float>(pl, hidden, weight_strip, v_begin, v_len, targets, lse, d_hidden,
                               accumulate, d_weight_strip, ws, steps, stream);
}

lce_status_t lce_backward(const lce_problem_t* p, const void* hidden, const void* weight,
                          const int32_t* targets, const float* lse, const float* grad_out,
                          float* d_hidden, float* d_weight, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  if ((s = check_ws(pl, ws, ws_bytes)) != LCE_OK) return s;
  if (!hidden || !weight || !targets || !lse || !grad_out || !d_hidden || !d_weight)
    return LCE_ERR_INVALID_VALUE;
  if (!aligned(hidden) || !aligned(weight) || !aligned(d_hidden) || !aligned(d_weight))
    return LCE_ERR_INVALID_VALUE;
  if ((s = lce_backward_begin(p, targets, grad_out, ws, ws_bytes, stream)) != LCE_OK) return s;
  const char* w = static_cast<const char*>(weight);
  for (int64_t v0 = 0; v0 < pl.V; v0 += pl.Vs) {
    const int64_t len = pl.V - v0 < pl.Vs ? pl.V - v0 : pl.Vs;
    s = lce_backward_fold(p, hidden, w + (size_t)v0 * pl.H * pl.elt, v0, len, targets, lse,
                          d_hidden, v0 != 0 ? LCE_ACC_DHIDDEN : LCE_ACC_NONE,
                          d_weight + (size_t)v0 * pl.H, ws, ws_bytes, stream);
    if (s != LCE_OK) return s;
  }
  return LCE_OK;
}

size_t lce_backward_fused_workspace_bytes(const lce_problem_t* p, int mode) {
  Plan pl;
  FusedPlan fp;
  if (make_plan(p, &pl) != LCE_OK || make_fused_plan(pl, mode, &fp) != LCE_OK) return 0;
  return fp.total;
}

lce_status_t lce_backward_fused(const lce_problem_t* p, const void* hidden, const void* weight,
                                const int32_t* targets, const float* lse, const float* grad_out,
                                float* d_hidden, float* d_weight, int mode, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  Plan pl;
  lce_status_t s = make_plan(p, &pl);
  if (s != LCE_OK) return s;
  FusedPlan fp;
  if ((s = make_fused_plan(pl, mode, &fp)) != LCE_OK) return s;
  if (!ws || !aligned(ws) || ws_bytes < fp.total) return LCE_ERR_WORKSPACE;
  if (!hidden || !weight || !targets || !lse || !grad_out || !d_hidden || !d_weight)
    return LCE_ERR_INVALID_VALUE;
  if (!aligned(hidden) || !aligned(weight) || !aligned(d_hidden) || !aligned(d_weight))
    return LCE_ERR_INVALID_VALUE;
  if (pl.H % 4 != 0) return LCE_ERR_UNSUPPORTED;  // the partial sums move 4 floats at a time
  Carve c = carve(pl, ws);
  if ((s = launched(lce::launch_grad_scale(targets, pl.N, pl.ignore_index, pl.reduction, grad_out,
                                           c.ctrl, stream))) != LCE_OK)
    return s;
  return pl.dtype == LCE_BF16
             ? fused_backward<__bf16>(pl, fp, hidden, weight, targets, lse, d_hidden, d_weight, ws,
                                      stream)
             : fused_backward<float>(pl, fp, hidden, weight, targets, lse, d_hidden, d_weight, ws,
                                     stream);
}

}  // extern "C"
