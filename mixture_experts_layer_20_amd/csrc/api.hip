// Host side of the C ABI: validation, capacity arithmetic, workspace layout
// and the launch sequence of the layer on the caller's stream.  Nothing here
// allocates device memory, synchronises or copies to the host.
//
// Sources: "Lab 18 -- Mixture of experts" s.3 (C = ceil(cf*T*k/E)) and "What
// to implement" (route, load_balancing_loss, router_z_loss, capacity_mask,
// MoE.forward); "Lab 01" "The traps" (capacity_factor < 1 must raise).
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "common.hpp"

namespace moe {
namespace {

thread_local std::string g_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

int64_t capacity_of(const moe_config& c) {
  // dropless: no expert receives more than T choices (a token picks an expert
  // at most once), so C = T never binds
  if (c.dropless) return c.T;
  if (c.capacity_override > 0) return c.capacity_override;
  // evaluated in IEEE double in this order, then rounded up; a value that is
  // not a finite non-negative number below 2^62 (an infinite or huge
  // capacity_factor) gives -1, which validation rejects before any use
  const double v = ceil(c.capacity_factor * static_cast<double>(c.T) * static_cast<double>(c.k) /
                        static_cast<double>(c.E));
  if (!(v >= 0.0 && v < 4.611686018427387904e18)) return -1;
  return static_cast<int64_t>(v);
}

size_t dsize(const moe_config& c) { return c.dtype == MOE_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status check_ptr(const void* p, const char* name, size_t align, bool required = true) {
  if (p == nullptr) {
    if (required) return fail(MOE_EINVAL, "%s must not be NULL", name);
    return MOE_OK;
  }
  if (!aligned(p, align)) return fail(MOE_EINVAL, "%s must be %zu-byte aligned", name, align);
  return MOE_OK;
}

#define MOE_TRY(expr)                  \
  do {                                 \
    moe_status _s = (expr);            \
    if (_s != MOE_OK) return _s;       \
  } while (0)

moe_status validate(const moe_config* cfg, int64_t* cap) {
  if (!cfg) return fail(MOE_EINVAL, "config is NULL");
  const moe_config& c = *cfg;
  if (c.T < 0) return fail(MOE_EINVAL, "T must be >= 0 (got %lld)", static_cast<long long>(c.T));
  if (c.d < 8 || c.d % 8) return fail(MOE_EINVAL, "d must be a positive multiple of 8 (got %d)", c.d);
  if (c.E < 1 || c.E > 256) return fail(MOE_EINVAL, "E must be in [1, 256] (got %d)", c.E);
  if (c.k < 1 || c.k > c.E || c.k > 32)
    return fail(MOE_EINVAL, "k must be in [1, min(E, 32)] (got k=%d, E=%d)", c.k, c.E);
  if (c.d_ff < 8 || c.d_ff % 8) return fail(MOE_EINVAL, "d_ff must be a positive multiple of 8 (got %d)", c.d_ff);
  if (c.n_shared < 0) return fail(MOE_EINVAL, "n_shared must be >= 0");
  if (c.n_shared > 0 && (c.d_ff_shared < 8 || c.d_ff_shared % 8))
    return fail(MOE_EINVAL, "d_ff_shared must be a positive multiple of 8 (got %d)", c.d_ff_shared);
  if (c.T * static_cast<int64_t>(c.k) >= (int64_t{1} << 31))
    return fail(MOE_EINVAL, "T*k must be < 2^31");
  if (c.dropless != 0 && c.dropless != 1) return fail(MOE_EINVAL, "dropless must be 0 or 1");
  if (c.routing != MOE_TOKEN_CHOICE && c.routing != MOE_EXPERT_CHOICE)
    return fail(MOE_EINVAL, "unknown routing %d", c.routing);
  if (c.routing == MOE_EXPERT_CHOICE && c.dropless)
    return fail(MOE_EINVAL, "expert-choice routing has no dropless mode (no choice is ever dropped)");
  if (c.save_preact != 0 && c.save_preact != 1) return fail(MOE_EINVAL, "save_preact must be 0 or 1");
  if (c.save_preact && c.dtype != MOE_BF16)
    return fail(MOE_EINVAL, "save_preact is built for bf16 storage (the backward pass's mode)");
  if (c.capacity_override < 0) return fail(MOE_EINVAL, "capacity_override must be >= 0");
  if (!c.dropless && c.capacity_override == 0 && !(c.capacity_factor >= 1.0))
    return fail(MOE_EINVAL,
                "capacity_factor must be >= 1.0 (got %g): below 1 it drops tokens even under "
                "perfect balance",
                c.capacity_factor);
  if (c.renormalize < -1 || c.renormalize > 1) return fail(MOE_EINVAL, "renormalize must be -1, 0 or 1");
  if (c.score != MOE_SOFTMAX && c.score != MOE_SIGMOID) return fail(MOE_EINVAL, "unknown score %d", c.score);
  if (c.act != MOE_GELU && c.act != MOE_SWIGLU) return fail(MOE_EINVAL, "unknown act %d", c.act);
  if (c.dtype != MOE_F32 && c.dtype != MOE_BF16) return fail(MOE_EINVAL, "unknown dtype %d", c.dtype);
  if (c.priority != MOE_RANK_MAJOR && c.priority != MOE_TOKEN_MAJOR && c.priority != MOE_SCORE_PRIORITY)
    return fail(MOE_EINVAL, "unknown priority %d", c.priority);
  if (c.dropped_output != 0 && c.dropped_output != 1) return fail(MOE_EINVAL, "dropped_output must be 0 or 1");
  const int64_t C = capacity_of(c);
  // capacity buffers hold E*C rows (dropless: T*k, bounded above)
  if (!c.dropless && C < 0)
    return fail(MOE_EINVAL, "capacity_factor %g gives no finite capacity for T=%lld, k=%d, E=%d",
                c.capacity_factor, static_cast<long long>(c.T), c.k, c.E);
  if (!c.dropless && C > (int64_t{1} << 31) / c.E)
    return fail(MOE_EINVAL, "capacity %lld too large", static_cast<long long>(C));
  if (cap) *cap = C;
  return MOE_OK;
}

int resolved_renorm(const moe_config& c) { return c.renormalize < 0 ? (c.k > 1) : c.renormalize; }

// Parts of the k range for the expert down projection when its tiles would
// not fill the GPU (few experts' rows, a narrow model): enough parts to reach
// about 256 workgroups, each part at least 512 wide and a multiple of 64.
// The weights are then streamed by every CU instead of a few.
struct KSplit {
  int parts;
  int64_t slice;
};
KSplit down_ksplit(int64_t groups, int64_t rpg, int64_t N, int64_t K) {
  const int64_t tiles = groups * ((rpg + 255) / 256) * ((N + 255) / 256);
  KSplit k{1, K};
  if (tiles >= 192 || tiles == 0) return k;
  const int64_t want = std::min<int64_t>({8, (256 + tiles - 1) / tiles, K / 512});
  if (want <= 1) return k;
  k.slice = ((K + want - 1) / want + 63) / 64 * 64;
  k.parts = static_cast<int>((K + k.slice - 1) / k.slice);
  return k;
}

// Batch-prioritised capacity in effect (in dropless mode nothing is dropped
// and the kept choices are numbered in rank-major order, as without it).
bool by_score(const moe_config& c) {
  return c.priority == MOE_SCORE_PRIORITY && !c.dropless && c.routing == MOE_TOKEN_CHOICE;
}

// ------------------------------------------------------------------ workspace
struct Workspace {
  int32_t* hist;
  int32_t* kept;
  int32_t* counts_tmp;
  double* p_partial;
  double* lse2_partial;
  int32_t* fallback_partial;
  double* psum;
  double* seq_partial;
  bf16_t* wplanes;
  float* zraw;
  int32_t* idx_tmp;
  float* gates_tmp;
  int32_t* row_token;
  uint32_t* ec_keys;
  int32_t* ec_selT;
  float* ec_probs;
  int32_t* ec_fallback;
  int32_t* score_queue;
  void* pre0;
  void* pre1;
  void* pres;
  float* kpart;
  float* tailpart;
  void* h;
  void* ye;
  void* hs;
  void* s;
  size_t bytes;
};

size_t align_up(size_t v) { return (v + 255) & ~size_t{255}; }

Workspace carve(const moe_config& c, int64_t C, void* base) {
  const int64_t n_tiles = (c.T + kTileTokens - 1) / kTileTokens;
  const int64_t n_rtiles = (c.T + kMinRouteTile - 1) / kMinRouteTile;
  const size_t ds = dsize(c);
  const int64_t fs = static_cast<int64_t>(c.n_shared) * c.d_ff_shared;
  Workspace w{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t n) -> void* {
    void* p = b ? b + off : nullptr;
    off += align_up(n);
    return p;
  };
  w.hist = static_cast<int32_t*>(take(sizeof(int32_t) * c.k * n_tiles * c.E));
  w.kept = static_cast<int32_t*>(take(sizeof(int32_t) * c.E));
  w.counts_tmp = static_cast<int32_t*>(take(sizeof(int32_t) * c.E));
  w.p_partial = static_cast<double*>(take(sizeof(double) * n_rtiles * c.E));
  w.lse2_partial = static_cast<double*>(take(sizeof(double) * n_rtiles));
  w.fallback_partial = static_cast<int32_t*>(take(sizeof(int32_t) * n_tiles));
  w.psum = static_cast<double*>(take(sizeof(double) * (c.E + 1)));
  w.seq_partial = static_cast<double*>(take(sizeof(double) * std::max<int64_t>(c.T, 1)));
  w.wplanes = static_cast<bf16_t*>(take(sizeof(bf16_t) * 4 * c.E * c.d));
  w.zraw = static_cast<float*>(take(sizeof(float) * router_splits(c.T, c.E, c.d) * c.T * c.E));
  w.idx_tmp = static_cast<int32_t*>(take(sizeof(int32_t) * c.T * c.k));
  w.gates_tmp = static_cast<float*>(take(sizeof(float) * c.T * c.k));
  // expert rows: E*C (capacity), or T*k packed (dropless)
  const int64_t xrows = c.dropless ? c.T * c.k : c.E * C;
  w.row_token = static_cast<int32_t*>(take(sizeof(int32_t) * xrows));
  if (c.routing == MOE_EXPERT_CHOICE || by_score(c)) {
    w.ec_keys = static_cast<uint32_t*>(take(sizeof(uint32_t) * c.T * c.E));
    w.ec_selT = static_cast<int32_t*>(take(sizeof(int32_t) * c.T * c.E));
  }
  if (c.routing == MOE_EXPERT_CHOICE) {
    w.ec_probs = static_cast<float*>(take(sizeof(float) * c.T * c.E));
    w.ec_fallback = static_cast<int32_t*>(take(sizeof(int32_t)));
  }
  if (by_score(c)) w.score_queue = static_cast<int32_t*>(take(sizeof(int32_t) * c.T * c.k));

  if (c.save_preact) {
    w.pre0 = take(ds * xrows * c.d_ff);
    if (c.act == MOE_SWIGLU) w.pre1 = take(ds * xrows * c.d_ff);
    if (fs > 0) w.pres = take(ds * c.T * fs);
  }
  if (!c.dropless && c.dtype == MOE_BF16) {
    const KSplit ksp = down_ksplit(c.E, C, c.d, c.d_ff);
    if (ksp.parts > 1) w.kpart = static_cast<float*>(take(sizeof(float) * ksp.parts * c.E * C * c.d));
  }
  if (c.dtype == MOE_BF16) w.tailpart = static_cast<float*>(take(kTailPartBytes));
  w.h = take(ds * xrows * c.d_ff);
  w.ye = take(ds * xrows * c.d);
  w.hs = fs > 0 ? take(ds * c.T * fs) : nullptr;
  w.s = fs > 0 ? take(ds * c.T * c.d) : nullptr;
  w.bytes = off;
  return w;
}

RouteArgs route_args(const moe_config& c, Workspace* w) {
  RouteArgs r{};
  r.T = c.T;
  r.d = c.d;
  r.E = c.E;
  r.k = c.k;
  r.score = c.score;
  r.renorm = resolved_renorm(c);
  r.zsplits = 1;
  if (w) {
    r.p_partial = w->p_partial;
    r.lse2_partial = w->lse2_partial;
    r.wplanes = w->wplanes;
    r.zraw = w->zraw;
  }
  return r;
}

// router partial sums come in one row per router workgroup
int router_tiles(const moe_config& c) { return static_cast<int>((c.T + kRouteTokens - 1) / kRouteTokens); }

CapArgs cap_args(const moe_config& c, int64_t C, const Workspace& w) {
  CapArgs a{};
  a.hist = w.hist;
  a.kept = w.kept;
  a.fallback_partial = w.fallback_partial;
  a.T = c.T;
  a.C = C;
  a.E = c.E;
  a.k = c.k;
  a.d = c.d;
  a.n_tiles = static_cast<int>((c.T + kTileTokens - 1) / kTileTokens);
  a.n_rtiles = static_cast<int>((c.T + kRouteTokens - 1) / kRouteTokens);
  a.token_major = c.priority == MOE_TOKEN_MAJOR;
  a.packed = c.dropless;
  return a;
}

LossArgs loss_args(const moe_config& c, int64_t C, const Workspace& w, const int32_t* counts) {
  LossArgs l{};
  l.psum = w.psum;
  l.counts = counts;
  l.fallback_partial = w.fallback_partial;
  l.T = c.T;
  l.C = C;
  l.E = c.E;
  l.k = c.k;
  l.n_tiles = static_cast<int>((c.T + kTileTokens - 1) / kTileTokens);
  l.has_shared = c.n_shared > 0;
  l.packed = c.dropless;
  return l;
}

// The gate/up launch of the expert FFN (h = act(a w_in^T + b_in), or the
// SwiGLU pair, with the pre-activations into pre0/pre1 when given).  The
// backward pass recomputes pre-activations with exactly this launch, so that
// they equal the forward's bit for bit (same tiles, same k order, the same
// split of a last round when tail_part is given).
GemmArgs up_args(const moe_config& c, int act, int groups, int64_t rpg, const int32_t* rows, const void* a,
                 const int32_t* gather, int64_t a_rows, const void* w_in, const void* w_gate, const void* b_in, int F,
                 void* h, bool packed, void* pre0, void* pre1, float* tail_part) {
  GemmArgs g1{};
  g1.A = a;
  g1.gather = gather;
  g1.a_rows = a_rows;
  g1.B0 = w_in;
  g1.B1 = w_gate;
  g1.bias = act == MOE_SWIGLU ? nullptr : b_in;
  g1.C = h;
  g1.rows = rows;
  g1.rows_per_group = rpg;
  g1.packed = packed;
  g1.total_rows = packed ? rpg : 0;
  g1.groups = groups;
  g1.N = F;
  g1.K = c.d;
  g1.act = act == MOE_SWIGLU ? 2 : 1;
  g1.pre0 = pre0;
  g1.pre1 = pre1;
  // a last, mostly empty round of tiles split along k (the launch decides on
  // the device, from the row counts)
  if (tail_part && rows && c.dtype == MOE_BF16) {
    g1.tail_part = tail_part;
    g1.tail_parts = 8;
  }
  return g1;
}

// Expert FFN on `groups` groups of rows: h = act(a w_in^T (+ b_in)) (or the
// SwiGLU pair), out = h w_out^T (+ b_out).  With `gather`, row m of group g
// is row gather[base_g + m] of a ([a_rows, d]), base_g = g*rpg, or with
// `packed` rows[0] + ... + rows[g-1] (then rpg is the bound on their sum).
moe_status ffn(const moe_config& c, int act, int groups, int64_t rpg, const int32_t* rows, const void* a,
               const int32_t* gather, int64_t a_rows, const void* w_in, const void* w_gate,
               const void* b_in, const void* w_out, const void* b_out, int F, void* h, void* out,
               hipStream_t s, bool packed = false, int64_t group_rows = 0, void* pre0 = nullptr,
               void* pre1 = nullptr, float* kpart = nullptr, float* tail_part = nullptr) {
  // each operand a GEMM launch addresses through one buffer descriptor (one
  // group's rows) stays below 2^30 elements (2^31 bytes); packed groups hold
  // at most group_rows rows
  const int64_t lim = int64_t{1} << 30;
  const int64_t gr = packed && group_rows > 0 ? std::min(group_rows, rpg) : rpg;
  if (gr * c.d >= lim || gr * F >= lim || static_cast<int64_t>(F) * c.d >= lim ||
      (gather && a_rows * c.d >= lim))
    return fail(MOE_EINVAL, "one expert's operands must hold < 2^30 elements");
  if (packed && groups > 256) return fail(MOE_EINVAL, "packed rows take at most 256 groups");
  const GemmArgs g1 = up_args(c, act, groups, rpg, rows, a, gather, a_rows, w_in, w_gate, b_in, F, h, packed, pre0,
                              pre1, tail_part);
  MOE_TRY(hip_status(launch_gemm(g1, c.dtype, s), "expert GEMM 1"));
  GemmArgs g2{};
  g2.A = h;
  g2.B0 = w_out;
  g2.bias = b_out;
  g2.C = out;
  g2.rows = rows;
  g2.rows_per_group = rpg;
  g2.packed = packed;
  g2.total_rows = packed ? rpg : 0;
  g2.groups = groups;
  g2.N = c.d;
  g2.K = F;
  g2.act = 0;
  if (kpart && !packed && c.dtype == MOE_BF16) {
    const KSplit ksp = down_ksplit(groups, rpg, c.d, F);
    if (ksp.parts > 1) {
      g2.ksplit = ksp.parts;
      g2.kslice = ksp.slice;
      g2.kpart = kpart;
      g2.kpart_stride = static_cast<int64_t>(groups) * rpg * c.d;
    }
  }
  // a last, mostly empty round of tiles split along k (the launch decides on
  // the device, from the row counts)
  if (tail_part && rows && g2.ksplit <= 1 && c.dtype == MOE_BF16) {
    g2.tail_part = tail_part;
    g2.tail_parts = 8;
  }
  return hip_status(launch_gemm(g2, c.dtype, s), "expert GEMM 2");
}

// Capacity and dispatch.  Score priority: the histogram/scan/permute pass
// first gives every assignment its rank-major queue position with room for
// all (into the workspace), then the kept set is chosen by score and numbered
// (launch_score_priority); the row copy into xe, if asked for, follows.
moe_status capacity_step(const moe_config& c, int64_t C, const Workspace& w, const CapArgs& a, const float* gates,
                         hipStream_t s) {
  if (!by_score(c)) return hip_status(launch_capacity(a, c.dtype, s), "capacity");
  CapArgs q = a;
  q.C = std::max<int64_t>(c.T, 1);
  q.slot = w.score_queue;
  q.row_token = nullptr;
  q.kept = nullptr;
  q.fallback_partial = nullptr;
  q.x = nullptr;
  q.xe = nullptr;
  q.token_major = 0;
  q.packed = 0;
  MOE_TRY(hip_status(launch_capacity(q, c.dtype, s), "capacity queue"));
  ScoreArgs sa{};
  sa.idx = a.idx;
  sa.gates = gates;
  sa.queue = w.score_queue;
  sa.counts = a.counts;
  sa.keys = w.ec_keys;
  sa.selT = w.ec_selT;
  sa.slot = a.slot;
  sa.dropped = a.dropped;
  sa.row_token = a.row_token;
  sa.kept = w.kept;
  sa.fallback_partial = a.fallback_partial;
  sa.T = c.T;
  sa.C = C;
  sa.E = c.E;
  sa.k = c.k;
  sa.n_tiles = a.n_tiles;
  MOE_TRY(hip_status(launch_score_priority(sa, s), "score-priority capacity"));
  if (a.xe && a.row_token && c.T > 0)
    MOE_TRY(hip_status(launch_gather_rows(a.x, a.xe, a.row_token, w.kept, C, c.E, static_cast<int>(c.d * dsize(c)), s),
                       "dispatch copy"));
  return MOE_OK;
}

// Expert choice after the router: each expert's picks, the routed FFNs on
// the picked rows (gathered straight from x), the shared experts, the
// probability-weighted combine and the losses.
// Phase boundaries of one forward pass, for moe_forward_events: 0 start,
// 1 routed, 2 capacity (or expert-choice selection) done, 3 routed expert
// FFN done (both grouped GEMM launches), 4 shared experts done, 5 combined,
// 6 losses done.
constexpr int kForwardEvents = 7;
struct PhaseMarks {
  void* const* ev;
  hipStream_t s;
  moe_status mark(int i) const {
    if (!ev || !ev[i]) return MOE_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(ev[i]), s), "hipEventRecord");
  }
};

moe_status forward_expert_choice(const moe_config& c, int64_t C, const moe_weights& wt, const void* x,
                                 const float* probs, const moe_outputs& out, const Workspace& w, hipStream_t s,
                                 const PhaseMarks& pm) {
  EcArgs e{};
  e.probs = probs;
  e.keys = w.ec_keys;
  e.selT = w.ec_selT;
  e.row_token = w.row_token;
  e.sel = out.sel;
  e.counts = out.counts;
  e.p_partial = w.p_partial;
  e.lse2_partial = w.lse2_partial;
  e.psum = w.psum;
  e.fallback_count = w.ec_fallback;
  e.T = c.T;
  e.C = C;
  e.E = c.E;
  e.n_rtiles = router_tiles(c);
  MOE_TRY(hip_status(launch_expert_choice(e, s), "expert choice"));   // T = 0: zero counts and sums
  MOE_TRY(pm.mark(2));
  if (c.T > 0) {
    MOE_TRY(ffn(c, c.act, c.E, C, out.counts, x, w.row_token, c.T, wt.w_in, wt.w_gate, wt.b_in, wt.w_out,
                wt.b_out, c.d_ff, w.h, w.ye, s, false, 0, w.pre0, w.pre1, w.kpart, w.tailpart));
    MOE_TRY(pm.mark(3));
    if (c.n_shared > 0)
      MOE_TRY(ffn(c, MOE_GELU, 1, c.T, nullptr, x, nullptr, 0, wt.ws_in, nullptr, wt.bs_in, wt.ws_out,
                  wt.bs_out, c.n_shared * c.d_ff_shared, w.hs, w.s, s, false, 0, w.pres));
    MOE_TRY(pm.mark(4));
    CombineArgs cb{};
    cb.x = x;
    cb.ye = w.ye;
    cb.shared_out = c.n_shared > 0 ? w.s : nullptr;
    cb.sel = out.sel;
    cb.probs = probs;
    cb.fallback_count = w.ec_fallback;
    cb.y = out.y;
    cb.T = c.T;
    cb.C = C;
    cb.d = c.d;
    cb.k = c.k;
    cb.E = c.E;
    cb.zero_fallback = c.dropped_output;
    MOE_TRY(hip_status(launch_combine(cb, c.dtype, s), "expert-choice combine"));
  } else {
    MOE_TRY(pm.mark(3));
    MOE_TRY(pm.mark(4));
  }
  MOE_TRY(pm.mark(5));
  LossArgs l = loss_args(c, C, w, out.counts);
  l.fallback_partial = nullptr;
  l.ec = 1;
  l.fallback_count = w.ec_fallback;
  l.losses = out.losses;
  l.stats = out.stats;
  MOE_TRY(hip_status(launch_losses(l, s), "loss finaliser"));
  return pm.mark(6);
}

// ------------------------------------------------------------------ backward
int64_t round8(int64_t v) { return (v + 7) / 8 * 8; }

struct BwdWorkspace {
  float* dgates;
  float* dz;
  bf16_t* dYe;
  bf16_t* U;
  bf16_t* U2;
  bf16_t* dH;
  bf16_t* dact;
  bf16_t* dA;
  bf16_t* wiT;
  bf16_t* AT;
  bf16_t* xT;
  bf16_t* planes;
  float* slabs;
  float* wrT;
  bf16_t* Us;
  bf16_t* dHs;
  bf16_t* dUs;
  bf16_t* dAs;
  int32_t* pstart;
  int32_t* kstart;
  float* tailpart;
  int64_t Kw;                 // columns of the transposed expert operands (packed along k)
  int S;
  size_t bytes;
};

// Upper bound of the expert rows the backward pass contracts over: kept
// (capacity), routed (dropless) or picked (expert choice) choices.
int64_t expert_rows_bound(const moe_config& c, int64_t C) {
  const int64_t Tk = c.T * c.k;
  if (c.routing == MOE_EXPERT_CHOICE) return static_cast<int64_t>(c.E) * std::min<int64_t>(C, c.T);
  if (c.dropless) return Tk;
  return std::min<int64_t>(Tk, static_cast<int64_t>(c.E) * C);
}

BwdWorkspace carve_bwd(const moe_config& c, int64_t C, void* base) {
  const int64_t T = c.T, d = c.d, E = c.E, F = c.d_ff, Tp = round8(T);
  const int64_t ga = c.act == MOE_SWIGLU ? 2 : 1;
  const int64_t Fs = static_cast<int64_t>(c.n_shared) * c.d_ff_shared;
  BwdWorkspace b{};
  size_t off = 0;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t n) -> void* {
    void* q = p ? p + off : nullptr;
    off += align_up(n);
    return q;
  };
  const size_t h2 = sizeof(bf16_t);
  b.S = router_splits(d, c.E, Tp);
  // expert choice: the gate gradients are those of the probabilities, [T,E]
  const int64_t ng = c.routing == MOE_EXPERT_CHOICE ? E : c.k;
  b.dgates = static_cast<float*>(take(sizeof(float) * T * ng));
  b.dz = static_cast<float*>(take(sizeof(float) * T * E));
  const int64_t R = c.dropless ? T * c.k : E * C;   // rows of the expert buffers (packed when dropless)
  b.dYe = static_cast<bf16_t*>(take(h2 * R * d));
  if (!c.save_preact) {
    b.U = static_cast<bf16_t*>(take(h2 * R * F));
    b.U2 = ga == 2 ? static_cast<bf16_t*>(take(h2 * R * F)) : nullptr;
  }
  b.dH = static_cast<bf16_t*>(take(h2 * R * F));
  b.dact = static_cast<bf16_t*>(take(h2 * R * ga * F));
  b.dA = static_cast<bf16_t*>(take(h2 * R * d));
  b.tailpart = static_cast<float*>(take(kTailPartBytes));
  if (c.dropless) b.pstart = static_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
  b.kstart = static_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));
  // the transposed expert operands of the weight gradients, packed along k:
  // expert e's max(8, round8(rows_e)) columns start at kstart[e]
  b.Kw = round8(expert_rows_bound(c, C)) + 8 * E;
  // (SwiGLU with F not a multiple of 64: the input-gradient weights transposed)
  if (ga == 2 && F % 64 != 0) b.wiT = static_cast<bf16_t*>(take(h2 * E * d * ga * F));
  b.AT = static_cast<bf16_t*>(take(h2 * d * b.Kw));
  b.xT = static_cast<bf16_t*>(take(h2 * d * Tp));
  b.planes = static_cast<bf16_t*>(take(h2 * 4 * E * Tp));
  b.slabs = static_cast<float*>(take(sizeof(float) * b.S * d * E));
  b.wrT = static_cast<float*>(take(sizeof(float) * E * d));
  if (Fs > 0) {
    if (!c.save_preact) b.Us = static_cast<bf16_t*>(take(h2 * T * Fs));
    b.dHs = static_cast<bf16_t*>(take(h2 * T * Fs));
    b.dUs = static_cast<bf16_t*>(take(h2 * T * Fs));
    b.dAs = static_cast<bf16_t*>(take(h2 * T * d));
  }
  b.bytes = off;
  return b;
}

moe_status check_backward_config(const moe_config& c, int64_t C) {
  if (c.dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "the backward pass is built for bf16 storage");
  const int64_t lim = int64_t{1} << 30;
  const int64_t ga = c.act == MOE_SWIGLU ? 2 : 1;
  const int64_t Fs = static_cast<int64_t>(c.n_shared) * c.d_ff_shared;
  // (one expert's transposed block: [cols, round8(C)] at most; dropless C = T)
  const int64_t Cp = round8(C), Tp = round8(c.T);
  const int64_t big = std::max({C * c.d, C * ga * c.d_ff, static_cast<int64_t>(c.d) * Cp, ga * c.d_ff * Cp,
                                static_cast<int64_t>(c.d) * Tp, Fs * Tp, c.T * std::max<int64_t>(Fs, c.d),
                                static_cast<int64_t>(c.d_ff) * c.d * ga});
  if (big >= lim) return fail(MOE_EINVAL, "one backward GEMM operand would hold 2^30 elements or more");
  return MOE_OK;
}

// C[g] = A[g] B[g]^T (+ bias) on the bf16 grouped GEMM, operands K-contiguous.
moe_status bgemm(const char* what, const void* A, int64_t lda, int64_t a_gs, const int32_t* gather, int64_t a_rows,
                 const void* B, int64_t ldb, int64_t b_gs, const void* bias, void* Cout, const int32_t* rows,
                 int64_t rpg, int groups, int N, int K, hipStream_t s, const int32_t* kvar = nullptr,
                 bool packed = false, const int32_t* koff = nullptr) {
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.a_gs = a_gs;
  g.gather = gather;
  g.a_rows = a_rows;
  g.B0 = B;
  g.ldb = ldb;
  g.b_gs = b_gs;
  g.bias = bias;
  g.C = Cout;
  g.rows = rows;
  g.rows_per_group = rpg;
  g.groups = groups;
  g.N = N;
  g.K = K;
  g.act = 0;
  g.kvar = kvar;
  g.koff = koff;
  g.packed = packed;
  g.total_rows = packed ? rpg : 0;
  return hip_status(launch_gemm(g, MOE_BF16, s), what);
}

// C[g] = A[g] B[g]^T on the bf16 grouped GEMM with k-major operands (kmaj
// bit 0: A is [K, M] per group, row length lda; bit 1: B is [K, N], row
// length ldb, or B0 for k < b_split and B1 from there), read through the LDS
// transpose loads instead of transposed copies.  A K-contiguous operand
// takes its usual strides (0: K).  With tail_part (k-major B only, device
// row counts) a sparse last round of tiles is split along k.
moe_status kgemm(const char* what, int kmaj, const void* A, int64_t lda, int64_t a_gs, const void* B0,
                 const void* B1, int64_t b_split, int64_t ldb, int64_t b_gs, void* Cout, const int32_t* rows,
                 int64_t rpg, int groups, int N, int K, hipStream_t s, const int32_t* kvar = nullptr,
                 const int32_t* kstart = nullptr, bool packed = false, const int32_t* koff = nullptr,
                 float* tail_part = nullptr) {
  GemmArgs g{};
  g.kmaj = kmaj;
  g.A = A;
  g.lda = lda;
  g.a_gs = a_gs;
  g.B0 = B0;
  g.B1 = B1;
  g.b_split = b_split;
  g.ldb = ldb;
  g.b_gs = b_gs;
  g.C = Cout;
  g.rows = rows;
  g.rows_per_group = rpg;
  g.groups = groups;
  g.N = N;
  g.K = K;
  g.act = 0;
  g.kvar = kvar;
  g.kstart = kstart;
  g.koff = koff;
  g.packed = packed;
  g.total_rows = packed ? rpg : 0;
  if (tail_part && rows) {
    g.tail_part = tail_part;
    g.tail_parts = 8;
  }
  return hip_status(launch_gemm(g, MOE_BF16, s), what);
}

moe_status transpose(const char* what, const bf16_t* in, bf16_t* out, int G, int64_t R, int64_t Cc, int64_t Rpad,
                     int64_t in_gs, int64_t ld_in, int64_t out_gs, int64_t ld_out, const int32_t* valid,
                     const int32_t* gather, int64_t gather_gs, hipStream_t s, const int32_t* ocol = nullptr,
                     const int32_t* gstart = nullptr) {
  TransposeArgs t{};
  t.in = in;
  t.out = out;
  t.gather = gather;
  t.valid = valid;
  t.R = R;
  t.Cc = Cc;
  t.Rpad = Rpad;
  t.in_gs = in_gs;
  t.ld_in = ld_in;
  t.gather_gs = gather_gs;
  t.out_gs = out_gs;
  t.ld_out = ld_out;
  t.G = G;
  t.ocol = ocol;
  t.gstart = gstart;
  return hip_status(launch_transpose(t, s), what);
}

// ------------------------------------------------------------------ no-alloc
// Scratch of the entry point that allocates nothing (moe_dispatch_noalloc):
// the capacity histograms, kept counts and fallback partials live in this
// file-scope device array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code never
// uses the array's name as an address: its device address is looked up once
// per device (hipGetSymbolAddress with that device current) and kept here.
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_address(void** out) {
  int dev = -1;
  MOE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p) return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The dispatch scratch: histograms [k, ceil(T/64), E], kept [E] and fallback
// partials [ceil(T/64)], 256-byte aligned pieces from `base` (NULL: sizes only).
struct DispatchScratch {
  int32_t* hist;
  int32_t* kept;
  int32_t* fallback_partial;
  size_t bytes;
};
DispatchScratch carve_dispatch(const moe_config& c, void* base) {
  const int64_t n_tiles = (c.T + kTileTokens - 1) / kTileTokens;
  DispatchScratch d{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t n) -> void* {
    void* p = b ? b + off : nullptr;
    off += align_up(n);
    return p;
  };
  d.hist = static_cast<int32_t*>(take(sizeof(int32_t) * c.k * n_tiles * c.E));
  d.kept = static_cast<int32_t*>(take(sizeof(int32_t) * c.E));
  d.fallback_partial = static_cast<int32_t*>(take(sizeof(int32_t) * std::max<int64_t>(n_tiles, 1)));
  d.bytes = off;
  return d;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_error.c_str(); }

moe_status moe_validate(const moe_config* cfg, int64_t* capacity) { return validate(cfg, capacity); }

size_t moe_workspace_bytes(const moe_config* cfg) {
  int64_t C = 0;
  if (validate(cfg, &C) != MOE_OK) return 0;
  return carve(*cfg, C, nullptr).bytes;
}

moe_status moe_route(const moe_config* cfg, const void* x, const float* w_router, const float* logit_bias,
                     const float* select_bias, float* logits, float* probs, int32_t* idx, float* gates,
                     float* lse, void* ws, void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  const bool needT = c.T > 0;   // T-sized buffers may be NULL when T == 0
  MOE_TRY(check_ptr(idx, "idx", 4, needT));
  MOE_TRY(check_ptr(gates, "gates", 4, needT));
  MOE_TRY(check_ptr(logit_bias, "logit_bias", 4, false));
  MOE_TRY(check_ptr(select_bias, "select_bias", 4, false));
  MOE_TRY(check_ptr(probs, "probs", 4, false));
  MOE_TRY(check_ptr(lse, "lse", 4, false));
  MOE_TRY(check_ptr(ws, "ws", 256, false));
  if (x) {
    MOE_TRY(check_ptr(x, "x", 16));
    MOE_TRY(check_ptr(w_router, "w_router", 4));
    MOE_TRY(check_ptr(logits, "logits", 4, false));
    if (c.dtype == MOE_BF16 && !ws)
      return fail(MOE_EINVAL, "ws must not be NULL when routing bf16 x (it holds the split router weight "
                              "and the logits)");
  } else {
    MOE_TRY(check_ptr(logits, "logits (input when x is NULL)", 4, needT));
  }
  Workspace w = carve(c, C, ws);
  RouteArgs r = route_args(c, ws ? &w : nullptr);
  r.x = x;
  r.w_router = w_router;
  r.logit_bias = logit_bias;
  r.select_bias = select_bias;
  r.logits = x ? nullptr : logits;
  r.logits_out = x ? logits : nullptr;
  r.probs = probs;
  r.idx = idx;
  r.gates = gates;
  r.lse = lse;
  return hip_status(launch_route(r, c.dtype, static_cast<hipStream_t>(stream)), "router");
}

moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* idx, int32_t* slot, uint8_t* dropped,
                        int32_t* counts, int32_t* row_token, void* xe, void* ws, void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  const bool needT = c.T > 0;
  MOE_TRY(check_ptr(idx, "idx", 4, needT));
  MOE_TRY(check_ptr(slot, "slot", 4, needT));
  MOE_TRY(check_ptr(dropped, "dropped", 1, needT));
  MOE_TRY(check_ptr(counts, "counts", 4));
  MOE_TRY(check_ptr(row_token, "row_token", 4, false));
  MOE_TRY(check_ptr(ws, "ws", 256));
  if ((xe || x) && needT) {
    MOE_TRY(check_ptr(x, "x", 16));
    MOE_TRY(check_ptr(xe, "xe", 16, C > 0));
  }
  if (by_score(c)) return fail(MOE_EINVAL, "score priority needs the scores: call moe_dispatch_by_score");
  Workspace w = carve(c, C, ws);
  CapArgs a = cap_args(c, C, w);
  a.idx = idx;
  a.slot = slot;
  a.dropped = dropped;
  a.counts = counts;
  a.row_token = row_token;
  a.x = x;
  a.xe = xe;
  return hip_status(launch_capacity(a, c.dtype, static_cast<hipStream_t>(stream)), "capacity");
}

moe_status moe_dispatch_noalloc(const moe_config* cfg, const void* x, const int32_t* idx, int32_t* slot,
                                uint8_t* dropped, int32_t* counts, int32_t* row_token, void* xe, void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  const bool needT = c.T > 0;
  MOE_TRY(check_ptr(idx, "idx", 4, needT));
  MOE_TRY(check_ptr(slot, "slot", 4, needT));
  MOE_TRY(check_ptr(dropped, "dropped", 1, needT));
  MOE_TRY(check_ptr(counts, "counts", 4));
  MOE_TRY(check_ptr(row_token, "row_token", 4, false));
  if ((xe || x) && needT) {
    MOE_TRY(check_ptr(x, "x", 16));
    MOE_TRY(check_ptr(xe, "xe", 16, C > 0));
  }
  if (by_score(c)) return fail(MOE_EINVAL, "score priority needs the scores: call moe_dispatch_by_score");
  const size_t need = carve_dispatch(c, nullptr).bytes;
  if (need > kNoAllocScratchBytes)
    return fail(MOE_EINVAL,
                "moe_dispatch_noalloc: this configuration needs %zu bytes of scratch (k*ceil(T/64)*E*4 plus "
                "E*4 and ceil(T/64)*4, 256-byte aligned), more than its fixed %zu; use moe_dispatch with a workspace",
                need, kNoAllocScratchBytes);
  void* base = nullptr;
  MOE_TRY(scratch_address(&base));
  const DispatchScratch d = carve_dispatch(c, base);
  CapArgs a{};
  a.hist = d.hist;
  a.kept = d.kept;
  a.fallback_partial = d.fallback_partial;
  a.T = c.T;
  a.C = C;
  a.E = c.E;
  a.k = c.k;
  a.d = c.d;
  a.n_tiles = static_cast<int>((c.T + kTileTokens - 1) / kTileTokens);
  a.n_rtiles = static_cast<int>((c.T + kRouteTokens - 1) / kRouteTokens);
  a.token_major = c.priority == MOE_TOKEN_MAJOR;
  a.packed = c.dropless;
  a.idx = idx;
  a.slot = slot;
  a.dropped = dropped;
  a.counts = counts;
  a.row_token = row_token;
  a.x = x;
  a.xe = xe;
  return hip_status(launch_capacity(a, c.dtype, static_cast<hipStream_t>(stream)), "capacity");
}

moe_status moe_dispatch_by_score(const moe_config* cfg, const void* x, const int32_t* idx, const float* gates,
                                 int32_t* slot, uint8_t* dropped, int32_t* counts, int32_t* row_token, void* xe,
                                 void* ws, void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  if (c.priority != MOE_SCORE_PRIORITY || c.routing != MOE_TOKEN_CHOICE)
    return fail(MOE_EINVAL, "moe_dispatch_by_score needs priority = MOE_SCORE_PRIORITY under token choice");
  const bool needT = c.T > 0;
  MOE_TRY(check_ptr(idx, "idx", 4, needT));
  MOE_TRY(check_ptr(gates, "gates", 4, needT));
  MOE_TRY(check_ptr(slot, "slot", 4, needT));
  MOE_TRY(check_ptr(dropped, "dropped", 1, needT));
  MOE_TRY(check_ptr(counts, "counts", 4));
  MOE_TRY(check_ptr(row_token, "row_token", 4, false));
  MOE_TRY(check_ptr(ws, "ws", 256));
  if ((xe || x) && needT) {
    MOE_TRY(check_ptr(x, "x", 16));
    MOE_TRY(check_ptr(xe, "xe", 16, C > 0));
    if (!row_token) return fail(MOE_EINVAL, "row_token is needed to copy rows into xe under score priority");
  }
  Workspace w = carve(c, C, ws);
  CapArgs a = cap_args(c, C, w);
  a.idx = idx;
  a.slot = slot;
  a.dropped = dropped;
  a.counts = counts;
  a.row_token = row_token;
  a.x = x;
  a.xe = xe;
  return capacity_step(c, C, w, a, gates, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn(const moe_config* cfg, int32_t act, int32_t groups, int64_t rows_per_group,
                          const int32_t* rows, const void* a, const int32_t* gather, int64_t a_rows,
                          const void* w_in, const void* w_gate, const void* b_in, const void* w_out,
                          const void* b_out, int32_t F, void* h, void* out, void* stream) {
  MOE_TRY(validate(cfg, nullptr));
  const moe_config& c = *cfg;
  if (act != MOE_GELU && act != MOE_SWIGLU) return fail(MOE_EINVAL, "unknown act %d", act);
  if (groups < 0 || rows_per_group < 0) return fail(MOE_EINVAL, "groups and rows_per_group must be >= 0");
  if (F < 8 || F % 8) return fail(MOE_EINVAL, "F must be a positive multiple of 8 (got %d)", F);
  if (static_cast<int64_t>(groups) * rows_per_group >= (int64_t{1} << 31))
    return fail(MOE_EINVAL, "groups*rows_per_group must be < 2^31");
  MOE_TRY(check_ptr(a, "a", 16));
  MOE_TRY(check_ptr(w_in, "w_in", 16));
  MOE_TRY(check_ptr(w_out, "w_out", 16));
  MOE_TRY(check_ptr(h, "h", 16));
  MOE_TRY(check_ptr(out, "out", 16));
  MOE_TRY(check_ptr(rows, "rows", 4, false));
  MOE_TRY(check_ptr(gather, "gather", 4, false));
  if (gather && a_rows <= 0) return fail(MOE_EINVAL, "a_rows must be > 0 when gathering");
  MOE_TRY(check_ptr(b_in, "b_in", 16, false));
  MOE_TRY(check_ptr(b_out, "b_out", 16, false));
  if (act == MOE_SWIGLU) {
    MOE_TRY(check_ptr(w_gate, "w_gate", 16));
    if (b_in) return fail(MOE_EUNSUPPORTED, "SwiGLU experts take no b_in");
  }
  return ffn(c, act, groups, rows_per_group, rows, a, gather, a_rows, w_in, w_gate, b_in, w_out, b_out, F, h,
             out, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_packed(const moe_config* cfg, int32_t act, int32_t groups, const int32_t* rows,
                                 int64_t total_rows, const void* a, const int32_t* gather, int64_t a_rows,
                                 const void* w_in, const void* w_gate, const void* b_in, const void* w_out,
                                 const void* b_out, int32_t F, void* h, void* out, void* stream) {
  MOE_TRY(validate(cfg, nullptr));
  const moe_config& c = *cfg;
  if (act != MOE_GELU && act != MOE_SWIGLU) return fail(MOE_EINVAL, "unknown act %d", act);
  if (groups < 0 || groups > 256) return fail(MOE_EINVAL, "groups must be in [0, 256] (got %d)", groups);
  if (total_rows < 0 || total_rows >= (int64_t{1} << 31)) return fail(MOE_EINVAL, "total_rows must be in [0, 2^31)");
  if (F < 8 || F % 8) return fail(MOE_EINVAL, "F must be a positive multiple of 8 (got %d)", F);
  if (groups == 0 || total_rows == 0) return MOE_OK;
  MOE_TRY(check_ptr(rows, "rows", 4));
  MOE_TRY(check_ptr(a, "a", 16));
  MOE_TRY(check_ptr(w_in, "w_in", 16));
  MOE_TRY(check_ptr(w_out, "w_out", 16));
  MOE_TRY(check_ptr(h, "h", 16));
  MOE_TRY(check_ptr(out, "out", 16));
  MOE_TRY(check_ptr(gather, "gather", 4, false));
  if (gather && a_rows <= 0) return fail(MOE_EINVAL, "a_rows must be > 0 when gathering");
  MOE_TRY(check_ptr(b_in, "b_in", 16, false));
  MOE_TRY(check_ptr(b_out, "b_out", 16, false));
  if (act == MOE_SWIGLU) {
    MOE_TRY(check_ptr(w_gate, "w_gate", 16));
    if (b_in) return fail(MOE_EUNSUPPORTED, "SwiGLU experts take no b_in");
  }
  return ffn(c, act, groups, total_rows, rows, a, gather, a_rows, w_in, w_gate, b_in, w_out, b_out, F, h, out,
             static_cast<hipStream_t>(stream), true);
}

moe_status moe_combine(const moe_config* cfg, const void* x, const void* ye, const void* shared_out,
                       const int32_t* idx, const float* gates, const int32_t* slot, const uint8_t* dropped, void* y,
                       void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  const bool needT = c.T > 0;
  MOE_TRY(check_ptr(x, "x", 16, needT));
  MOE_TRY(check_ptr(ye, "ye", 16, needT && C > 0));
  MOE_TRY(check_ptr(shared_out, "shared_out", 16, false));
  MOE_TRY(check_ptr(idx, "idx", 4, needT));
  MOE_TRY(check_ptr(gates, "gates", 4, needT));
  MOE_TRY(check_ptr(slot, "slot", 4, needT));
  MOE_TRY(check_ptr(dropped, "dropped", 1, needT));
  MOE_TRY(check_ptr(y, "y", 16, needT));
  CombineArgs a{};
  a.x = x;
  a.ye = ye;
  a.shared_out = shared_out;
  a.idx = idx;
  a.gates = gates;
  a.slot = slot;
  a.dropped = dropped;
  a.y = y;
  a.T = c.T;
  a.C = C;
  a.d = c.d;
  a.k = c.k;
  a.E = c.E;
  a.zero_fallback = c.dropped_output;
  a.packed = c.dropless;
  return hip_status(launch_combine(a, c.dtype, static_cast<hipStream_t>(stream)), "combine");
}

moe_status moe_expert_choice(const moe_config* cfg, const float* probs, int32_t* row_token, int32_t* sel,
                             int32_t* counts, void* ws, void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  if (c.routing != MOE_EXPERT_CHOICE) return fail(MOE_EINVAL, "moe_expert_choice needs routing = MOE_EXPERT_CHOICE");
  const bool needT = c.T > 0;
  MOE_TRY(check_ptr(probs, "probs", 4, needT));
  MOE_TRY(check_ptr(row_token, "row_token", 4, needT));
  MOE_TRY(check_ptr(sel, "sel", 4, needT));
  MOE_TRY(check_ptr(counts, "counts", 4));
  MOE_TRY(check_ptr(ws, "ws", 256));
  Workspace w = carve(c, C, ws);
  EcArgs e{};
  e.probs = probs;
  e.keys = w.ec_keys;
  e.selT = w.ec_selT;
  e.row_token = row_token;
  e.sel = sel;
  e.counts = counts;
  e.T = c.T;
  e.C = C;
  e.E = c.E;
  return hip_status(launch_expert_choice(e, static_cast<hipStream_t>(stream)), "expert choice");
}

moe_status moe_combine_expert_choice(const moe_config* cfg, const void* x, const void* ye, const void* shared_out,
                                     const float* probs, const int32_t* sel, void* y, void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  if (c.routing != MOE_EXPERT_CHOICE)
    return fail(MOE_EINVAL, "moe_combine_expert_choice needs routing = MOE_EXPERT_CHOICE");
  const bool needT = c.T > 0;
  MOE_TRY(check_ptr(x, "x", 16, needT));
  MOE_TRY(check_ptr(ye, "ye", 16, needT));
  MOE_TRY(check_ptr(shared_out, "shared_out", 16, false));
  MOE_TRY(check_ptr(probs, "probs", 4, needT));
  MOE_TRY(check_ptr(sel, "sel", 4, needT));
  MOE_TRY(check_ptr(y, "y", 16, needT));
  CombineArgs a{};
  a.x = x;
  a.ye = ye;
  a.shared_out = shared_out;
  a.sel = sel;
  a.probs = probs;
  a.y = y;
  a.T = c.T;
  a.C = C;
  a.d = c.d;
  a.k = c.k;
  a.E = c.E;
  a.zero_fallback = c.dropped_output;
  return hip_status(launch_combine(a, c.dtype, static_cast<hipStream_t>(stream)), "expert-choice combine");
}

moe_status moe_aux_losses(const moe_config* cfg, const float* logits, const int32_t* idx, float* losses, void* ws,
                          void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  MOE_TRY(check_ptr(logits, "logits", 4, c.T > 0));
  MOE_TRY(check_ptr(idx, "idx", 4, c.T > 0));
  MOE_TRY(check_ptr(losses, "losses", 4));
  MOE_TRY(check_ptr(ws, "ws", 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w = carve(c, C, ws);
  // probabilities and LSE partials from the given logits (the re-derived
  // selection goes to scratch and is not used)
  RouteArgs r = route_args(c, &w);
  r.logits = const_cast<float*>(logits);
  r.idx = w.idx_tmp;
  r.gates = w.gates_tmp;
  MOE_TRY(hip_status(launch_route(r, c.dtype, s), "aux-loss statistics"));
  // f_i from the given choices: the capacity histogram + scan (no dispatch)
  CapArgs a = cap_args(c, C, w);
  a.idx = idx;
  a.counts = w.counts_tmp;
  a.slot = w.idx_tmp;                         // scratch, overwritten
  a.dropped = reinterpret_cast<uint8_t*>(w.gates_tmp);
  a.fallback_partial = nullptr;
  a.p_partial = w.p_partial;
  a.lse2_partial = w.lse2_partial;
  a.psum = w.psum;
  a.n_rtiles = router_tiles(c);
  MOE_TRY(hip_status(launch_capacity(a, c.dtype, s), "aux-loss counts"));
  LossArgs l = loss_args(c, C, w, w.counts_tmp);
  l.fallback_partial = nullptr;
  l.losses = losses;
  return hip_status(launch_losses(l, s), "aux-loss finaliser");
}

moe_status moe_sequence_aux_loss(const moe_config* cfg, int64_t seq_len, const float* probs, const int32_t* idx,
                                 float* loss, void* ws, void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  if (c.T == 0) return fail(MOE_EINVAL, "the sequence-wise loss needs T > 0");
  if (seq_len <= 0 || c.T % seq_len)
    return fail(MOE_EINVAL, "seq_len must be positive and divide T (T=%lld, seq_len=%lld)",
                static_cast<long long>(c.T), static_cast<long long>(seq_len));
  MOE_TRY(check_ptr(probs, "probs", 4));
  MOE_TRY(check_ptr(idx, "idx", 4));
  MOE_TRY(check_ptr(loss, "loss", 4));
  MOE_TRY(check_ptr(ws, "ws", 256));
  Workspace w = carve(c, C, ws);
  SeqLossArgs a{};
  a.probs = probs;
  a.idx = idx;
  a.partial = w.seq_partial;
  a.loss = loss;
  a.seq_len = seq_len;
  a.n_seq = c.T / seq_len;
  a.E = c.E;
  a.k = c.k;
  return hip_status(launch_seq_loss(a, static_cast<hipStream_t>(stream)), "sequence-wise loss");
}

moe_status moe_update_select_bias(const moe_config* cfg, const int32_t* counts, float* select_bias, float gamma,
                                  void* stream) {
  MOE_TRY(validate(cfg, nullptr));
  const moe_config& c = *cfg;
  if (!(gamma >= 0.0f) || gamma == __builtin_huge_valf())
    return fail(MOE_EINVAL, "gamma must be finite and >= 0 (got %g)", static_cast<double>(gamma));
  MOE_TRY(check_ptr(counts, "counts", 4));
  MOE_TRY(check_ptr(select_bias, "select_bias", 4));
  return hip_status(launch_bias_update(counts, select_bias, c.E, c.T * c.k, gamma, static_cast<hipStream_t>(stream)),
                    "selection-bias update");
}

static moe_status forward_impl(const moe_config* cfg, const moe_weights* wt, const void* x, moe_outputs* out, void* ws,
                               void* stream, void* const* events) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  if (!wt || !out) return fail(MOE_EINVAL, "weights and outputs must not be NULL");
  const bool needT = c.T > 0;   // T-sized buffers may be NULL when T == 0
  MOE_TRY(check_ptr(x, "x", 16, needT));
  MOE_TRY(check_ptr(ws, "ws", 256));
  MOE_TRY(check_ptr(wt->w_router, "w_router", 4));
  MOE_TRY(check_ptr(wt->logit_bias, "logit_bias", 4, false));
  MOE_TRY(check_ptr(wt->select_bias, "select_bias", 4, false));
  MOE_TRY(check_ptr(wt->w_in, "w_in", 16));
  MOE_TRY(check_ptr(wt->w_out, "w_out", 16));
  MOE_TRY(check_ptr(wt->b_in, "b_in", 16, false));
  MOE_TRY(check_ptr(wt->b_out, "b_out", 16, false));
  if (c.act == MOE_SWIGLU) {
    MOE_TRY(check_ptr(wt->w_gate, "w_gate", 16));
    if (wt->b_in) return fail(MOE_EUNSUPPORTED, "SwiGLU experts take no b_in");
  }
  if (c.n_shared > 0) {
    MOE_TRY(check_ptr(wt->ws_in, "ws_in", 16));
    MOE_TRY(check_ptr(wt->ws_out, "ws_out", 16));
    MOE_TRY(check_ptr(wt->bs_in, "bs_in", 16, false));
    MOE_TRY(check_ptr(wt->bs_out, "bs_out", 16, false));
  }
  const bool ec = c.routing == MOE_EXPERT_CHOICE;
  MOE_TRY(check_ptr(out->y, "y", 16, needT));
  MOE_TRY(check_ptr(out->idx, "idx", 4, needT && !ec));
  MOE_TRY(check_ptr(out->gates, "gates", 4, needT && !ec));
  MOE_TRY(check_ptr(out->slot, "slot", 4, needT && !ec));
  MOE_TRY(check_ptr(out->dropped, "dropped", 1, needT && !ec));
  MOE_TRY(check_ptr(out->sel, "sel", 4, needT && ec));
  MOE_TRY(check_ptr(out->counts, "counts", 4));
  MOE_TRY(check_ptr(out->losses, "losses", 4));
  MOE_TRY(check_ptr(out->stats, "stats", 4, false));
  MOE_TRY(check_ptr(out->logits, "logits", 4, false));
  MOE_TRY(check_ptr(out->probs, "probs", 4, false));
  MOE_TRY(check_ptr(out->lse, "lse", 4, false));
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w = carve(c, C, ws);
  const PhaseMarks pm{events, s};
  MOE_TRY(pm.mark(0));

  RouteArgs r = route_args(c, &w);
  r.x = x;
  r.w_router = wt->w_router;
  r.logit_bias = wt->logit_bias;
  r.select_bias = wt->select_bias;
  r.logits_out = out->logits;
  r.probs = out->probs;
  r.idx = out->idx;
  r.gates = out->gates;
  r.lse = out->lse;
  if (ec) {
    // the top-k of the router is still formed (into idx/gates when given)
    if (!r.probs) r.probs = w.ec_probs;
    if (!r.idx) r.idx = w.idx_tmp;
    if (!r.gates) r.gates = w.gates_tmp;
  }
  MOE_TRY(hip_status(launch_route(r, c.dtype, s), "router"));
  MOE_TRY(pm.mark(1));
  if (ec) return forward_expert_choice(c, C, *wt, x, r.probs, *out, w, s, pm);

  CapArgs a = cap_args(c, C, w);
  a.idx = out->idx;
  a.counts = out->counts;
  a.slot = out->slot;
  a.dropped = out->dropped;
  a.row_token = w.row_token;
  a.p_partial = w.p_partial;
  a.lse2_partial = w.lse2_partial;
  a.psum = w.psum;
  a.n_rtiles = router_tiles(c);
  // the up-projection gathers token rows straight into its tiles through
  // row_token, so no dispatched copy of x is made
  a.x = nullptr;
  a.xe = nullptr;
  MOE_TRY(capacity_step(c, C, w, a, out->gates, s));
  MOE_TRY(pm.mark(2));

  if (c.dropless) {
    // packed rows: expert e's rows start after the counts of the lower experts
    if (c.T > 0)
      MOE_TRY(ffn(c, c.act, c.E, c.T * c.k, out->counts, x, w.row_token, c.T, wt->w_in, wt->w_gate, wt->b_in,
                  wt->w_out, wt->b_out, c.d_ff, w.h, w.ye, s, true, c.T, w.pre0, w.pre1, nullptr, w.tailpart));
  } else if (C > 0) {
    MOE_TRY(ffn(c, c.act, c.E, C, w.kept, x, w.row_token, c.T, wt->w_in, wt->w_gate, wt->b_in, wt->w_out,
                wt->b_out, c.d_ff, w.h, w.ye, s, false, 0, w.pre0, w.pre1, w.kpart, w.tailpart));
  }
  MOE_TRY(pm.mark(3));
  if (c.n_shared > 0 && c.T > 0)
    MOE_TRY(ffn(c, MOE_GELU, 1, c.T, nullptr, x, nullptr, 0, wt->ws_in, nullptr, wt->bs_in, wt->ws_out,
                wt->bs_out, c.n_shared * c.d_ff_shared, w.hs, w.s, s, false, 0, w.pres));
  MOE_TRY(pm.mark(4));

  CombineArgs cb{};
  cb.x = x;
  cb.ye = w.ye;
  cb.shared_out = c.n_shared > 0 ? w.s : nullptr;
  cb.idx = out->idx;
  cb.gates = out->gates;
  cb.slot = out->slot;
  cb.dropped = out->dropped;
  cb.y = out->y;
  cb.T = c.T;
  cb.C = C;
  cb.d = c.d;
  cb.k = c.k;
  cb.E = c.E;
  cb.zero_fallback = c.dropped_output;
  cb.packed = c.dropless;
  MOE_TRY(hip_status(launch_combine(cb, c.dtype, s), "combine"));
  MOE_TRY(pm.mark(5));

  LossArgs l = loss_args(c, C, w, out->counts);
  l.losses = out->losses;
  l.stats = out->stats;
  MOE_TRY(hip_status(launch_losses(l, s), "loss finaliser"));
  return pm.mark(6);
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* wt, const void* x, moe_outputs* out, void* ws,
                       void* stream) {
  return forward_impl(cfg, wt, x, out, ws, stream, nullptr);
}

moe_status moe_forward_events(const moe_config* cfg, const moe_weights* wt, const void* x, moe_outputs* out,
                              void* ws, void* stream, void* const* events, int32_t n_events) {
  if (n_events != kForwardEvents || !events)
    return fail(MOE_EINVAL, "moe_forward_events takes %d event handles (got %d)", kForwardEvents, n_events);
  return forward_impl(cfg, wt, x, out, ws, stream, events);
}

size_t moe_backward_workspace_bytes(const moe_config* cfg) {
  int64_t C = 0;
  if (validate(cfg, &C) != MOE_OK || check_backward_config(*cfg, C) != MOE_OK) return 0;
  return carve_bwd(*cfg, C, nullptr).bytes;
}

moe_status moe_backward(const moe_config* cfg, const moe_weights* wt, const void* x, const moe_outputs* fwd,
                        const void* fwd_ws, const void* dy, float alpha_aux, float alpha_z, moe_grads* gr, void* bws,
                        void* stream) {
  int64_t C = 0;
  MOE_TRY(validate(cfg, &C));
  const moe_config& c = *cfg;
  MOE_TRY(check_backward_config(c, C));
  if (!wt || !fwd || !gr) return fail(MOE_EINVAL, "weights, forward outputs and gradients must not be NULL");
  if (!(alpha_aux == alpha_aux) || !(alpha_z == alpha_z)) return fail(MOE_EINVAL, "alpha_aux and alpha_z must not be NaN");
  const bool needT = c.T > 0;
  const bool glu = c.act == MOE_SWIGLU;
  const int64_t Fs = static_cast<int64_t>(c.n_shared) * c.d_ff_shared;
  MOE_TRY(check_ptr(x, "x", 16, needT));
  MOE_TRY(check_ptr(dy, "dy", 16, needT));
  MOE_TRY(check_ptr(fwd_ws, "fwd_ws", 256));
  MOE_TRY(check_ptr(bws, "bws", 256));
  MOE_TRY(check_ptr(wt->w_router, "w_router", 4));
  MOE_TRY(check_ptr(wt->w_in, "w_in", 16));
  MOE_TRY(check_ptr(wt->w_out, "w_out", 16));
  MOE_TRY(check_ptr(wt->b_in, "b_in", 16, false));
  if (glu) MOE_TRY(check_ptr(wt->w_gate, "w_gate", 16));
  if (Fs > 0) {
    MOE_TRY(check_ptr(wt->ws_in, "ws_in", 16));
    MOE_TRY(check_ptr(wt->ws_out, "ws_out", 16));
    MOE_TRY(check_ptr(wt->bs_in, "bs_in", 16, false));
  }
  const bool ec = c.routing == MOE_EXPERT_CHOICE;
  MOE_TRY(check_ptr(fwd->idx, "fwd idx", 4, needT && !ec));
  MOE_TRY(check_ptr(fwd->gates, "fwd gates", 4, needT && !ec));
  MOE_TRY(check_ptr(fwd->slot, "fwd slot", 4, needT && !ec));
  MOE_TRY(check_ptr(fwd->dropped, "fwd dropped", 1, needT && !ec));
  MOE_TRY(check_ptr(fwd->sel, "fwd sel", 4, needT && ec));
  MOE_TRY(check_ptr(fwd->probs, "fwd probs", 4, false));
  MOE_TRY(check_ptr(fwd->counts, "fwd counts", 4));
  MOE_TRY(check_ptr(fwd->logits, "fwd logits", 4, needT));
  MOE_TRY(check_ptr(gr->dx, "dx", 16, needT));
  MOE_TRY(check_ptr(gr->dw_router, "dw_router", 4));
  MOE_TRY(check_ptr(gr->dlogit_bias, "dlogit_bias", 4, false));
  MOE_TRY(check_ptr(gr->dw_in, "dw_in", 16));
  MOE_TRY(check_ptr(gr->dw_out, "dw_out", 16));
  if (glu) MOE_TRY(check_ptr(gr->dw_gate, "dw_gate", 16));
  MOE_TRY(check_ptr(gr->db_in, "db_in", 2, false));
  MOE_TRY(check_ptr(gr->db_out, "db_out", 2, false));
  if (glu && gr->db_in) return fail(MOE_EINVAL, "SwiGLU experts have no b_in (db_in must be NULL)");
  if (Fs > 0) {
    MOE_TRY(check_ptr(gr->dws_in, "dws_in", 16));
    MOE_TRY(check_ptr(gr->dws_out, "dws_out", 16));
    MOE_TRY(check_ptr(gr->dbs_in, "dbs_in", 2, false));
    MOE_TRY(check_ptr(gr->dbs_out, "dbs_out", 2, false));
  }
  MOE_TRY(check_ptr(gr->dgates, "dgates", 4, false));
  MOE_TRY(check_ptr(gr->dlogits, "dlogits", 4, false));
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w = carve(c, C, const_cast<void*>(fwd_ws));
  BwdWorkspace b = carve_bwd(c, C, bws);
  const int64_t T = c.T, d = c.d, F = c.d_ff, Tp = round8(T);
  const int E = c.E;
  const int ga = glu ? 2 : 1;

  BwdArgs a{};
  a.idx = fwd->idx;
  a.gates = fwd->gates;
  a.slot = fwd->slot;
  a.dropped = fwd->dropped;
  a.counts = fwd->counts;
  a.logits = fwd->logits;
  a.dy = dy;
  a.ye = w.ye;
  a.dYe = b.dYe;
  a.dgates = gr->dgates ? gr->dgates : b.dgates;
  a.dz = gr->dlogits ? gr->dlogits : b.dz;
  a.dA = b.dA;
  a.dAs = Fs > 0 ? b.dAs : nullptr;
  a.wrT = b.wrT;
  a.dx = gr->dx;
  a.T = T;
  a.C = C;
  a.d = c.d;
  a.E = E;
  a.k = ec ? 0 : c.k;
  a.score = c.score;
  a.renorm = resolved_renorm(c);
  if (ec) {
    // the forward kept the probabilities in the caller's buffer when given,
    // else in its workspace; every expert picked min(C, T) tokens
    a.sel = fwd->sel;
    a.probs = fwd->probs ? fwd->probs : w.ec_probs;
    a.dprobs = a.dgates;
    a.fden = static_cast<int64_t>(E) * std::min<int64_t>(C, T);
  }
  a.zero_fallback = c.dropped_output;
  a.packed = c.dropless;
  a.alpha_aux = alpha_aux;
  a.alpha_z = alpha_z;

  // gates and logits
  MOE_TRY(hip_status(launch_combine_bwd(a, s), "combine backward"));
  MOE_TRY(hip_status(launch_router_bwd(a, s), "router backward"));
  if (gr->dlogit_bias) MOE_TRY(hip_status(launch_dz_colsum(a.dz, gr->dlogit_bias, T, E, s), "logit-bias gradient"));
  // router weight: dW_r = x^T dz on the matrix cores, dz split into exact bf16
  // planes, K = tokens split into S slabs summed in order
  MOE_TRY(transpose("x transpose", static_cast<const bf16_t*>(x), b.xT, 1, T, d, Tp, 0, d, 0, Tp, nullptr, nullptr,
                    0, s));
  MOE_TRY(hip_status(launch_router_weight_prep(a.dz, b.planes, T, Tp, E, wt->w_router, b.wrT, c.d, s),
                     "router planes"));
  {
    const int S = b.S;
    const int64_t kc = Tp / S;
    GemmArgs g{};
    g.A = b.xT;
    g.B0 = b.planes;
    g.C = b.slabs;
    g.rows_per_group = d;
    g.groups = S;
    g.N = 4 * E;
    g.K = static_cast<int>(kc);
    g.lda = Tp;
    g.ldb = Tp;
    g.a_gs = kc;
    g.b_gs = kc;
    g.c_gs = d * E;
    g.act = 3;
    if (T > 0) MOE_TRY(hip_status(launch_gemm(g, MOE_BF16, s), "router weight gradient"));
    else MOE_TRY(hip_status(launch_zero(b.slabs, sizeof(float) * S * d * E, s), "router weight gradient"));
    MOE_TRY(hip_status(launch_slab_sum(b.slabs, gr->dw_router, d * E, S, s), "router weight slabs"));
  }

  // routed experts: rows = kept (expert choice: picked) per expert in [E, C]
  // slabs, or (dropless) every choice in packed rows; gathered from x
  // through row_token
  if (C > 0 && T > 0) {
    const bool dl = c.dropless != 0;
    const int32_t* rows = dl || ec ? fwd->counts : w.kept;   // rows of each expert
    const int64_t R = dl ? T * c.k : E * C;            // rows of the expert buffers
    const int64_t rpg = dl ? R : C;                    // GEMM rows per group (packed: the bound)
    const bf16_t* W_in = static_cast<const bf16_t*>(wt->w_in);
    // the GEMMs over the expert rows: slabs, or packed rows
    auto rgemm = [&](const char* what, const void* A, const int32_t* gather, int64_t a_rows, const void* B,
                     const void* bias, void* out, int N, int K) -> moe_status {
      return bgemm(what, A, 0, 0, gather, a_rows, B, 0, 0, bias, out, rows, rpg, E, N, K, s, nullptr, dl);
    };
    if (!c.save_preact) {
      // the forward's gate/up launch again, with its activations into the dH
      // buffer (scratch until dH is formed) and the pre-activations kept
      const GemmArgs g1 = up_args(c, c.act, E, rpg, rows, x, w.row_token, T, wt->w_in, wt->w_gate, wt->b_in,
                                  static_cast<int>(F), b.dH, dl, b.U, glu ? b.U2 : nullptr, b.tailpart);
      MOE_TRY(hip_status(launch_gemm(g1, MOE_BF16, s), "recompute pre-activations"));
    }
    // dH = dYe W_out, W_out [E, d, F] read k-major (k = d)
    MOE_TRY(kgemm("expert hidden gradient", 2, b.dYe, 0, 0, wt->w_out, nullptr, 0, F, d * F, b.dH, rows, rpg, E,
                  static_cast<int>(F), c.d, s, nullptr, nullptr, dl, nullptr, b.tailpart));
    ActBwdArgs ab{};
    ab.dH = b.dH;
    ab.U = c.save_preact ? static_cast<const bf16_t*>(w.pre0) : b.U;
    ab.U2 = c.save_preact ? static_cast<const bf16_t*>(w.pre1) : b.U2;
    ab.dact = b.dact;
    ab.valid = dl ? nullptr : rows;                    // packed rows are all valid
    ab.rpg = dl ? R : C;
    ab.groups = dl ? 1 : E;
    ab.F = static_cast<int>(F);
    MOE_TRY(hip_status(launch_act_bwd(ab, c.act, s), "activation backward"));
    // dA = dact W_in (SwiGLU: [dGp | dUp] [W_gate; W_up]), the weights read
    // k-major (k = F; SwiGLU: the gate matrix for k < F, the up matrix from
    // there, which needs F to be a multiple of the 64-k stage; otherwise they
    // are transposed into [E, d, 2F] first)
    if (!glu) {
      MOE_TRY(kgemm("expert input gradient", 2, b.dact, 0, 0, W_in, nullptr, 0, d, F * d, b.dA, rows, rpg, E, c.d,
                    static_cast<int>(F), s, nullptr, nullptr, dl, nullptr, b.tailpart));
    } else if (F % 64 == 0) {
      MOE_TRY(kgemm("expert input gradient", 2, b.dact, 0, 0, wt->w_gate, W_in, F, d, F * d, b.dA, rows, rpg, E,
                    c.d, static_cast<int>(2 * F), s, nullptr, nullptr, dl, nullptr, b.tailpart));
    } else {
      MOE_TRY(transpose("w_gate transpose", static_cast<const bf16_t*>(wt->w_gate), b.wiT, E, F, d, F, F * d, d,
                        d * 2 * F, 2 * F, nullptr, nullptr, 0, s));
      MOE_TRY(transpose("w_up transpose", W_in, b.wiT + F, E, F, d, F, F * d, d, d * 2 * F, 2 * F, nullptr, nullptr, 0,
                        s));
      MOE_TRY(rgemm("expert input gradient", b.dact, nullptr, 0, b.wiT, nullptr, b.dA, c.d, static_cast<int>(2 * F)));
    }
    // dW_out = dYe^T H and dW_in = dact^T A: contractions over each expert's
    // own rows (kvar).  dYe, H and dact are read k-major from the expert
    // buffers (dropless: from each expert's packed start); the token rows,
    // gathered through row_token, are transposed into per-expert blocks
    // packed one after another: expert e's block is [d, n_e], n_e = max(8,
    // round8(rows_e)) (zero past rows_e), kstart[e]*d elements in
    MOE_TRY(hip_status(launch_group_starts(rows, b.kstart, E, 1, s), "packed columns"));
    if (dl) MOE_TRY(hip_status(launch_group_starts(rows, b.pstart, E, 0, s), "packed rows"));
    const int32_t* gst = dl ? b.pstart : nullptr;
    const int64_t Kw = b.Kw;
    const int64_t rmax = dl ? T : C;                   // rows of one expert at most
    const int Kmax = static_cast<int>(std::max<int64_t>(8, round8(rmax)));
    MOE_TRY(kgemm("w_out gradient", 3, b.dYe, d, dl ? 0 : C * d, w.h, nullptr, 0, F, dl ? 0 : C * F, gr->dw_out,
                  nullptr, d, E, static_cast<int>(F), Kmax, s, rows, gst));
    MOE_TRY(transpose("token rows transpose", static_cast<const bf16_t*>(x), b.AT, E, rmax, d, round8(rmax), 0, d, 0,
                      Kw, rows, w.row_token, C, s, b.kstart, gst));
    // (SwiGLU: the gate half of the activation gradient, then the up half, F
    // columns in)
    for (int h = 0; h < ga; ++h) {
      void* dw = glu && h == 0 ? gr->dw_gate : gr->dw_in;
      MOE_TRY(kgemm(glu ? (h == 0 ? "w_gate gradient" : "w_up gradient") : "w_in gradient", 1, b.dact + h * F,
                    ga * F, dl ? 0 : C * ga * F, b.AT, nullptr, 0, 0, 0, dw, nullptr, F, E, c.d,
                    static_cast<int>(Kw), s, rows, gst, false, b.kstart));
    }
    const int32_t* starts = dl ? b.pstart : nullptr;
    if (gr->db_out)
      MOE_TRY(hip_status(launch_colsum(b.dYe, gr->db_out, rows, E, rpg, d, 0, s, starts), "b_out gradient"));
    if (gr->db_in)
      MOE_TRY(hip_status(launch_colsum(b.dact, gr->db_in, rows, E, rpg, F, 0, s, starts), "b_in gradient"));
  } else {
    // no expert row: every expert-weight gradient is zero
    const size_t ew = sizeof(bf16_t) * E * F * d;
    MOE_TRY(hip_status(launch_zero(gr->dw_in, ew, s), "zero gradients"));
    MOE_TRY(hip_status(launch_zero(gr->dw_out, ew, s), "zero gradients"));
    if (glu) MOE_TRY(hip_status(launch_zero(gr->dw_gate, ew, s), "zero gradients"));
    if (gr->db_in) MOE_TRY(hip_status(launch_zero(gr->db_in, sizeof(bf16_t) * E * F, s), "zero gradients"));
    if (gr->db_out) MOE_TRY(hip_status(launch_zero(gr->db_out, sizeof(bf16_t) * E * d, s), "zero gradients"));
  }

  // shared experts: every token, output gradient dy itself
  if (Fs > 0 && T > 0) {
    if (!c.save_preact)
      MOE_TRY(bgemm("recompute shared pre-activation", x, 0, 0, nullptr, 0, wt->ws_in, 0, 0, wt->bs_in, b.Us, nullptr,
                    T, 1, static_cast<int>(Fs), c.d, s));
    // the shared weights and the activations read k-major: no transposed copies
    MOE_TRY(kgemm("shared hidden gradient", 2, dy, 0, 0, wt->ws_out, nullptr, 0, Fs, 0, b.dHs, nullptr, T, 1,
                  static_cast<int>(Fs), c.d, s));
    ActBwdArgs ab{};
    ab.dH = b.dHs;
    ab.U = c.save_preact ? static_cast<const bf16_t*>(w.pres) : b.Us;
    ab.dact = b.dUs;
    ab.rpg = T;
    ab.groups = 1;
    ab.F = static_cast<int>(Fs);
    MOE_TRY(hip_status(launch_act_bwd(ab, MOE_GELU, s), "shared activation backward"));
    MOE_TRY(kgemm("shared input gradient", 2, b.dUs, 0, 0, wt->ws_in, nullptr, 0, d, 0, b.dAs, nullptr, T, 1, c.d,
                  static_cast<int>(Fs), s));
    MOE_TRY(kgemm("ws_out gradient", 3, dy, d, 0, w.hs, nullptr, 0, Fs, 0, gr->dws_out, nullptr, d, 1,
                  static_cast<int>(Fs), static_cast<int>(T), s));
    MOE_TRY(kgemm("ws_in gradient", 3, b.dUs, Fs, 0, x, nullptr, 0, d, 0, gr->dws_in, nullptr, Fs, 1, c.d,
                  static_cast<int>(T), s));
    if (gr->dbs_in) MOE_TRY(hip_status(launch_colsum(b.dUs, gr->dbs_in, nullptr, 1, T, Fs, 0, s), "bs_in gradient"));
    if (gr->dbs_out)
      MOE_TRY(hip_status(launch_colsum(static_cast<const bf16_t*>(dy), gr->dbs_out, nullptr, 1, T, d, 0, s),
                         "bs_out gradient"));
  }
  if (Fs > 0 && T == 0) {
    const size_t sw = sizeof(bf16_t) * Fs * d;
    MOE_TRY(hip_status(launch_zero(gr->dws_in, sw, s), "zero gradients"));
    MOE_TRY(hip_status(launch_zero(gr->dws_out, sw, s), "zero gradients"));
    if (gr->dbs_in) MOE_TRY(hip_status(launch_zero(gr->dbs_in, sizeof(bf16_t) * Fs, s), "zero gradients"));
    if (gr->dbs_out) MOE_TRY(hip_status(launch_zero(gr->dbs_out, sizeof(bf16_t) * d, s), "zero gradients"));
  }
  return hip_status(launch_dx(a, s), "input gradient");
}

}  // extern "C"
