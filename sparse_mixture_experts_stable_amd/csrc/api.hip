// C ABI of libmoe.so: host-side validation, workspace carve-up and the launch sequence of
// every entry point. No entry point allocates device memory or synchronises (except
// moe_read_error and moe_profile_read, which exist to wait).

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

using namespace moe;

// ------------------------------------------------------------------------------------
// profiling hooks
// ------------------------------------------------------------------------------------
namespace {
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
bool g_prof = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
hipEvent_t g_pending = nullptr;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

namespace moe_prof {
void before(const char*, hipStream_t s) {
  if (!g_prof) return;
  g_pending = take_event();
  if (g_pending) (void)hipEventRecord(g_pending, s);
}
void after(const char* name, hipStream_t s) {
  if (!g_prof || !g_pending) return;
  hipEvent_t stop = take_event();
  if (!stop) return;
  (void)hipEventRecord(stop, s);
  g_recs.push_back({name, g_pending, stop});
  g_pending = nullptr;
}
}  // namespace moe_prof

// ------------------------------------------------------------------------------------
// helpers
// ------------------------------------------------------------------------------------
namespace {

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

int elem_size(int dt) { return dt == MOE_BF16 ? 2 : 4; }

bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }

bool valid_kind(int k) {
  return k == MOE_EXPERT_LINEAR || k == MOE_EXPERT_GELU_MLP || k == MOE_EXPERT_SWIGLU;
}

// Validates an expert set. Returns MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED.
moe_status_t check_experts(const moe_experts_t* ex) {
  if (!ex) return MOE_ERR_INVALID_ARG;
  if (!valid_kind(ex->kind) || !valid_dtype(ex->dtype)) return MOE_ERR_INVALID_ARG;
  if (ex->num_experts < 1 || ex->d_model < 1 || ex->d_hidden < 1) return MOE_ERR_INVALID_ARG;
  if (!ex->w_in) return MOE_ERR_INVALID_ARG;
  if (ex->kind == MOE_EXPERT_LINEAR && ex->d_hidden != ex->d_model) return MOE_ERR_INVALID_ARG;
  if (ex->kind == MOE_EXPERT_SWIGLU && (!ex->w_up || !ex->w_out)) return MOE_ERR_INVALID_ARG;
  if (ex->kind == MOE_EXPERT_GELU_MLP && !ex->w_out) return MOE_ERR_INVALID_ARG;
  if (ex->w_in_layout != MOE_LAYOUT_IN_OUT && ex->w_in_layout != MOE_LAYOUT_OUT_IN)
    return MOE_ERR_INVALID_ARG;
  if (ex->w_out_layout != MOE_LAYOUT_IN_OUT && ex->w_out_layout != MOE_LAYOUT_OUT_IN)
    return MOE_ERR_INVALID_ARG;
  const int q = ex->dtype == MOE_BF16 ? 64 : 16;
  if (ex->d_model % q || ex->d_hidden % q) return MOE_ERR_UNSUPPORTED;
  if ((ex->w_in_layout == MOE_LAYOUT_OUT_IN || ex->w_out_layout == MOE_LAYOUT_OUT_IN) &&
      ex->dtype != MOE_BF16)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t hidden_bytes(const moe_experts_t* ex, int rows) {
  if (ex->kind == MOE_EXPERT_LINEAR) return 0;
  return size_t(ex->num_experts) * rows * ex->d_hidden * elem_size(ex->dtype);
}

// The bf16 tile loader forms each lane's A and B byte offsets from a group's base in 32
// bits (the base itself is 64-bit), so every row of a bf16 operand it reads must start
// below 4 GiB from its group's base: rows * leading dimension * 2 bytes < 2^32.
bool bf16_rows_fit(int64_t rows, int64_t ld) {
  return rows >= 0 && ld >= 0 && rows * ld * 2 < (int64_t(1) << 32);
}

// The bf16 operands of one expert set run through that loader: x (rows of T, leading
// dimension ldx), the hidden activation of each group (C rows routed, T dense, of F),
// and each expert's weight matrices (D x F either way round).
bool bf16_expert_offsets_fit(const moe_experts_t* ex, int64_t T, int64_t ldx, int64_t rows) {
  if (ex->dtype != MOE_BF16) return true;
  const int64_t D = ex->d_model, F = ex->d_hidden;
  return bf16_rows_fit(T, ldx) && bf16_rows_fit(rows, F) && bf16_rows_fit(D, F) &&
         bf16_rows_fit(F, D);
}

// The expert GEMM problems for one expert set. dense: slot_assign == NULL (all T rows).
struct ExpertPlan {
  GemmProblem g1, g2;       // bf16
  GemmF32Problem f1, f2;    // fp32
  bool two_stage;
};

// h_pieces: the hidden activation is the library's own (not a caller's hidden_cache),
// so the bf16 GEMMs keep it in 32-column pieces (GemmProblem::c_pstride / a_pstride).
void plan_experts(const moe_experts_t* ex, const void* x, int64_t ldx, int T, int k, int C,
                  const int32_t* slot_assign, const int32_t* used, void* hidden, void* out,
                  bool h_pieces, ExpertPlan& pl) {
  const bool dense = slot_assign == nullptr;
  const int rows = dense ? T : C;
  const int E = ex->num_experts, D = ex->d_model, F = ex->d_hidden;
  pl.two_stage = ex->kind != MOE_EXPERT_LINEAR;
  if (ex->dtype == MOE_BF16) {
    GemmProblem a{};
    a.A = x;
    a.lda = ldx;
    a.a_gstride = 0;
    a.row_map = slot_assign;
    a.row_map_ld = C;
    a.row_div = k;
    a.m_count = dense ? nullptr : used;
    a.m_const = T;
    a.m_tiles_rows = rows;
    a.B0 = ex->w_in;
    a.B1 = ex->kind == MOE_EXPERT_SWIGLU ? ex->w_up : nullptr;
    a.b_gstride = int64_t(D) * (pl.two_stage ? F : D);
    a.b_kmajor = ex->w_in_layout == MOE_LAYOUT_OUT_IN;
    a.bias = ex->kind == MOE_EXPERT_GELU_MLP ? ex->b_in : nullptr;
    a.bias_gstride = F;
    a.K = D;
    a.N = pl.two_stage ? F : D;
    a.groups = E;
    a.epi = ex->kind == MOE_EXPERT_GELU_MLP ? EPI_GELU_BIAS
          : ex->kind == MOE_EXPERT_SWIGLU  ? EPI_SWIGLU
                                           : EPI_STORE;
    a.out_f32 = 0;
    a.C = pl.two_stage ? hidden : out;
    a.ldc = a.N;
    a.c_gstride = int64_t(rows) * a.N;
    const int64_t pieces = pl.two_stage && h_pieces ? int64_t(rows) * 32 : 0;
    a.c_pstride = pieces;
    pl.g1 = a;
    if (pl.two_stage) {
      GemmProblem b{};
      b.A = hidden;
      b.lda = F;
      b.a_gstride = int64_t(rows) * F;
      b.a_pstride = pieces;
      b.row_map = nullptr;
      b.row_div = 1;
      b.m_count = dense ? nullptr : used;
      b.m_const = T;
      b.m_tiles_rows = rows;
      b.B0 = ex->w_out;
      b.b_gstride = int64_t(F) * D;
      b.b_kmajor = ex->w_out_layout == MOE_LAYOUT_OUT_IN;
      b.bias = ex->kind == MOE_EXPERT_GELU_MLP ? ex->b_out : nullptr;
      b.bias_gstride = D;
      b.K = F;
      b.N = D;
      b.groups = E;
      b.epi = ex->kind == MOE_EXPERT_GELU_MLP ? EPI_BIAS : EPI_STORE;
      b.C = out;
      b.ldc = D;
      b.c_gstride = int64_t(rows) * D;
      pl.g2 = b;
    }
  } else {
    GemmF32Problem a{};
    a.A = static_cast<const float*>(x);
    a.lda = ldx;
    a.row_map = slot_assign;
    a.row_map_ld = C;
    a.row_div = k;
    a.g_count = dense ? nullptr : used;
    a.g_const = T;
    a.m_rows = rows;
    a.B = static_cast<const float*>(ex->w_in);
    a.B1 = static_cast<const float*>(ex->kind == MOE_EXPERT_SWIGLU ? ex->w_up : nullptr);
    a.N = pl.two_stage ? F : D;
    a.ldb = a.N;
    a.b_gstride = int64_t(D) * a.N;
    a.bias = static_cast<const float*>(ex->kind == MOE_EXPERT_GELU_MLP ? ex->b_in : nullptr);
    a.bias_gstride = F;
    a.K = D;
    a.groups = E;
    a.epi = ex->kind == MOE_EXPERT_GELU_MLP ? EPI_GELU_BIAS
          : ex->kind == MOE_EXPERT_SWIGLU  ? EPI_SWIGLU
                                           : EPI_STORE;
    a.C = static_cast<float*>(pl.two_stage ? hidden : out);
    a.ldc = a.N;
    a.c_gstride = int64_t(rows) * a.N;
    pl.f1 = a;
    if (pl.two_stage) {
      GemmF32Problem b{};
      b.A = static_cast<const float*>(hidden);
      b.lda = F;
      b.a_gstride = int64_t(rows) * F;
      b.row_div = 1;
      b.g_count = dense ? nullptr : used;
      b.g_const = T;
      b.m_rows = a.m_rows;
      b.B = static_cast<const float*>(ex->w_out);
      b.ldb = D;
      b.b_gstride = int64_t(F) * D;
      b.bias = static_cast<const float*>(ex->kind == MOE_EXPERT_GELU_MLP ? ex->b_out : nullptr);
      b.bias_gstride = D;
      b.K = F;
      b.N = D;
      b.groups = E;
      b.epi = EPI_BIAS;
      b.C = static_cast<float*>(out);
      b.ldc = D;
      b.c_gstride = int64_t(rows) * D;
      pl.f2 = b;
    }
  }
}

// Runs one or two expert sets (routed + shared) with shared launches per stage.
moe_status_t run_experts(const ExpertPlan* plans, const moe_experts_t* const* exs, int n,
                         hipStream_t s) {
  if (exs[0]->dtype == MOE_BF16) {
    GemmBatch b1{};
    b1.nprob = n;
    for (int i = 0; i < n; ++i) b1.p[i] = plans[i].g1;
    const bool gated = exs[0]->kind == MOE_EXPERT_SWIGLU;
    if (n == 2 && (exs[1]->kind == MOE_EXPERT_SWIGLU) != gated) {
      // different kinds cannot share a launch
      for (int i = 0; i < n; ++i) {
        GemmBatch one{};
        one.nprob = 1;
        one.p[0] = plans[i].g1;
        moe_status_t st = launch_gemm_bf16(one, exs[i]->kind == MOE_EXPERT_SWIGLU, "expert_gemm1", s);
        if (st != MOE_OK) return st;
      }
    } else {
      moe_status_t st = launch_gemm_bf16(b1, gated, gated ? "expert_gemm1_swiglu" : "expert_gemm1", s);
      if (st != MOE_OK) return st;
    }
    GemmBatch b2{};
    for (int i = 0; i < n; ++i)
      if (plans[i].two_stage) b2.p[b2.nprob++] = plans[i].g2;
    if (b2.nprob) return launch_gemm_bf16(b2, false, "expert_gemm2", s);
    return MOE_OK;
  }
  for (int i = 0; i < n; ++i) {
    ExpertPlan p = plans[i];
    // a dense set (the shared expert) runs under names of its own
    const bool dense = p.f1.row_map == nullptr;
    const char* n1 = p.f1.epi == EPI_SWIGLU ? (dense ? "shared_gemm1_swiglu_f32" : "expert_gemm1_swiglu_f32")
                                            : (dense ? "shared_gemm1_f32" : "expert_gemm1_f32");
    moe_status_t st = launch_gemm_f32(p.f1, A_ROWS, B_KN, n1, s);
    if (st != MOE_OK) return st;
    if (p.two_stage) {
      st = launch_gemm_f32(p.f2, A_ROWS, B_KN, dense ? "shared_gemm2_f32" : "expert_gemm2_f32", s);
      if (st != MOE_OK) return st;
    }
  }
  return MOE_OK;
}

moe_status_t router_gemm(const void* x, int dt, int64_t ldx, const void* w, int T, int D, int E,
                         float* logits, hipStream_t s) {
  if (dt == MOE_BF16 && D % kBf16BK == 0 && E % 8 == 0) {
    GemmBatch b{};
    b.nprob = 1;
    GemmProblem& p = b.p[0];
    p.A = x;
    p.lda = ldx;
    p.row_div = 1;
    p.m_const = T;
    p.m_tiles_rows = T;
    p.B0 = w;
    p.K = D;
    p.N = E;
    p.groups = 1;
    p.epi = EPI_STORE;
    p.out_f32 = 1;
    p.C = logits;
    p.ldc = E;
    return launch_gemm_bf16(b, false, "router_gemm", s);
  }
  if (dt == MOE_F32 && D % 4 == 0 && E % 4 == 0 && ldx % 4 == 0) {
    GemmF32Problem p{};
    p.A = static_cast<const float*>(x);
    p.lda = ldx;
    p.row_div = 1;
    p.g_const = T;
    p.m_rows = T;
    p.B = static_cast<const float*>(w);
    p.ldb = E;
    p.K = D;
    p.N = E;
    p.groups = 1;
    p.epi = EPI_STORE;
    p.C = logits;
    p.ldc = E;
    return launch_gemm_f32(p, A_ROWS, B_KN, "router_gemm_f32", s);
  }
  return launch_router_simt(x, dt, ldx, w, T, D, E, logits, s);
}

bool opts_ok(const moe_router_opts_t* o) {
  return !o || o->scoring == MOE_SCORE_SOFTMAX || o->scoring == MOE_SCORE_SIGMOID;
}

RouteOpts route_opts(const moe_router_opts_t* o) {
  RouteOpts r{};
  r.scoring = o ? o->scoring : MOE_SCORE_SOFTMAX;
  r.bias = o ? o->selection_bias : nullptr;
  r.with_z = (o && o->z_loss) ? 1 : 0;
  return r;
}

bool route_shape_ok(int T, int E, int k) {
  return T >= 1 && E >= 1 && E <= 1024 && k >= 1 && k <= E;
}

}  // namespace

// ------------------------------------------------------------------------------------
// SIMT router GEMM for shapes the MFMA tiles do not cover
// ------------------------------------------------------------------------------------
namespace moe {
template <typename TX>
__global__ __launch_bounds__(64) void router_simt_kernel(const TX* __restrict__ x, int64_t ldx,
                                                         const TX* __restrict__ w, int D, int E,
                                                         float* __restrict__ logits) {
  const int t = blockIdx.x;
  const int e = blockIdx.y * 64 + threadIdx.x;
  if (e >= E) return;
  float acc = 0.f;
  for (int d = 0; d < D; ++d) {
    float xv, wv;
    if constexpr (sizeof(TX) == 2) {
      xv = bf16_to_f32(x[size_t(t) * ldx + d]);
      wv = bf16_to_f32(w[size_t(d) * E + e]);
    } else {
      xv = x[size_t(t) * ldx + d];
      wv = w[size_t(d) * E + e];
    }
    acc = fmaf(xv, wv, acc);
  }
  logits[size_t(t) * E + e] = acc;
}

moe_status_t launch_router_simt(const void* x, int dtype, int64_t ldx, const void* w, int T,
                                int D, int E, float* logits, hipStream_t s) {
  const dim3 grid(T, (E + 63) / 64), block(64);
  if (dtype == MOE_BF16) {
    MOE_LAUNCH("router_simt", router_simt_kernel<bf16_t>, grid, block, 0, s,
               static_cast<const bf16_t*>(x), ldx, static_cast<const bf16_t*>(w), D, E, logits);
  } else {
    MOE_LAUNCH("router_simt", router_simt_kernel<float>, grid, block, 0, s,
               static_cast<const float*>(x), ldx, static_cast<const float*>(w), D, E, logits);
  }
  return MOE_OK;
}
}  // namespace moe

// ------------------------------------------------------------------------------------
// C ABI
// ------------------------------------------------------------------------------------
extern "C" {

const char* moe_version(void) { return "moe-gfx950 0.1"; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double cf) {
  if (T < 1 || T >= (int64_t(1) << 40) || E < 1 || k < 1 || k > E) return -1;
  if (!std::isfinite(cf) || cf < 0.0) return -1;
  if (cf == 0.0) return 0;
  // cf = mant * 2^ex exactly, mant a 53-bit integer
  int ex = 0;
  const double fr = std::frexp(cf, &ex);
  const uint64_t mant = static_cast<uint64_t>(std::ldexp(fr, 53));
  ex -= 53;
  unsigned __int128 num = static_cast<unsigned __int128>(T) * static_cast<unsigned>(k) * mant;
  if (ex > 0) {
    if (ex > 40) return -1;
    num <<= ex;
  }
  unsigned __int128 q = (num + static_cast<unsigned>(E) - 1) / static_cast<unsigned>(E);
  if (ex < 0) {
    const int sh = -ex;
    if (sh >= 127) {
      q = q > 0 ? 1 : 0;
    } else {
      const unsigned __int128 one = 1;
      q = (q + (one << sh) - 1) >> sh;
    }
  }
  if (q > static_cast<unsigned __int128>(INT32_MAX)) return -1;
  return static_cast<int64_t>(q);
}

size_t moe_route_workspace_size(int32_t T, int32_t E) {
  if (T < 1 || E < 1) return 0;
  return carve_route_ws(nullptr, T, E).bytes;
}

moe_status_t moe_route(const void* x, int32_t x_dtype, int64_t ldx, const void* w_router,
                       float* logits, int32_t T, int32_t D, int32_t E, int32_t k,
                       int32_t* topk_idx, float* topk_gate, int32_t* expert_count,
                       float* prob_sum, float* aux_loss, const moe_router_opts_t* opts,
                       void* ws, size_t ws_bytes, void* stream) {
  if (!route_shape_ok(T, E, k)) return k > 256 && k <= E ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG;
  if (k > 256) return MOE_ERR_UNSUPPORTED;
  if (!logits || !topk_idx || !topk_gate || !expert_count || !prob_sum || !aux_loss || !ws)
    return MOE_ERR_INVALID_ARG;
  if (w_router) {
    if (!x || !valid_dtype(x_dtype) || D < 1 || ldx < D) return MOE_ERR_INVALID_ARG;
    if (x_dtype == MOE_BF16 && !bf16_rows_fit(T, ldx)) return MOE_ERR_UNSUPPORTED;
  }
  if (!opts_ok(opts)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe_route_workspace_size(T, E)) return MOE_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  RouteWs w = carve_route_ws(ws, T, E);
  moe_status_t st;
  if (w_router) {
    st = router_gemm(x, x_dtype, ldx, w_router, T, D, E, logits, s);
    if (st != MOE_OK) return st;
  }
  st = launch_route(logits, T, E, k, topk_idx, topk_gate, route_opts(opts), w, s);
  if (st != MOE_OK) return st;
  const LoadStats ls{opts ? opts->token_fraction : nullptr,
                     opts ? opts->probability_mass : nullptr};
  return launch_reduce_scan(T, k, E, -1, true, expert_count, prob_sum, aux_loss, nullptr, nullptr,
                            nullptr, opts ? opts->z_loss : nullptr, ls, w, s);
}

size_t moe_dispatch_workspace_size(int32_t T, int32_t k, int32_t E) {
  if (T < 1 || E < 1 || k < 1) return 0;
  return carve_route_ws(nullptr, T, E).bytes;
}

moe_status_t moe_dispatch(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t C,
                          int32_t* slot, uint8_t* kept, int32_t* slot_assign,
                          int32_t* expert_used, int32_t* expert_overflow,
                          int32_t* token_drops, void* ws, size_t ws_bytes, void* stream) {
  if (T < 1 || E < 1 || E > 1024 || k < 1 || C < 0) return MOE_ERR_INVALID_ARG;
  if (!topk_idx || !slot || !kept || !expert_used || !expert_overflow || !token_drops || !ws)
    return MOE_ERR_INVALID_ARG;
  if (C > 0 && !slot_assign) return MOE_ERR_INVALID_ARG;
  if (int64_t(T) * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < moe_dispatch_workspace_size(T, k, E)) return MOE_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  RouteWs w = carve_route_ws(ws, T, E);
  moe_status_t st = launch_count(topk_idx, T, k, E, w, s);
  if (st != MOE_OK) return st;
  // expert_count is not an output of moe_dispatch; the totals land in fp scratch space
  return launch_dispatch(topk_idx, T, k, E, C, false, reinterpret_cast<int32_t*>(w.fp), nullptr,
                         nullptr, expert_used, expert_overflow, nullptr, LoadStats{}, slot, kept,
                         slot_assign, token_drops, w, s);
}

size_t moe_expert_mlp_workspace_size(const moe_experts_t* ex, int32_t rows) {
  if (!ex || rows < 0) return 0;
  return align_up(hidden_bytes(ex, rows), 256) + 256;
}

moe_status_t moe_expert_mlp(const moe_experts_t* ex, const void* x, int64_t ldx, int32_t T,
                            int32_t k, int32_t C, const int32_t* slot_assign,
                            const int32_t* expert_used, void* hidden_cache, void* expert_out,
                            void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_experts(ex);
  if (st != MOE_OK) return st;
  if (!x || !expert_out || T < 1 || ldx < ex->d_model) return MOE_ERR_INVALID_ARG;
  const bool dense = slot_assign == nullptr;
  if (dense && ex->num_experts != 1) return MOE_ERR_INVALID_ARG;
  if (!dense && (k < 1 || C < 0 || !expert_used)) return MOE_ERR_INVALID_ARG;
  if (ldx % (ex->dtype == MOE_BF16 ? 8 : 4)) return MOE_ERR_UNSUPPORTED;
  const int rows = dense ? T : C;
  if (!bf16_expert_offsets_fit(ex, T, ldx, rows)) return MOE_ERR_UNSUPPORTED;
  void* hidden = hidden_cache;
  if (!hidden && hidden_bytes(ex, rows)) {
    if (!ws || ws_bytes < moe_expert_mlp_workspace_size(ex, rows)) return MOE_ERR_WORKSPACE;
    hidden = ws;
  }
  if (rows == 0) return MOE_OK;
  ExpertPlan pl;
  plan_experts(ex, x, ldx, T, k, C, slot_assign, expert_used, hidden, expert_out,
               hidden_cache == nullptr, pl);
  const moe_experts_t* exs[1] = {ex};
  return run_experts(&pl, exs, 1, S(stream));
}

moe_status_t moe_combine(int32_t dt, const void* residual, const void* shared_out,
                         const void* expert_out, const int32_t* topk_idx, const int32_t* slot,
                         const float* topk_gate, int32_t T, int32_t k, int32_t E, int32_t C,
                         int32_t D, int32_t renormalize_kept, void* y, void* stream) {
  if (!valid_dtype(dt) || T < 1 || k < 1 || E < 1 || D < 1) return MOE_ERR_INVALID_ARG;
  if (!topk_idx || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  const bool dense = slot == nullptr;
  if (dense ? !expert_out : (C < 0 || (C > 0 && !expert_out))) return MOE_ERR_INVALID_ARG;
  if (dense && int64_t(T) * E >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return launch_combine(dt, residual, D, shared_out, expert_out, topk_idx, slot, topk_gate, T, k,
                        E, dense ? 1 : C, D, renormalize_kept ? 1 : 0, y, S(stream));
}

// ---- forward ------------------------------------------------------------------------
namespace {
struct FwdWs {
  RouteWs rw;
  void* hidden;
  void* shared_hidden;
  void* shared_out;
  size_t bytes;
};

FwdWs carve_fwd(const moe_forward_args_t* a, void* ws) {
  FwdWs f{};
  const int E = a->experts.num_experts;
  f.rw = carve_route_ws(ws, a->T, E);
  size_t off = f.rw.bytes;
  char* base = static_cast<char*>(ws);
  f.hidden = nullptr;
  if (!a->hidden_cache) {
    const size_t hb = hidden_bytes(&a->experts, a->capacity);
    if (hb) {
      f.hidden = base ? base + off : nullptr;
      off = align_up(off + hb, 256);
    }
  }
  f.shared_hidden = nullptr;
  f.shared_out = nullptr;
  if (a->shared.w_in) {
    f.shared_hidden = base ? base + off : nullptr;
    off = align_up(off + hidden_bytes(&a->shared, a->T), 256);
    if (!a->shared_out) {
      f.shared_out = base ? base + off : nullptr;
      off = align_up(off + size_t(a->T) * a->experts.d_model * elem_size(a->experts.dtype), 256);
    }
  }
  f.bytes = off;
  return f;
}

moe_status_t check_forward(const moe_forward_args_t* a) {
  if (!a) return MOE_ERR_INVALID_ARG;
  moe_status_t st = check_experts(&a->experts);
  if (st != MOE_OK) return st;
  const int T = a->T, E = a->experts.num_experts, k = a->k, C = a->capacity;
  const int D = a->experts.d_model;
  if (!route_shape_ok(T, E, k) || C < 0 || !opts_ok(&a->router)) return MOE_ERR_INVALID_ARG;
  if (k > 256 || int64_t(T) * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!a->x || a->ldx < D || !a->logits || !a->y) return MOE_ERR_INVALID_ARG;
  if (!a->topk_idx || !a->topk_gate || !a->expert_count || !a->prob_sum || !a->aux_loss ||
      !a->slot || !a->kept || !a->expert_used || !a->expert_overflow || !a->token_drops ||
      (C > 0 && (!a->slot_assign || !a->expert_out)))
    return MOE_ERR_INVALID_ARG;
  if (a->ldx % (a->experts.dtype == MOE_BF16 ? 8 : 4)) return MOE_ERR_UNSUPPORTED;
  if (!bf16_expert_offsets_fit(&a->experts, T, a->ldx, C)) return MOE_ERR_UNSUPPORTED;
  if (a->shared.w_in && !bf16_expert_offsets_fit(&a->shared, T, a->ldx, T))
    return MOE_ERR_UNSUPPORTED;
  if (a->shared.w_in) {
    st = check_experts(&a->shared);
    if (st != MOE_OK) return st;
    if (a->shared.kind != MOE_EXPERT_SWIGLU || a->shared.num_experts != 1 ||
        a->shared.dtype != a->experts.dtype || a->shared.d_model != D ||
        a->shared.w_in_layout != a->experts.w_in_layout ||
        a->shared.w_out_layout != a->experts.w_out_layout)
      return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}
}  // namespace

size_t moe_forward_workspace_size(const moe_forward_args_t* a) {
  if (!a || a->T < 1 || a->experts.num_experts < 1) return 0;
  return carve_fwd(a, nullptr).bytes;
}

moe_status_t moe_forward(const moe_forward_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_forward(a);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < moe_forward_workspace_size(a)) return MOE_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  const int T = a->T, E = a->experts.num_experts, k = a->k, C = a->capacity;
  const int D = a->experts.d_model;
  FwdWs f = carve_fwd(a, ws);
  if (a->w_router) {
    st = router_gemm(a->x, a->experts.dtype, a->ldx, a->w_router, T, D, E, a->logits, s);
    if (st != MOE_OK) return st;
  }
  st = launch_route(a->logits, T, E, k, a->topk_idx, a->topk_gate, route_opts(&a->router), f.rw,
                    s);
  if (st != MOE_OK) return st;
  st = launch_dispatch(a->topk_idx, T, k, E, C, true, a->expert_count, a->prob_sum, a->aux_loss,
                       a->expert_used, a->expert_overflow, a->router.z_loss,
                       LoadStats{a->router.token_fraction, a->router.probability_mass}, a->slot,
                       a->kept, a->slot_assign, a->token_drops, f.rw, s);
  if (st != MOE_OK) return st;

  ExpertPlan plans[2];
  const moe_experts_t* exs[2] = {&a->experts, &a->shared};
  int n = 0;
  if (C > 0) {
    plan_experts(&a->experts, a->x, a->ldx, T, k, C, a->slot_assign, a->expert_used,
                 a->hidden_cache ? a->hidden_cache : f.hidden, a->expert_out,
                 a->hidden_cache == nullptr, plans[n]);
    exs[n++] = &a->experts;
  }
  void* shared_out = nullptr;
  if (a->shared.w_in) {
    shared_out = a->shared_out ? a->shared_out : f.shared_out;
    plan_experts(&a->shared, a->x, a->ldx, T, 1, 0, nullptr, nullptr, f.shared_hidden,
                 shared_out, true, plans[n]);
    exs[n++] = &a->shared;
  }
  if (n) {
    st = run_experts(plans, exs, n, s);
    if (st != MOE_OK) return st;
  }
  return launch_combine(a->experts.dtype, a->use_residual ? a->x : nullptr, a->ldx, shared_out,
                        a->expert_out, a->topk_idx, a->slot, a->topk_gate, T, k, E, C, D,
                        a->router.renormalize_kept ? 1 : 0, a->y, s);
}

// ---- backward -----------------------------------------------------------------------
namespace {
// One expert set seen by the backward: routed (rows of expert e are its kept
// assignments, slot_assign order, output gradient gate * dy) or dense (the shared expert:
// all T rows, output gradient dy).
// Kernel names of one set's launches (static storage: the profiler keeps the pointers).
struct BwdNames {
  const char *dh, *recompute_gelu, *recompute_swiglu, *dw_out, *dw_in, *dw_up, *dx;
};
constexpr BwdNames kRoutedNames{"bwd_dh_gemm", "bwd_gelu_recompute", "bwd_swiglu_recompute",
                                "bwd_dw_out_gemm", "bwd_dw_in_gemm", "bwd_dw_up_gemm",
                                "bwd_dx_gemm"};
constexpr BwdNames kSharedNames{"bwd_shared_dh_gemm", "bwd_shared_gelu_recompute",
                                "bwd_shared_swiglu_recompute", "bwd_shared_dw_out_gemm",
                                "bwd_shared_dw_in_gemm", "bwd_shared_dw_up_gemm",
                                "bwd_shared_dx_gemm"};

struct BwdSet {
  const BwdNames* names;
  const moe_experts_t* ex;
  int rows;                  // C (routed) or T (dense)
  const int32_t* row_map;    // slot_assign or NULL
  int row_div;               // k or 1
  const int32_t* count;      // expert_used or NULL (then every group has `cnt_const` rows)
  int cnt_const;
  const float* gate;         // topk_gate or NULL
  float* kpart;              // split-K workspace for constant-K weight gradients, or NULL
  float *dw_in, *dw_up, *dw_out, *db_in, *db_out;
  float *h, *g, *u;          // [E, rows, F] scratch: H, dH -> dZ / dA, dU
  float* dxr;                // [E, rows, D] input gradient of each row
};

struct BwdWs {
  float* eff_gate;           // [T, k] survivor-renormalised gates (renormalize_kept only)
  float* dxe;
  float *h, *g, *u;
  float *sh_h, *sh_g, *sh_u, *sh_dx;
  float* part;
  float* kpart;              // split-K partials of the constant-K weight gradients
  size_t bytes;
};

BwdWs carve_bwd(const moe_backward_args_t* a, void* ws) {
  BwdWs w{};
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t floats) -> float* {
    float* p = base ? reinterpret_cast<float*>(base + off) : nullptr;
    off = align_up(off + floats * 4, 256);
    return p;
  };
  const moe_experts_t& ex = a->experts;
  const size_t E = ex.num_experts, C = a->capacity, D = ex.d_model, F = ex.d_hidden;
  const size_t T = a->T;
  if (a->router.renormalize_kept) w.eff_gate = take(T * size_t(a->k));
  w.dxe = take(E * C * D);
  if (ex.kind != MOE_EXPERT_LINEAR) {
    w.h = take(E * C * F);
    w.g = take(E * C * F);
    if (ex.kind == MOE_EXPERT_SWIGLU) w.u = take(E * C * F);
  }
  if (a->shared.w_in) {
    const size_t Fs = a->shared.d_hidden;
    w.sh_h = take(T * Fs);
    w.sh_g = take(T * Fs);
    w.sh_u = take(T * Fs);
    w.sh_dx = take(T * D);
  }
  if (ex.kind == MOE_EXPERT_GELU_MLP) {
    const size_t pf = colsum_part_floats(int(E), int(C), int(F));
    const size_t pd = colsum_part_floats(int(E), int(C), int(D));
    w.part = take(pf > pd ? pf : pd);
  }
  // the shared expert's and the router's weight gradients reduce over all T rows
  size_t kp = 0;
  if (a->shared.w_in) {
    const int Fs = a->shared.d_hidden;
    kp = std::max(f32_kpart_floats(1, Fs, int(D), int(T)), f32_kpart_floats(1, int(D), Fs, int(T)));
  }
  if (a->w_router) kp = std::max(kp, f32_kpart_floats(1, int(D), int(E), int(T)));
  if (kp) w.kpart = take(kp);
  w.bytes = off + 256;
  return w;
}

// Backward through the MLPs of one expert set: parameter gradients and set.dxr.
moe_status_t mlp_backward(const BwdSet& S, const float* x, const float* dy, int64_t ld,
                          float* part, hipStream_t s) {
  const moe_experts_t* ex = S.ex;
  const int E = ex->num_experts, D = ex->d_model, F = ex->d_hidden, R = S.rows;
  const bool swiglu = ex->kind == MOE_EXPERT_SWIGLU;
  moe_status_t st;

  // dH = dO W_out^T, ungated here (the gate is applied in the recompute epilogue)
  GemmF32Problem p{};
  p.A = dy;
  p.lda = ld;
  p.row_map = S.row_map;
  p.row_map_ld = R;
  p.row_div = S.row_div;
  p.g_count = S.count;
  p.g_const = S.cnt_const;
  p.m_rows = R;
  p.B = static_cast<const float*>(ex->w_out);
  p.ldb = D;
  p.b_gstride = int64_t(F) * D;
  p.K = D;
  p.N = F;
  p.groups = E;
  p.epi = EPI_STORE;
  p.C = S.g;
  p.ldc = F;
  p.c_gstride = int64_t(R) * F;
  const BwdNames& nm = *S.names;
  st = launch_gemm_f32(p, A_ROWS, B_NK, nm.dh, s);
  if (st != MOE_OK) return st;

  // recompute the pre-activation; epilogue writes H and dZ (GELU) or H, dA, dU (SwiGLU)
  p = GemmF32Problem{};
  p.A = x;
  p.lda = ld;
  p.row_map = S.row_map;
  p.row_map_ld = R;
  p.row_div = S.row_div;
  p.g_count = S.count;
  p.g_const = S.cnt_const;
  p.m_rows = R;
  p.B = static_cast<const float*>(ex->w_in);
  p.B1 = swiglu ? static_cast<const float*>(ex->w_up) : nullptr;
  p.ldb = F;
  p.b_gstride = int64_t(D) * F;
  p.gate = S.gate;
  p.bias = swiglu ? nullptr : static_cast<const float*>(ex->b_in);
  p.bias_gstride = F;
  p.K = D;
  p.N = F;
  p.groups = E;
  p.epi = swiglu ? EPI_SWIGLU_BWD : EPI_GELU_BWD;
  p.C = S.h;
  p.G = S.g;
  p.C2 = S.u;
  p.ldc = F;
  p.c_gstride = int64_t(R) * F;
  st = launch_gemm_f32(p, A_ROWS, B_KN, swiglu ? nm.recompute_swiglu : nm.recompute_gelu, s);
  if (st != MOE_OK) return st;

  // dW_out = H^T dO (K = the group's rows; dO rows gathered and gated)
  p = GemmF32Problem{};
  p.A = S.h;
  p.lda = F;
  p.a_gstride = int64_t(R) * F;
  p.row_map_ld = R;
  p.row_div = S.row_div;
  p.g_count = S.count;
  p.g_const = S.cnt_const;
  p.M = F;
  p.m_rows = F;
  p.B = dy;
  p.ldb = ld;
  p.b_row_map = S.row_map;
  p.gate = S.gate;
  p.N = D;
  p.groups = E;
  p.epi = EPI_STORE;
  p.C = S.dw_out;
  p.ldc = D;
  p.c_gstride = int64_t(F) * D;
  p.kpart = S.kpart;
  st = launch_gemm_f32(p, A_KROWS, B_KROWS, nm.dw_out, s);
  if (st != MOE_OK) return st;

  // dW_in = X^T dZ (dA); dW_up = X^T dU
  for (int w = 0; w < (swiglu ? 2 : 1); ++w) {
    p = GemmF32Problem{};
    p.A = x;
    p.lda = ld;
    p.row_map = S.row_map;
    p.row_map_ld = R;
    p.row_div = S.row_div;
    p.g_count = S.count;
    p.g_const = S.cnt_const;
    p.M = D;
    p.m_rows = D;
    p.B = w == 0 ? S.g : S.u;
    p.ldb = F;
    p.b_gstride = int64_t(R) * F;
    p.N = F;
    p.groups = E;
    p.epi = EPI_STORE;
    p.C = w == 0 ? S.dw_in : S.dw_up;
    p.ldc = F;
    p.c_gstride = int64_t(D) * F;
    p.kpart = S.kpart;
    st = launch_gemm_f32(p, A_KROWS, B_KROWS, w == 0 ? nm.dw_in : nm.dw_up, s);
    if (st != MOE_OK) return st;
  }

  if (!swiglu) {
    if (S.db_out) {
      st = launch_colsum(dy, ld, 0, S.row_map, R, S.row_div, S.gate, S.count, S.cnt_const, R, E,
                         D, part, S.db_out, D, s);
      if (st != MOE_OK) return st;
    }
    if (S.db_in) {
      st = launch_colsum(S.g, F, int64_t(R) * F, nullptr, R, 1, nullptr, S.count, S.cnt_const, R,
                         E, F, part, S.db_in, F, s);
      if (st != MOE_OK) return st;
    }
  }

  // input gradient of each row: dZ W_in^T (+ dU W_up^T)
  for (int w = 0; w < (swiglu ? 2 : 1); ++w) {
    p = GemmF32Problem{};
    p.A = w == 0 ? S.g : S.u;
    p.lda = F;
    p.a_gstride = int64_t(R) * F;
    p.row_div = 1;
    p.g_count = S.count;
    p.g_const = S.cnt_const;
    p.m_rows = R;
    p.B = static_cast<const float*>(w == 0 ? ex->w_in : ex->w_up);
    p.ldb = F;
    p.b_gstride = int64_t(D) * F;
    p.K = F;
    p.N = D;
    p.groups = E;
    p.epi = w == 0 ? EPI_STORE : EPI_ACCUM;
    p.C = S.dxr;
    p.ldc = D;
    p.c_gstride = int64_t(R) * D;
    st = launch_gemm_f32(p, A_ROWS, B_NK, nm.dx, s);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status_t check_backward(const moe_backward_args_t* a) {
  if (!a) return MOE_ERR_INVALID_ARG;
  moe_status_t st = check_experts(&a->experts);
  if (st != MOE_OK) return st;
  const moe_experts_t& ex = a->experts;
  if (ex.dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  const int T = a->T, E = ex.num_experts, k = a->k, C = a->capacity;
  const int D = ex.d_model;
  if (!route_shape_ok(T, E, k) || C < 0 || !opts_ok(&a->router)) return MOE_ERR_INVALID_ARG;
  if (k > 256 || int64_t(T) * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!a->dy || !a->x || a->ld < D || !a->logits || !a->topk_idx || !a->topk_gate ||
      !a->expert_count || !a->slot || !a->expert_used || !a->dx || !a->dW || !a->dgate ||
      !a->dlogits || (C > 0 && (!a->slot_assign || !a->expert_out)))
    return MOE_ERR_INVALID_ARG;
  if (ex.kind != MOE_EXPERT_LINEAR && !a->dW_out) return MOE_ERR_INVALID_ARG;
  if (ex.kind == MOE_EXPERT_SWIGLU && !a->dW_up) return MOE_ERR_INVALID_ARG;
  if (ex.kind == MOE_EXPERT_GELU_MLP && ((ex.b_in && !a->db_in) || (ex.b_out && !a->db_out)))
    return MOE_ERR_INVALID_ARG;
  if (a->ld != D) return MOE_ERR_UNSUPPORTED;
  const int per_row = D / 4;
  if ((per_row > 256 && per_row % 256) || (per_row < 256 && 256 % per_row)) return MOE_ERR_UNSUPPORTED;
  if (a->shared.w_in) {
    st = check_experts(&a->shared);
    if (st != MOE_OK) return st;
    if (a->shared.kind != MOE_EXPERT_SWIGLU || a->shared.num_experts != 1 ||
        a->shared.dtype != MOE_F32 || a->shared.d_model != D)
      return MOE_ERR_UNSUPPORTED;
    if (!a->dshared_w_in || !a->dshared_w_up || !a->dshared_w_out) return MOE_ERR_INVALID_ARG;
  }
  if (a->w_router) {
    if (!a->dw_router) return MOE_ERR_INVALID_ARG;
    if (E % 4) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}
}  // namespace

size_t moe_backward_workspace_size(const moe_backward_args_t* a) {
  if (!a || a->T < 1 || a->experts.num_experts < 1 || a->capacity < 0) return 0;
  return carve_bwd(a, nullptr).bytes;
}

moe_status_t moe_backward(const moe_backward_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_backward(a);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < moe_backward_workspace_size(a)) return MOE_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  const moe_experts_t& ex = a->experts;
  const int T = a->T, E = ex.num_experts, k = a->k, C = a->capacity;
  const int D = ex.d_model;
  const float* dy = static_cast<const float*>(a->dy);
  const float* x = static_cast<const float*>(a->x);
  BwdWs w = carve_bwd(a, ws);

  DgateArgs da{};
  da.dy = dy;
  da.o = static_cast<const float*>(a->expert_out);
  da.logits = a->logits;
  da.idx = a->topk_idx;
  da.gate = a->topk_gate;
  da.slot = a->slot;
  da.count = a->expert_count;
  da.T = T;
  da.k = k;
  da.E = E;
  da.C = C;
  da.D = D;
  da.aux_scale = a->aux_grad_scale;
  da.z_scale = a->z_grad_scale;
  da.scoring = a->router.scoring;
  da.renorm = a->router.renormalize_kept ? 1 : 0;
  da.dgate = a->dgate;
  da.dlogits = a->dlogits;
  da.eff_gate = w.eff_gate;
  st = launch_dgate_router_bwd(da, s);
  if (st != MOE_OK) return st;
  // the gates the experts saw in the forward
  const float* gate_eff = w.eff_gate ? w.eff_gate : a->topk_gate;

  // with C == 0 no row is kept: every weight gradient is zero (K = 0 products)
  const int32_t* used = C > 0 ? a->expert_used : nullptr;
  if (ex.kind == MOE_EXPERT_LINEAR) {
    // dX_e = dY_e W_e^T on the slot rows (ungated; the combine below applies the gate)
    GemmF32Problem px{};
    px.A = dy;
    px.lda = a->ld;
    px.row_map = a->slot_assign;
    px.row_map_ld = C;
    px.row_div = k;
    px.g_count = a->expert_used;
    px.m_rows = C;
    px.B = static_cast<const float*>(ex.w_in);
    px.ldb = D;
    px.b_gstride = int64_t(D) * D;
    px.K = D;
    px.N = D;
    px.groups = E;
    px.epi = EPI_STORE;
    px.C = w.dxe;
    px.ldc = D;
    px.c_gstride = int64_t(C) * D;
    if (C > 0) {
      st = launch_gemm_f32(px, A_ROWS, B_NK, "bwd_dx_gemm", s);
      if (st != MOE_OK) return st;
    }
    // dW_e = X_e^T (gate * dY_e), K = used_e gathered rows
    GemmF32Problem pw{};
    pw.A = x;
    pw.lda = a->ld;
    pw.row_map = a->slot_assign;
    pw.row_map_ld = C;
    pw.row_div = k;
    pw.g_count = used;
    pw.g_const = 0;
    pw.M = D;
    pw.m_rows = D;
    pw.B = dy;
    pw.ldb = a->ld;
    pw.b_row_map = a->slot_assign;
    pw.gate = gate_eff;
    pw.N = D;
    pw.groups = E;
    pw.epi = EPI_STORE;
    pw.C = static_cast<float*>(a->dW);
    pw.ldc = D;
    pw.c_gstride = int64_t(D) * D;
    st = launch_gemm_f32(pw, A_KROWS, B_KROWS, "bwd_dw_gemm", s);
    if (st != MOE_OK) return st;
  } else {
    BwdSet r{};
    r.names = &kRoutedNames;
    r.ex = &ex;
    r.rows = C;
    r.row_map = a->slot_assign;
    r.row_div = k;
    r.count = used;
    r.cnt_const = 0;
    r.gate = gate_eff;
    r.dw_in = static_cast<float*>(a->dW);
    r.dw_up = static_cast<float*>(a->dW_up);
    r.dw_out = static_cast<float*>(a->dW_out);
    r.db_in = ex.b_in ? static_cast<float*>(a->db_in) : nullptr;
    r.db_out = ex.b_out ? static_cast<float*>(a->db_out) : nullptr;
    r.h = w.h;
    r.g = w.g;
    r.u = w.u;
    r.dxr = w.dxe;
    st = mlp_backward(r, x, dy, a->ld, w.part, s);
    if (st != MOE_OK) return st;
  }

  if (a->shared.w_in) {
    BwdSet sh{};
    sh.names = &kSharedNames;
    sh.ex = &a->shared;
    sh.rows = T;
    sh.row_div = 1;
    sh.cnt_const = T;
    sh.dw_in = static_cast<float*>(a->dshared_w_in);
    sh.dw_up = static_cast<float*>(a->dshared_w_up);
    sh.dw_out = static_cast<float*>(a->dshared_w_out);
    sh.h = w.sh_h;
    sh.g = w.sh_g;
    sh.u = w.sh_u;
    sh.dxr = w.sh_dx;
    sh.kpart = w.kpart;
    st = mlp_backward(sh, x, dy, a->ld, nullptr, s);
    if (st != MOE_OK) return st;
  }

  // dx = r dy + shared input gradient + sum over kept choices of the routed rows'
  // input gradients (gated here for single-linear experts, already gated for MLPs)
  st = launch_combine(MOE_F32, a->use_residual ? a->dy : nullptr, a->ld, w.sh_dx, w.dxe,
                      a->topk_idx, a->slot, ex.kind == MOE_EXPERT_LINEAR ? gate_eff : nullptr,
                      T, k, E, C, D, 0, a->dx, s);
  if (st != MOE_OK) return st;

  if (a->w_router) {
    // dW_r = x^T dlogits
    GemmF32Problem pr{};
    pr.A = x;
    pr.lda = a->ld;
    pr.row_div = 1;
    pr.g_const = T;
    pr.M = D;
    pr.m_rows = D;
    pr.B = a->dlogits;
    pr.ldb = E;
    pr.N = E;
    pr.groups = 1;
    pr.epi = EPI_STORE;
    pr.C = static_cast<float*>(a->dw_router);
    pr.ldc = E;
    pr.kpart = w.kpart;
    st = launch_gemm_f32(pr, A_KROWS, B_KROWS, "bwd_dw_router_gemm", s);
    if (st != MOE_OK) return st;
    // dx += dlogits W_r^T
    GemmF32Problem pd{};
    pd.A = a->dlogits;
    pd.lda = E;
    pd.row_div = 1;
    pd.g_const = T;
    pd.m_rows = T;
    pd.B = static_cast<const float*>(a->w_router);
    pd.ldb = E;
    pd.K = E;
    pd.N = D;
    pd.groups = 1;
    pd.epi = EPI_ACCUM;
    pd.C = static_cast<float*>(a->dx);
    pd.ldc = D;
    st = launch_gemm_f32(pd, A_ROWS, B_NK, "bwd_dx_router_gemm", s);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

// ---- errors and profiling -------------------------------------------------------------
int32_t moe_read_error(const void* ws, void* stream) {
  if (!ws) return -1;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, S(stream)) != hipSuccess) return -1;
  if (hipStreamSynchronize(S(stream)) != hipSuccess) return -1;
  return v;
}

void moe_profile_enable(int32_t on) { g_prof = on != 0; }

int32_t moe_profile_read(char* names, int32_t name_stride, int32_t* counts, double* total_ms,
                         int32_t max_entries) {
  std::vector<std::string> order;
  std::map<std::string, std::pair<int, double>> acc;
  for (auto& r : g_recs) {
    float ms = 0.f;
    (void)hipEventSynchronize(r.stop);
    (void)hipEventElapsedTime(&ms, r.start, r.stop);
    auto it = acc.find(r.name);
    if (it == acc.end()) {
      order.push_back(r.name);
      acc[r.name] = {1, double(ms)};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  int n = 0;
  for (auto& nm : order) {
    if (n >= max_entries) break;
    if (names && name_stride > 0) {
      std::strncpy(names + size_t(n) * name_stride, nm.c_str(), name_stride - 1);
      names[size_t(n) * name_stride + name_stride - 1] = 0;
    }
    if (counts) counts[n] = acc[nm].first;
    if (total_ms) total_ms[n] = acc[nm].second;
    ++n;
  }
  return n;
}

}  // extern "C"
