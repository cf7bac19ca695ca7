// Internal launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.h"

namespace moe {

// ---- routing / dispatch ---------------------------------------------------------
// Tokens per routing block. The per-block partial counts and probability sums are
// stored block-major, [nb][E], nb = ceil(T / kRouteTokens).
constexpr int kRouteTokens = 32;
inline int route_blocks(int T) { return (T + kRouteTokens - 1) / kRouteTokens; }
// Routing blocks per scan chunk (the first level of the two-level offset scan).
constexpr int kScanRows = 16;
inline int scan_chunks(int T) { return (route_blocks(T) + kScanRows - 1) / kScanRows; }
// Routing blocks per dispatch (slot assignment) block.
inline int assign_group(int k) {
  int g = 512 / (kRouteTokens * k);
  return g < 1 ? 1 : g;
}

// Workspace carve-up shared by route and dispatch.
struct RouteWs {
  int32_t* flags;      // [0] error word
  int32_t* cnt_part;   // [nb][E]
  float* prob_part;    // [nb][E]
  int32_t* chunk_cnt;  // [nc][E] counts per chunk of kScanRows routing blocks
  float* chunk_prob;   // [nc][E]
  int32_t* chunk_off;  // [nc][E] exclusive offsets of the chunks
  float* fp;           // [E] f_e * P_e
  float* zpart;        // [nb] per routing block, sum of lse_t^2 over its tokens
  size_t bytes;
};

// Router variants seen by the routing kernel (moe_router_opts_t, device side).
struct RouteOpts {
  int32_t scoring;       // MOE_SCORE_SOFTMAX / MOE_SCORE_SIGMOID
  const float* bias;     // [E] selection bias or NULL
  int32_t with_z;        // 1: write the per-block z partials
};
RouteWs carve_route_ws(void* ws, int T, int E);

moe_status_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                          const RouteOpts& o, const RouteWs& w, hipStream_t s);
moe_status_t launch_count(const int32_t* idx, int T, int k, int E, const RouteWs& w,
                          hipStream_t s);
// Optional per-expert load statistics written by the scan: token_fraction = count / T,
// probability_mass = prob_sum / T (each may be NULL).
struct LoadStats {
  float* token_fraction;
  float* probability_mass;
};
// with_prob: prob_part is valid (computes prob_sum and aux); C < 0: routing only;
// z_loss != NULL: zpart is valid, z_loss = sum of zpart / T.
moe_status_t launch_reduce_scan(int T, int k, int E, int C, bool with_prob, int32_t* count,
                                float* prob_sum, float* aux, int32_t* used, int32_t* overflow,
                                int32_t* slot_assign, float* z_loss, const LoadStats& ls,
                                const RouteWs& w, hipStream_t s);
// `used` (from launch_reduce_scan) also drives the -1 fill of unfilled slots.
moe_status_t launch_assign(const int32_t* idx, int T, int k, int E, int C, int32_t* slot,
                           uint8_t* kept, int32_t* slot_assign, int32_t* drops,
                           const int32_t* used, const RouteWs& w, hipStream_t s);
// The scan (launch_reduce_scan's outputs) and the slot assignment after routing or
// counting. With E <= 256 and at most kFusedScanEntries chunk sums the scan runs inside
// the assignment launch (chunk sums, then one kernel); otherwise as three launches.
constexpr int64_t kFusedScanEntries = 16384;
moe_status_t launch_dispatch(const int32_t* idx, int T, int k, int E, int C, bool with_prob,
                             int32_t* count, float* prob_sum, float* aux, int32_t* used,
                             int32_t* overflow, float* z_loss, const LoadStats& ls,
                             int32_t* slot, uint8_t* kept, int32_t* slot_assign, int32_t* drops,
                             const RouteWs& w, hipStream_t s);

// ---- grouped GEMMs ----------------------------------------------------------------
enum Epi : int32_t {
  EPI_STORE = 0,      // C = acc (output dtype of the kernel)
  EPI_BIAS = 1,       // C = acc + bias[n]
  EPI_GELU_BIAS = 2,  // C = gelu(acc + bias[n]) (bias may be NULL)
  EPI_SWIGLU = 3,     // C = silu(acc_gate) * acc_up
  EPI_SCALE_ROW = 4   // C = acc * rowscale (unused)
};

// One grouped problem: for group g and row r < M_g, C[g, r, :] = A_row(g, r) . B[g].
// A_row(g, r) = A + g*a_gstride + src*lda, src = row_map ? row_map[g*row_map_ld + r] /
// row_div : r. M_g = m_count ? m_count[g] : m_const. B[g] = B + g*b_gstride, [K][N].
struct GemmProblem {
  const void* A;
  int64_t lda;
  int64_t a_gstride;
  const int32_t* row_map;
  int32_t row_map_ld;
  int32_t row_div;
  const int32_t* m_count;
  int32_t m_const;
  int32_t m_tiles_rows;  // upper bound of rows per group (C, or T when dense)
  int32_t m_tiles;       // filled by the launcher for its tile height
  const void* B0;
  const void* B1;  // SwiGLU up projection (gated kernel only)
  int64_t b_gstride;
  const void* bias;
  int64_t bias_gstride;
  void* C;
  int64_t ldc;
  int64_t c_gstride;
  int32_t K;
  int32_t N;
  int32_t n_tiles;
  int32_t groups;
  int32_t epi;
  int32_t out_f32;  // bf16 kernel: 1 = store fp32 (router logits)
  int32_t tiles;    // groups * m_tiles * n_tiles (filled by the launcher)
  int32_t b_kmajor; // bf16 kernel: B stored [N][K] per group (k contiguous), else [K][N]
  // bf16 kernel: A (a_pstride) or C (c_pstride) stored in 32-column pieces when nonzero,
  // element (r, c) of group g at g*gstride + (c / 32)*pstride + r*32 + c % 32, pstride =
  // 32 * rows of the group's buffer (lda / ldc unused). The hidden activation between the
  // two expert GEMMs when it stays inside the library: a 32-column output strip of a wave
  // then fills whole 128-byte lines, two rows each, and the next GEMM still reads whole
  // lines per K step.
  int64_t a_pstride;
  int64_t c_pstride;
};

struct GemmBatch {
  GemmProblem p[2];
  int32_t nprob;
  int32_t total;
  int32_t chunk;     // tiles per chunk dealt to one XCD (one group's tiles of problem 0)
  int32_t xcd_max;   // most tiles any XCD receives
  int32_t list_cap;  // persistent kernel: entries of a block's tile list (LDS)
};

constexpr int kBf16BM = 128, kBf16BN = 128, kBf16BK = 64;
moe_status_t launch_gemm_bf16(GemmBatch& b, bool gated, const char* name, hipStream_t s);

// fp32 grouped GEMM (fp32 MFMA). Modes select the operand layouts.
// Every operand row is addressed as X + g*x_gstride + src*ldx, where src is the row's
// index or, with a row map, map[g*row_map_ld + i] / row_div (callers pass gstride 0
// with a map: the map then indexes one shared tensor).
//   A_ROWS : row r < M_g of C[g] is the product of A row r (mapped by row_map); K = P.K.
//   A_KROWS: the K index walks rows of A (an A^T operand), mapped by row_map;
//            M = P.M columns of A; K_g = g_count ? g_count[g] : g_const.
//   B_KN   : B[g] = B + g*b_gstride, [K][N] (N contiguous); B1 likewise (gated kernels).
//   B_NK   : B[g] = B + g*b_gstride, [N][K] (K contiguous): C = A B^T.
//   B_KROWS: the K index walks rows of B, mapped by b_row_map; a mapped row a is scaled
//            by gate[a] when gate != NULL.
enum AMode : int32_t { A_ROWS = 0, A_KROWS = 1 };
enum BMode : int32_t { B_KN = 0, B_NK = 1, B_KROWS = 2 };
// Epilogues of the fp32 kernel beyond those of the bf16 one. With an A_ROWS row map,
// rgate(m) = gate[row_map[g*row_map_ld + m]], else 1.
//   EPI_ACCUM      : C += acc
//   EPI_GELU_BWD   : z = acc + bias; dh = G * rgate(m); C = gelu(z); G = dh * gelu'(z)
//   EPI_SWIGLU_BWD : a = acc (B), u = acc1 (B1); dh = G * rgate(m); C = silu(a) u;
//                    G = dh u silu'(a); C2 = dh silu(a)
constexpr int32_t EPI_ACCUM = 5, EPI_GELU_BWD = 6, EPI_SWIGLU_BWD = 7;
struct GemmF32Problem {
  const float* A;
  int64_t lda;
  int64_t a_gstride;
  const int32_t* row_map;   // A_ROWS: maps M rows; A_KROWS: maps K rows; NULL: identity
  int32_t row_map_ld;
  int32_t row_div;
  const int32_t* g_count;   // A_ROWS: M per group; A_KROWS: K per group (NULL: g_const)
  int32_t g_const;
  int32_t M;                // A_KROWS: fixed M
  int32_t m_rows;           // rows to tile: A_ROWS the most rows of any group, A_KROWS M
  int32_t m_tiles;          // filled by the launcher for its tile height
  const float* B;
  const float* B1;          // gated kernels: second weight (the SwiGLU up projection)
  int64_t ldb;
  int64_t b_gstride;
  const int32_t* b_row_map; // B_KROWS: maps K rows (shares row_map_ld / row_div); NULL: identity
  const float* gate;        // B_KROWS: row scales by assignment; *_BWD: rgate source
  const float* bias;
  int64_t bias_gstride;
  float* C;
  int64_t ldc;
  int64_t c_gstride;
  float* G;                 // *_BWD: incoming dH, overwritten (layout of C)
  float* C2;                // EPI_SWIGLU_BWD: dU (layout of C)
  int32_t K;                // A_ROWS: inner size
  int32_t N;
  int32_t n_tiles;
  int32_t groups;
  int32_t epi;
  int32_t tiles;
  // A_KROWS with a constant K (g_count NULL), EPI_STORE and C dense ([groups][M][N]):
  // when the output has too few tiles to fill the GPU, the launcher splits K into
  // k_splits ranges of k_chunk rows, each writing a partial to kpart, and sums them in a
  // fixed order into C. kpart (caller-owned, >= f32_kpart_floats(...) floats) may be
  // NULL, which disables the split. k_splits and k_chunk are filled by the launcher.
  float* kpart;
  int32_t k_splits;
  int32_t k_chunk;
};
moe_status_t launch_gemm_f32(GemmF32Problem& p, int amode, int bmode, const char* name,
                             hipStream_t s);
// Floats of kpart that launch_gemm_f32 uses for a constant-K A_KROWS product of this
// shape (0 if it does not split it).
size_t f32_kpart_floats(int groups, int M, int N, int K);
// Column sums per group: out[g*out_gstride + n] = sum over rows r < M_g (in row order,
// fixed chunking) of scale(r) * row(r)[n], rows addressed like B_KROWS (map / identity,
// gate). Deterministic. part: >= colsum_part_floats(groups, max_rows, N) floats.
size_t colsum_part_floats(int groups, int max_rows, int N);
moe_status_t launch_colsum(const float* src, int64_t ld, int64_t gstride, const int32_t* map,
                           int32_t map_ld, int32_t div, const float* gate,
                           const int32_t* g_count, int32_t g_const, int max_rows, int groups,
                           int N, float* part, float* out, int64_t out_gstride, hipStream_t s);

// Plain SIMT router GEMM for shapes the MFMA kernels do not tile (any E).
moe_status_t launch_router_simt(const void* x, int dtype, int64_t ldx, const void* w, int T,
                                int D, int E, float* logits, hipStream_t s);

// ---- combine / backward --------------------------------------------------------------
moe_status_t launch_combine(int dt, const void* residual, int64_t ldr, const void* shared_out,
                            const void* expert_out, const int32_t* idx, const int32_t* slot,
                            const float* gate, int T, int k, int E, int C, int D, int renorm,
                            void* y, hipStream_t s);
struct DgateArgs {
  const float* dy;
  const float* o;          // [E, C, D] expert outputs (ungated)
  const float* logits;
  const int32_t* idx;
  const float* gate;       // topk_gate
  const int32_t* slot;
  const int32_t* count;
  int T, k, E, C, D;
  float aux_scale;
  float z_scale;
  int scoring;
  int renorm;
  float* dgate;
  float* dlogits;
  float* eff_gate;         // [T, k] effective gates (written when non-NULL)
};
moe_status_t launch_dgate_router_bwd(const DgateArgs& a, hipStream_t s);

}  // namespace moe
