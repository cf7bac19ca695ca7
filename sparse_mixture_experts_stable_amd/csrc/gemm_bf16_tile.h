// Pieces shared by the grouped bf16 GEMM kernels: the tile configuration, the LDS
// layouts and their swizzles, the DMA requests that fill one LDS stage, the decoding of
// a block's tile, and the epilogue.
//
// LDS stage layout (one K step of BK = 64 or 32):
//   A (expert rows, k contiguous) is stored [m][k], 2 BK bytes per row (128 or 64), and
//   read as one 16-byte fragment per lane. Each lane fetches source chunk c ^ f(m), with
//   f(m) = m % 8 for 128-byte rows and (m / 4) % 4 for 64-byte rows, so that the lanes
//   of a fragment read hit distinct bank groups.
//   B (weights, n contiguous: [k][n] per expert, as stored) is copied unchanged apart
//   from a per-row XOR of the 16-byte chunk index (hswz); the k-major fragment each MFMA
//   needs is assembled with two ds_read_b64_tr_b16 transpose reads. Within a 16-lane
//   group that instruction hands lane l element l % 4 of the 8-byte pieces addressed by
//   lanes l/4 + 4v (v = 0..3), so lane s of group g points at row 8g + (s%16)/4 (+4 for
//   the second read) and column 4 (s % 4) of its 16-column slice.
//   B stored [n][k] (k contiguous, BKM) is laid out and read like A instead.
// Both operands move HBM -> LDS with global_load_lds_dwordx4: one instruction moves
// 1 KiB (64 lanes x 16 bytes) to a contiguous LDS range.
#pragma once

#include "internal.h"

namespace moe {
namespace tile {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// k-contiguous rows of RB bytes (A, and B in the OUT_IN layout): chunk c of row m sits at
// c ^ fswz(m). 128-byte rows: m % 8 (measured on gfx950 with the LDS bank-conflict
// counter: conflict-free for the 16-row fragment reads, where c ^ ((m ^ m/8) % 8) is
// not). 64-byte rows: (m / 4) % 4, which gives the 16 rows of a fragment read 16
// distinct 16-byte bank groups (rows m and m + 4 share the byte offset m % 4 * 64 of a
// 256-byte bank line, and the swizzle separates them).
template <int RB>
__device__ __forceinline__ int fswz(int m) {
  static_assert(RB == 128 || RB == 64, "k-contiguous row of 64 or 32 bf16");
  if constexpr (RB == 128) return m & 7;
  return (m >> 2) & 3;
}
// B rows: the 16-byte chunk index is XORed with an even value that differs for the four
// rows one 16-lane group reads together and, in addition, between groups 0 and 1 (rows
// k and k + 8), so that both 16 and 32 lanes per LDS cycle are conflict free.
template <int RB>
__device__ __forceinline__ int hswz(int k) {
  if constexpr (RB == 128) return ((k ^ (k >> 3)) & 3) << 1;
  return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
}

// Tiles are dealt to the 8 XCDs in chunks of `chunk` consecutive logical tiles (one
// group's tiles, which share weight panels): chunk c goes to XCD c % 8. The hardware
// dispatches workgroup h to XCD h % 8, so the j-th tile of XCD x is taken by a block
// with h % 8 == x. This keeps the tiles of one expert in one XCD's L2 and spreads
// busy and empty groups evenly over the XCDs. Returns -1 past the end of XCD x's list.
__device__ __forceinline__ int xcd_tile(int total, int chunk, int x, int j) {
  const int c = x + 8 * (j / chunk);
  const int t = c * chunk + (j % chunk);
  return t < total ? t : -1;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt with the vector-memory and LDS counters both at zero.
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8));
}

template <int BM_, int BNE_, bool GATED_, int WGM_ = 2, int WGN_ = 2, int STAGES_ = 3,
          int BK_ = 64>
struct TileCfg {
  static constexpr int STAGES = STAGES_;           // LDS ring depth
  static constexpr int BK = BK_;                   // K per step (64 or 32)
  static constexpr int K_RB = BK * 2;              // bytes per k-contiguous LDS row
  static constexpr int K_RPI = 1024 / K_RB;        // such rows per 1 KiB DMA load
  static constexpr int K_CPR = K_RB / 16;          // 16-byte chunks per such row
  static constexpr int BM = BM_;                 // rows per block
  static constexpr int BNE = BNE_;               // B columns staged per step (all matrices)
  static constexpr bool GATED = GATED_;
  static constexpr int WGM = WGM_, WGN = WGN_;   // wave grid (rows x columns)
  static constexpr int WAVES = WGM * WGN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NB = GATED ? 2 : 1;       // B matrices
  static constexpr int BNQ = BNE / NB;           // columns per B matrix = output columns
  static constexpr int WROWS = BM / WGM;         // rows per wave
  static constexpr int WCOLS = BNQ / WGN;        // output columns per wave
  static constexpr int TM = WROWS / 16;          // MFMA tiles per wave, rows
  static constexpr int TN = WCOLS / 16;          // MFMA tiles per wave, columns per matrix
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int BQ_BYTES = BK * BNQ * 2;  // one B matrix
  static constexpr int STAGE = A_BYTES + NB * BQ_BYTES;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int A_INST = BM / K_RPI / WAVES;  // 1 KiB DMA loads of A per wave per step
  static constexpr int B_RB = BNQ * 2;           // bytes per B row
  static constexpr int B_RPI = 1024 / B_RB;      // B rows per 1 KiB load
  static constexpr int B_IPQ = BK / B_RPI;       // loads per B matrix per step
  static constexpr int B_INST = NB * B_IPQ / WAVES;  // per wave per step
  static constexpr int LOADS = A_INST + B_INST;  // vector-memory ops per thread per step
  static_assert(BM % (K_RPI * WAVES) == 0, "A loads split evenly over the waves");
  static_assert(NB * B_IPQ % WAVES == 0, "B loads split evenly over the waves");
};

// DMA sources of a tile: uniform group bases (scalar registers) and this lane's byte
// offsets from them.
template <class CF>
struct DmaSrc {
  const char* a;              // A of the group (uniform)
  const char* b[CF::NB];      // B matrices of the group (uniform)
  uint32_t ka_step;           // bytes from one K step of A to the next (uniform)
  uint32_t ao[CF::A_INST];    // per lane: gathered row and swizzled chunk
  uint32_t bo[CF::B_INST];    // per lane: k row and swizzled chunk
};

// Requests the A tile of step kt into `dst` (one 1 KiB DMA per instruction). `wv` is
// the wave index (uniform).
template <class CF>
__device__ __forceinline__ void issue_a(char* __restrict__ dst, const DmaSrc<CF>& S, int kt, int wv) {
  const size_t ka = size_t(kt) * S.ka_step;
#pragma unroll
  for (int t = 0; t < CF::A_INST; ++t) {
    const char* g = S.a + ka + S.ao[t];
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(dst + (wv * CF::A_INST + t) * 1024), 16, 0, 0);
  }
}

// Requests the B tiles of step kt into `dst` (matrix q at q * BQ_BYTES). BKM: B is stored
// [N][K] (k contiguous, like A).
template <class CF, bool BKM = false>
__device__ __forceinline__ void issue_b(char* __restrict__ dst, const DmaSrc<CF>& S, int kt, int N,
                                        int wv) {
  const size_t kb = BKM ? size_t(kt) * CF::BK * 2 : size_t(kt) * CF::BK * size_t(N) * 2;
#pragma unroll
  for (int t = 0; t < CF::B_INST; ++t) {
    const int u = wv * CF::B_INST + t;
    const char* bq = (CF::NB > 1 && u / CF::B_IPQ) ? S.b[CF::NB - 1] : S.b[0];
    const char* g = bq + kb + S.bo[t];
    __builtin_amdgcn_global_load_lds(
        g, (lds_void*)(dst + (u / CF::B_IPQ) * CF::BQ_BYTES + (u % CF::B_IPQ) * 1024), 16, 0, 0);
  }
}

// Requests the tiles of step kt into the LDS stage `dst`: A, then B at A_BYTES.
template <class CF, bool BKM = false>
__device__ __forceinline__ void issue_stage(char* __restrict__ dst, const DmaSrc<CF>& S, int kt,
                                            int N, int wv) {
  issue_a<CF>(dst, S, kt, wv);
  issue_b<CF, BKM>(dst + CF::A_BYTES, S, kt, N, wv);
}

// A tile of a grouped batch: problem, group (expert), first row and column, row count.
struct TileId {
  int pi, g, m0, n0, M;
};

// Decodes logical tile id `lid`: problems in order, then groups, then column tiles, then
// row tiles (consecutive ids share a weight panel). M (the group's row count) is left at
// 0: group_rows reads it.
template <class CF>
__device__ __forceinline__ TileId decode_tile_id(const GemmBatch& batch, int lid) {
  TileId t;
  t.pi = (batch.nprob > 1 && lid >= batch.p[0].tiles) ? 1 : 0;
  const GemmProblem& P = batch.p[t.pi];
  int rem = t.pi ? lid - batch.p[0].tiles : lid;
  const int per_group = P.m_tiles * P.n_tiles;
  t.g = rem / per_group;
  rem -= t.g * per_group;
  const int nt = rem / P.m_tiles;
  const int mt = rem - nt * P.m_tiles;
  t.M = 0;
  t.m0 = mt * CF::BM;
  t.n0 = nt * CF::BNQ;
  return t;
}

// The row count of tile t's group (a load when the problem has per-group counts).
__device__ __forceinline__ int group_rows(const GemmProblem& P, const TileId& t) {
  return P.m_count ? P.m_count[t.g] : P.m_const;
}
// The same as a scalar load (t uniform; the counts are only read during the kernel).
__device__ __forceinline__ int group_rows_scalar(const GemmProblem& P, const TileId& t) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  return P.m_count ? ((cptr)P.m_count)[t.g] : P.m_const;
}

// decode_tile_id with M. The same value in every lane: keep it (and all tile bookkeeping)
// in scalar registers.
template <class CF>
__device__ __forceinline__ TileId decode_tile(const GemmBatch& batch, int lid) {
  TileId t = decode_tile_id<CF>(batch, lid);
  t.M = __builtin_amdgcn_readfirstlane(group_rows(batch.p[t.pi], t));
  return t;
}

// Whether logical tile `lid` holds rows (its first row is below the group's row count),
// evaluated per lane: lanes may look at different tiles and problems.
template <class CF>
__device__ __forceinline__ bool tile_nonempty(const GemmBatch& batch, int lid) {
  const bool second = batch.nprob > 1 && lid >= batch.p[0].tiles;
  const int rem = second ? lid - batch.p[0].tiles : lid;
  const int mtiles = second ? batch.p[1].m_tiles : batch.p[0].m_tiles;
  const int ntiles = second ? batch.p[1].n_tiles : batch.p[0].n_tiles;
  const int32_t* cnt = second ? batch.p[1].m_count : batch.p[0].m_count;
  const int mconst = second ? batch.p[1].m_const : batch.p[0].m_const;
  const int per_group = mtiles * ntiles;
  const int g = rem / per_group;
  const int mt = (rem - g * per_group) % mtiles;
  const int M = cnt ? cnt[g] : mconst;
  return mt * CF::BM < M;
}

// The A source row of DMA load i of this lane for tile t: load i of wave wv fills LDS
// rows (wv*A_INST + i)*K_RPI .. +K_RPI, this lane row (lane / K_CPR); rows past M repeat
// row m0 (never stored); with a row map the row is the gathered token (or slot) row.
template <class CF>
__device__ __forceinline__ int tile_a_row(const GemmProblem& P, const TileId& t, int wv, int lane,
                                          int i) {
  const int row = (wv * CF::A_INST + i) * CF::K_RPI + lane / CF::K_CPR;
  int r = t.m0 + row;
  if (r >= t.M) r = t.m0;
  return P.row_map ? P.row_map[size_t(t.g) * P.row_map_ld + r] / P.row_div : r;
}

// The row map entries of the A rows that wave wv stages for tile t, read with scalar
// loads (the same for every lane; the map is only read during the kernel): rows
// m0 + NR*wv .. +NR, NR = A_INST * K_RPI, or the last NR rows of the group's map when
// that window runs past it (those rows are past M). `first` is the row of e[0]. Without
// a map nothing is read.
template <class CF>
struct WaveRows {
  static constexpr int NR = CF::A_INST * CF::K_RPI;
  int e[NR];
  int first;
};

template <class CF>
__device__ __forceinline__ void wave_row_entries(const GemmProblem& P, const TileId& t, int wv,
                                                 WaveRows<CF>& w) {
  constexpr int NR = WaveRows<CF>::NR;
  const int r0 = t.m0 + wv * NR;
  w.first = r0;
  if (!P.row_map) return;
  const int last = P.row_map_ld - NR;  // row_map_ld >= NR (checked on the host)
  if (r0 > last) w.first = last;
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  const cptr p = (cptr)(P.row_map + size_t(t.g) * P.row_map_ld + w.first);
#pragma unroll
  for (int j = 0; j < NR; ++j) w.e[j] = p[j];
}

// The source row of DMA load i of this lane from those entries: as tile_a_row, except
// that gathered rows past M read row 0 (never stored either way).
template <class CF>
__device__ __forceinline__ int a_row_from_entries(const GemmProblem& P, const TileId& t, int wv,
                                                  int lane, int i, const WaveRows<CF>& w) {
  const int r = t.m0 + (wv * CF::A_INST + i) * CF::K_RPI + lane / CF::K_CPR;
  if (!P.row_map) return r < t.M ? r : t.m0;
  const int j = r - w.first;  // in [0, NR) for every row below M
  int e = 0;
#pragma unroll
  for (int q = 0; q < WaveRows<CF>::NR; ++q) e = j == q ? w.e[q] : e;
  return r < t.M ? e / P.row_div : 0;
}

// DMA sources of tile t from the A rows of tile_a_row. A: this lane's physical chunk
// p = lane % K_CPR holds source chunk p ^ f(row). B: load i of wave wv is load
// u = wv*B_INST + i overall: matrix u / B_IPQ, rows (u % B_IPQ) * B_RPI .. +B_RPI;
// columns past N read column 0 (never stored). BKM (B stored [N][K]): B is staged like
// A, [n][k] with K_RB-byte rows and the same chunk swizzle; load u covers the K_RPI rows
// (u % B_IPQ) * K_RPI .. +K_RPI of its matrix, and rows past N read row 0.
template <class CF>
__device__ __forceinline__ void tile_a_sources(const GemmProblem& P, const TileId& t, int wv, int lane,
                                               const int* rows, DmaSrc<CF>& S) {
  S.a = static_cast<const char*>(P.A) + size_t(t.g) * P.a_gstride * 2;
  const int64_t ps = P.a_pstride;
  S.ka_step = ps ? uint32_t(ps * (CF::BK / 32) * 2) : uint32_t(CF::BK * 2);
#pragma unroll
  for (int i = 0; i < CF::A_INST; ++i) {
    const int row = (wv * CF::A_INST + i) * CF::K_RPI + lane / CF::K_CPR;
    const int c = (lane % CF::K_CPR) ^ fswz<CF::K_RB>(row);  // source chunk of 8 columns
    S.ao[i] = ps ? uint32_t((size_t(c >> 2) * ps + size_t(rows[i]) * 32 + 8 * (c & 3)) * 2)
                 : uint32_t((size_t(rows[i]) * P.lda + 8 * c) * 2);
  }
}

template <class CF, bool BKM = false>
__device__ __forceinline__ void tile_b_sources(const GemmProblem& P, const TileId& t, int wv, int lane,
                                               DmaSrc<CF>& S) {
  S.b[0] = static_cast<const char*>(P.B0) + size_t(t.g) * P.b_gstride * 2;
  if constexpr (CF::NB > 1) S.b[CF::NB - 1] = static_cast<const char*>(P.B1) + size_t(t.g) * P.b_gstride * 2;
  if constexpr (BKM) {
    static_assert(CF::B_IPQ * CF::K_RPI == CF::BNQ, "one 1 KiB load per K_RPI rows");
#pragma unroll
    for (int i = 0; i < CF::B_INST; ++i) {
      const int u = wv * CF::B_INST + i;
      const int nl = (u % CF::B_IPQ) * CF::K_RPI + lane / CF::K_CPR;
      int n = t.n0 + nl;
      if (n >= P.N) n = 0;
      S.bo[i] = uint32_t((size_t(n) * P.K + 8 * ((lane % CF::K_CPR) ^ fswz<CF::K_RB>(nl))) * 2);
    }
  } else {
    constexpr int CPR = CF::B_RB / 16;  // chunks per row
#pragma unroll
    for (int i = 0; i < CF::B_INST; ++i) {
      const int u = wv * CF::B_INST + i;
      const int k = (u % CF::B_IPQ) * CF::B_RPI + lane / CPR;
      const int c = (lane % CPR) ^ hswz<CF::B_RB>(k);
      int col = t.n0 + 8 * c;
      if (col >= P.N) col = 0;
      S.bo[i] = uint32_t((size_t(k) * P.N + col) * 2);
    }
  }
}

template <class CF, bool BKM = false>
__device__ __forceinline__ void tile_sources_from_rows(const GemmProblem& P, const TileId& t,
                                                       int wv, int lane, const int* rows,
                                                       DmaSrc<CF>& S) {
  tile_a_sources<CF>(P, t, wv, lane, rows, S);
  tile_b_sources<CF, BKM>(P, t, wv, lane, S);
}

template <class CF, bool BKM = false>
__device__ __forceinline__ void tile_sources(const GemmProblem& P, const TileId& t, int wv,
                                             int lane, DmaSrc<CF>& S) {
  int rows[CF::A_INST];
#pragma unroll
  for (int i = 0; i < CF::A_INST; ++i) rows[i] = tile_a_row<CF>(P, t, wv, lane, i);
  tile_sources_from_rows<CF, BKM>(P, t, wv, lane, rows, S);
}

// fp32 epilogue (the router logits, EPI_STORE): lane holds C[m][n..n+3] of every MFMA
// tile (the MFMA ran with B as its first operand, so each tile comes out transposed),
// stored as 16 bytes per lane.
template <class CF>
__device__ __forceinline__ void store_tile_f32(const GemmProblem& P, const TileId& t, int wm,
                                               int wn, int lane,
                                               const f32x4 (&acc)[CF::NB][CF::TM][CF::TN]) {
  static_assert(!CF::GATED, "plain products only");
  const int fr = lane & 15, fc = lane >> 4;
  char* Cb = static_cast<char*>(P.C);
#pragma unroll
  for (int i = 0; i < CF::TM; ++i) {
    const int m = t.m0 + wm * CF::WROWS + i * 16 + fr;
    if (m >= t.M) continue;
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) {
      const int n = t.n0 + wn * CF::WCOLS + j * 16 + fc * 4;
      if (n >= P.N) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[0][i][j][r];
      char* dst = Cb + (size_t(t.g) * P.c_gstride + size_t(m) * P.ldc + n) * 4;
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Epilogue of a bf16 tile without LDS staging: 16-byte stores straight from registers,
// after the epilogue math (bias from `sbias`, the block's BNQ columns staged in LDS as
// fp32 with zeros past N; GELU; SwiGLU). After the MFMAs lane (r, g) (r = lane % 16,
// g = lane / 16) holds columns 16 j + 4 g .. + 3 of row r of every 16 x 16 tile j. For a
// pair of tiles j0 = 2 p, j1 = j0 + 1 one v_permlane16_swap per dword exchanges the odd
// 16-lane groups' j0 pieces with the even groups' j1 pieces, after which lane (r, g) holds
// the 8 consecutive columns 16 (j0 + g % 2) + 8 (g / 2) .. + 7 of row r: one 16-byte
// chunk per pair. With two pairs (64 columns per wave) lanes r and r + 8 then trade one
// chunk (a DPP rotation by 8 within each 16-lane row), so that each store instruction
// covers 8 whole 128-byte rows rather than 16 half rows. Every lane takes part in the
// exchanges (they read other lanes); stores past M or N are skipped. NT: non-temporal
// stores (an output read once, later, by a streaming kernel). With C in 32-column pieces
// (c_pstride) the same chunks land in that layout: the 16 rows of one 32-column strip
// are then 1 KiB of contiguous memory, one store instruction.
template <class CF, int EPI, bool NT>
__device__ __forceinline__ void store_tile_swapped(const GemmProblem& P, const TileId& t, int wm,
                                                   int wn, int lane, const float* sbias,
                                                   const f32x4 (&acc)[CF::NB][CF::TM][CF::TN]) {
  static_assert(CF::TN == 2 || CF::TN == 4, "one or two pairs of tiles");
  constexpr int NP = CF::TN / 2;
  // the lane's addresses are formed here, not hoisted out of the caller's tile loop
  asm volatile("" : "+v"(lane));
  const int fr = lane & 15, fc = lane >> 4;
  const bool lo = fr < 8;
  char* Cb = static_cast<char*>(P.C);
  const int n = t.n0 + wn * CF::WCOLS + 8 * (fc >> 1) + 16 * (fc & 1) + (NP == 2 && !lo ? 32 : 0);
  const int64_t cps = P.c_pstride;
  auto put = [&](int m, const u32x4& val) {
    if (m < t.M && n < P.N) {
      const size_t e = cps ? size_t(n >> 5) * cps + size_t(m) * 32 + (n & 31) : size_t(m) * P.ldc + n;
      u32x4* dst = reinterpret_cast<u32x4*>(Cb + (size_t(t.g) * P.c_gstride + e) * 2);
      if constexpr (NT)
        __builtin_nontemporal_store(val, dst);
      else
        *dst = val;
    }
  };
#pragma unroll
  for (int i = 0; i < CF::TM; ++i) {
    u32x4 ch[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint32_t w[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[0][i][2 * p + h][r];
          if constexpr (EPI == EPI_SWIGLU) v[r] = silu(v[r]) * acc[CF::NB - 1][i][2 * p + h][r];
        }
        if constexpr (EPI == EPI_BIAS || EPI == EPI_GELU_BIAS) {
          const float4 bb = *reinterpret_cast<const float4*>(sbias + wn * CF::WCOLS + (2 * p + h) * 16 + fc * 4);
          v[0] += bb.x;
          v[1] += bb.y;
          v[2] += bb.z;
          v[3] += bb.w;
        }
        if constexpr (EPI == EPI_GELU_BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = gelu_erf(v[r]);
        }
        w[h][0] = pack_bf16x2(v[0], v[1]);
        w[h][1] = pack_bf16x2(v[2], v[3]);
      }
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const auto sw = __builtin_amdgcn_permlane16_swap(w[0][d], w[1][d], false, false);
        ch[p][d] = sw[0];      // columns + 0..3 of the lane's chunk
        ch[p][2 + d] = sw[1];  // columns + 4..7
      }
    }
    const int m = t.m0 + wm * CF::WROWS + i * 16;
    if constexpr (NP == 1) {
      put(m + fr, ch[0]);
    } else {
      // lane r < 8 keeps its first chunk (row r) and sends its second (row r) to lane
      // r + 8; lane r + 8 keeps its second (row r + 8) and sends its first to lane r
      u32x4 got;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        got[d] = uint32_t(__builtin_amdgcn_update_dpp(0, int(lo ? ch[1][d] : ch[0][d]), 0x128, 0xF, 0xF, false));
      put(m + (fr & 7), lo ? ch[0] : got);
      put(m + 8 + (fr & 7), lo ? got : ch[1]);
    }
  }
}

// Stages the bias of the block's BNQ columns in LDS as fp32 (zeros past N or without a
// bias). The caller synchronises before the epilogue reads it.
template <class CF>
__device__ __forceinline__ void stage_bias(const GemmProblem& P, const TileId& t, int tid,
                                           float* sbias) {
  const bf16_t* bias = static_cast<const bf16_t*>(P.bias);
  for (int c = tid; c < CF::BNQ; c += CF::THREADS)
    sbias[c] = (bias && t.n0 + c < P.N) ? bf16_to_f32(bias[size_t(t.g) * P.bias_gstride + t.n0 + c]) : 0.f;
}

}  // namespace tile
}  // namespace moe
