// Pieces shared by the grouped bf16 GEMM kernels: the tile configuration, the LDS
// layouts and their swizzles, the DMA requests that fill one LDS stage, the decoding of
// a block's tile, and the epilogue.
//
// LDS stage layout (one K step of BK = 64):
//   A (expert rows, k contiguous) is stored [m][k], 128 bytes per row, and read as one
//   16-byte fragment per lane. Each lane fetches source chunk c ^ f(m), f(m) = m % 8,
//   so that the lanes of a fragment read hit distinct bank groups.
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

constexpr int BK = kBf16BK;  // 64

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// A rows: chunk c of row m sits at c ^ (m % 8). (Measured on gfx950 with the LDS
// bank-conflict counter: this pattern reads conflict-free for the 16-row fragment
// reads, where c ^ ((m ^ m/8) % 8) does not.)
__device__ __forceinline__ int fswz(int m) { return m & 7; }
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

template <int BM_, int BNE_, bool GATED_, int WGM_ = 2, int WGN_ = 2, int STAGES_ = 3>
struct TileCfg {
  static constexpr int STAGES = STAGES_;           // LDS ring depth
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
  static constexpr int A_INST = BM / 8 / WAVES;  // 1 KiB DMA loads of A per wave per step
  static constexpr int B_RB = BNQ * 2;           // bytes per B row
  static constexpr int B_RPI = 1024 / B_RB;      // B rows per 1 KiB load
  static constexpr int B_IPQ = BK / B_RPI;       // loads per B matrix per step
  static constexpr int B_INST = NB * B_IPQ / WAVES;  // per wave per step
  static constexpr int LOADS = A_INST + B_INST;  // vector-memory ops per thread per step
  static_assert(BM % (8 * WAVES) == 0, "A loads split evenly over the waves");
  static_assert(NB * B_IPQ % WAVES == 0, "B loads split evenly over the waves");
};

// DMA sources of a tile: uniform group bases (scalar registers) and this lane's byte
// offsets from them.
template <class CF>
struct DmaSrc {
  const char* a;              // A of the group (uniform)
  const char* b[CF::NB];      // B matrices of the group (uniform)
  uint32_t ao[CF::A_INST];    // per lane: gathered row and swizzled chunk
  uint32_t bo[CF::B_INST];    // per lane: k row and swizzled chunk
};

// Requests the tiles of step kt into the LDS stage `dst` (one 1 KiB DMA per instruction).
// `wv` is the wave index (uniform). BKM: B is stored [N][K] (k contiguous, like A).
template <class CF, bool BKM = false>
__device__ __forceinline__ void issue_stage(char* __restrict__ dst, const DmaSrc<CF>& S, int kt,
                                            int N, int wv) {
  const size_t ka = size_t(kt) * BK * 2;
  const size_t kb = BKM ? ka : size_t(kt) * BK * size_t(N) * 2;
#pragma unroll
  for (int t = 0; t < CF::A_INST; ++t) {
    const char* g = S.a + ka + S.ao[t];
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(dst + (wv * CF::A_INST + t) * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < CF::B_INST; ++t) {
    const int u = wv * CF::B_INST + t;
    const char* bq = (CF::NB > 1 && u / CF::B_IPQ) ? S.b[CF::NB - 1] : S.b[0];
    const char* g = bq + kb + S.bo[t];
    __builtin_amdgcn_global_load_lds(
        g, (lds_void*)(dst + CF::A_BYTES + (u / CF::B_IPQ) * CF::BQ_BYTES + (u % CF::B_IPQ) * 1024),
        16, 0, 0);
  }
}

// A tile of a grouped batch: problem, group (expert), first row and column, row count.
struct TileId {
  int pi, g, m0, n0, M;
};

// Decodes logical tile id `lid`: problems in order, then groups, then column tiles, then
// row tiles (consecutive ids share a weight panel). M is the row count of the group.
template <class CF>
__device__ __forceinline__ TileId decode_tile(const GemmBatch& batch, int lid) {
  TileId t;
  t.pi = (batch.nprob > 1 && lid >= batch.p[0].tiles) ? 1 : 0;
  const GemmProblem& P = batch.p[t.pi];
  int rem = t.pi ? lid - batch.p[0].tiles : lid;
  const int per_group = P.m_tiles * P.n_tiles;
  t.g = rem / per_group;
  rem -= t.g * per_group;
  const int nt = rem / P.m_tiles;
  const int mt = rem - nt * P.m_tiles;
  // the same value in every lane: keep it (and all tile bookkeeping) in scalar registers
  t.M = P.m_count ? __builtin_amdgcn_readfirstlane(P.m_count[t.g]) : P.m_const;
  t.m0 = mt * CF::BM;
  t.n0 = nt * CF::BNQ;
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
// rows (wv*A_INST + i)*8 .. +8, this lane row (lane / 8); rows past M repeat row m0
// (never stored); with a row map the row is the gathered token (or slot) row.
template <class CF>
__device__ __forceinline__ int tile_a_row(const GemmProblem& P, const TileId& t, int wv, int lane,
                                          int i) {
  const int row = (wv * CF::A_INST + i) * 8 + (lane >> 3);
  int r = t.m0 + row;
  if (r >= t.M) r = t.m0;
  return P.row_map ? P.row_map[size_t(t.g) * P.row_map_ld + r] / P.row_div : r;
}

// DMA sources of tile t from the A rows of tile_a_row. A: this lane's physical chunk
// p = lane % 8 holds source chunk p ^ f(row). B: load i of wave wv is load
// u = wv*B_INST + i overall: matrix u / B_IPQ, rows (u % B_IPQ) * B_RPI .. +B_RPI;
// columns past N read column 0 (never stored). BKM (B stored [N][K]): B is staged like
// A, [n][k] with 128-byte rows and the same chunk swizzle; load u covers the 8 rows
// (u % B_IPQ) * 8 .. +8 of its matrix, and rows past N read row 0.
template <class CF, bool BKM = false>
__device__ __forceinline__ void tile_sources_from_rows(const GemmProblem& P, const TileId& t,
                                                       int wv, int lane, const int* rows,
                                                       DmaSrc<CF>& S) {
  S.a = static_cast<const char*>(P.A) + size_t(t.g) * P.a_gstride * 2;
  S.b[0] = static_cast<const char*>(P.B0) + size_t(t.g) * P.b_gstride * 2;
  if constexpr (CF::NB > 1) S.b[CF::NB - 1] = static_cast<const char*>(P.B1) + size_t(t.g) * P.b_gstride * 2;
#pragma unroll
  for (int i = 0; i < CF::A_INST; ++i) {
    const int row = (wv * CF::A_INST + i) * 8 + (lane >> 3);
    S.ao[i] = uint32_t((size_t(rows[i]) * P.lda + 8 * ((lane & 7) ^ fswz(row))) * 2);
  }
  if constexpr (BKM) {
    static_assert(CF::B_IPQ * 8 == CF::BNQ, "one 1 KiB load per 8 rows of 128 bytes");
#pragma unroll
    for (int i = 0; i < CF::B_INST; ++i) {
      const int u = wv * CF::B_INST + i;
      const int nl = (u % CF::B_IPQ) * 8 + (lane >> 3);
      int n = t.n0 + nl;
      if (n >= P.N) n = 0;
      S.bo[i] = uint32_t((size_t(n) * P.K + 8 * ((lane & 7) ^ fswz(nl))) * 2);
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
__device__ __forceinline__ void tile_sources(const GemmProblem& P, const TileId& t, int wv,
                                             int lane, DmaSrc<CF>& S) {
  int rows[CF::A_INST];
#pragma unroll
  for (int i = 0; i < CF::A_INST; ++i) rows[i] = tile_a_row<CF>(P, t, wv, lane, i);
  tile_sources_from_rows<CF, BKM>(P, t, wv, lane, rows, S);
}

// Epilogue: lane holds C[m][n..n+3] of every MFMA tile (the MFMA ran with B as its first
// operand, so each tile comes out transposed). For EPI_BIAS / EPI_GELU_BIAS the bias
// comes from `sbias` (the block's BNQ values staged in LDS) or, when `sbias` is null,
// straight from the problem's bias vector.
template <class CF, int EPI, bool OF32>
__device__ __forceinline__ void store_tile(const GemmProblem& P, const TileId& t, int wm, int wn,
                                           int lane, const float* sbias,
                                           const f32x4 (&acc)[CF::NB][CF::TM][CF::TN]) {
  const int fr = lane & 15, fc = lane >> 4;
  char* Cb = static_cast<char*>(P.C);
  constexpr int es = OF32 ? 4 : 2;
#pragma unroll
  for (int i = 0; i < CF::TM; ++i) {
    const int m = t.m0 + wm * CF::WROWS + i * 16 + fr;
    if (m >= t.M) continue;
#pragma unroll
    for (int j = 0; j < CF::TN; ++j) {
      const int nl = wn * CF::WCOLS + j * 16 + fc * 4;
      const int n = t.n0 + nl;
      if (n >= P.N) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[0][i][j][r];
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = silu(v[r]) * acc[CF::NB - 1][i][j][r];
      }
      if constexpr (EPI == EPI_BIAS || EPI == EPI_GELU_BIAS) {
        if (sbias) {
          const float4 bb = *reinterpret_cast<const float4*>(sbias + nl);
          v[0] += bb.x;
          v[1] += bb.y;
          v[2] += bb.z;
          v[3] += bb.w;
        } else if (P.bias) {
          // n .. n+3 < N: N is a multiple of 64
          const uint2 bw = *reinterpret_cast<const uint2*>(
              static_cast<const bf16_t*>(P.bias) + size_t(t.g) * P.bias_gstride + n);
          v[0] += bf16_to_f32(bf16_t(bw.x & 0xffff));
          v[1] += bf16_to_f32(bf16_t(bw.x >> 16));
          v[2] += bf16_to_f32(bf16_t(bw.y & 0xffff));
          v[3] += bf16_to_f32(bf16_t(bw.y >> 16));
        }
      }
      if constexpr (EPI == EPI_GELU_BIAS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = gelu_erf(v[r]);
      }
      char* dst = Cb + (size_t(t.g) * P.c_gstride + size_t(m) * P.ldc + n) * es;
      if constexpr (OF32) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

// The epilogue math for 4 consecutive outputs n..n+3 of row m: SwiGLU product, bias
// (staged `sbias` or, when null, read from the problem's bias vector), GELU.
template <class CF, int EPI>
__device__ __forceinline__ void epi_math(const GemmProblem& P, const TileId& t, int nl, int n,
                                         const float* sbias, const float (&a)[4],
                                         const float (&b)[4], float (&v)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = a[r];
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = silu(a[r]) * b[r];
  }
  if constexpr (EPI == EPI_BIAS || EPI == EPI_GELU_BIAS) {
    if (sbias) {
      const float4 bb = *reinterpret_cast<const float4*>(sbias + nl);
      v[0] += bb.x;
      v[1] += bb.y;
      v[2] += bb.z;
      v[3] += bb.w;
    } else if (P.bias) {
      // n .. n+3 < N: N is a multiple of 64
      const uint2 bw = *reinterpret_cast<const uint2*>(
          static_cast<const bf16_t*>(P.bias) + size_t(t.g) * P.bias_gstride + n);
      v[0] += bf16_to_f32(bf16_t(bw.x & 0xffff));
      v[1] += bf16_to_f32(bf16_t(bw.x >> 16));
      v[2] += bf16_to_f32(bf16_t(bw.y & 0xffff));
      v[3] += bf16_to_f32(bf16_t(bw.y >> 16));
    }
  }
  if constexpr (EPI == EPI_GELU_BIAS) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = gelu_erf(v[r]);
  }
}

// bf16 epilogue through LDS: the tile is written to `stage` (the whole LDS ring,
// CF::LDS bytes, free once the K loop is done) in rounds of R = min(BM, CF::LDS / (2 BNQ))
// rows (one round for the 256-row tiles: every wave writes its accumulators at once), each
// lane's 8-byte pieces placed with the 16-byte chunk index XORed by (row % 16), then
// read back as 16 bytes per lane along whole rows and stored (non-temporal), so every
// store instruction writes complete row segments. All threads of the block take part
// (it synchronises); `stage` must be free on entry and is free again on return.
template <class CF, int EPI>
__device__ __forceinline__ void store_tile_staged(const GemmProblem& P, const TileId& t, int wm,
                                                  int wn, int wv, int lane, const float* sbias,
                                                  char* stage,
                                                  const f32x4 (&acc)[CF::NB][CF::TM][CF::TN]) {
  constexpr int RB = CF::BNQ * 2;         // bytes per output row
  constexpr int CPR = RB / 16;            // 16-byte chunks per row
  constexpr int R = CF::LDS / RB < CF::BM ? CF::LDS / RB : CF::BM;  // rows per round
  constexpr int ROUNDS = CF::BM / R;
  constexpr int LPR = 64 / CPR;           // rows per wave instruction when reading back
  static_assert(CPR >= 16 && R % CF::WROWS == 0 && CF::BM % R == 0 && CF::WAVES == 16,
                "staged epilogue shape");
  const int fr = lane & 15, fc = lane >> 4;
  char* Cb = static_cast<char*>(P.C);
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    __syncthreads();  // stage free (previous round stored, or the K loop done with it)
    if (wm * CF::WROWS >= rd * R && wm * CF::WROWS < (rd + 1) * R) {
#pragma unroll
      for (int i = 0; i < CF::TM; ++i) {
        const int ml = wm * CF::WROWS + i * 16 + fr - rd * R;
        const int m = t.m0 + rd * R + ml;
#pragma unroll
        for (int j = 0; j < CF::TN; ++j) {
          const int nl = wn * CF::WCOLS + j * 16 + fc * 4;
          const int n = t.n0 + nl;
          float a[4], b[4], v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            a[r] = acc[0][i][j][r];
            b[r] = acc[CF::NB - 1][i][j][r];
          }
          if (m < t.M && n < P.N) {
            epi_math<CF, EPI>(P, t, nl, n, sbias, a, b, v);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = 0.f;
          }
          const int bc = nl * 2;  // byte column
          *reinterpret_cast<uint2*>(stage + ml * RB + 16 * ((bc >> 4) ^ (ml & 15)) + (bc & 15)) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < R / (16 * LPR); ++q) {
      const int ml = (wv * (R / 16)) + q * LPR + lane / CPR;  // 16 waves, R/16 rows each
      const int c = lane % CPR;
      const int m = t.m0 + rd * R + ml;
      const int n = t.n0 + 8 * c;
      // non-temporal: the tile is read back once, by a later kernel, long after this
      // launch has streamed far more than the caches hold
      if (m < t.M && n < P.N)
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4*>(stage + ml * RB + 16 * (c ^ (ml & 15))),
            reinterpret_cast<u32x4*>(Cb + (size_t(t.g) * P.c_gstride + size_t(m) * P.ldc + n) * 2));
    }
  }
  __syncthreads();  // every wave has read the stage back
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
