// Grouped bf16 GEMM on gfx950 MFMA (v_mfma_f32_16x16x32_bf16), fp32 accumulate.
//
// This is the one dense contraction on the MoE path: each expert's slot buffer times
// its weights ("Module 7", swiglu_expert and the EducationalMoE expert loop, done as
// one grouped launch instead of a loop). Rows of A are gathered by indirection
// (slot -> assignment -> token), so each expert's input rows are assembled directly in
// LDS tiles from x without a separate gather pass.
//
// Data movement. Both operands go from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging), through a three-stage ring: the tile
// for step k+2 is requested while step k is multiplied (ring depth S: step k+S-1), so
// S-1 steps of MFMA cover the memory latency and one barrier per step publishes the
// next tile.
//   A (expert rows, k contiguous) is stored [m][k], 128 bytes per row (BK = 64), and
//   read as one 16-byte fragment per lane. Each lane fetches the source chunk
//   c ^ (m % 8), so that the lanes of a fragment read hit distinct bank groups.
//   B (weights, n contiguous: [k][n] per expert, as stored) is copied unchanged apart
//   from a per-row XOR of the 16-byte chunk index (hswz); the k-major fragment
//   each MFMA needs is assembled with two ds_read_b64_tr_b16 transpose reads. Within a
//   16-lane group that instruction hands lane l element l % 4 of the 8-byte pieces
//   addressed by lanes l/4 + 4v (v = 0..3), so lane s of group g points at row
//   8g + (s%16)/4 (+4 for the second read) and column 4 (s % 4) of its 16-column slice.
//   B stored [n][k] per expert instead (the OUT_IN weight layout, BKM) is staged and
//   read exactly like A: one ds_read_b128 per fragment.
//
// Tiles: the large tile is 256 rows x 256 staged B columns (SwiGLU: 128 gate + 128 up
// columns of the same outputs) on 16 waves (4 x 4, four per SIMD, each 64 rows x 64
// staged columns) with a two-stage ring (128 KiB of LDS): large enough that each byte
// staged feeds 128 FLOPs. The small tile (128 x 128, 4 waves, three stages) serves
// narrow problems. The gated variant holds gate and up accumulators of the same outputs
// in one lane, so silu(x Wg) * (x Wu) is formed in the epilogue and only the product is
// written.
//
// The MFMA is issued with the B fragment as its first operand, which yields C^T per
// tile: each lane then holds 4 consecutive output columns of one row, so the epilogue
// stores 8 (bf16) or 16 (fp32) contiguous bytes per lane.
//
// Block scheduling: the hardware deals workgroups to the 8 XCDs round-robin; the
// kernel remaps the hardware id so that each XCD works through a contiguous range of
// tiles. Consecutive tiles belong to the same expert, so the tiles of one expert share
// their weight panels in one XCD's L2.

#include "gemm_bf16_tile.h"

namespace moe {

namespace {

using namespace tile;

// One K step: request step `nxt` into slot `nxt_slot`, then multiply the tiles in slot
// `cur`. The two slots are distinct, which the restrict qualifiers state; that lets the
// compiler order the LDS reads of `cur` freely against the DMA writes still in flight.
// BKM: B is staged [n][k] like A, and its fragments are read like A's.
template <class CF, bool BKM>
__device__ __forceinline__ void step_compute_issue(const char* __restrict__ cur,
                                                   char* __restrict__ nxt_slot,
                                                   const DmaSrc<CF>& S, int nxt, int N,
                                                   int wv, int wm, int wn, int lane,
                                                   f32x4 (&acc)[CF::NB][CF::TM][CF::TN],
                                                   bool issue = true) {
  constexpr int NB = CF::NB, TM = CF::TM, TN = CF::TN;
  if (issue) issue_stage<CF, BKM>(nxt_slot, S, nxt, N, wv);
  const int fr = lane & 15, fc = lane >> 4;
  const int arow = wm * CF::WROWS + fr;
  // B transpose-read coordinates of this lane: k row within the 32-wide k step and the
  // column offset inside a 16-column fragment
  const int bk = 8 * fc + (fr >> 2);
  const int bcol = 4 * (fr & 3);
  const char* As = cur;
  const char* Bs = cur + CF::A_BYTES;
#pragma unroll
  for (int ks = 0; ks < CF::BK / 32; ++ks) {
    bf16x8 bfr[NB][TN];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (BKM) {
          const int n = wn * CF::WCOLS + j * 16 + fr;
          bfr[q][j] = *reinterpret_cast<const bf16x8*>(Bs + q * CF::BQ_BYTES + n * CF::K_RB +
                                                      16 * ((ks * 4 + fc) ^ fswz<CF::K_RB>(n)));
        } else {
          const int col = wn * CF::WCOLS + j * 16 + bcol;
          const int k0 = ks * 32 + bk;
          const int k1 = k0 + 4;
          const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(Bs + q * CF::BQ_BYTES + k0 * CF::B_RB + 16 * ((col >> 3) ^ hswz<CF::B_RB>(k0)) + 2 * (col & 7)));
          const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(Bs + q * CF::BQ_BYTES + k1 * CF::B_RB + 16 * ((col >> 3) ^ hswz<CF::B_RB>(k1)) + 2 * (col & 7)));
          bfr[q][j] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = arow + i * 16;
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(As + m * CF::K_RB +
                                                         16 * ((ks * 4 + fc) ^ fswz<CF::K_RB>(m)));
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[q][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[q][j], af, acc[q][i][j], 0, 0, 0);
    }
  }
}

}  // namespace

// The 16-wave, 256-row tile with a bf16 output leaves through the LDS-staged epilogue.
template <class CF, bool OF32>
constexpr bool staged_epilogue() {
  return !OF32 && CF::WAVES == 16 && CF::BM == 256;
}
// Dynamic LDS of gemm_bf16_kernel: the ring, plus the block's bias columns (fp32) above
// it when the staged epilogue, which uses the whole ring, needs a bias.
template <class CF, int EPI, bool OF32>
constexpr int kernel_lds() {
  return CF::LDS + (staged_epilogue<CF, OF32>() && (EPI == EPI_BIAS || EPI == EPI_GELU_BIAS)
                        ? int(sizeof(float)) * CF::BNQ
                        : 0);
}

// EPI: EPI_STORE / EPI_BIAS / EPI_GELU_BIAS / EPI_SWIGLU; OF32: store fp32 instead of bf16;
// BKM: B stored [N][K]
template <class CF, int EPI, bool OF32, bool BKM>
__global__ __launch_bounds__(CF::THREADS, 1) void gemm_bf16_kernel(GemmBatch batch) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int NB = CF::NB, TM = CF::TM, TN = CF::TN;

  const int lt = xcd_tile(batch.total, batch.chunk, blockIdx.x & 7, blockIdx.x >> 3);
  if (lt < 0) return;
  const TileId tl = decode_tile<CF>(batch, lt);
  if (tl.m0 >= tl.M) return;
  const GemmProblem& P = batch.p[tl.pi];
  const int N = P.N;
  const int K = P.K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % CF::WGM, wn = wv / CF::WGM;

  DmaSrc<CF> S;
  tile_sources<CF, BKM>(P, tl, wv, lane, S);

  f32x4 acc[NB][TM][TN];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[q][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / CF::BK;
  const int last = nk - 1;
  constexpr int NS = CF::STAGES;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    issue_stage<CF, BKM>(smem + st * CF::STAGE, S, st <= last ? st : last, N, wv);
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's loads for step kt have landed (S-2 later steps may still be in
    // flight); after the barrier everyone's have, and every wave is done with step kt-1,
    // whose slot the next request reuses
    wait_vmcnt<CF::LOADS * (NS - 2)>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int nxt = kt + NS - 1 <= last ? kt + NS - 1 : last;
    step_compute_issue<CF, BKM>(smem + (kt % NS) * CF::STAGE,
                                smem + ((kt + NS - 1) % NS) * CF::STAGE, S, nxt, N, wv, wm, wn,
                                lane, acc);
  }
  wait_vmcnt<0>();  // the clamped tail loads still target LDS
  __syncthreads();

  constexpr bool STAGED = staged_epilogue<CF, OF32>();
  // bias of this block's columns, staged once in LDS (in the ring, free after the main
  // loop; above it when the staged epilogue uses the whole ring)
  float* sbias = reinterpret_cast<float*>(smem + (STAGED ? CF::LDS : 0));
  if constexpr (EPI == EPI_BIAS || EPI == EPI_GELU_BIAS) {
    stage_bias<CF>(P, tl, tid, sbias);
    __syncthreads();
  }
  if constexpr (STAGED)
    store_tile_staged<CF, EPI>(P, tl, wm, wn, wv, lane, sbias, smem, acc);
  else
    store_tile<CF, EPI, OF32>(P, tl, wm, wn, lane, sbias, acc);
}

// Persistent form of the two-stage kernel: one block per CU works through a list of
// tiles. XCD x (hardware blocks x, x+8, ...) owns a contiguous range of logical tiles, so
// the blocks running together on one XCD work on neighbouring tiles, which share weight
// panels in that XCD's L2. At the start the block ranks the non-empty tiles of its XCD's
// range in order (a block-wide prefix count) and keeps those of rank bi, bi + nb_x, ...
// in LDS, so skewed groups (many nearly empty experts) still spread evenly over the
// XCD's blocks. On the last K step of a tile the DMA request already targets step 0 of
// the block's next tile, so that tile's first stage streams in while the epilogue of the
// current one runs; the next tile's gathered row indices are read at the start of the
// current tile.
template <class CF, int EPI, bool OF32, bool BKM>
__global__ __launch_bounds__(CF::THREADS, 1) void gemm_bf16_persistent_kernel(GemmBatch batch) {
  static_assert(CF::STAGES == 2, "two-stage ring");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int NB = CF::NB, TM = CF::TM, TN = CF::TN;
  const int nblk = gridDim.x;
  const int x = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int nb_x = (nblk >> 3) + ((nblk & 7) > x ? 1 : 0);
  int ranked = 0;  // non-empty tiles in XCD x's range
  {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    int* s_list = reinterpret_cast<int*>(smem + CF::LDS);
    int* s_wsum = s_list + batch.list_cap;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j0 = 0;; j0 += CF::THREADS) {
      const int lt = xcd_tile(batch.total, batch.chunk, x, j0 + tid);
      const bool ne = lt >= 0 && tile_nonempty<CF>(batch, lt);
      const uint64_t bal = __ballot(ne);
      if (lane == 0) s_wsum[wv] = __popcll(bal);
      __syncthreads();
      int before = 0, tot = 0;
#pragma unroll
      for (int w2 = 0; w2 < CF::WAVES; ++w2) {
        const int c = s_wsum[w2];
        before += w2 < wv ? c : 0;
        tot += c;
      }
      if (ne) {
        const int r = ranked + before + __popcll(bal & below);
        if (r % nb_x == bi) s_list[r / nb_x] = lt;
      }
      ranked += tot;
      __syncthreads();  // s_wsum is rewritten by the next pass; s_list complete after the last
      if (xcd_tile(batch.total, batch.chunk, x, j0 + CF::THREADS) < 0) break;
    }
  }
  const int* s_list = reinterpret_cast<const int*>(smem + CF::LDS);
  const int nmine = ranked > bi ? (ranked - bi + nb_x - 1) / nb_x : 0;
  if (nmine == 0) return;
  int qi = 0;  // position in the block's tile list
  TileId tl = decode_tile<CF>(batch, __builtin_amdgcn_readfirstlane(s_list[0]));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % CF::WGM, wn = wv / CF::WGM;

  DmaSrc<CF> S;
  tile_sources<CF, BKM>(batch.p[tl.pi], tl, wv, lane, S);
  f32x4 acc[NB][TM][TN];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[q][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue_stage<CF, BKM>(smem, S, 0, batch.p[tl.pi].N, wv);
  int g = 0;  // steps done by this block: stage g & 1 holds the current one
  while (true) {
    const GemmProblem& P = batch.p[tl.pi];
    // the block's next tile, and its gathered A rows
    const bool more = qi + 1 < nmine;
    TileId tl2 = tl;
    if (more) tl2 = decode_tile<CF>(batch, __builtin_amdgcn_readfirstlane(s_list[qi + 1]));
    int rows2[CF::A_INST];
    if (more) {
#pragma unroll
      for (int i = 0; i < CF::A_INST; ++i) rows2[i] = tile_a_row<CF>(batch.p[tl2.pi], tl2, wv, lane, i);
    }
    const int nk = P.K / CF::BK;
    for (int kt = 0; kt < nk; ++kt, ++g) {
      // this thread's loads for step kt have landed; after the barrier everyone's have,
      // and every wave is done with the previous step, whose stage the next request uses
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      int knext = kt + 1, nN = P.N;
      bool issue = true;
      if (knext == nk) {
        if (more) {
          tile_sources_from_rows<CF, BKM>(batch.p[tl2.pi], tl2, wv, lane, rows2, S);
          knext = 0;
          nN = batch.p[tl2.pi].N;
        } else {
          issue = false;
        }
      }
      step_compute_issue<CF, BKM>(smem + (g & 1) * CF::STAGE, smem + ((g + 1) & 1) * CF::STAGE,
                                  S, knext, nN, wv, wm, wn, lane, acc, issue);
    }
    store_tile<CF, EPI, OF32>(P, tl, wm, wn, lane, nullptr, acc);
    if (!more) break;
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[q][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    ++qi;
    tl = tl2;
  }
}

namespace {
// Tile counts of every problem, the chunk dealt to one XCD and the longest XCD list.
template <class CF>
void plan_tiles(GemmBatch& b) {
  b.total = 0;
  for (int i = 0; i < b.nprob; ++i) {
    GemmProblem& p = b.p[i];
    p.m_tiles = (p.m_tiles_rows + CF::BM - 1) / CF::BM;
    p.n_tiles = (p.N + CF::BNQ - 1) / CF::BNQ;
    p.tiles = p.groups * p.m_tiles * p.n_tiles;
    b.total += p.tiles;
  }
  // one group's tiles, but at least 256 chunks overall (32 per XCD) for balance
  const int group = b.p[0].m_tiles * b.p[0].n_tiles;
  const int cap = b.total / 256;
  int ch = group < cap ? group : cap;
  b.chunk = ch < 1 ? 1 : ch;
  b.xcd_max = 0;
  const int nchunks = (b.total + b.chunk - 1) / b.chunk;
  for (int x = 0; x < 8; ++x) {
    int n = 0;
    for (int c = x; c < nchunks; c += 8) n += (c == nchunks - 1) ? b.total - c * b.chunk : b.chunk;
    if (n > b.xcd_max) b.xcd_max = n;
  }
}

template <class CF, int EPI, bool OF32, bool BKM>
moe_status_t launch_cfg(GemmBatch& b, const char* name, hipStream_t s) {
  plan_tiles<CF>(b);
  if (b.total == 0) return MOE_OK;
  constexpr int lds = kernel_lds<CF, EPI, OF32>();
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel<CF, EPI, OF32, BKM>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
      return MOE_ERR_HIP;
    attr_set = true;
  }
  MOE_LAUNCH(name, (gemm_bf16_kernel<CF, EPI, OF32, BKM>), dim3(8 * b.xcd_max), dim3(CF::THREADS),
             lds, s, b);
  return MOE_OK;
}

// LDS of a persistent block: the ring plus its tile list (at most 24 KiB of entries)
constexpr int kPersistentLdsMax = 2 * 65536 + 24576;

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
  }
  return n;
}

template <class CF, int EPI, bool OF32, bool BKM>
moe_status_t launch_persistent(GemmBatch& b, const char* name, hipStream_t s) {
  plan_tiles<CF>(b);
  if (b.total == 0) return MOE_OK;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(
            reinterpret_cast<const void*>(gemm_bf16_persistent_kernel<CF, EPI, OF32, BKM>),
            hipFuncAttributeMaxDynamicSharedMemorySize, kPersistentLdsMax) != hipSuccess)
      return MOE_ERR_HIP;
    attr_set = true;
  }
  const int grid = b.total < cu_count() ? int(b.total) : cu_count();
  const int nb_min = grid / 8 > 0 ? grid / 8 : 1;  // blocks of the XCD with the fewest
  b.list_cap = (b.xcd_max + nb_min - 1) / nb_min;
  const size_t lds = CF::LDS + sizeof(int) * (size_t(b.list_cap) + CF::WAVES);
  if (lds > size_t(kPersistentLdsMax)) return launch_cfg<CF, EPI, OF32, BKM>(b, name, s);
  MOE_LAUNCH(name, (gemm_bf16_persistent_kernel<CF, EPI, OF32, BKM>), dim3(grid),
             dim3(CF::THREADS), lds, s, b);
  return MOE_OK;
}

template <class CF, bool BKM>
moe_status_t launch_epi(GemmBatch& b, const char* name, hipStream_t s) {
  const int epi = b.p[0].epi;
  for (int i = 1; i < b.nprob; ++i)
    if (b.p[i].epi != epi || b.p[i].out_f32 != b.p[0].out_f32) return MOE_ERR_UNSUPPORTED;
  if (b.p[0].out_f32) {
    if (epi != EPI_STORE || BKM) return MOE_ERR_UNSUPPORTED;
    return launch_cfg<CF, EPI_STORE, true, false>(b, name, s);
  }
  switch (epi) {
    case EPI_STORE: return launch_cfg<CF, EPI_STORE, false, BKM>(b, name, s);
    case EPI_BIAS: return launch_cfg<CF, EPI_BIAS, false, BKM>(b, name, s);
    case EPI_GELU_BIAS: return launch_cfg<CF, EPI_GELU_BIAS, false, BKM>(b, name, s);
    default: return MOE_ERR_UNSUPPORTED;
  }
}

template <bool BKM>
moe_status_t launch_layout(GemmBatch& b, bool gated, bool large, const char* name,
                           hipStream_t s) {
  if (gated) {
    for (int i = 0; i < b.nprob; ++i)
      if (b.p[i].epi != EPI_SWIGLU || b.p[i].out_f32) return MOE_ERR_UNSUPPORTED;
    return large ? launch_persistent<TileCfg<256, 256, true, 4, 4, 2>, EPI_SWIGLU, false, BKM>(b, name, s)
                 : launch_cfg<TileCfg<128, 128, true, 2, 2, 3>, EPI_SWIGLU, false, BKM>(b, name, s);
  }
  return large ? launch_epi<TileCfg<256, 256, false, 4, 4, 2>, BKM>(b, name, s)
               : launch_epi<TileCfg<128, 128, false, 2, 2, 3>, BKM>(b, name, s);
}
}  // namespace

moe_status_t launch_gemm_bf16(GemmBatch& b, bool gated, const char* name, hipStream_t s) {
  // Large tiles (256 x 256, 16 waves, two stages) when every problem has enough rows per
  // group and the grid has at least 128 of them (half the CUs: the large tile's higher
  // rate per CU outweighs the idle CUs, e.g. 192 tiles with K = 4096 run in 115 us against
  // 139 us as 640 small tiles); else 128 x 128 tiles. The
  // gated (SwiGLU) GEMM, with long K loops and small output tiles, runs persistent blocks;
  // the others (K as short as d_hidden, 128 KiB output tiles) run one block per tile with
  // the LDS-staged epilogue, whose stores overlap the next block's start.
  using Large = TileCfg<256, 256, true, 4, 4, 2>;
  bool large = true;
  long tiles = 0;
  for (int i = 0; i < b.nprob; ++i) {
    const GemmProblem& p = b.p[i];
    if (p.m_tiles_rows < 192) large = false;
    const int bnq = gated ? Large::BNQ : 2 * Large::BNQ;
    tiles += long(p.groups) * ((p.m_tiles_rows + 255) / 256) * ((p.N + bnq - 1) / bnq);
  }
  if (tiles < 128) large = false;
  // B layout: every problem of a batch stores B the same way
  for (int i = 1; i < b.nprob; ++i)
    if (b.p[i].b_kmajor != b.p[0].b_kmajor) return MOE_ERR_UNSUPPORTED;
  return b.p[0].b_kmajor ? launch_layout<true>(b, gated, large, name, s)
                         : launch_layout<false>(b, gated, large, name, s);
}

}  // namespace moe
