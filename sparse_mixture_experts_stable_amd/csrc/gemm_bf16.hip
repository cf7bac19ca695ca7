// Grouped bf16 GEMM on gfx950 MFMA (v_mfma_f32_16x16x32_bf16), fp32 accumulate.
//
// This is the one dense contraction on the MoE path: each expert's slot buffer times
// its weights ("Module 7", swiglu_expert and the EducationalMoE expert loop, done as
// one grouped launch instead of a loop). Rows of A are gathered by indirection
// (slot -> assignment -> token), so each expert's input rows are assembled directly in
// LDS tiles from x without a separate gather pass.
//
// Data movement. Both operands go from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging), with one barrier per K step to publish
// the next tiles. The small tile uses a ring of S stages: the tiles of step k+S-1 are
// requested while step k is multiplied, so S-1 steps of MFMA cover the memory latency.
// The large tile keeps its A and B tiles in separate operand slots so that the weights
// can be requested two steps ahead (see kSlotBytes).
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
// staged columns) with five 32 KiB operand slots (160 KiB of LDS, below): large enough
// that each byte staged feeds 128 FLOPs. The small tile (128 x 128) serves narrow
// problems, on 8 waves (64 x 32 each) with four stages for plain products such as the
// router GEMM (4.5 us faster there than 4 waves of 64 x 64; four stages 30.3 us, three
// 31.7, two 34.7) and on 4 waves with three stages for gated ones. The gated
// variant holds gate and up accumulators of the same outputs in one lane, so
// silu(x Wg) * (x Wu) is formed in the epilogue and only the product is written.
//
// The MFMA is issued with the B fragment as its first operand, which yields C^T per
// tile: each lane then holds 4 consecutive output columns of one row, so the epilogue
// stores 8 (bf16) or 16 (fp32) contiguous bytes per lane; the persistent kernel first
// pairs those pieces across lanes into 16-byte chunks (store_tile_swapped).
//
// Block scheduling: the hardware deals workgroups to the 8 XCDs round-robin; the
// kernels remap the hardware id so that each XCD works through a contiguous range of
// tiles. Consecutive tiles belong to the same expert, so the tiles of one expert share
// their weight panels in one XCD's L2. The persistent kernel runs one block per CU over
// the non-empty tiles of its XCD's range.

#include "gemm_bf16_tile.h"

namespace moe {

namespace {

using namespace tile;

// B fragment (matrix q, column fragment j, 32-wide k slice ks) of this lane from the B
// tiles at `Bs` (matrix q at q * BQ_BYTES). BKM: B is staged [n][k] like A, and its
// fragments are read like A's; otherwise [k][n], read with two transpose reads: within a
// 16-lane group lane s points at k row 8 (s / 16) + (s % 16) / 4 (+4 for the second read)
// and column 4 (s % 4) of its 16-column slice.
template <class CF, bool BKM>
__device__ __forceinline__ bf16x8 b_frag(const char* Bs, int q, int j, int ks, int wn, int lane) {
  const int fr = lane & 15, fc = lane >> 4;
  if constexpr (BKM) {
    const int n = wn * CF::WCOLS + j * 16 + fr;
    return *reinterpret_cast<const bf16x8*>(Bs + q * CF::BQ_BYTES + n * CF::K_RB +
                                            16 * ((ks * 4 + fc) ^ fswz<CF::K_RB>(n)));
  } else {
    const int col = wn * CF::WCOLS + j * 16 + 4 * (fr & 3);
    const int k0 = ks * 32 + 8 * fc + (fr >> 2);
    const int k1 = k0 + 4;
    const bf16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(Bs + q * CF::BQ_BYTES + k0 * CF::B_RB + 16 * ((col >> 3) ^ hswz<CF::B_RB>(k0)) + 2 * (col & 7)));
    const bf16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(Bs + q * CF::BQ_BYTES + k1 * CF::B_RB + 16 * ((col >> 3) ^ hswz<CF::B_RB>(k1)) + 2 * (col & 7)));
    return __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// A fragment (row fragment i, k slice ks) of this lane from the A tile at `As`.
template <class CF>
__device__ __forceinline__ bf16x8 a_frag(const char* As, int i, int ks, int wm, int lane) {
  const int m = wm * CF::WROWS + i * 16 + (lane & 15);
  return *reinterpret_cast<const bf16x8*>(As + m * CF::K_RB + 16 * ((ks * 4 + (lane >> 4)) ^ fswz<CF::K_RB>(m)));
}

// The MFMAs of one K step on the A tile at `As` and the B tiles at `Bs`. Per 32-wide k
// slice: AFIRST = false reads the wave's NB x TN B fragments, then per row fragment one A
// fragment and its NB x TN MFMAs; AFIRST = true reads the TM A fragments, then per B
// fragment its TM MFMAs, which holds fewer fragment registers (the same reads and MFMAs).
template <class CF, bool BKM, bool AFIRST = false>
__device__ __forceinline__ void mma_step(const char* As, const char* Bs, int wm, int wn, int lane,
                                         f32x4 (&acc)[CF::NB][CF::TM][CF::TN]) {
  constexpr int NB = CF::NB, TM = CF::TM, TN = CF::TN;
#pragma unroll
  for (int ks = 0; ks < CF::BK / 32; ++ks) {
    if constexpr (AFIRST) {
      bf16x8 af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = a_frag<CF>(As, i, ks, wm, lane);
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const bf16x8 bf = b_frag<CF, BKM>(Bs, q, j, ks, wn, lane);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[q][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[i], acc[q][i][j], 0, 0, 0);
        }
    } else {
      bf16x8 bfr[NB][TN];
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[q][j] = b_frag<CF, BKM>(Bs, q, j, ks, wn, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const bf16x8 af = a_frag<CF>(As, i, ks, wm, lane);
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[q][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[q][j], af, acc[q][i][j], 0, 0, 0);
      }
    }
  }
}

// One K step: request step `nxt` into slot `nxt_slot` (if `issue`), then multiply the
// tiles in slot `cur`. The two slots are distinct, which the restrict qualifiers state;
// that lets the compiler order the LDS reads of `cur` freely against the DMA writes still
// in flight.
template <class CF, bool BKM>
__device__ __forceinline__ void step_compute_issue(const char* __restrict__ cur,
                                                   char* __restrict__ nxt_slot,
                                                   const DmaSrc<CF>& S, int nxt, int N,
                                                   int wv, int wm, int wn, int lane,
                                                   f32x4 (&acc)[CF::NB][CF::TM][CF::TN],
                                                   bool issue) {
  if (issue) issue_stage<CF, BKM>(nxt_slot, S, nxt, N, wv);
  mma_step<CF, BKM>(cur, cur + CF::A_BYTES, wm, wn, lane, acc);
}

// The same for the operand slots: request the A tile of step `ka` into `dA` (if `ia`) and
// the B tiles of step `kb` into `dB` (if `ib`), then multiply the A tile at `As` with the B
// tiles at `Bs`. The four slots are distinct (restrict: the compiler need not wait for the
// requests before the fragment reads).
template <class CF, bool BKM>
__device__ __forceinline__ void step_compute_issue_split(
    char* __restrict__ As, char* __restrict__ Bs, char* __restrict__ dA, char* __restrict__ dB,
    const DmaSrc<CF>& SA, const DmaSrc<CF>& SB, int ka, int kb, int N, bool ia, bool ib, int wv,
    int wm, int wn, int lane, f32x4 (&acc)[CF::NB][CF::TM][CF::TN]) {
  if (ia) issue_a<CF>(dA, SA, ka, wv);
  if (ib) issue_b<CF, BKM>(dB, SB, kb, N, wv);
  mma_step<CF, BKM, false>(As, Bs, wm, wn, lane, acc);
}

// Entry q of a block's tile list held in a register: lane j holds entries j (low 16 bits)
// and 64 + j (high 16 bits).
__device__ __forceinline__ int list_entry(int l, int q) {
  const int v = __builtin_amdgcn_readlane(l, q & 63);
  return q < 64 ? (v & 0xffff) : int(uint32_t(v) >> 16);
}

}  // namespace

// Operand slots: the large tiles (256 x 256, 64-wide K step) keep the A tile and the B
// tiles of a K step in separate 32 KiB slots, five of them (the whole 160 KiB of a CU),
// requested in the order B(0), A(0), B(1), A(1), ...: step s reads slots 2s % 5 (B) and
// (2s + 1) % 5 (A), and while it is multiplied A(s + 1) and B(s + 2) are in flight. The
// weights, which come from HBM, are thus requested two steps ahead and the A rows one
// step ahead (three whole 64 KiB stages would not fit).
constexpr int kSlotBytes = 32768;
constexpr int kSlots = 5;
constexpr int kPersistentLds = kSlots * kSlotBytes;
template <class CF>
constexpr bool uses_slots() {
  return CF::STAGES == 2 && CF::A_BYTES == kSlotBytes && CF::NB * CF::BQ_BYTES == kSlotBytes;
}

// Dynamic LDS of gemm_bf16_kernel: the ring, or the five operand slots.
template <class CF, int EPI, bool OF32>
constexpr int kernel_lds() {
  return uses_slots<CF>() ? kPersistentLds : CF::LDS;
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
  if constexpr (uses_slots<CF>()) {
    issue_b<CF, BKM>(smem, S, 0, N, wv);
    issue_a<CF>(smem + kSlotBytes, S, 0, wv);
    if (last >= 1) issue_b<CF, BKM>(smem + 2 * kSlotBytes, S, 1, N, wv);
    int sb = 0, sa = 1;  // slots of the current step's B and A tiles
    for (int kt = 0; kt < nk; ++kt) {
      // step kt's loads have landed once at most the newest requests (B of step kt + 1,
      // if there is one) are outstanding; after the barrier everyone's have, and every
      // wave is done with step kt - 1, whose two slots the requests below reuse. Nothing
      // is requested past the last step (no vector load is outstanding in this loop apart
      // from the DMA, so the count depends on the step only).
      if (kt + 1 <= last)
        wait_vmcnt<CF::B_INST>();
      else
        wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int da = sa + 2 < kSlots ? sa + 2 : sa + 2 - kSlots;  // (2s + 3) % 5
      const int db = sb + 4 < kSlots ? sb + 4 : sb + 4 - kSlots;  // (2s + 4) % 5
      step_compute_issue_split<CF, BKM>(smem + sa * kSlotBytes, smem + sb * kSlotBytes,
                                        smem + da * kSlotBytes, smem + db * kSlotBytes, S, S,
                                        kt + 1, kt + 2, N, kt + 1 <= last, kt + 2 <= last, wv, wm,
                                        wn, lane, acc);
      sa = da;
      sb = sb + 2 < kSlots ? sb + 2 : sb + 2 - kSlots;
    }
  } else {
    constexpr int NS = CF::STAGES;
    static_assert(NS >= 2 && NS <= 4, "ring depth");
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st <= last) issue_stage<CF, BKM>(smem + st * CF::STAGE, S, st, N, wv);
    for (int kt = 0; kt < nk; ++kt) {
      // this thread's loads for step kt have landed once only those of the later steps
      // already requested (up to S-2, none past the last step) are outstanding; after
      // the barrier everyone's have, and every wave is done with step kt-1, whose slot
      // the next request reuses
      const int ahead = last - kt < NS - 2 ? last - kt : NS - 2;
      if (NS > 3 && ahead >= 2)
        wait_vmcnt<CF::LOADS * 2>();
      else if (NS > 2 && ahead >= 1)
        wait_vmcnt<CF::LOADS>();
      else
        wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int nxt = kt + NS - 1;
      step_compute_issue<CF, BKM>(smem + (kt % NS) * CF::STAGE,
                                  smem + ((kt + NS - 1) % NS) * CF::STAGE, S, nxt, N, wv, wm, wn,
                                  lane, acc, nxt <= last);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // bias of this block's columns, staged once in LDS (in the ring, free after the main
  // loop)
  float* sbias = reinterpret_cast<float*>(smem);
  if constexpr (EPI == EPI_BIAS || EPI == EPI_GELU_BIAS) {
    stage_bias<CF>(P, tl, tid, sbias);
    __syncthreads();
  }
  // bf16: lane pairs into 16-byte chunks (non-temporal for the large plain tiles, whose
  // outputs the combine or GEMM-2 stream once); fp32: 16 bytes per lane as they are
  if constexpr (!OF32) {
    store_tile_swapped<CF, EPI, !CF::GATED && CF::BM == 256>(P, tl, wm, wn, lane, sbias, acc);
  } else {
    static_assert(EPI == EPI_STORE, "fp32 output without epilogue math");
    store_tile_f32<CF>(P, tl, wm, wn, lane, acc);
  }
}

// Longest tile list a persistent block holds (one register per lane, 16-bit tile ids).
constexpr int kPersistentListMax = 128;

// Persistent form of the large tile (gated, or plain without bias): one block per CU
// works through a list of tiles. XCD x (hardware blocks x, x+8, ...) owns a contiguous range of logical tiles, so
// the blocks running together on one XCD work on neighbouring tiles, which share weight
// panels in that XCD's L2. At the start the block ranks the non-empty tiles of its XCD's
// range in order (a block-wide prefix count) and keeps those of rank bi, bi + nb_x, ...;
// so skewed groups (many nearly empty experts) still spread evenly over the XCD's blocks.
// The list then moves to registers, since the operand ring takes the whole LDS.
//
// The operand slots (above): the block's steps run on as one stream across its tiles,
// so the requests cross into the block's next tile the same way and its first steps
// stream in while the epilogue of the current one runs. The epilogue needs no LDS and
// no barrier: lanes pair their pieces into 16-byte chunks and store them from registers
// (store_tile_swapped; 128-byte rows for the plain tile). Every tile has at least two
// K steps (the host checks).
template <class CF, int EPI, bool OF32, bool BKM>
__global__ __launch_bounds__(CF::THREADS, 1) void gemm_bf16_persistent_kernel(GemmBatch batch) {
  static_assert(CF::A_BYTES == kSlotBytes && CF::NB * CF::BQ_BYTES == kSlotBytes,
                "one slot per operand tile");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int NB = CF::NB, TM = CF::TM, TN = CF::TN;
  const int nblk = gridDim.x;
  const int x = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int nb_x = (nblk >> 3) + ((nblk & 7) > x ? 1 : 0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  int ranked = 0;  // non-empty tiles in XCD x's range
  {
    const int wv = tid >> 6;
    int* s_list = reinterpret_cast<int*>(smem);
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
  const int nmine = ranked > bi ? (ranked - bi + nb_x - 1) / nb_x : 0;
  if (nmine == 0) return;
  int lst;  // entries lane (low half) and 64 + lane (high half); ids below 2^16
  {
    const int* s_list = reinterpret_cast<const int*>(smem);
    const int e0 = lane < nmine ? s_list[lane] : 0;
    const int e1 = 64 + lane < nmine ? s_list[64 + lane] : 0;
    lst = e0 | (e1 << 16);
  }
  __syncthreads();  // the ring below overwrites the list

  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % CF::WGM, wn = wv / CF::WGM;
  int qi = 0;  // position in the block's tile list
  TileId tl = decode_tile<CF>(batch, list_entry(lst, 0));

  DmaSrc<CF> SA, SB;  // sources of the A requests and of the B requests
  tile_sources<CF, BKM>(batch.p[tl.pi], tl, wv, lane, SA);
  SB = SA;
  int nb = batch.p[tl.pi].N;  // N of the problem the B requests read
  f32x4 acc[NB][TM][TN];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[q][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue_b<CF, BKM>(smem + 0 * kSlotBytes, SB, 0, nb, wv);
  issue_a<CF>(smem + 1 * kSlotBytes, SA, 0, wv);
  issue_b<CF, BKM>(smem + 2 * kSlotBytes, SB, 1, nb, wv);
  int sb = 0, sa = 1;  // slots of the current step's B and A tiles
  while (true) {
    const GemmProblem& P = batch.p[tl.pi];
    const bool more = qi + 1 < nmine;
    // The next tile: its decode, and scalar loads of its row count and of the row map
    // entries of this wave's A rows (its A rows are formed when its first A request is
    // made). No vector load is outstanding in the loop apart from the DMA: the compiler,
    // which does not count DMA requests, would wait for all of them before using a loaded
    // register.
    TileId tl2 = tl;
    int m2 = 0;
    WaveRows<CF> wr2;
    if (more) {
      tl2 = decode_tile_id<CF>(batch, list_entry(lst, qi + 1));
      m2 = group_rows_scalar(batch.p[tl2.pi], tl2);
      wave_row_entries<CF>(batch.p[tl2.pi], tl2, wv, wr2);
    }
    const int nk = P.K / CF::BK;
    // not peeled (a copy of the step body per iteration kind would exhaust the registers)
#pragma clang loop unroll(disable)
    for (int kt = 0; kt < nk; ++kt) {
      // the current step's loads have landed once at most the B loads of the next step
      // (the newest requests) are outstanding; after the barrier everyone's have, and
      // every wave is done with the previous step, whose two slots are reused. One wait
      // count on every step: past the block's last step the B requests repeat that step
      // (into a free slot, never read), so the count stays exact.
      wait_vmcnt<CF::B_INST>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // A one step ahead: the next step of this tile, or the first of the next tile
      int ka = kt + 1;
      bool ia = true;
      if (ka == nk) {
        if (more) {
          tl2.M = m2;
          int rows2[CF::A_INST];
#pragma unroll
          for (int i = 0; i < CF::A_INST; ++i) rows2[i] = a_row_from_entries<CF>(batch.p[tl2.pi], tl2, wv, lane, i, wr2);
          tile_a_sources<CF>(batch.p[tl2.pi], tl2, wv, lane, rows2, SA);
          ka = 0;
        } else {
          ia = false;
        }
      }
      // B two steps ahead (clamped to the last step at the end of the block's tiles)
      int kb = kt + 2;
      if (kb >= nk) {
        if (more) {
          if (kb == nk) {
            tile_b_sources<CF, BKM>(batch.p[tl2.pi], tl2, wv, lane, SB);
            nb = batch.p[tl2.pi].N;
          }
          kb -= nk;
        } else {
          kb = nk - 1;
        }
      }
      const int da = sa + 2 < kSlots ? sa + 2 : sa + 2 - kSlots;  // (2s + 3) % 5
      const int db = sb + 4 < kSlots ? sb + 4 : sb + 4 - kSlots;  // (2s + 4) % 5
      step_compute_issue_split<CF, BKM>(smem + sa * kSlotBytes, smem + sb * kSlotBytes,
                                        smem + da * kSlotBytes, smem + db * kSlotBytes, SA, SB,
                                        ka, kb, nb, ia, true, wv, wm, wn, lane, acc);
      sa = da;
      sb = sb + 2 < kSlots ? sb + 2 : sb + 2 - kSlots;
    }
    // straight from registers, no LDS: the next tile's first requests are in flight.
    // Non-temporal: H and the expert outputs are read once, by the next kernel (H with
    // normal stores held L2 lines the operand loads share: GEMM-1 about 1% slower).
    static_assert((EPI == EPI_SWIGLU || EPI == EPI_STORE) && !OF32, "bf16 SwiGLU or plain tiles");
    store_tile_swapped<CF, EPI, true>(P, tl, wm, wn, lane, nullptr, acc);
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
  wait_vmcnt<0>();  // the repeated tail requests still target LDS
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
  const int grid = b.total < cu_count() ? int(b.total) : cu_count();
  const int nb_min = grid / 8 > 0 ? grid / 8 : 1;  // blocks of the XCD with the fewest
  b.list_cap = (b.xcd_max + nb_min - 1) / nb_min;
  // the slot ring needs two K steps per tile; the list lives in two registers per lane
  bool fits = b.list_cap <= kPersistentListMax && b.total <= 65536 &&
              sizeof(int) * (size_t(b.list_cap) + CF::WAVES) <= size_t(kPersistentLds);
  for (int i = 0; i < b.nprob; ++i) {
    if (b.p[i].K < 2 * CF::BK) fits = false;
    if (b.p[i].row_map && b.p[i].row_map_ld < CF::A_INST * CF::K_RPI) fits = false;
  }
  if (!fits) return launch_cfg<CF, EPI, OF32, BKM>(b, name, s);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(
            reinterpret_cast<const void*>(gemm_bf16_persistent_kernel<CF, EPI, OF32, BKM>),
            hipFuncAttributeMaxDynamicSharedMemorySize, kPersistentLds) != hipSuccess)
      return MOE_ERR_HIP;
    attr_set = true;
  }
  MOE_LAUNCH(name, (gemm_bf16_persistent_kernel<CF, EPI, OF32, BKM>), dim3(grid),
             dim3(CF::THREADS), kPersistentLds, s, b);
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
    case EPI_STORE:
      if constexpr (uses_slots<CF>()) return launch_persistent<CF, EPI_STORE, false, BKM>(b, name, s);
      return launch_cfg<CF, EPI_STORE, false, BKM>(b, name, s);
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
               : launch_epi<TileCfg<128, 128, false, 2, 4, 4>, BKM>(b, name, s);
}
}  // namespace

moe_status_t launch_gemm_bf16(GemmBatch& b, bool gated, const char* name, hipStream_t s) {
  // Large tiles (256 x 256, 16 waves, operand slots) when every problem has enough rows
  // per group and the grid has at least 128 of them (half the CUs: the large tile's
  // higher rate per CU outweighs the idle CUs, e.g. 192 tiles with K = 4096 run in 115 us
  // against 139 us as 640 small tiles); else 128 x 128 tiles. On the large tiles the
  // gated (SwiGLU) GEMM and the plain one without bias run persistent blocks (skipping
  // empty tiles, the next tile's first steps requested during the epilogue); with a bias,
  // one block per tile (the bias is staged in LDS after the K loop).
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
