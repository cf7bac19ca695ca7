// Grouped bf16 GEMM on gfx950 MFMA (v_mfma_f32_16x16x32_bf16), fp32 accumulate.
//
// This is the one dense contraction on the MoE path: each expert's slot buffer times
// its weights ("Module 7", swiglu_expert and the EducationalMoE expert loop, done as
// one grouped launch instead of a loop). Rows of A are gathered by indirection
// (slot -> assignment -> token), so each expert's input rows are assembled directly in
// LDS tiles from x without a separate gather pass.
//
// Tile: 128 x 128 x 64 per 256-thread block, four waves in a 2 x 2 grid, each wave a
// 64 x 64 patch of 4 x 4 MFMA tiles. The gated (SwiGLU) variant carries a second B
// operand and a second accumulator set so that silu(x Wg) * (x Wu) is formed in the
// epilogue and only the product is written.
//
// Operand layouts in LDS: A is [m][k] and B is [n][k] (k contiguous), 128 bytes per
// row, with the 16-byte chunk index XOR-swizzled by (row / 2) % 8 so that the 16 lanes
// reading one MFMA fragment hit 16 distinct bank groups. B arrives from HBM as [k][n]
// (n contiguous); each thread loads a 4 x 8 or 8 x 8 sub-block and transposes it in
// registers before the LDS store.
//
// The MFMA is issued with the B fragment as its first operand, which yields C^T per
// tile: each lane then holds 4 consecutive output columns of one row, so the epilogue
// stores 8 (bf16) or 16 (fp32) contiguous bytes per lane.
//
// Block scheduling: the hardware deals workgroups to the 8 XCDs round-robin; the
// kernel remaps the hardware id so that each XCD works through a contiguous range of
// tiles. Consecutive tiles belong to the same expert, so the tiles of one expert share
// their weight panels in one XCD's L2.

#include "internal.h"

namespace moe {

namespace {

constexpr int BM = kBf16BM, BN = kBf16BN, BK = kBf16BK;
constexpr int kRowBytes = BK * 2;  // 128
constexpr int kTileBytes = BM * kRowBytes;  // 16 KiB

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ int logical_block(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// 2 bf16 (16-bit halves h of words a and b) -> one word: low = a's half, high = b's half.
__device__ __forceinline__ uint32_t pick2(uint32_t a, uint32_t b, int hi) {
  return hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

template <bool GATED>
struct Stage {
  static constexpr int KR = GATED ? 8 : 4;  // k rows per B sub-block
  uint4 a[4];
  uint4 b[KR];
};

}  // namespace

template <bool GATED>
__global__ __launch_bounds__(256, GATED ? 1 : 2) void gemm_bf16_kernel(GemmBatch batch) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NB = GATED ? 2 : 1;
  constexpr int KR = Stage<GATED>::KR;
  constexpr int kStageBytes = kTileBytes * (1 + NB);

  const int lid = logical_block(blockIdx.x, gridDim.x);
  const int pi = (batch.nprob > 1 && lid >= batch.p[0].tiles) ? 1 : 0;
  const GemmProblem& P = batch.p[pi];
  int rem = pi ? lid - batch.p[0].tiles : lid;
  const int per_group = P.m_tiles * P.n_tiles;
  const int g = rem / per_group;
  rem -= g * per_group;
  const int nt = rem / P.m_tiles;
  const int mt = rem - nt * P.m_tiles;
  const int M = P.m_count ? P.m_count[g] : P.m_const;
  const int m0 = mt * BM;
  if (m0 >= M) return;
  const int n0 = nt * BN;
  const int N = P.N;
  const int K = P.K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;

  // ---- A row sources (4 rows per thread, 16 bytes each per stage) ----
  const bf16_t* a_src[4];
  const int a_chunk = tid & 7;
  {
    const bf16_t* Ab = static_cast<const bf16_t*>(P.A) + size_t(g) * P.a_gstride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = m0 + (tid >> 3) + 32 * i;
      if (r >= M) r = m0;
      int src = r;
      if (P.row_map) src = P.row_map[size_t(g) * P.row_map_ld + r] / P.row_div;
      a_src[i] = Ab + size_t(src) * P.lda + a_chunk * 8;
    }
  }
  // ---- B sub-block: KR k-rows x 8 n-columns per thread ----
  const int b_sel = GATED ? (tid >> 7) : 0;
  const int b_t = GATED ? (tid & 127) : tid;
  const int b_nb = b_t & 15;           // n block of 8
  const int b_kb = b_t >> 4;           // k block of KR
  const int b_n = n0 + b_nb * 8;
  const bool b_ok = b_n < N;           // N is a multiple of 8
  const bf16_t* b_src =
      static_cast<const bf16_t*>(b_sel ? P.B1 : P.B0) + size_t(g) * P.b_gstride + (b_ok ? b_n : 0);

  Stage<GATED> st;
  auto load = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.a[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int kk = k0 + b_kb * KR + r;
      st.b[r] = b_ok ? *reinterpret_cast<const uint4*>(b_src + size_t(kk) * N) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
    char* As = smem + buf * kStageBytes;
    char* Bs = As + kTileBytes + b_sel * kTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(As + swz((tid >> 3) + 32 * i, a_chunk)) = st.a[i];
    // transpose KR x 8 -> 8 columns of KR k-values
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int wsel = c >> 1, hi = c & 1;
      uint32_t w[KR / 2];
#pragma unroll
      for (int r = 0; r < KR; r += 2) {
        const uint32_t lo_w = reinterpret_cast<const uint32_t*>(&st.b[r])[wsel];
        const uint32_t hi_w = reinterpret_cast<const uint32_t*>(&st.b[r + 1])[wsel];
        w[r / 2] = pick2(lo_w, hi_w, hi);
      }
      const int n = b_nb * 8 + c;
      if constexpr (KR == 8) {
        *reinterpret_cast<uint4*>(Bs + swz(n, b_kb)) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        *reinterpret_cast<uint2*>(Bs + swz(n, b_kb >> 1) + ((b_kb & 1) << 3)) = make_uint2(w[0], w[1]);
      }
    }
  };

  f32x4 acc[NB][4][4];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[q][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  load(0);
  store(0);
  __syncthreads();
  const int fr = lane & 15, fc = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    const char* As = smem + cur * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[4], bfr[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * 64 + i * 16 + fr, ks * 4 + fc));
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[q][j] = *reinterpret_cast<const bf16x8*>(As + kTileBytes * (1 + q) +
                                                       swz(wn * 64 + j * 16 + fr, ks * 4 + fc));
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[q][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[q][j], af[i], acc[q][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[m][n..n+3] ----
  char* Cb = static_cast<char*>(P.C);
  const int es = P.out_f32 ? 4 : 2;
  const bf16_t* bias = static_cast<const bf16_t*>(P.bias);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 64 + i * 16 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + fc * 4;
      if (n >= N) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[0][i][j][r];
      if (GATED) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = silu(v[r]) * acc[NB - 1][i][j][r];
      } else if (P.epi == EPI_BIAS || P.epi == EPI_GELU_BIAS) {
        if (bias) {
          const uint2 bb = *reinterpret_cast<const uint2*>(bias + size_t(g) * P.bias_gstride + n);
          v[0] += bf16_to_f32(bb.x & 0xffff);
          v[1] += bf16_to_f32(bb.x >> 16);
          v[2] += bf16_to_f32(bb.y & 0xffff);
          v[3] += bf16_to_f32(bb.y >> 16);
        }
        if (P.epi == EPI_GELU_BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = gelu_erf(v[r]);
        }
      }
      char* dst = Cb + (size_t(g) * P.c_gstride + size_t(m) * P.ldc + n) * es;
      if (P.out_f32) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

moe_status_t launch_gemm_bf16(GemmBatch& b, bool gated, const char* name, hipStream_t s) {
  b.total = 0;
  for (int i = 0; i < b.nprob; ++i) {
    GemmProblem& p = b.p[i];
    p.n_tiles = (p.N + BN - 1) / BN;
    p.tiles = p.groups * p.m_tiles * p.n_tiles;
    b.total += p.tiles;
  }
  if (b.total == 0) return MOE_OK;
  const size_t shmem = size_t(2) * kTileBytes * (gated ? 3 : 2);
  static bool attr_set[2] = {false, false};
  if (!attr_set[gated]) {
    hipError_t e = gated ? hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel<true>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem))
                         : hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel<false>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem));
    if (e != hipSuccess) return MOE_ERR_HIP;
    attr_set[gated] = true;
  }
  if (gated) {
    MOE_LAUNCH(name, gemm_bf16_kernel<true>, dim3(b.total), dim3(256), shmem, s, b);
  } else {
    MOE_LAUNCH(name, gemm_bf16_kernel<false>, dim3(b.total), dim3(256), shmem, s, b);
  }
  return MOE_OK;
}

}  // namespace moe
