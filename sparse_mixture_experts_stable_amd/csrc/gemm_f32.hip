// Grouped fp32 GEMM on gfx950 fp32 MFMA (v_mfma_f32_16x16x4_f32). gfx950 has no
// reduced-precision xf32 path, so fp32 experts run on true fp32 matrix cores.
//
// Forward: the fp32 expert MLPs ("Sparse MoE Layer in NumPy", section 2 forward einsum
// for single-linear experts; llm-atlas "Mixture of Experts", Expert; "Module 7",
// swiglu_expert), the gated kernel computing silu(X Wg) * (X Wu) in one pass.
// Backward (the chain rule through those experts; single-linear form in "Sparse MoE
// Layer in NumPy", section 2 moe_backward), with dO = gate * dY on the kept rows:
//   dH   = dO W2^T                           A_ROWS x B_NK
//   Z    = X W1 + b1, then H, dZ             A_ROWS x B_KN, EPI_GELU_BWD / EPI_SWIGLU_BWD
//   dW2  = H^T dO,  dW1 = X^T dZ             A_KROWS x B_KROWS (K = the expert's rows)
//   dX_e = dZ W1^T                           A_ROWS x B_NK (+ EPI_ACCUM for SwiGLU's 2nd)
//
// Tiles of BM x BN x 32 (BM, BN each 64 or 128) per 256-thread block; four waves in
// 2 x 2, each (BM/2) x (BN/2) in 16 x 16 MFMA tiles. An operand keeps its HBM
// orientation in LDS, so every global load is a float4 and every LDS store a float4 (no
// transposition):
//   k-contiguous operands (A_ROWS, B_NK) as [row][k], rows padded to 36 floats: eight
//     threads read one full 128-byte line of a row per k-tile;
//   m/n-contiguous operands (A_KROWS, B_KN, B_KROWS) as [k][m|n], rows padded to 16
//     floats beyond the tile width.
// MFMA step ks (of 8) takes k = 4 ks + lane / 16, so lane l reads the A value
// (row l % 16, that k) and the B value (that k, column l % 16) one float at a time; both
// paddings make these 64-lane reads conflict-free (36 r mod 64 runs over distinct
// multiples of 4; a row of 80 or 144 floats is 16 mod 64, which separates the four k
// rows of one read). The 128-wide tiles read half as many fragment values per MFMA as
// the 64-wide ones, which is what bounds the small tile (LDS read bandwidth). Loads are
// guarded per float4 against M, N and K, so those sizes need only be multiples of 4.

#include "internal.h"

namespace moe {

namespace {
constexpr int BK = 32;
constexpr int KP = BK + 4;  // LDS row of a [row][k] operand (floats)

__device__ __forceinline__ int logical_block_f32(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

__device__ __forceinline__ float4 ld4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ f32x4 ld4v(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// d/dz of z * Phi(z): Phi(z) + z phi(z), with the standard normal cdf / pdf.
__device__ __forceinline__ float gelu_erf_grad(float z) {
  const float pdf = 0.39894228040143267794f * __expf(-0.5f * z * z);
  return normal_cdf(z) + z * pdf;
}
}  // namespace

// SINGLE: one LDS buffer and two barriers per k-tile (half the LDS, so three blocks
// share a CU instead of two); else a double buffer and one barrier.
template <int AM, int BMODE, bool GATED, int BM, int BN, bool SINGLE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Problem P) {
  constexpr int NB = GATED ? 2 : 1;
  constexpr bool AK = AM == A_ROWS;     // A stored [m][k]
  constexpr bool BK_ = BMODE == B_NK;   // B stored [n][k]
  constexpr int NPA = BM + 16, NPB = BN + 16;  // LDS rows of [k][m|n] operands (floats)
  constexpr int A_SZ = AK ? BM * KP : BK * NPA;
  constexpr int B_SZ = BK_ ? BN * KP : BK * NPB;
  constexpr int TM = BM / 32, TN = BN / 32;    // 16 x 16 MFMA tiles per wave
  constexpr int AL = BM / 32, BL = BN / 32;    // float4 loads per thread per k-tile
  static_assert((BM == 64 || BM == 128) && (BN == 64 || BN == 128), "tile size");
  constexpr int NBUF = SINGLE ? 1 : 2;
  __shared__ float As[NBUF][A_SZ];
  __shared__ float Bs[NB][NBUF][B_SZ];
  int lid = logical_block_f32(blockIdx.x, gridDim.x);
  const int per_group = P.m_tiles * P.n_tiles;
  // split K: blocks split * tiles .. + tiles - 1 take k rows [split * k_chunk, + k_chunk)
  const bool split_k = AM == A_KROWS && P.k_splits > 1;
  int split = 0;
  if (split_k) {
    split = lid / (P.groups * per_group);
    lid -= split * (P.groups * per_group);
  }
  const int g = lid / per_group;
  int rem = lid - g * per_group;
  const int nt = rem / P.m_tiles;
  const int mt = rem - nt * P.m_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;

  // sizes
  int M, Kg;
  if (AM == A_ROWS) {
    M = P.g_count ? P.g_count[g] : P.g_const;
    Kg = P.K;
    if (m0 >= M) return;
  } else {
    M = P.M;
    Kg = P.g_count ? P.g_count[g] : P.g_const;
  }
  const int N = P.N;
  int kbeg = 0, kend = Kg;  // this block's k rows
  if (split_k) {
    kbeg = split * P.k_chunk;
    kend = min(Kg, kbeg + P.k_chunk);
  }

  // ---- per-thread load coordinates ----
  // [row][k] operands: row = tid / 8 + 32 h, k quad = tid % 8
  // [k][m|n] operands of width W: k row = tid / (W/4) + (1024 / W) h, quad = tid % (W/4)
  const int kr_row = tid >> 3, kr_q = tid & 7;
  const int am_q = tid % (BM / 4), am_k = tid / (BM / 4);
  const int bn_q = tid % (BN / 4), bn_k = tid / (BN / 4);
  constexpr int AM_STEP = 1024 / BM, BN_STEP = 1024 / BN;

  const float* a_base = P.A + size_t(g) * P.a_gstride;
  const float* a_row_ptr[AL];  // A_ROWS
  if (AM == A_ROWS) {
#pragma unroll
    for (int h = 0; h < AL; ++h) {
      int r = m0 + kr_row + 32 * h;
      if (r >= M) r = m0;
      const int src = P.row_map ? P.row_map[size_t(g) * P.row_map_ld + r] / P.row_div : r;
      a_row_ptr[h] = a_base + size_t(src) * P.lda + kr_q * 4;
    }
  }
  const float* b_base = P.B + size_t(g) * P.b_gstride;
  const float* b1_base = GATED ? P.B1 + size_t(g) * P.b_gstride : nullptr;
  const int* a_map = (AM == A_KROWS && P.row_map) ? P.row_map + size_t(g) * P.row_map_ld : nullptr;
  const int* b_map = (BMODE == B_KROWS && P.b_row_map) ? P.b_row_map + size_t(g) * P.row_map_ld : nullptr;
  const float* b_gate = b_map ? P.gate : nullptr;

  // Staging registers are plain vectors, each filled by one guarded 16-byte load; a
  // zero default keeps the guard a predicated load (no select between addresses, which
  // would turn into generic-address-space loads).
  // Gathered K rows (A_KROWS, B_KROWS): the map entries of a k-tile are fetched one step
  // before its data, and load() first takes them into source rows, then requests the
  // entries of the following k-tile, then the data; the gate of a B row is applied when
  // the row is written to LDS. So no load waits on a load issued in the same step.
  f32x4 ra[AL], rb[NB][BL];
  int ia[AL], ib[BL];  // raw map entries (or k itself without a map) of the next k-tile
  float sc[BL];        // gates of the B rows held in rb
  auto fetch_map = [&](int kt) {
    const int k0 = kbeg + kt * BK;
    if constexpr (AM == A_KROWS) {
#pragma unroll
      for (int h = 0; h < AL; ++h) {
        const int kk = k0 + am_k + AM_STEP * h;
        ia[h] = kk;
        if (a_map && kk < kend) ia[h] = a_map[kk];
      }
    }
    if constexpr (BMODE == B_KROWS) {
#pragma unroll
      for (int h = 0; h < BL; ++h) {
        const int kk = k0 + bn_k + BN_STEP * h;
        ib[h] = kk;
        if (b_map && kk < kend) ib[h] = b_map[kk];
      }
    }
  };
  auto load = [&](int kt, bool fetch_next) {
    const int k0 = kbeg + kt * BK;
    int sa[AL], sb[BL], gb[BL];
    if constexpr (AM == A_KROWS) {
#pragma unroll
      for (int h = 0; h < AL; ++h) sa[h] = a_map ? ia[h] / P.row_div : ia[h];
    }
    if constexpr (BMODE == B_KROWS) {
#pragma unroll
      for (int h = 0; h < BL; ++h) {
        gb[h] = ib[h];
        sb[h] = b_map ? ib[h] / P.row_div : ib[h];
      }
    }
    if ((AM == A_KROWS || BMODE == B_KROWS) && fetch_next) fetch_map(kt + 1);
#pragma unroll
    for (int h = 0; h < AL; ++h) {
      ra[h] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (AM == A_ROWS) {
        if (k0 + kr_q * 4 < kend) ra[h] = ld4v(a_row_ptr[h] + k0);
      } else {
        const int kk = k0 + am_k + AM_STEP * h;
        if (kk < kend && m0 + am_q * 4 < M) ra[h] = ld4v(a_base + size_t(sa[h]) * P.lda + m0 + am_q * 4);
      }
    }
#pragma unroll
    for (int h = 0; h < BL; ++h) {
#pragma unroll
      for (int b = 0; b < NB; ++b) rb[b][h] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (BMODE == B_KN) {
        const int kk = k0 + bn_k + BN_STEP * h;
        const int n = n0 + bn_q * 4;
        if (kk < kend && n < N) {
          rb[0][h] = ld4v(b_base + size_t(kk) * P.ldb + n);
          if constexpr (GATED) rb[NB - 1][h] = ld4v(b1_base + size_t(kk) * P.ldb + n);
        }
      } else if (BMODE == B_NK) {
        const int n = n0 + kr_row + 32 * h;
        const int kq = k0 + kr_q * 4;
        if (n < N && kq < kend) rb[0][h] = ld4v(b_base + size_t(n) * P.ldb + kq);
      } else {
        const int kk = k0 + bn_k + BN_STEP * h;
        const int n = n0 + bn_q * 4;
        sc[h] = 1.f;
        if (kk < kend && n < N) {
          if (b_gate) sc[h] = b_gate[gb[h]];
          rb[0][h] = ld4v(b_base + size_t(sb[h]) * P.ldb + n);
        }
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int h = 0; h < AL; ++h) {
      const int off = AK ? (kr_row + 32 * h) * KP + kr_q * 4 : (am_k + AM_STEP * h) * NPA + am_q * 4;
      *reinterpret_cast<f32x4*>(&As[buf][off]) = ra[h];
    }
#pragma unroll
    for (int h = 0; h < BL; ++h) {
      const int off = BK_ ? (kr_row + 32 * h) * KP + kr_q * 4 : (bn_k + BN_STEP * h) * NPB + bn_q * 4;
      if constexpr (BMODE == B_KROWS) {
        *reinterpret_cast<f32x4*>(&Bs[0][buf][off]) = rb[0][h] * sc[h];
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(&Bs[b][buf][off]) = rb[b][h];
      }
    }
  };

  f32x4 acc[NB][TM][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int fr = lane & 15, fc = lane >> 4;
  if (nk > 0) {
    fetch_map(0);
    load(0, nk > 1);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = SINGLE ? 0 : (kt & 1);
      if (kt + 1 < nk) load(kt + 1, kt + 2 < nk);
#pragma unroll
      for (int ks = 0; ks < BK / 4; ++ks) {
        const int kl = ks * 4 + fc;
        float af[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * (BM / 2) + i * 16 + fr;
          af[i] = As[cur][AK ? row * KP + kl : kl * NPA + row];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float bf[TN];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = wn * (BN / 2) + j * 16 + fr;
            bf[j] = Bs[b][cur][BK_ ? col * KP + kl : kl * NPB + col];
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[b][i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j], af[i], acc[b][i][j], 0, 0, 0);
        }
      }
      if constexpr (SINGLE) {
        __syncthreads();  // every wave is done with the buffer the next k-tile overwrites
        if (kt + 1 < nk) store(0);
      } else {
        if (kt + 1 < nk) store(cur ^ 1);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds C[m][n..n+3] (a split-K block: its partial) ----
  const int epi = P.epi;
  float* Cout = P.C;
  int64_t ldc = P.ldc, c_gstride = P.c_gstride;
  if (split_k) {
    Cout = P.kpart + size_t(split) * P.groups * size_t(P.M) * N;
    ldc = N;
    c_gstride = int64_t(P.M) * N;
  }
  const bool bwd = epi == EPI_GELU_BWD || epi == EPI_SWIGLU_BWD;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * (BM / 2) + i * 16 + fr;
    if (m >= M) continue;
    float rg = 1.f;
    if (bwd && AM == A_ROWS && P.gate && P.row_map)
      rg = P.gate[P.row_map[size_t(g) * P.row_map_ld + m]];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * (BN / 2) + j * 16 + fc * 4;
      if (n >= N) continue;
      const size_t off = size_t(g) * c_gstride + size_t(m) * ldc + n;
      float v[4] = {acc[0][i][j][0], acc[0][i][j][1], acc[0][i][j][2], acc[0][i][j][3]};
      if ((epi == EPI_BIAS || epi == EPI_GELU_BIAS || epi == EPI_GELU_BWD) && P.bias) {
        const float4 bb = ld4(P.bias + size_t(g) * P.bias_gstride + n);
        v[0] += bb.x;
        v[1] += bb.y;
        v[2] += bb.z;
        v[3] += bb.w;
      }
      if (epi == EPI_GELU_BIAS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = gelu_erf(v[r]);
      } else if (epi == EPI_ACCUM) {
        const float4 c = ld4(P.C + off);
        v[0] += c.x;
        v[1] += c.y;
        v[2] += c.z;
        v[3] += c.w;
      } else if (epi == EPI_GELU_BWD) {
        const float4 gi = ld4(P.G + off);
        const float dh[4] = {gi.x * rg, gi.y * rg, gi.z * rg, gi.w * rg};
        float dz[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dz[r] = dh[r] * gelu_erf_grad(v[r]);
          v[r] = gelu_erf(v[r]);
        }
        *reinterpret_cast<float4*>(P.G + off) = make_float4(dz[0], dz[1], dz[2], dz[3]);
      }
      if constexpr (GATED) {
        const float u[4] = {acc[1][i][j][0], acc[1][i][j][1], acc[1][i][j][2], acc[1][i][j][3]};
        if (epi == EPI_SWIGLU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = silu(v[r]) * u[r];
        } else if (epi == EPI_SWIGLU_BWD) {
          const float4 gi = ld4(P.G + off);
          const float dh[4] = {gi.x * rg, gi.y * rg, gi.z * rg, gi.w * rg};
          float da[4], du[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = v[r];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
            const float sa = a * sg;
            du[r] = dh[r] * sa;
            da[r] = dh[r] * u[r] * (sg * (1.0f + a * (1.0f - sg)));
            v[r] = sa * u[r];
          }
          *reinterpret_cast<float4*>(P.G + off) = make_float4(da[0], da[1], da[2], da[3]);
          *reinterpret_cast<float4*>(P.C2 + off) = make_float4(du[0], du[1], du[2], du[3]);
        }
      }
      *reinterpret_cast<float4*>(Cout + off) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Sum of the split-K partials in split order: out[i] = part[0][i] + part[1][i] + ...
__global__ __launch_bounds__(256) void ksum_kernel(const float* __restrict__ part, int splits,
                                                   size_t n4, float* __restrict__ out) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += size_t(gridDim.x) * 256) {
    f32x4 v = ld4v(part + 4 * i);
    for (int q = 1; q < splits; ++q) v += ld4v(part + (size_t(q) * n4 + i) * 4);
    *reinterpret_cast<f32x4*>(out + 4 * i) = v;
  }
}

namespace {
// K split of a constant-K A_KROWS product: enough splits for about two blocks per CU
// (512 blocks), each split keeping at least 512 k rows (16 k-tiles), at most 16 splits.
// The tiles are 128 x 128 when both M and N allow it, else 64 x 64.
struct KSplitPlan {
  int splits, chunk;
  bool big;
};
KSplitPlan ksplit_plan(int groups, int M, int N, int K) {
  KSplitPlan r{1, 0, M >= 128 && N >= 128};
  const int bm = r.big ? 128 : 64;
  const long tiles = long(groups) * ((M + bm - 1) / bm) * ((N + bm - 1) / bm);
  if (tiles <= 0 || tiles >= 256 || K < 1024) return r;
  long sp = (512 + tiles - 1) / tiles;
  if (sp > K / 512) sp = K / 512;
  if (sp > 16) sp = 16;
  if (sp < 2) return r;
  const int chunk = int((K + sp - 1) / sp + BK - 1) / BK * BK;
  r.splits = (K + chunk - 1) / chunk;
  r.chunk = chunk;
  return r;
}

template <int AM, int BMODE, bool GATED, int BM, int BN>
moe_status_t launch_tile(GemmF32Problem& p, const char* name, hipStream_t s) {
  p.m_tiles = (p.m_rows + BM - 1) / BM;
  p.n_tiles = (p.N + BN - 1) / BN;
  p.tiles = p.groups * p.m_tiles * p.n_tiles;
  if (p.tiles == 0) return MOE_OK;
  const int blocks = p.tiles * (p.k_splits > 1 ? p.k_splits : 1);
  // Three blocks per CU (single LDS buffer) pay off for the weight gradients (short,
  // gathered K) and for grids of many blocks; a smaller grid divides better into rounds
  // of two blocks per CU.
  if (AM == A_KROWS || blocks >= 4096)
    MOE_LAUNCH(name, (gemm_f32_kernel<AM, BMODE, GATED, BM, BN, true>), dim3(blocks), dim3(256), 0,
               s, p);
  else
    MOE_LAUNCH(name, (gemm_f32_kernel<AM, BMODE, GATED, BM, BN, false>), dim3(blocks), dim3(256),
               0, s, p);
  return MOE_OK;
}

// 128 x 128 tiles when the grid still holds two of them per CU (they read half as many
// LDS values per MFMA as 64 x 64 tiles); gated products take 128 x 64 (two B matrices).
template <int AM, int BMODE, bool GATED>
moe_status_t launch_sized(GemmF32Problem& p, const char* name, hipStream_t s) {
  const long big = long(p.groups) * ((p.m_rows + 127) / 128) * ((p.N + 127) / 128);
  if (p.m_rows >= 128 && p.N >= 128 && big >= 512) {
    if constexpr (GATED)
      return launch_tile<AM, BMODE, GATED, 128, 64>(p, name, s);
    else
      return launch_tile<AM, BMODE, GATED, 128, 128>(p, name, s);
  }
  return launch_tile<AM, BMODE, GATED, 64, 64>(p, name, s);
}
}  // namespace

moe_status_t launch_gemm_f32(GemmF32Problem& p, int amode, int bmode, const char* name,
                             hipStream_t s) {
  const bool gated = p.epi == EPI_SWIGLU || p.epi == EPI_SWIGLU_BWD;
  if (gated && (!p.B1 || amode != A_ROWS || bmode != B_KN)) return MOE_ERR_UNSUPPORTED;
  if ((p.epi == EPI_GELU_BWD || p.epi == EPI_SWIGLU_BWD) && (!p.G || amode != A_ROWS))
    return MOE_ERR_UNSUPPORTED;
  if (p.epi == EPI_SWIGLU_BWD && !p.C2) return MOE_ERR_UNSUPPORTED;
  if (p.m_rows < 0) return MOE_ERR_INVALID_ARG;
  if (amode == A_ROWS && bmode == B_KN) {
    if (gated) return launch_sized<A_ROWS, B_KN, true>(p, name, s);
    return launch_sized<A_ROWS, B_KN, false>(p, name, s);
  }
  if (amode == A_ROWS && bmode == B_NK) return launch_sized<A_ROWS, B_NK, false>(p, name, s);
  if (amode == A_KROWS && bmode == B_KROWS) {
    p.k_splits = 1;
    p.k_chunk = 0;
    const bool dense_c = p.ldc == p.N && (p.groups == 1 || p.c_gstride == int64_t(p.M) * p.N);
    if (p.kpart && !p.g_count && p.epi == EPI_STORE && dense_c && p.M == p.m_rows) {
      const KSplitPlan kp = ksplit_plan(p.groups, p.M, p.N, p.g_const);
      if (kp.splits > 1) {
        p.k_splits = kp.splits;
        p.k_chunk = kp.chunk;
        const moe_status_t st = kp.big ? launch_tile<A_KROWS, B_KROWS, false, 128, 128>(p, name, s)
                                       : launch_tile<A_KROWS, B_KROWS, false, 64, 64>(p, name, s);
        if (st != MOE_OK || p.tiles == 0) return st;
        const size_t n4 = size_t(p.groups) * p.M * p.N / 4;
        const int grid = int(n4 / 256 < 2048 ? (n4 + 255) / 256 : 2048);
        MOE_LAUNCH("ksum_f32", ksum_kernel, dim3(grid), dim3(256), 0, s, p.kpart, p.k_splits, n4, p.C);
        return MOE_OK;
      }
    }
    return launch_sized<A_KROWS, B_KROWS, false>(p, name, s);
  }
  return MOE_ERR_UNSUPPORTED;
}

size_t f32_kpart_floats(int groups, int M, int N, int K) {
  const KSplitPlan kp = ksplit_plan(groups, M, N, K);
  return kp.splits > 1 ? size_t(kp.splits) * groups * size_t(M) * N : 0;
}

}  // namespace moe
