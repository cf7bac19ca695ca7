// Grouped fp32 GEMM on gfx950 fp32 MFMA (v_mfma_f32_16x16x4_f32). gfx950 has no
// reduced-precision xf32 path, so fp32 experts run on true fp32 matrix cores.
//
// Used for the fp32 expert MLPs ("Sparse MoE Layer in NumPy", section 2 forward
// einsum for single-linear experts; llm-atlas "Mixture of Experts", Expert) and for the
// two GEMMs of the single-linear backward (same page, section 2 moe_backward):
//   dX_e = (dY rows of e) W_e^T               A_ROWS x B_NK  (rows gathered by slot)
//   dW_e = X_e^T (gate * dY_e)                A_KROWS x B_KROWS_GATE (K gathered)
//
// Tile 64 x 64 x 16 per 256-thread block; four waves in 2 x 2, each 32 x 32 (2 x 2
// MFMA tiles). LDS holds A as [k][m] and B as [k][n] (m / n contiguous, rows padded to
// 68 floats), so every fragment read is one conflict-free 4-byte read per lane; operands
// that arrive k-contiguous from HBM are transposed on the LDS store.

#include "internal.h"

namespace moe {

namespace {
constexpr int BM = kF32BM, BN = kF32BN, BK = kF32BK;
constexpr int LDP = 68;  // padded LDS row (floats)

__device__ __forceinline__ int logical_block_f32(int bid, int nblk) {
  const int q = nblk >> 3, r = nblk & 7;
  const int x = bid & 7, i = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}
}  // namespace

template <int AM, int BMODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Problem P) {
  __shared__ float As[2][BK][LDP];
  __shared__ float Bs[2][BK][LDP];
  const int lid = logical_block_f32(blockIdx.x, gridDim.x);
  const int per_group = P.m_tiles * P.n_tiles;
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

  // ---- per-thread load coordinates ----
  // transposing loads (k contiguous in HBM): row = tid / 4, k quad = tid % 4
  // direct loads (m / n contiguous in HBM): k row = tid / 16, quad = tid % 16
  const int tr_row = tid >> 2, tr_kq = tid & 3;
  const int dr_k = tid >> 4, dr_q = tid & 15;

  const float* a_row_ptr = nullptr;  // A_ROWS
  if (AM == A_ROWS) {
    int r = m0 + tr_row;
    if (r >= M) r = m0;
    int src = P.row_map ? P.row_map[size_t(g) * P.row_map_ld + r] / P.row_div : r;
    a_row_ptr = P.A + size_t(g) * P.a_gstride + size_t(src) * P.lda + tr_kq * 4;
  }
  const float* b_base = P.B + size_t(g) * P.b_gstride;

  float4 ra, rb;
  auto load = [&](int kt) {
    const int k0 = kt * BK;
    if (AM == A_ROWS) {
      ra = *reinterpret_cast<const float4*>(a_row_ptr + k0);
    } else {
      const int kk = k0 + dr_k;
      if (kk < Kg && m0 + dr_q * 4 < M) {
        const int a = P.row_map[size_t(g) * P.row_map_ld + kk];
        ra = *reinterpret_cast<const float4*>(P.A + size_t(a / P.row_div) * P.lda + m0 + dr_q * 4);
      } else {
        ra = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    if (BMODE == B_KN) {
      const int kk = k0 + dr_k;
      const int n = n0 + dr_q * 4;
      rb = (n < N) ? *reinterpret_cast<const float4*>(b_base + size_t(kk) * P.ldb + n)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    } else if (BMODE == B_NK) {
      const int n = n0 + tr_row;
      rb = (n < N) ? *reinterpret_cast<const float4*>(b_base + size_t(n) * P.ldb + k0 + tr_kq * 4)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      const int kk = k0 + dr_k;
      if (kk < Kg && n0 + dr_q * 4 < N) {
        const int a = P.row_map[size_t(g) * P.row_map_ld + kk];
        const float gs = P.gate[a];
        float4 v = *reinterpret_cast<const float4*>(P.B + size_t(a / P.row_div) * P.ldb + n0 + dr_q * 4);
        rb = make_float4(v.x * gs, v.y * gs, v.z * gs, v.w * gs);
      } else {
        rb = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto store = [&](int buf) {
    if (AM == A_ROWS) {
      As[buf][tr_kq * 4 + 0][tr_row] = ra.x;
      As[buf][tr_kq * 4 + 1][tr_row] = ra.y;
      As[buf][tr_kq * 4 + 2][tr_row] = ra.z;
      As[buf][tr_kq * 4 + 3][tr_row] = ra.w;
    } else {
      *reinterpret_cast<float4*>(&As[buf][dr_k][dr_q * 4]) = ra;
    }
    if (BMODE == B_NK) {
      Bs[buf][tr_kq * 4 + 0][tr_row] = rb.x;
      Bs[buf][tr_kq * 4 + 1][tr_row] = rb.y;
      Bs[buf][tr_kq * 4 + 2][tr_row] = rb.z;
      Bs[buf][tr_kq * 4 + 3][tr_row] = rb.w;
    } else {
      *reinterpret_cast<float4*>(&Bs[buf][dr_k][dr_q * 4]) = rb;
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (Kg + BK - 1) / BK;
  const int fr = lane & 15, fc = lane >> 4;
  if (nk > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) load(kt + 1);
#pragma unroll
      for (int ks = 0; ks < BK / 4; ++ks) {
        float af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = As[cur][ks * 4 + fc][wm * 32 + i * 16 + fr];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = Bs[cur][ks * 4 + fc][wn * 32 + j * 16 + fr];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j], af[i], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds C[m][n..n+3] ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 32 + i * 16 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 32 + j * 16 + fc * 4;
      if (n >= N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (P.epi == EPI_BIAS || P.epi == EPI_GELU_BIAS) {
        if (P.bias) {
          const float4 bb = *reinterpret_cast<const float4*>(P.bias + size_t(g) * P.bias_gstride + n);
          v[0] += bb.x;
          v[1] += bb.y;
          v[2] += bb.z;
          v[3] += bb.w;
        }
        if (P.epi == EPI_GELU_BIAS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = gelu_erf(v[r]);
        }
      }
      float* dst = P.C + size_t(g) * P.c_gstride + size_t(m) * P.ldc + n;
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

moe_status_t launch_gemm_f32(GemmF32Problem& p, int amode, int bmode, const char* name,
                             hipStream_t s) {
  p.n_tiles = (p.N + BN - 1) / BN;
  p.tiles = p.groups * p.m_tiles * p.n_tiles;
  if (p.tiles == 0) return MOE_OK;
  const dim3 grid(p.tiles), block(256);
  if (amode == A_ROWS && bmode == B_KN) {
    MOE_LAUNCH(name, (gemm_f32_kernel<A_ROWS, B_KN>), grid, block, 0, s, p);
  } else if (amode == A_ROWS && bmode == B_NK) {
    MOE_LAUNCH(name, (gemm_f32_kernel<A_ROWS, B_NK>), grid, block, 0, s, p);
  } else if (amode == A_KROWS && bmode == B_KROWS_GATE) {
    MOE_LAUNCH(name, (gemm_f32_kernel<A_KROWS, B_KROWS_GATE>), grid, block, 0, s, p);
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

}  // namespace moe
