// Gate-weighted combine and the router-side backward, both HBM-bound.
//
// combine_kernel: y_t = residual_t + shared_t + sum_{j kept} gate_tj * o[e_tj, slot_tj]
// ("Sparse MoE Layer in NumPy", trap 4: dropped choices leave the residual untouched;
// "Top-k MoE Router with Load Statistics", y equation; "32. Sparse MoE Token Dispatch &
// Combine", step 6), accumulated in fp32 in that fixed order and rounded once. Each
// thread owns 16 bytes of one output row; a row's expert outputs are gathered straight
// from the [E, C, D] slot buffers, so no token-ordered copy of them is ever written.
//
// dgate_router_kernel: one wavefront per token ("Sparse MoE Layer in NumPy", section 2
// moe_backward and trap 7):
//   dgate_tj = kept_tj <dy_t, o[e_tj, slot_tj]>
//   dq_j = (dgate_j - sum_r g_r dgate_r) / S_t,  S_t = sum_r p[t, e_tr]
//   dlogits[t, i] = p_i (dp_i - sum_l p_l dp_l), dp[t, e_tj] = dq_j
//   (+ aux_scale * (E / T) p_i (f_i - sum_l f_l p_l), f = count / (T k))
// with the variants of "Module 7. Mixture of Experts": sigmoid scores (S_t sums the
// chosen sigmoid(s), and dlogits[t, e_tj] = dq_j q_j (1 - q_j) without the softmax
// coupling), survivor renormalisation (dgate through the quotient by the kept gate
// mass) and the z-loss term z_scale (2 / T) lse_t p_i.

#include "internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Loads of rows that are read exactly once (the expert output rows): non-temporal, so the
// streamed rows do not evict the rows of x and the shared output the same tokens need.
__device__ __forceinline__ u32x4 load_once(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  typedef float4 Raw;
  __device__ static Raw load_raw(const void* p) {
    const u32x4 q = load_once(p);
    return make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
                       __uint_as_float(q.w));
  }
  __device__ static void fma_raw(float g, const Raw& r, float* acc) {
    acc[0] = fmaf(g, r.x, acc[0]);
    acc[1] = fmaf(g, r.y, acc[1]);
    acc[2] = fmaf(g, r.z, acc[2]);
    acc[3] = fmaf(g, r.w, acc[3]);
  }
  __device__ static void load(const void* p, float* v) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static void store(void* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct Vec<bf16_t> {
  static constexpr int N = 8;
  typedef uint4 Raw;
  __device__ static Raw load_raw(const void* p) {
    const u32x4 q = load_once(p);
    return make_uint4(q.x, q.y, q.z, q.w);
  }
  __device__ static void fma_raw(float g, const Raw& r, float* acc) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(g, __uint_as_float(w[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(g, __uint_as_float(w[i] & 0xffff0000u), acc[2 * i + 1]);
    }
  }
  __device__ static void load(const void* p, float* v) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(void* p, const float* v) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
};

// Expert rows are fetched in batches of KB choices: first the batch's (expert, slot,
// gate) triples, then all its row loads at once (kept packed until used), then the
// fused multiply-adds in choice order, so a token costs ceil(k / KB) dependent round
// trips instead of k. gate == NULL weights every choice by 1 (exact: fma(1, v, acc) is
// acc + v), for expert rows that already carry their gate. With renorm each kept gate
// is divided by the token's kept gate sum ("Module 7. Mixture of Experts",
// dispatch_with_capacity with renormalize_kept_gates). A dropped choice is skipped (not added as zero), so a fully
// dropped token keeps y == residual bit for bit, signed zeros included.
template <typename T, int KB>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ residual,
                                                      const T* __restrict__ shared_out,
                                                      const T* __restrict__ expert_out,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ gate, int T_,
                                                      int k, int E, int C, int D, int64_t ldr,
                                                      int renorm, T* __restrict__ y) {
  constexpr int V = Vec<T>::N;
  const bool dense = slot == nullptr;
  const int per_row = D / V;
  int t, col;
  if (per_row >= 256) {
    const int chunks = per_row / 256;
    t = blockIdx.x / chunks;
    col = ((blockIdx.x % chunks) * 256 + threadIdx.x) * V;
  } else {
    const int rows_per_block = 256 / per_row;
    t = blockIdx.x * rows_per_block + threadIdx.x / per_row;
    col = (threadIdx.x % per_row) * V;
    if (int(threadIdx.x) >= rows_per_block * per_row) return;
  }
  if (t >= T_) return;
  float acc[V];
  if (residual) {
    Vec<T>::load(residual + size_t(t) * ldr + col, acc);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
  }
  if (shared_out) {
    float v[V];
    Vec<T>::load(shared_out + size_t(t) * D + col, v);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += v[i];
  }
  // survivor renormalisation: the token's kept gate mass
  float K = 1.0f;
  if (renorm) {
    K = 0.f;
    for (int j = 0; j < k; ++j) {
      const int e = idx[size_t(t) * k + j];
      const int sl = dense ? 0 : slot[size_t(t) * k + j];
      if (sl >= 0 && sl < C && e >= 0 && e < E) K += gate[size_t(t) * k + j];
    }
  }
  for (int j0 = 0; j0 < k; j0 += KB) {
    int64_t off[KB];
    float g[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      off[b] = -1;
      g[b] = 0.f;
      const int j = j0 + b;
      if (j < k) {
        const int e = idx[size_t(t) * k + j];
        const int sl = dense ? 0 : slot[size_t(t) * k + j];
        if (sl >= 0 && sl < C && e >= 0 && e < E) {
          off[b] = dense ? int64_t(t) * E + e : int64_t(e) * C + sl;
          g[b] = gate ? gate[size_t(t) * k + j] : 1.0f;
          if (renorm) g[b] = g[b] / K;
        }
      }
    }
    typename Vec<T>::Raw v[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b)
      if (off[b] >= 0) v[b] = Vec<T>::load_raw(expert_out + size_t(off[b]) * D + col);
#pragma unroll
    for (int b = 0; b < KB; ++b)
      if (off[b] >= 0) Vec<T>::fma_raw(g[b], v[b], acc);
  }
  Vec<T>::store(y + size_t(t) * D + col, acc);
}

__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const bf16_t* p) { return bf16_to_f32(*p); }

// The same sum for any d_model: one output element per thread, the token's choices
// read by every thread of its row. Used where a row cannot be split into 16-byte
// pieces that tile the 256-thread block evenly.
template <typename T>
__global__ __launch_bounds__(256) void combine_generic_kernel(
    const T* __restrict__ residual, const T* __restrict__ shared_out,
    const T* __restrict__ expert_out, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ slot, const float* __restrict__ gate, int T_, int k, int E,
    int C, int D, int64_t ldr, int renorm, T* __restrict__ y) {
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (g >= int64_t(T_) * D) return;
  const int t = int(g / D), c = int(g - int64_t(t) * D);
  const bool dense = slot == nullptr;
  float acc = residual ? load_f32(residual + size_t(t) * ldr + c) : 0.f;
  if (shared_out) acc += load_f32(shared_out + size_t(t) * D + c);
  float K = 1.0f;
  if (renorm) {
    K = 0.f;
    for (int j = 0; j < k; ++j) {
      const int e = idx[size_t(t) * k + j];
      const int sl = dense ? 0 : slot[size_t(t) * k + j];
      if (sl >= 0 && sl < C && e >= 0 && e < E) K += gate[size_t(t) * k + j];
    }
  }
  for (int j = 0; j < k; ++j) {
    const int e = idx[size_t(t) * k + j];
    const int sl = dense ? 0 : slot[size_t(t) * k + j];
    if (sl < 0 || sl >= C || e < 0 || e >= E) continue;
    float gj = gate ? gate[size_t(t) * k + j] : 1.0f;
    if (renorm) gj = gj / K;
    const int64_t row = dense ? int64_t(t) * E + e : int64_t(e) * C + sl;
    acc = fmaf(gj, load_f32(expert_out + size_t(row) * D + c), acc);
  }
  if constexpr (sizeof(T) == 2) reinterpret_cast<bf16_t*>(y)[size_t(t) * D + c] = f32_to_bf16(acc);
  else y[size_t(t) * D + c] = acc;
}

// Whether the 16-byte combine tiles rows of d_model D: D a multiple of the vector width
// and D / width dividing 256 or a multiple of 256. Otherwise the generic kernel runs.
bool combine_vector_shape(int dt, int D) {
  const int V = dt == MOE_BF16 ? 8 : 4;
  const int per_row = D / V;
  return D % V == 0 && ((per_row >= 256 && per_row % 256 == 0) || (per_row < 256 && 256 % per_row == 0));
}

moe_status_t launch_combine(int dt, const void* residual, int64_t ldr, const void* shared_out,
                            const void* expert_out, const int32_t* idx, const int32_t* slot,
                            const float* gate, int T, int k, int E, int C, int D, int renorm,
                            void* y, hipStream_t s) {
  const int rn = renorm && gate ? 1 : 0;
  // vector loads also need 16-byte aligned rows of the residual
  if (!combine_vector_shape(dt, D) || (residual && ldr % (dt == MOE_BF16 ? 8 : 4))) {
    const int64_t n = int64_t(T) * D;
    const dim3 grid(unsigned((n + 255) / 256));
    if (dt == MOE_BF16) {
      MOE_LAUNCH("combine", combine_generic_kernel<bf16_t>, grid, dim3(256), 0, s,
                 static_cast<const bf16_t*>(residual), static_cast<const bf16_t*>(shared_out),
                 static_cast<const bf16_t*>(expert_out), idx, slot, gate, T, k, E, C, D, ldr, rn,
                 static_cast<bf16_t*>(y));
    } else {
      MOE_LAUNCH("combine", combine_generic_kernel<float>, grid, dim3(256), 0, s,
                 static_cast<const float*>(residual), static_cast<const float*>(shared_out),
                 static_cast<const float*>(expert_out), idx, slot, gate, T, k, E, C, D, ldr, rn,
                 static_cast<float*>(y));
    }
    return MOE_OK;
  }
  const int V = dt == MOE_BF16 ? 8 : 4;
  const int per_row = D / V;
  int blocks;
  if (per_row >= 256) {
    blocks = T * (per_row / 256);
  } else {
    const int rpb = 256 / per_row;
    blocks = (T + rpb - 1) / rpb;
  }
  if (dt == MOE_BF16) {
    MOE_LAUNCH("combine", (combine_kernel<bf16_t, 4>), dim3(blocks), dim3(256), 0, s,
               static_cast<const bf16_t*>(residual), static_cast<const bf16_t*>(shared_out),
               static_cast<const bf16_t*>(expert_out), idx, slot, gate, T, k, E, C, D,
               ldr, rn, static_cast<bf16_t*>(y));
  } else {
    MOE_LAUNCH("combine", (combine_kernel<float, 4>), dim3(blocks), dim3(256), 0, s,
               static_cast<const float*>(residual), static_cast<const float*>(shared_out),
               static_cast<const float*>(expert_out), idx, slot, gate, T, k, E, C, D,
               ldr, rn, static_cast<float*>(y));
  }
  return MOE_OK;
}

// One wavefront per token (4 tokens per block). EPL = experts per lane (E <= 64*EPL).
// Three passes over the token's k choices: d'_j = kept <dy, o_j> (with the kept gate
// mass K and sum_kept g_j d'_j), then dgate_j (d'_j, or with survivor renormalisation
// its quotient-rule image (d'_j - sum_kept g'_r d'_r) / K) with G = sum_j g_j dgate_j,
// then dq_j = (dgate_j - G) / S into the score derivative (softmax Jacobian, or
// q (1 - q) of the chosen sigmoid scores). Aux and z-loss terms are added per expert.
// DQ > 0: the token's dy row is held in registers (DQ float4 per lane, D <= 256 DQ) and
// read from HBM once for all k choices; DQ = 0 streams it again for every choice.
template <int EPL, int DQ>
__global__ __launch_bounds__(256) void dgate_router_kernel(DgateArgs A) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= A.T) return;
  const int k = A.k, E = A.E, C = A.C, D = A.D;
  const bool sig = A.scoring == MOE_SCORE_SIGMOID;
  // softmax row
  const float* row = A.logits + size_t(t) * E;
  float s[EPL], p[EPL], dp[EPL];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    s[i] = e < E ? row[e] : -INFINITY;
    mx = fmaxf(mx, s[i]);
    dp[i] = 0.f;
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    p[i] = e < E ? __expf(s[i] - mx) : 0.f;
    sum += p[i];
  }
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
#pragma unroll
  for (int i = 0; i < EPL; ++i) p[i] *= inv;

  // pass 1: d'_j kept in lane (j % 64), register slot j / 64 (k <= 256); S over the
  // chosen clean scores; K and sum_kept g d' for the survivor quotient
  const float* dyr = A.dy + size_t(t) * D;
  const int32_t* idr = A.idx + size_t(t) * k;
  const int32_t* slr = A.slot + size_t(t) * k;
  const float* gr = A.gate + size_t(t) * k;
  float S = 0.f, K = 0.f, Gk = 0.f;
  float dreg[4] = {0.f, 0.f, 0.f, 0.f};
  float4 dyv[DQ > 0 ? DQ : 1];
#pragma unroll
  for (int q = 0; q < DQ; ++q) {
    const int c = lane * 4 + 256 * q;
    dyv[q] = c < D ? *reinterpret_cast<const float4*>(dyr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // choice metadata: with k <= 64, lane j holds choice j's expert, slot and gate, which
  // every lane reads back with readlane, so no round waits on a load of its own
  const bool meta_in_lanes = k <= 64;
  int me = 0, msl = -1;
  float mg = 0.f;
  if (meta_in_lanes && lane < k) {
    me = idr[lane];
    msl = slr[lane];
    mg = gr[lane];
  }
  auto choice = [&](int j, int& e, int& sl, float& g) {
    if (meta_in_lanes) {
      e = __builtin_amdgcn_readlane(me, j);
      sl = __builtin_amdgcn_readlane(msl, j);
      g = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mg), j));
    } else {
      e = idr[j];
      sl = slr[j];
      g = gr[j];
    }
  };
  // <dy, o_j> of this lane's columns
  auto dot_part = [&](const float* orow) {
    float d = 0.f;
    if constexpr (DQ > 0) {
      float4 ov[DQ];
#pragma unroll
      for (int q = 0; q < DQ; ++q) {
        const int c = lane * 4 + 256 * q;
        ov[q] = c < D ? *reinterpret_cast<const float4*>(orow + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int q = 0; q < DQ; ++q) {
        if (lane * 4 + 256 * q < D) {
          d = fmaf(dyv[q].x, ov[q].x, d);
          d = fmaf(dyv[q].y, ov[q].y, d);
          d = fmaf(dyv[q].z, ov[q].z, d);
          d = fmaf(dyv[q].w, ov[q].w, d);
        }
      }
    } else {
      for (int c = lane * 4; c < D; c += 256) {
        const float4 a = *reinterpret_cast<const float4*>(dyr + c);
        const float4 b = *reinterpret_cast<const float4*>(orow + c);
        d = fmaf(a.x, b.x, d);
        d = fmaf(a.y, b.y, d);
        d = fmaf(a.z, b.z, d);
        d = fmaf(a.w, b.w, d);
      }
    }
    return d;
  };
  // the sums over choices, in choice order
  auto account = [&](int j, int e, bool kept, float g, float d) {
    if (kept) {
      K += g;
      Gk += g * d;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lane == (j & 63) && r == (j >> 6)) dreg[r] = d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i == (e >> 6)) q = sig ? s[i] : p[i];
    q = __shfl(q, e & 63, kWave);
    if (sig) q = 1.0f / (1.0f + __expf(-q));
    S += q;
  };
  // two choices per round: both expert rows are requested before either is reduced
  for (int j = 0; j < k; j += 2) {
    const bool two = j + 1 < k;
    int e0, sl0, e1 = 0, sl1 = -1;
    float g0, g1 = 0.f;
    choice(j, e0, sl0, g0);
    if (two) choice(j + 1, e1, sl1, g1);
    const bool kept0 = sl0 >= 0 && sl0 < C;
    const bool kept1 = two && sl1 >= 0 && sl1 < C;
    float d0 = kept0 ? dot_part(A.o + (size_t(e0) * C + sl0) * D) : 0.f;
    float d1 = kept1 ? dot_part(A.o + (size_t(e1) * C + sl1) * D) : 0.f;
    if (kept0) d0 = wave_sum(d0);
    if (kept1) d1 = wave_sum(d1);
    account(j, e0, kept0, g0, d0);
    if (two) account(j + 1, e1, kept1, g1, d1);
  }
  // pass 2: dgate_j and G = sum_j g_j dgate_j; effective gates
  float G = 0.f;
  for (int j = 0; j < k; ++j) {
    float dv = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r == (j >> 6)) dv = dreg[r];
    float d = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(dv), j & 63));
    int e, sl;
    float g;
    choice(j, e, sl, g);
    const bool kept = sl >= 0 && sl < C;
    if (A.renorm) d = (kept && K > 0.f) ? (d - Gk / K) / K : 0.f;
    G += g * d;
    if (lane == 0) {
      A.dgate[size_t(t) * k + j] = d;
      if (A.eff_gate)
        A.eff_gate[size_t(t) * k + j] = kept ? (A.renorm ? (K > 0.f ? g / K : 0.f) : g) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lane == (j & 63) && r == (j >> 6)) dreg[r] = d;
  }
  // pass 3: dq_j into the score derivative at the chosen experts
  for (int j = 0; j < k; ++j) {
    int e, sl;
    float g;
    choice(j, e, sl, g);
    float dv = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r == (j >> 6)) dv = dreg[r];
    const float d = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(dv), j & 63));
    const float dq = (d - G) / S;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (lane + 64 * i == e) {
        if (sig) {
          const float q = 1.0f / (1.0f + __expf(-s[i]));
          dp[i] += dq * q * (1.0f - q);
        } else {
          dp[i] += dq;
        }
      }
    }
  }
  float pdp = 0.f;
  if (!sig) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) pdp += p[i] * dp[i];
    pdp = wave_sum(pdp);
  }
  float pf = 0.f;
  float f[EPL];
  if (A.aux_scale != 0.f) {
    const float inv_tk = 1.0f / (float(A.T) * float(k));
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      f[i] = e < E ? float(A.count[e]) * inv_tk : 0.f;
      pf += p[i] * f[i];
    }
    pf = wave_sum(pf);
  }
  const float zc = A.z_scale != 0.f ? A.z_scale * (2.0f / float(A.T)) * (mx + __logf(sum)) : 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) continue;
    float v = sig ? dp[i] : p[i] * (dp[i] - pdp);
    if (A.aux_scale != 0.f) v += A.aux_scale * (float(E) / float(A.T)) * p[i] * (f[i] - pf);
    if (A.z_scale != 0.f) v += zc * p[i];
    A.dlogits[size_t(t) * E + e] = v;
  }
}

moe_status_t launch_dgate_router_bwd(const DgateArgs& a, hipStream_t s) {
  const dim3 grid((a.T + 3) / 4), block(256);
#define MOE_DGQ(EPLV, DQV) \
  MOE_LAUNCH("dgate_router_bwd", (dgate_router_kernel<EPLV, DQV>), grid, block, 0, s, a)
#define MOE_DG(EPLV)          \
  if (a.D <= 1024) {          \
    MOE_DGQ(EPLV, 4);         \
  } else if (a.D <= 2048) {   \
    MOE_DGQ(EPLV, 8);         \
  } else {                    \
    MOE_DGQ(EPLV, 0);         \
  }
  if (a.E <= 64) {
    MOE_DG(1);
  } else if (a.E <= 128) {
    MOE_DG(2);
  } else if (a.E <= 256) {
    MOE_DG(4);
  } else if (a.E <= 512) {
    MOE_DG(8);
  } else {
    MOE_DG(16);
  }
#undef MOE_DG
#undef MOE_DGQ
  return MOE_OK;
}

// ---- bias gradients: grouped column sums -------------------------------------------
// Stage 1: block (x, c, g) sums rows [c*kColRows, (c+1)*kColRows) of group g for 1024
// columns (4 per thread), in row order, into part[g][c][n]. Stage 2 adds the chunks in
// chunk order. The result depends only on the shapes, never on scheduling.
namespace {
constexpr int kColRows = 64;
inline int col_chunks(int max_rows) { return (max_rows + kColRows - 1) / kColRows; }
}  // namespace

size_t colsum_part_floats(int groups, int max_rows, int N) {
  return size_t(groups) * (col_chunks(max_rows) > 0 ? col_chunks(max_rows) : 1) * N;
}

__global__ __launch_bounds__(256) void colsum_part_kernel(
    const float* __restrict__ src, int64_t ld, int64_t gstride, const int32_t* __restrict__ map,
    int32_t map_ld, int32_t div, const float* __restrict__ gate,
    const int32_t* __restrict__ g_count, int32_t g_const, int N, float* __restrict__ part) {
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int c = blockIdx.y, g = blockIdx.z, nch = gridDim.y;
  if (n >= N) return;
  const int Mg = g_count ? g_count[g] : g_const;
  const int r0 = c * kColRows;
  const int r1 = min(r0 + kColRows, Mg);
  const float* base = src + size_t(g) * gstride + n;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int r = r0; r < r1; ++r) {
    int row = r;
    float sc = 1.f;
    if (map) {
      const int a = map[size_t(g) * map_ld + r];
      row = a / div;
      if (gate) sc = gate[a];
    }
    const float4 v = *reinterpret_cast<const float4*>(base + size_t(row) * ld);
    acc.x += sc * v.x;
    acc.y += sc * v.y;
    acc.z += sc * v.z;
    acc.w += sc * v.w;
  }
  *reinterpret_cast<float4*>(part + (size_t(g) * nch + c) * N + n) = acc;
}

__global__ __launch_bounds__(256) void colsum_finish_kernel(const float* __restrict__ part,
                                                            int nch, int N,
                                                            float* __restrict__ out,
                                                            int64_t out_gstride) {
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int g = blockIdx.y;
  if (n >= N) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < nch; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(part + (size_t(g) * nch + c) * N + n);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>(out + size_t(g) * out_gstride + n) = acc;
}

moe_status_t launch_colsum(const float* src, int64_t ld, int64_t gstride, const int32_t* map,
                           int32_t map_ld, int32_t div, const float* gate,
                           const int32_t* g_count, int32_t g_const, int max_rows, int groups,
                           int N, float* part, float* out, int64_t out_gstride, hipStream_t s) {
  if (groups < 1 || N < 1) return MOE_OK;
  if (N % 4 || max_rows < 0) return MOE_ERR_UNSUPPORTED;
  const int nch = col_chunks(max_rows) > 0 ? col_chunks(max_rows) : 1;
  const int xb = (N + 1023) / 1024;
  MOE_LAUNCH("colsum_part", colsum_part_kernel, dim3(xb, nch, groups), dim3(256), 0, s, src, ld,
             gstride, map, map_ld, div, gate, g_count, g_const, N, part);
  MOE_LAUNCH("colsum_finish", colsum_finish_kernel, dim3(xb, groups), dim3(256), 0, s, part, nch,
             N, out, out_gstride);
  return MOE_OK;
}

}  // namespace moe
