// Routing and position-priority dispatch for gfx950.
//
// route_kernel     fp32 softmax over the E logits of a token, top-k by logit with exact
//                  ties to the lower expert index, gates renormalised over the k
//                  choices ("Top-k MoE Router with Load Statistics", alpha equation;
//                  "Sparse MoE Layer in NumPy", top_k_gating), plus per-block pre-drop
//                  counts and probability sums (trap 6 of the same page). A token is
//                  handled by a group of L lanes (8..64) holding V <= 16 logits each, so
//                  a wavefront works on 64/L tokens at once and every reduction stays
//                  inside the group. The variants of "Module 7. Mixture of Experts"
//                  (route_logits, router_z_loss): a selection bias added to the fp32
//                  clean score in the top-k key only; sigmoid scoring with gates
//                  normalised in log space; per-block sums of lse_t^2 for the z-loss.
// count_kernel     per-block expert histogram of caller-supplied choices.
// chunk_sum        per chunk of kScanRows routing blocks, the per-expert sums.
// scan_kernel      one block: per expert, the exclusive scan of the chunk sums in chunk
//                  order, totals, used/overflow, prob_sum, and the aux loss, all summed
//                  in a fixed order (bitwise reproducible, no atomics or fences).
// assign_kernel    slots: a stable rank of each assignment among earlier assignments to
//                  the same expert inside the block (wave ballots, then a per-wave
//                  prefix), plus the block's scanned offset. This reproduces the serial
//                  token-then-choice loop of position_priority_dispatch ("Sparse MoE
//                  Layer in NumPy", trap 3) exactly. The grid also writes -1 into the
//                  unfilled tail of every expert's slot table.
//
// Per-block partial arrays are block-major, [nb][E], so every block writes and the scan
// reads whole rows.

#include "internal.h"

namespace moe {

RouteWs carve_route_ws(void* ws, int T, int E) {
  RouteWs w;
  const int nb = route_blocks(T);
  char* p = static_cast<char*>(ws);
  size_t off = 0;
  w.flags = reinterpret_cast<int32_t*>(p + off);
  off += 256;
  w.cnt_part = reinterpret_cast<int32_t*>(p + off);
  off = align_up(off + sizeof(int32_t) * size_t(E) * nb, 256);
  w.prob_part = reinterpret_cast<float*>(p + off);
  off = align_up(off + sizeof(float) * size_t(E) * nb, 256);
  const int nc = scan_chunks(T);
  w.chunk_cnt = reinterpret_cast<int32_t*>(p + off);
  off = align_up(off + sizeof(int32_t) * size_t(E) * nc, 256);
  w.chunk_prob = reinterpret_cast<float*>(p + off);
  off = align_up(off + sizeof(float) * size_t(E) * nc, 256);
  w.chunk_off = reinterpret_cast<int32_t*>(p + off);
  off = align_up(off + sizeof(int32_t) * size_t(E) * nc, 256);
  w.fp = reinterpret_cast<float*>(p + off);
  off = align_up(off + sizeof(float) * size_t(E), 256);
  w.zpart = reinterpret_cast<float*>(p + off);
  off = align_up(off + sizeof(float) * size_t(nb), 256);
  w.bytes = off;
  return w;
}

namespace {

// Logistic function without overflow, and log(sigmoid(s)) = min(s, 0) - log(1 + e^-|s|),
// finite for every finite s ("Module 7. Mixture of Experts", stable_sigmoid and
// _log_sigmoid).
__device__ __forceinline__ float sigmoid_stable(float s) {
  if (s >= 0.f) return 1.0f / (1.0f + __expf(-s));
  const float e = __expf(s);
  return e / (1.0f + e);
}
__device__ __forceinline__ float log_sigmoid(float s) {
  return fminf(s, 0.f) - log1pf(__expf(-fabsf(s)));
}

// Lane exchanges inside 16-lane rows (DPP): quad permutations [1,0,3,2] and [2,3,0,1],
// the half-row mirror (lane i <-> 7 - i) and the row mirror (i <-> 15 - i).
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141,
              kDppRowMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float(dpp32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return (uint64_t(dpp32<CTRL>(uint32_t(v >> 32))) << 32) | dpp32<CTRL>(uint32_t(v));
}
struct MaxF {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumF {
  __device__ float operator()(float a, float b) const { return a + b; }
};
struct MaxU64 {
  __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return b > a ? b : a; }
};
template <int CTRL, class T>
__device__ __forceinline__ T dpp_any(T v) {
  if constexpr (sizeof(T) == 8) return dpp_u64<CTRL>(v);
  else return dpp_f<CTRL>(v);
}
// All-reduce over aligned groups of L lanes (L a power of two): partner exchanges inside
// each 16-lane row through DPP (pairs, quads, the two quads of a half-row, the two halves
// of a row), then cross-row shuffles. At every step the two partners combine the same two
// values, so every lane of the group ends with the same result, bit for bit.
template <int L, class OP, class T>
__device__ __forceinline__ T group_reduce(T v, OP op) {
  if constexpr (L >= 2) v = op(v, dpp_any<kDppQuadXor1>(v));
  if constexpr (L >= 4) v = op(v, dpp_any<kDppQuadXor2>(v));
  if constexpr (L >= 8) v = op(v, dpp_any<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = op(v, dpp_any<kDppRowMirror>(v));
  if constexpr (L >= 32) v = op(v, T(__shfl_xor(v, 16, L)));
  if constexpr (L >= 64) v = op(v, T(__shfl_xor(v, 32, L)));
  return v;
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
  return group_reduce<L>(v, MaxF{});
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  return group_reduce<L>(v, SumF{});
}
template <int L>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  return group_reduce<L>(v, MaxU64{});
}
// Inverse of orderable() (negative zero comes back as +0).
__device__ __forceinline__ float from_orderable(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

}  // namespace

// L lanes per token, V logits per lane (E <= L*V), KR result slots per lane (k <= L*KR),
// NT threads per block (NT / L tokens per round; the block's kRouteTokens tokens take
// kRouteTokens * L / NT rounds, one when NT = kRouteTokens * L, so more waves are in
// flight for the latency-bound selection rounds).
// VAR: the router variants are compiled in (sigmoid scoring, selection bias, z partials,
// chosen at run time from o); without it the kernel is the plain softmax router.
template <int L, int V, int KR, bool VAR, int NT>
__global__ __launch_bounds__(NT) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ gate_out,
                                                    int32_t* __restrict__ cnt_part,
                                                    float* __restrict__ prob_part, RouteOpts o,
                                                    float* __restrict__ zpart) {
  constexpr int TPR = NT / L;  // tokens per round of the block
  static_assert(kRouteTokens % TPR == 0, "whole rounds");
  __shared__ int s_hist[L * V];
  __shared__ float s_prob[TPR][L * V];
  __shared__ float s_z[TPR];
  // rows of E fp32 logits start 16-byte aligned when E % 4 == 0 (logits is)
  const bool vec_rows = V % 4 == 0 && (E & 3) == 0;
  const bool sig = VAR && o.scoring == MOE_SCORE_SIGMOID;
  const bool with_z = VAR && o.with_z;
  const float* bias = VAR ? o.bias : nullptr;
  float zacc = 0.f;
  const int tid = threadIdx.x;
  const int grp = tid / L;
  const int li = tid % L;
  for (int e = tid; e < L * V; e += NT) s_hist[e] = 0;
  __syncthreads();

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;

  const int t0 = blockIdx.x * kRouteTokens;
  for (int r = 0; r < kRouteTokens / TPR; ++r) {
    const int t = t0 + r * TPR + grp;
    if (t >= T) break;  // uniform across the group
    const float* row = logits + size_t(t) * E + li * V;
    float s[V];
    if (vec_rows && li * V + V <= E) {
      // the lane's V logits are in range and 16-byte aligned: V / 4 vector loads
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(row + i);
        s[i] = q[0];
        s[i + 1] = q[1];
        s[i + 2] = q[2];
        s[i + 3] = q[3];
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) s[i] = (li * V + i < E) ? row[i] : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < V; ++i) mx = fmaxf(mx, s[i]);
    mx = group_max<L>(mx);
    float p[V];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      p[i] = (li * V + i < E) ? __expf(s[i] - mx) : 0.f;
      sum += p[i];
    }
    sum = group_sum<L>(sum);
    const float inv = 1.0f / sum;
    if (with_z) {
      const float lse = mx + __logf(sum);
      zacc = fmaf(lse, lse, zacc);
    }
    uint64_t key[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      p[i] *= inv;
      acc[i] += p[i];
      const int e = li * V + i;
      float kv = s[i];
      if (bias && e < E) kv = (sig ? sigmoid_stable(s[i]) : p[i]) + bias[e];
      key[i] = (e < E) ? ((uint64_t(orderable(kv)) << 32) | uint32_t(0xffffffffu - uint32_t(e))) : 0ull;
    }

    int my_e[KR];
    float my_p[KR];
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      my_e[q] = 0;
      my_p[q] = 0.f;
    }
    // Selection: each lane keeps its best remaining key; a round takes the group maximum,
    // and only the lane that held it retires that key (its high word cleared, which
    // ranks it below every live key) and finds its next best.
    auto lane_best = [&]() {
      uint64_t b = key[0];
#pragma unroll
      for (int i = 1; i < V; ++i) b = key[i] > b ? key[i] : b;
      return b;
    };
    uint64_t lb = lane_best();
    float gsum = 0.f;
    for (int j = 0; j < k; ++j) {
      const uint64_t best = group_max_u64<L>(lb);
      const int e = int(0xffffffffu - uint32_t(best));
      float pe;
      if (!bias && !sig) {
        // the key holds the logit: every lane forms p_e exactly as the owner did
        pe = __expf(from_orderable(uint32_t(best >> 32)) - mx) * inv;
      } else {
        const int owner = e / V;
        const int si = e - owner * V;
        float pv = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (li == owner && i == si) pv = sig ? log_sigmoid(s[i]) : p[i];
        pe = __shfl(pv, owner, L);
      }
      if (lb == best) {
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (uint32_t(key[i]) == uint32_t(best)) key[i] &= 0xffffffffull;
        lb = lane_best();
      }
      gsum += pe;
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        if (li == (j % L) && q == (j / L)) {
          my_e[q] = e;
          my_p[q] = pe;
        }
      }
    }
    if (sig) {
      // gates = softmax over the chosen experts of log sigmoid(s)
      float lm = -INFINITY;
#pragma unroll
      for (int q = 0; q < KR; ++q)
        if (li + L * q < k) lm = fmaxf(lm, my_p[q]);
      lm = group_max<L>(lm);
      float ws = 0.f;
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        if (li + L * q < k) {
          my_p[q] = __expf(my_p[q] - lm);
          ws += my_p[q];
        }
      }
      gsum = group_sum<L>(ws);
    }
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      const int j = li + L * q;
      if (j < k) {
        idx_out[size_t(t) * k + j] = my_e[q];
        gate_out[size_t(t) * k + j] = my_p[q] / gsum;
        atomicAdd(&s_hist[my_e[q]], 1);
      }
    }
  }
  if (li == 0) s_z[grp] = zacc;

#pragma unroll
  for (int i = 0; i < V; ++i) s_prob[grp][li * V + i] = acc[i];
  __syncthreads();
  const size_t base = size_t(blockIdx.x) * E;
  for (int e = tid; e < E; e += NT) {
    float v = 0.f;
    for (int g2 = 0; g2 < TPR; ++g2) v += s_prob[g2][e];
    prob_part[base + e] = v;
    cnt_part[base + e] = s_hist[e];
  }
  if (with_z && tid == 0) {
    float z = 0.f;
    for (int g2 = 0; g2 < TPR; ++g2) z += s_z[g2];
    zpart[blockIdx.x] = z;
  }
}

// Per-block expert histogram over the same token partition as route_kernel. Indices
// outside [0, E) are skipped here and reported by assign_kernel.
__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int T,
                                                    int k, int E,
                                                    int32_t* __restrict__ cnt_part) {
  extern __shared__ int s_cnt[];
  for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kRouteTokens;
  const int t1 = min(T, t0 + kRouteTokens);
  for (int a = t0 * k + threadIdx.x; a < t1 * k; a += 256) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) cnt_part[size_t(blockIdx.x) * E + e] = s_cnt[e];
}

// Chunk sums: block c adds the per-block partials of routing blocks c*kScanRows ..
// (c+1)*kScanRows - 1 (in block order) for every expert.
// flags_reset != NULL: clear the error word here (the scan that would clear it runs
// inside the assignment kernel, whose blocks may set it).
__global__ __launch_bounds__(256) void chunk_sum_kernel(const int32_t* __restrict__ cnt_part,
                                                        const float* __restrict__ prob_part,
                                                        int nb, int E, int with_prob,
                                                        int32_t* __restrict__ chunk_cnt,
                                                        float* __restrict__ chunk_prob,
                                                        int32_t* __restrict__ flags_reset) {
  const int c = blockIdx.x;
  if (flags_reset && c == 0 && threadIdx.x == 0) flags_reset[0] = 0;
  const int b0 = c * kScanRows;
  const int b1 = min(nb, b0 + kScanRows);
  for (int e = threadIdx.x; e < E; e += 256) {
    // all kScanRows loads of the column in flight at once, then added in block order
    int cv[kScanRows];
    float pv[kScanRows];
#pragma unroll
    for (int i = 0; i < kScanRows; ++i) {
      const bool in = b0 + i < b1;
      cv[i] = in ? cnt_part[size_t(b0 + i) * E + e] : 0;
      pv[i] = (in && with_prob) ? prob_part[size_t(b0 + i) * E + e] : 0.f;
    }
    int cs = 0;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < kScanRows; ++i) {
      cs += cv[i];
      ps += pv[i];
    }
    chunk_cnt[size_t(c) * E + e] = cs;
    if (with_prob) chunk_prob[size_t(c) * E + e] = ps;
  }
}

// One block of E*P threads (E*P <= 1024): thread (e, part) owns expert e and the chunk
// range part*seg .. +seg. It sums its chunks, takes the exclusive prefix of the earlier
// ranges, and writes each chunk's starting offset. Totals, prob_sum (ranges added in
// order) and the aux loss (fixed tree over experts) follow; all of it is reproducible
// bit for bit and needs no atomics or fences.
__global__ __launch_bounds__(1024) void scan_kernel(
    const int32_t* __restrict__ chunk_cnt, const float* __restrict__ chunk_prob,
    int32_t* __restrict__ chunk_off, int nchunks, int P, int T, int k, int E, int C,
    int with_prob, int32_t* __restrict__ count_out, float* __restrict__ prob_out,
    float* __restrict__ aux_out, int32_t* __restrict__ used_out,
    int32_t* __restrict__ overflow_out, int32_t* __restrict__ flags,
    const float* __restrict__ zpart, int nb, float* __restrict__ z_out, LoadStats ls) {
  __shared__ int s_c[1024];
  __shared__ float s_p[1024];
  const int tid = threadIdx.x;
  const int e = tid % E;
  const int part = tid / E;
  const bool active = part < P;
  const int seg = (nchunks + P - 1) / P;
  const int lo = min(nchunks, part * seg);
  const int hi = min(nchunks, lo + seg);
  int csum = 0;
  float psum = 0.f;
  if (active) {
    for (int c = lo; c < hi; ++c) {
      csum += chunk_cnt[size_t(c) * E + e];
      if (with_prob) psum += chunk_prob[size_t(c) * E + e];
    }
  }
  s_c[tid] = csum;
  s_p[tid] = psum;
  __syncthreads();
  if (active && chunk_off != nullptr) {
    int run = 0;
    for (int q = 0; q < part; ++q) run += s_c[q * E + e];
    for (int c = lo; c < hi; ++c) {
      chunk_off[size_t(c) * E + e] = run;
      run += chunk_cnt[size_t(c) * E + e];
    }
  }
  float fpv = 0.f;
  if (part == 0) {
    int total = 0;
    float P_e = 0.f;
    for (int q = 0; q < P; ++q) {
      total += s_c[q * E + e];
      P_e += s_p[q * E + e];
    }
    count_out[e] = total;
    if (ls.token_fraction) ls.token_fraction[e] = float(total) / float(T);
    if (with_prob) {
      prob_out[e] = P_e;
      if (ls.probability_mass) ls.probability_mass[e] = P_e / float(T);
      fpv = (float(total) / (float(T) * float(k))) * (P_e / float(T));
    }
    if (C >= 0) {
      const int used = min(total, C);
      used_out[e] = used;
      overflow_out[e] = total - used;
    }
  }
  if (tid == 0) flags[0] = 0;
  if (!with_prob) return;
  __syncthreads();
  s_p[tid] = (part == 0) ? fpv : 0.f;
  __syncthreads();
  for (int d = 512; d >= 1; d >>= 1) {
    if (tid < d) s_p[tid] += s_p[tid + d];
    __syncthreads();
  }
  if (tid == 0) aux_out[0] = float(E) * s_p[0];
  if (!z_out) return;
  // z-loss: thread tid adds the block partials tid, tid + 1024, ... in order, then a
  // fixed tree over the threads
  float z = 0.f;
  for (int b = tid; b < nb; b += 1024) z += zpart[b];
  __syncthreads();
  s_p[tid] = z;
  __syncthreads();
  for (int d = 512; d >= 1; d >>= 1) {
    if (tid < d) s_p[tid] += s_p[tid + d];
    __syncthreads();
  }
  if (tid == 0) z_out[0] = s_p[0] / float(T);
}

template <class T>
struct Vec4;
template <>
struct Vec4<int> {
  typedef int type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec4<float> {
  typedef float type __attribute__((ext_vector_type(4)));
};

// Per-expert sums over a chunk table [nchunks][E] with the block's 256 threads: `all`
// over every chunk, `below` over the chunks c < lim. Thread (g, part) covers column
// group g (four experts read as one 16-byte load when E % 4 == 0, else one expert) over
// the chunk range part*seg .. +seg in chunk order; the parts meet in LDS (s_a, s_b:
// 1024 entries each) and thread e < E adds them in part order, so every sum has a
// fixed order. Valid in threads e < E (E <= 256); the other threads get zeros.
template <class T>
struct ColSum {
  T all, below;
};
template <class T>
__device__ ColSum<T> chunk_column_sums(const T* __restrict__ tab, int nchunks, int E, int lim,
                                       T* s_a, T* s_b) {
  const int tid = threadIdx.x;
  const bool vec = (E & 3) == 0;
  const int EG = vec ? E >> 2 : E;
  const int P = 256 / EG;
  const int g = tid % EG, part = tid / EG;
  const int seg = (nchunks + P - 1) / P;
  const int lo = min(nchunks, part * seg), hi = min(nchunks, lo + seg);
  T a[4] = {T(0), T(0), T(0), T(0)}, b[4] = {T(0), T(0), T(0), T(0)};
  if (part < P) {
    if (vec) {
#pragma unroll 4
      for (int c = lo; c < hi; ++c) {
        const typename Vec4<T>::type v = reinterpret_cast<const typename Vec4<T>::type*>(tab + size_t(c) * E)[g];
        const bool lt = c < lim;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] += v[r];
          if (lt) b[r] += v[r];
        }
      }
    } else {
      for (int c = lo; c < hi; ++c) {
        const T v = tab[size_t(c) * E + g];
        a[0] += v;
        if (c < lim) b[0] += v;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s_a[tid * 4 + r] = a[r];
    s_b[tid * 4 + r] = b[r];
  }
  __syncthreads();
  ColSum<T> out{T(0), T(0)};
  if (tid < E) {
    const int gg = vec ? tid >> 2 : tid, comp = vec ? (tid & 3) : 0;
    for (int q = 0; q < P; ++q) {
      out.all += s_a[(q * EG + gg) * 4 + comp];
      out.below += s_b[(q * EG + gg) * 4 + comp];
    }
  }
  __syncthreads();
  return out;
}

// Slot assignment. Block b covers tokens [b*G*kRouteTokens, ...) (G routing blocks) and
// walks its assignments in chunks of 256 (a = t*k + j ascending). Within a chunk each
// wave finds, by ballots on the expert-id bits, the lanes holding the same expert, and
// ranks a lane by the equal lanes below it; waves are ordered through a per-wave
// histogram in LDS; chunks through a running per-expert count that starts at the
// offset of the block (its chunk's scanned offset plus the counts of the earlier routing
// blocks of that chunk). The grid then writes -1 into slot_assign[e, c] for
// c >= used[e] (a grid-stride pass over the E*C table).
//
// FUSED (E <= 256 and few chunks): there is no separate scan launch. Every assignment
// block adds up the chunk sums itself (integer sums, so the order does not matter): those
// of the chunks before its own give its chunk's offset, all of them the totals behind
// used[e]. One extra block, the last of the grid, writes the scan's outputs: totals,
// used/overflow, prob_sum (per expert, the chunk sums of a part of the chunk range in
// order, then the parts in order), the aux loss and the z-loss (fixed trees).
struct ScanOut {
  int32_t* count;
  float* prob_sum;
  float* aux;
  int32_t* used;
  int32_t* overflow;
  float* z_loss;     // NULL: no z-loss
  int with_prob;
  LoadStats ls;      // optional count / T and prob_sum / T
};

template <bool FUSED>
__global__ __launch_bounds__(256) void assign_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int C, int G,
    const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ cnt_part, int ebits,
    const int32_t* __restrict__ used,
    int32_t* __restrict__ slot, uint8_t* __restrict__ kept, int32_t* __restrict__ slot_assign,
    int32_t* __restrict__ drops, int32_t* __restrict__ flags,
    const int32_t* __restrict__ chunk_cnt, const float* __restrict__ chunk_prob, int nchunks,
    const float* __restrict__ zpart, int nb, ScanOut so) {
  extern __shared__ int smem[];
  int* s_run = smem;                // [E]
  int* s_wh = smem + E;             // [4][E]
  int* s_tk = smem + 5 * E;         // [G*kRouteTokens] kept choices per token
  __shared__ int s_ci[FUSED ? 256 : 1];
  __shared__ int s_cj[FUSED ? 256 : 1];
  __shared__ int s_x[FUSED ? 2 : 1][FUSED ? 1024 : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  if constexpr (FUSED) {
    if (blockIdx.x == gridDim.x - 1) {
      // the scan's outputs
      const ColSum<int> cnt = chunk_column_sums<int>(chunk_cnt, nchunks, E, 0, s_x[0], s_x[1]);
      ColSum<float> pr{0.f, 0.f};
      if (so.with_prob)
        pr = chunk_column_sums<float>(chunk_prob, nchunks, E, 0, reinterpret_cast<float*>(s_x[0]),
                                      reinterpret_cast<float*>(s_x[1]));
      float* s_f = reinterpret_cast<float*>(s_x[0]);
      float fpv = 0.f;
      if (tid < E) {
        const int total = cnt.all;
        so.count[tid] = total;
        const int u = min(total, C);
        so.used[tid] = u;
        so.overflow[tid] = total - u;
        if (so.ls.token_fraction) so.ls.token_fraction[tid] = float(total) / float(T);
        if (so.with_prob) {
          so.prob_sum[tid] = pr.all;
          if (so.ls.probability_mass) so.ls.probability_mass[tid] = pr.all / float(T);
          fpv = (float(total) / (float(T) * float(k))) * (pr.all / float(T));
        }
      }
      if (!so.with_prob) return;
      s_f[tid] = fpv;
      __syncthreads();
      for (int d = 128; d >= 1; d >>= 1) {
        if (tid < d) s_f[tid] += s_f[tid + d];
        __syncthreads();
      }
      if (tid == 0) so.aux[0] = float(E) * s_f[0];
      if (!so.z_loss) return;
      float z = 0.f;
      for (int b = tid; b < nb; b += 256) z += zpart[b];
      __syncthreads();
      s_f[tid] = z;
      __syncthreads();
      for (int d = 128; d >= 1; d >>= 1) {
        if (tid < d) s_f[tid] += s_f[tid + d];
        __syncthreads();
      }
      if (tid == 0) so.z_loss[0] = s_f[0] / float(T);
      return;
    }
  }
  const int tokens = G * kRouteTokens;
  const int tok0 = blockIdx.x * tokens;
  const int tok1 = min(T, tok0 + tokens);
  const int rb = blockIdx.x * G;    // first routing block of this block
  const int cb = rb / kScanRows;
  if constexpr (FUSED) {
    // per expert: the counts of the chunks before chunk cb (the chunk's offset) and
    // used[e] = min(total, C)
    const ColSum<int> cs = chunk_column_sums<int>(chunk_cnt, nchunks, E, cb, s_x[0], s_x[1]);
    if (tid < E) {
      s_ci[tid] = cs.below;
      s_cj[tid] = min(cs.all, C);
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += 256) {
    int run = FUSED ? s_ci[e] : chunk_off[size_t(cb) * E + e];
    for (int b = cb * kScanRows; b < rb; ++b) run += cnt_part[size_t(b) * E + e];
    s_run[e] = run;
    s_wh[e] = 0;
    s_wh[E + e] = 0;
    s_wh[2 * E + e] = 0;
    s_wh[3 * E + e] = 0;
  }
  for (int t = tid; t < tokens; t += 256) s_tk[t] = 0;
  __syncthreads();
  const int64_t a_end = int64_t(tok1) * k;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = int64_t(tok0) * k; base < a_end; base += 256) {
    const int64_t a = base + tid;
    const bool valid = a < a_end;
    int e = valid ? idx[a] : -1;
    if (valid && (e < 0 || e >= E)) {
      atomicOr(&flags[0], 1);
      e = -1;
    }
    const bool has = e >= 0;
    uint64_t eq = __ballot(has);
    for (int bit = 0; bit < ebits; ++bit) {
      const bool v = has && ((e >> bit) & 1);
      const uint64_t bb = __ballot(v);
      eq &= v ? bb : ~bb;
    }
    int rank = 0;
    if (has) {
      rank = __popcll(eq & below);
      if (rank == 0) s_wh[wv * E + e] = __popcll(eq);
    }
    __syncthreads();
    if (has) {
      int pre = s_run[e];
      for (int w2 = 0; w2 < wv; ++w2) pre += s_wh[w2 * E + e];
      const int sl = pre + rank;
      const bool kp = sl < C;
      slot[a] = kp ? sl : -1;
      kept[a] = kp ? 1 : 0;
      if (kp) {
        slot_assign[size_t(e) * C + sl] = int32_t(a);
        atomicAdd(&s_tk[int(a / k) - tok0], 1);
      }
    } else if (valid) {
      slot[a] = -1;
      kept[a] = 0;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += 256) {
      s_run[e2] += s_wh[e2] + s_wh[E + e2] + s_wh[2 * E + e2] + s_wh[3 * E + e2];
      s_wh[e2] = 0;
      s_wh[E + e2] = 0;
      s_wh[2 * E + e2] = 0;
      s_wh[3 * E + e2] = 0;
    }
    __syncthreads();
  }
  for (int t = tid; t < tok1 - tok0; t += 256) drops[tok0 + t] = k - s_tk[t];
  // unfilled slots (FUSED: the last block of the grid is the scan block)
  const int64_t total = int64_t(E) * C;
  const int nab = FUSED ? gridDim.x - 1 : gridDim.x;
  for (int64_t i = int64_t(blockIdx.x) * 256 + tid; i < total; i += int64_t(nab) * 256) {
    const int e2 = int(i / C);
    const int c = int(i - int64_t(e2) * C);
    if (c >= (FUSED ? s_cj[e2] : used[e2])) slot_assign[i] = -1;
  }
}

template <int L, int V>
static moe_status_t launch_route_lv(const float* logits, int T, int E, int k, int32_t* idx,
                                    float* gate, const RouteOpts& o, const RouteWs& w,
                                    hipStream_t s) {
  const int nb = route_blocks(T);
  const bool var = o.scoring != MOE_SCORE_SOFTMAX || o.bias || o.with_z;
  // one round per block where the LDS staging of the probability sums fits
  constexpr int NT = (L == 16 || L == 32) ? 512 : 256;
#define MOE_ROUTE(KRV)                                                                        \
  if (var) {                                                                                \
    MOE_LAUNCH("route", (route_kernel<L, V, KRV, true, NT>), dim3(nb), dim3(NT), 0, s, logits, \
               T, E, k, idx, gate, w.cnt_part, w.prob_part, o, w.zpart);                     \
  } else {                                                                                  \
    MOE_LAUNCH("route", (route_kernel<L, V, KRV, false, NT>), dim3(nb), dim3(NT), 0, s,        \
               logits, T, E, k, idx, gate, w.cnt_part, w.prob_part, o, w.zpart);             \
  }
  if (k <= L) {
    MOE_ROUTE(1)
  } else if (k <= 4 * L) {
    MOE_ROUTE(4)
  } else {
    MOE_ROUTE(32)
  }
#undef MOE_ROUTE
  return MOE_OK;
}

moe_status_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                          const RouteOpts& o, const RouteWs& w, hipStream_t s) {
  // L lanes per token with V = E / L <= 16 logits each (L >= 8 so that a round of the
  // block covers at most kRouteTokens tokens)
  if (E <= 8) return launch_route_lv<8, 1>(logits, T, E, k, idx, gate, o, w, s);
  if (E <= 16) return launch_route_lv<8, 2>(logits, T, E, k, idx, gate, o, w, s);
  if (E <= 32) return launch_route_lv<8, 4>(logits, T, E, k, idx, gate, o, w, s);
  if (E <= 64) return launch_route_lv<8, 8>(logits, T, E, k, idx, gate, o, w, s);
  if (E <= 128) return launch_route_lv<8, 16>(logits, T, E, k, idx, gate, o, w, s);
  if (E <= 256) return launch_route_lv<16, 16>(logits, T, E, k, idx, gate, o, w, s);
  if (E <= 512) return launch_route_lv<32, 16>(logits, T, E, k, idx, gate, o, w, s);
  return launch_route_lv<64, 16>(logits, T, E, k, idx, gate, o, w, s);
}

moe_status_t launch_count(const int32_t* idx, int T, int k, int E, const RouteWs& w,
                          hipStream_t s) {
  const int nb = route_blocks(T);
  MOE_LAUNCH("count", count_kernel, dim3(nb), dim3(256), sizeof(int) * E, s, idx, T, k, E,
             w.cnt_part);
  return MOE_OK;
}

moe_status_t launch_reduce_scan(int T, int k, int E, int C, bool with_prob, int32_t* count,
                                float* prob_sum, float* aux, int32_t* used, int32_t* overflow,
                                int32_t* slot_assign, float* z_loss, const LoadStats& ls,
                                const RouteWs& w, hipStream_t s) {
  (void)slot_assign;
  const int nb = route_blocks(T);
  const int nchunks = scan_chunks(T);
  MOE_LAUNCH("chunk_sum", chunk_sum_kernel, dim3(nchunks), dim3(256), 0, s, w.cnt_part,
             w.prob_part, nb, E, with_prob ? 1 : 0, w.chunk_cnt, w.chunk_prob, nullptr);
  int P = 1024 / E;
  if (P < 1) P = 1;
  if (P > nchunks) P = nchunks;
  MOE_LAUNCH("scan", scan_kernel, dim3(1), dim3(1024), 0, s, w.chunk_cnt, w.chunk_prob,
             C >= 0 ? w.chunk_off : nullptr, nchunks, P, T, k, E, C, with_prob ? 1 : 0, count,
             prob_sum, aux, used, overflow, w.flags, w.zpart, nb, with_prob ? z_loss : nullptr,
             LoadStats{ls.token_fraction, with_prob ? ls.probability_mass : nullptr});
  return MOE_OK;
}

namespace {
int assign_ebits(int E) {
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  return ebits;
}
}  // namespace

moe_status_t launch_assign(const int32_t* idx, int T, int k, int E, int C, int32_t* slot,
                           uint8_t* kept, int32_t* slot_assign, int32_t* drops,
                           const int32_t* used, const RouteWs& w, hipStream_t s) {
  const int G = assign_group(k);
  const int tokens = G * kRouteTokens;
  const int blocks = (T + tokens - 1) / tokens;
  const size_t shmem = sizeof(int) * (5 * size_t(E) + tokens);
  MOE_LAUNCH("assign", assign_kernel<false>, dim3(blocks), dim3(256), shmem, s, idx, T, k, E, C,
             G, w.chunk_off, w.cnt_part, assign_ebits(E), used, slot, kept, slot_assign, drops,
             w.flags, nullptr, nullptr, 0, nullptr, 0, ScanOut{});
  return MOE_OK;
}

moe_status_t launch_dispatch(const int32_t* idx, int T, int k, int E, int C, bool with_prob,
                             int32_t* count, float* prob_sum, float* aux, int32_t* used,
                             int32_t* overflow, float* z_loss, const LoadStats& ls,
                             int32_t* slot, uint8_t* kept, int32_t* slot_assign, int32_t* drops,
                             const RouteWs& w, hipStream_t s) {
  const int nb = route_blocks(T);
  const int nchunks = scan_chunks(T);
  if (E > 256 || int64_t(nchunks) * E > kFusedScanEntries) {
    moe_status_t st = launch_reduce_scan(T, k, E, C, with_prob, count, prob_sum, aux, used,
                                         overflow, slot_assign, z_loss, ls, w, s);
    if (st != MOE_OK) return st;
    return launch_assign(idx, T, k, E, C, slot, kept, slot_assign, drops, used, w, s);
  }
  MOE_LAUNCH("chunk_sum", chunk_sum_kernel, dim3(nchunks), dim3(256), 0, s, w.cnt_part,
             w.prob_part, nb, E, with_prob ? 1 : 0, w.chunk_cnt, w.chunk_prob, w.flags);
  const int G = assign_group(k);
  const int tokens = G * kRouteTokens;
  const int blocks = (T + tokens - 1) / tokens;
  const size_t shmem = sizeof(int) * (5 * size_t(E) + tokens);
  ScanOut so{count, prob_sum, aux, used, overflow, with_prob ? z_loss : nullptr,
             with_prob ? 1 : 0,
             LoadStats{ls.token_fraction, with_prob ? ls.probability_mass : nullptr}};
  MOE_LAUNCH("assign", assign_kernel<true>, dim3(blocks + 1), dim3(256), shmem, s, idx, T, k, E,
             C, G, nullptr, w.cnt_part, assign_ebits(E), nullptr, slot, kept, slot_assign, drops,
             w.flags, w.chunk_cnt, w.chunk_prob, nchunks, w.zpart, nb, so);
  return MOE_OK;
}

}  // namespace moe
