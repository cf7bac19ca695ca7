// Routing and position-priority dispatch for gfx950.
//
// route_kernel     one wavefront per token: fp32 softmax over the E logits, top-k by
//                  logit with exact ties to the lower expert index, gates renormalised
//                  over the k choices ("Top-k MoE Router with Load Statistics", alpha
//                  equation; "Sparse MoE Layer in NumPy", top_k_gating), plus per-block
//                  pre-drop counts and probability sums (trap 6 of the same page).
// count_kernel     per-block expert histogram of caller-supplied choices.
// reduce_scan      one block per expert: exclusive scan of the per-block counts in
//                  block order, totals, used/overflow, prob_sum, and the aux loss
//                  (finished by the last block to arrive, in a fixed summation order).
// assign_kernel    slots: a stable rank of each assignment among earlier assignments to
//                  the same expert inside the block (wave ballots, then a per-wave
//                  prefix), plus the block's scanned offset. This reproduces the serial
//                  token-then-choice loop of position_priority_dispatch ("Sparse MoE
//                  Layer in NumPy", trap 3) exactly, with no serial pass.
//
// Everything that decides an integer is integer or comparison work, so the indices,
// slots and counts are bit-exact; the float reductions run in a fixed order so that
// repeated runs are bitwise identical.

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
  w.off_part = reinterpret_cast<int32_t*>(p + off);
  off = align_up(off + sizeof(int32_t) * size_t(E) * nb, 256);
  w.prob_part = reinterpret_cast<float*>(p + off);
  off = align_up(off + sizeof(float) * size_t(E) * nb, 256);
  w.fp = reinterpret_cast<float*>(p + off);
  off = align_up(off + sizeof(float) * size_t(E), 256);
  w.bytes = off;
  return w;
}

// EPL: experts held per lane (E <= 64 * EPL). KR: register slots for the k results per
// lane (k <= 64 * KR).
template <int EPL, int KR>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ gate_out,
                                                    int32_t* __restrict__ cnt_part,
                                                    float* __restrict__ prob_part,
                                                    int32_t* __restrict__ flags) {
  __shared__ int s_hist[64 * EPL];
  __shared__ float s_prob[4][64 * EPL];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nb = gridDim.x;
  for (int e = threadIdx.x; e < 64 * EPL; e += 256) s_hist[e] = 0;
  __syncthreads();

  float acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.f;

  const int t0 = blockIdx.x * kRouteTokens;
  for (int tt = wv; tt < kRouteTokens; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float* row = logits + size_t(t) * E;
    float s[EPL];
    uint64_t key[EPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      s[i] = (e < E) ? row[e] : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
    mx = wave_max(mx);
    float p[EPL];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      p[i] = (e < E) ? __expf(s[i] - mx) : 0.f;
      sum += p[i];
      key[i] = (e < E) ? ((uint64_t(orderable(s[i])) << 32) | uint32_t(0xffffffffu - uint32_t(e)))
                       : 0ull;
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      p[i] *= inv;
      acc[i] += p[i];
    }

    int my_e[KR];
    float my_p[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      my_e[r] = 0;
      my_p[r] = 0.f;
    }
    float gsum = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = int(0xffffffffu - uint32_t(best));
      const int owner = e & 63;
      const int si = e >> 6;
      float pv = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (i == si) {
          pv = p[i];
          if (lane == owner) key[i] = 0ull;
        }
      }
      const float pe = __shfl(pv, owner, kWave);
      gsum += pe;
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        if (lane == (j & 63) && r == (j >> 6)) {
          my_e[r] = e;
          my_p[r] = pe;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int j = lane + 64 * r;
      if (j < k) {
        idx_out[size_t(t) * k + j] = my_e[r];
        gate_out[size_t(t) * k + j] = my_p[r] / gsum;
        atomicAdd(&s_hist[my_e[r]], 1);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < EPL; ++i) s_prob[wv][lane + 64 * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const float v = ((s_prob[0][e] + s_prob[1][e]) + s_prob[2][e]) + s_prob[3][e];
    prob_part[size_t(e) * nb + blockIdx.x] = v;
    cnt_part[size_t(e) * nb + blockIdx.x] = s_hist[e];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    flags[0] = 0;
    flags[1] = 0;
  }
}

// Per-block expert histogram over the same token partition as route_kernel. Indices
// outside [0, E) are skipped here and reported by assign_kernel.
__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int T,
                                                    int k, int E,
                                                    int32_t* __restrict__ cnt_part,
                                                    int32_t* __restrict__ flags) {
  extern __shared__ int s_hist[];
  const int nb = gridDim.x;
  for (int e = threadIdx.x; e < E; e += 256) s_hist[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kRouteTokens;
  const int t1 = min(T, t0 + kRouteTokens);
  for (int a = t0 * k + threadIdx.x; a < t1 * k; a += 256) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&s_hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) cnt_part[size_t(e) * nb + blockIdx.x] = s_hist[e];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    flags[0] = 0;
    flags[1] = 0;
  }
}

// One block per expert. Exclusive scan over the nb per-block counts (in block order),
// totals and, when requested, dispatch bookkeeping. The last block to finish sums the
// per-expert aux terms in expert order.
__global__ __launch_bounds__(256) void reduce_scan_kernel(
    const int32_t* __restrict__ cnt_part, const float* __restrict__ prob_part,
    int32_t* __restrict__ off_part, int nb, int T, int k, int E, int C, int with_prob,
    int32_t* __restrict__ count_out, float* __restrict__ prob_out, float* __restrict__ aux_out,
    int32_t* __restrict__ used_out, int32_t* __restrict__ overflow_out,
    int32_t* __restrict__ slot_assign, float* __restrict__ fp, int32_t* __restrict__ flags) {
  __shared__ int s_c[256];
  __shared__ float s_p[256];
  __shared__ int s_last;
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int seg = (nb + 255) / 256;
  const int lo = min(nb, tid * seg);
  const int hi = min(nb, lo + seg);
  const int32_t* cp = cnt_part + size_t(e) * nb;
  int csum = 0;
  float psum = 0.f;
  for (int b = lo; b < hi; ++b) csum += cp[b];
  if (with_prob) {
    const float* pp = prob_part + size_t(e) * nb;
    for (int b = lo; b < hi; ++b) psum += pp[b];
  }
  s_c[tid] = csum;
  s_p[tid] = psum;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread sums (integer: order-free).
  for (int d = 1; d < 256; d <<= 1) {
    const int v = tid >= d ? s_c[tid - d] : 0;
    __syncthreads();
    s_c[tid] += v;
    __syncthreads();
  }
  const int total = s_c[255];
  int run = s_c[tid] - csum;
  if (off_part != nullptr) {
    int32_t* op = off_part + size_t(e) * nb;
    for (int b = lo; b < hi; ++b) {
      op[b] = run;
      run += cp[b];
    }
  }
  // fixed-shape tree for the probability sum
  for (int d = 128; d >= 1; d >>= 1) {
    if (tid < d) s_p[tid] += s_p[tid + d];
    __syncthreads();
  }
  if (tid == 0) {
    count_out[e] = total;
    if (with_prob) {
      const float P = s_p[0];
      prob_out[e] = P;
      fp[e] = (float(total) / (float(T) * float(k))) * (P / float(T));
    }
    if (C >= 0) {
      const int used = min(total, C);
      used_out[e] = used;
      overflow_out[e] = total - used;
    }
  }
  if (C >= 0) {
    const int used = min(total, C);
    for (int c = used + tid; c < C; c += 256) slot_assign[size_t(e) * C + c] = -1;
  }
  if (!with_prob) return;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&flags[1], 1) == int(gridDim.x) - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  float v = 0.f;
  for (int i = tid; i < E; i += 256) v += __builtin_nontemporal_load(&fp[i]);
  s_p[tid] = v;
  __syncthreads();
  for (int d = 128; d >= 1; d >>= 1) {
    if (tid < d) s_p[tid] += s_p[tid + d];
    __syncthreads();
  }
  if (tid == 0) {
    aux_out[0] = float(E) * s_p[0];
    flags[1] = 0;
  }
}

// Slot assignment. Block b covers tokens [b*G*16, (b+1)*G*16) (G routing blocks) and
// walks its assignments in chunks of 256 (a = t*k + j ascending). Within a chunk each
// wave finds, by ballots on the expert-id bits, the lanes holding the same expert, and
// ranks a lane by the equal lanes below it; waves are ordered through a per-wave
// histogram in LDS; chunks through a running per-expert count that starts at the
// scanned offset of the block.
__global__ __launch_bounds__(256) void assign_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int C, int G,
    const int32_t* __restrict__ off_part, int nb, int ebits, int32_t* __restrict__ slot,
    uint8_t* __restrict__ kept, int32_t* __restrict__ slot_assign, int32_t* __restrict__ drops,
    int32_t* __restrict__ flags) {
  extern __shared__ int smem[];
  int* s_run = smem;                // [E]
  int* s_wh = smem + E;             // [4][E]
  int* s_tk = smem + 5 * E;         // [G*16] kept choices per token
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int tokens = G * kRouteTokens;
  const int tok0 = blockIdx.x * tokens;
  const int tok1 = min(T, tok0 + tokens);
  const int rb = blockIdx.x * G;    // first routing block of this block
  for (int e = tid; e < E; e += 256) {
    s_run[e] = off_part[size_t(e) * nb + rb];
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
}

template <int EPL>
static moe_status_t launch_route_epl(const float* logits, int T, int E, int k, int32_t* idx,
                                     float* gate, const RouteWs& w, hipStream_t s) {
  const int nb = route_blocks(T);
  if (k <= 64) {
    MOE_LAUNCH("route", (route_kernel<EPL, 1>), dim3(nb), dim3(256), 0, s, logits, T, E, k, idx,
               gate, w.cnt_part, w.prob_part, w.flags);
  } else {
    MOE_LAUNCH("route", (route_kernel<EPL, 4>), dim3(nb), dim3(256), 0, s, logits, T, E, k, idx,
               gate, w.cnt_part, w.prob_part, w.flags);
  }
  return MOE_OK;
}

moe_status_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                          const RouteWs& w, hipStream_t s) {
  if (E <= 64) return launch_route_epl<1>(logits, T, E, k, idx, gate, w, s);
  if (E <= 128) return launch_route_epl<2>(logits, T, E, k, idx, gate, w, s);
  if (E <= 256) return launch_route_epl<4>(logits, T, E, k, idx, gate, w, s);
  if (E <= 512) return launch_route_epl<8>(logits, T, E, k, idx, gate, w, s);
  return launch_route_epl<16>(logits, T, E, k, idx, gate, w, s);
}

moe_status_t launch_count(const int32_t* idx, int T, int k, int E, const RouteWs& w,
                          hipStream_t s) {
  const int nb = route_blocks(T);
  MOE_LAUNCH("count", count_kernel, dim3(nb), dim3(256), sizeof(int) * E, s, idx, T, k, E,
             w.cnt_part, w.flags);
  return MOE_OK;
}

moe_status_t launch_reduce_scan(int T, int k, int E, int C, bool with_prob, int32_t* count,
                                float* prob_sum, float* aux, int32_t* used, int32_t* overflow,
                                int32_t* slot_assign, const RouteWs& w, hipStream_t s) {
  const int nb = route_blocks(T);
  MOE_LAUNCH("reduce_scan", reduce_scan_kernel, dim3(E), dim3(256), 0, s, w.cnt_part,
             w.prob_part, C >= 0 ? w.off_part : nullptr, nb, T, k, E, C, with_prob ? 1 : 0,
             count, prob_sum, aux, used, overflow, slot_assign, w.fp, w.flags);
  return MOE_OK;
}

moe_status_t launch_assign(const int32_t* idx, int T, int k, int E, int C, int32_t* slot,
                           uint8_t* kept, int32_t* slot_assign, int32_t* drops,
                           const RouteWs& w, hipStream_t s) {
  const int nb = route_blocks(T);
  const int G = assign_group(k);
  const int tokens = G * kRouteTokens;
  const int blocks = (T + tokens - 1) / tokens;
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  const size_t shmem = sizeof(int) * (5 * size_t(E) + tokens);
  MOE_LAUNCH("assign", assign_kernel, dim3(blocks), dim3(256), shmem, s, idx, T, k, E, C, G,
             w.off_part, nb, ebits, slot, kept, slot_assign, drops, w.flags);
  return MOE_OK;
}

}  // namespace moe
