// Top-K routing and its backward, one 64-lane wavefront per token, and the
// auxiliary load-balancing loss.
//
// Follows the fused router of the TransformerEngine MoE block pull request
// (Description / Changes: top-K with optional grouped/sigmoid scoring and an
// optional auxiliary load-balancing loss): experts are ranked on a float32
// key, the lower id winning a tie; weights are softmax over all experts or
// the logistic function, optionally renormalised over the K selected.  The
// key is the logit plus an optional per-expert bias, or (selection-only
// bias, the "pre_bias_logits" of the MaxText DeepSeek-V3 router) the score
// plus the bias with the weights taken from the unbiased scores.  Grouped
// selection keeps the topk_groups groups of consecutive experts with the
// largest sum of their two best keys and ranks experts inside them.
#include "common.h"

namespace moe {
namespace {

constexpr int kWaves = 4;  // tokens per 256-thread block

// Expert e lives in lane (e % 64), register slot (e / 64).
template <int V>
__device__ __forceinline__ void load_z(const float* lrow, const float* bias, int E, int lane,
                                       float z[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    float v = -INFINITY;
    if (e < E) {
      v = lrow[e];
      if (bias) v = __fadd_rn(v, bias[e]);
    }
    z[i] = v;
  }
}

// (value, id) total order: larger value first, then smaller id.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Wave-wide argmax of (value, id) over this lane's candidates of V slots
// (cid == INT_MAX: not a candidate); the result is wave-uniform.
template <int V>
__device__ __forceinline__ void wave_argmax(const float (&key)[V], const int (&cid)[V], float& bv,
                                            int& bi) {
  bv = -INFINITY;
  bi = INT_MAX;
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (cid[i] != INT_MAX && better(key[i], cid[i], bv, bi)) { bv = key[i]; bi = cid[i]; }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
}

template <int V>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int select,
                                                    int n_groups, int topk_groups, int64_t T,
                                                    int E, int K, int score, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  // z: the logits the weights are scores of (biased unless the bias only
  // moves the selection)
  const float* zb = select ? nullptr : bias;
  float z[V];
  load_z<V>(logits + t * E, zb, E, lane, z);
  float m = 0.f, ssum = 1.f;
  if (score == MOE_SOFTMAX) {
    m = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) m = fmaxf(m, z[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    ssum = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) ssum += (i * 64 + lane < E) ? expf(z[i] - m) : 0.f;
    ssum = wave_sum(ssum);
  }
  auto score_of = [&](float zv) {
    return score == MOE_SOFTMAX ? expf(zv - m) / ssum : 1.0f / (1.0f + expf(-zv));
  };
  float key[V];
  int cid[V];   // candidate id per register slot; INT_MAX = not a candidate (padding or taken)
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    cid[i] = e < E ? e : INT_MAX;
    key[i] = z[i];
    if (select && e < E) key[i] = __fadd_rn(score_of(z[i]), bias ? bias[e] : 0.f);
  }
  if (n_groups > 1) {
    // group gi = experts [gi eg, (gi + 1) eg): score = sum of its two best keys
    const int eg = E / n_groups;
    float gsc = -INFINITY;   // lane gi holds group gi's score
    for (int gi = 0; gi < n_groups; ++gi) {
      int gid[V];
#pragma unroll
      for (int i = 0; i < V; ++i) gid[i] = (cid[i] != INT_MAX && cid[i] / eg == gi) ? cid[i] : INT_MAX;
      float v1, v2 = 0.f;
      int i1, i2;
      wave_argmax<V>(key, gid, v1, i1);
      if (eg >= 2) {
#pragma unroll
        for (int i = 0; i < V; ++i) if (gid[i] == i1) gid[i] = INT_MAX;
        wave_argmax<V>(key, gid, v2, i2);
      }
      const float sc = eg >= 2 ? __fadd_rn(v1, v2) : v1;
      if (lane == gi) gsc = sc;
    }
    // keep the topk_groups best groups (ties: lower group id)
    uint64_t keep = 0;
    bool open = lane < n_groups;
    for (int r = 0; r < topk_groups; ++r) {
      float bv = open ? gsc : -INFINITY;
      int bi = open ? lane : INT_MAX;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      keep |= 1ull << bi;
      if (lane == bi) open = false;
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (cid[i] != INT_MAX && !((keep >> (cid[i] / eg)) & 1ull)) cid[i] = INT_MAX;
  }

  int my_id = 0;       // lane j < K keeps the j-th selection
  for (int j = 0; j < K; ++j) {
    float bv;
    int bi;
    wave_argmax<V>(key, cid, bv, bi);
    // bi is now wave-uniform; retire it
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (cid[i] == bi) cid[i] = INT_MAX;
    if (lane == j) my_id = bi;
  }

  float p = 0.f;
  if (lane < K) {
    const float zs = zb ? __fadd_rn(logits[t * E + my_id], zb[my_id]) : logits[t * E + my_id];
    p = score_of(zs);
  }
  if (renorm) {
    const float tot = wave_sum(p);
    p = p / tot;
  }
  if (lane < K) {
    ids[t * K + lane] = my_id;
    w[t * K + lane] = p;
  }
}

template <int V, typename TO>
__global__ __launch_bounds__(256) void route_bwd_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ ids, const float* __restrict__ dw, int64_t T, int E, int K,
    int score, int renorm, TO* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  float z[V];
  load_z<V>(logits + t * E, bias, E, lane, z);
  const int sel = (lane < K) ? ids[t * K + lane] : -1;
  const float g = (lane < K) ? dw[t * K + lane] : 0.f;
  const float zs = (lane < K && sel >= 0 && sel < E) ? __fadd_rn(logits[t * E + sel], bias ? bias[sel] : 0.f) : 0.f;

  float out_sel = 0.f;   // gradient for this lane's selected expert
  float others = 0.f;    // value for experts not selected (softmax without renorm)
  float m = 0.f, s = 1.f;
  if (score == MOE_SOFTMAX) {
    m = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) m = fmaxf(m, z[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    s = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) s += (i * 64 + lane < E) ? expf(z[i] - m) : 0.f;
    s = wave_sum(s);
    const float p = (lane < K) ? expf(zs - m) / s : 0.f;
    if (renorm) {
      const float tot = wave_sum(p);
      const float wj = p / tot;
      const float inner = wave_sum(wj * g);
      out_sel = wj * (g - inner);
    } else {
      const float inner = wave_sum(p * g);
      out_sel = p * g;        // plus the -p*inner term every expert gets
      others = inner;
    }
  } else {
    const float sj = (lane < K) ? 1.0f / (1.0f + expf(-zs)) : 0.f;
    if (renorm) {
      const float S = wave_sum(sj);
      const float inner = wave_sum(sj * g) / S;   // sum_i w_i dw_i
      out_sel = sj * (1.f - sj) * (g - inner) / S;
    } else {
      out_sel = g * sj * (1.f - sj);
    }
  }
  const bool dense = (score == MOE_SOFTMAX && !renorm);
  // every lane writes its own experts; a selected expert picks up out_sel
  // from the lane that selected it
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    float v = 0.f;
    if (dense) v = -(expf(z[i] - m) / s) * others;
    for (int j = 0; j < K; ++j) {
      const int idj = __shfl(sel, j, 64);
      const float oj = __shfl(out_sel, j, 64);
      if (idj == e) v += oj;
    }
    if (e < E) Elem<TO>::store(dlogits + t * E + e, v);
  }
}

// Balancing-loss probabilities of one token (lane-held experts): softmax of
// the logits, or the sigmoids normalised to sum one; sg receives the
// sigmoids (for the backward).
template <int V>
__device__ __forceinline__ void aux_probs(const float* lrow, int E, int lane, int score,
                                          float (&p)[V], float (&sg)[V], float& denom) {
  float z[V];
  load_z<V>(lrow, nullptr, E, lane, z);
  if (score == MOE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) m = fmaxf(m, z[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      p[i] = (i * 64 + lane < E) ? expf(z[i] - m) : 0.f;
      s += p[i];
    }
    denom = wave_sum(s);
#pragma unroll
    for (int i = 0; i < V; ++i) { p[i] /= denom; sg[i] = 0.f; }
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      sg[i] = (i * 64 + lane < E) ? 1.0f / (1.0f + expf(-z[i])) : 0.f;
      s += sg[i];
    }
    denom = wave_sum(s);
#pragma unroll
    for (int i = 0; i < V; ++i) p[i] = sg[i] / denom;
  }
}

constexpr int kAuxTok = 256;   // tokens per partial-sum workgroup (64 per wave)

// Per workgroup b: psum[b][e] = sum of p_te over its tokens (each wave in
// token order, the four waves added in wave order) and pcnt[b][e] = selected
// slots of e among its tokens (integer LDS atomics: exact).
template <int V>
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ ids,
                                                          int64_t T, int E, int K, int score,
                                                          float* __restrict__ psum,
                                                          int32_t* __restrict__ pcnt) {
  __shared__ float wsum[kWaves][1024];
  __shared__ int cnt[1024];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kAuxTok;
  const int64_t t1 = t0 + kAuxTok < T ? t0 + kAuxTok : T;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int64_t t = t0 + wv; t < t1; t += kWaves) {
    float p[V], sg[V], den;
    aux_probs<V>(logits + t * E, E, lane, score, p, sg, den);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += p[i];
  }
  for (int64_t q = t0 * K + threadIdx.x; q < t1 * K; q += 256) {
    const int e = ids[q];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (i * 64 + lane < E) wsum[wv][i * 64 + lane] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) v += wsum[q][e];
    psum[static_cast<int64_t>(blockIdx.x) * E + e] = v;
    pcnt[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
  }
}

// One workgroup: P_e = sum over partial blocks in order / T, counts_e, and
// loss = alpha E sum_e (counts_e / (T K)) P_e by a fixed-order tree.
__global__ __launch_bounds__(1024) void aux_final_kernel(const float* __restrict__ psum,
                                                         const int32_t* __restrict__ pcnt,
                                                         int nb, int64_t T, int E, int K,
                                                         float alpha, float* __restrict__ loss,
                                                         int32_t* __restrict__ counts,
                                                         float* __restrict__ probs) {
  __shared__ float term[1024];
  const int e = threadIdx.x;
  float tv = 0.f;
  if (e < E) {
    float P = 0.f;
    int c = 0;
    for (int b = 0; b < nb; ++b) {
      P += psum[static_cast<int64_t>(b) * E + e];
      c += pcnt[static_cast<int64_t>(b) * E + e];
    }
    P /= static_cast<float>(T);
    if (counts) counts[e] = c;
    if (probs) probs[e] = P;
    tv = static_cast<float>(c) / static_cast<float>(T * K) * P;
  }
  term[e] = tv;
  __syncthreads();
  for (int h = 512; h > 0; h >>= 1) {
    if (e < h) term[e] += term[e + h];
    __syncthreads();
  }
  if (e == 0) *loss = alpha * static_cast<float>(E) * term[0];
}

// d logits (+)= d(alpha E sum_e f_e P_e) / d logits with the counts fixed:
//   softmax: (alpha E / T) p_k (f_k - sum_e f_e p_e)
//   sigmoid: (alpha E / T) s_k (1 - s_k) / S (f_k - sum_e f_e p_e)
template <int V, typename TO>
__global__ __launch_bounds__(256) void aux_bwd_kernel(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ counts,
                                                      int64_t T, int E, int K, int score,
                                                      float alpha, TO* __restrict__ dlogits,
                                                      int accumulate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  float p[V], sg[V], den;
  aux_probs<V>(logits + t * E, E, lane, score, p, sg, den);
  const float inv_tk = 1.0f / static_cast<float>(T * K);
  float f[V];
  float inner = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    f[i] = e < E ? static_cast<float>(counts[e]) * inv_tk : 0.f;
    inner += f[i] * p[i];
  }
  inner = wave_sum(inner);
  const float scale = alpha * static_cast<float>(E) / static_cast<float>(T);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    if (e >= E) continue;
    const float d = score == MOE_SOFTMAX ? scale * p[i] * (f[i] - inner)
                                         : scale * sg[i] * (1.f - sg[i]) / den * (f[i] - inner);
    TO* o = dlogits + t * E + e;
    Elem<TO>::store(o, accumulate ? Elem<TO>::load(o) + d : d);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

#define ROUTE_LAUNCH(KERNEL, V, ...)                                                   \
  hipLaunchKernelGGL(KERNEL<V>, dim3(static_cast<unsigned>((T + kWaves - 1) / kWaves)), \
                     dim3(256), 0, st, __VA_ARGS__)

MOE_API int moe_route(const float* logits, const float* bias, int bias_mode, int n_groups,
                      int topk_groups, int64_t T, int E, int K, int score, int renorm,
                      int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || K < 1 || K > E || K > 64) return MOE_ERR_ARG;
  if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_ERR_ARG;
  if (bias_mode != MOE_BIAS_LOGIT && bias_mode != MOE_BIAS_SELECT) return MOE_ERR_ARG;
  if (n_groups > 1) {
    if (n_groups > 64 || E % n_groups || topk_groups < 1 || topk_groups > n_groups ||
        K > topk_groups * (E / n_groups))
      return MOE_ERR_ARG;
  } else {
    n_groups = 0;
  }
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int V = (E + 63) / 64;
  const int sel = bias_mode == MOE_BIAS_SELECT;
#define RF(VV) \
  ROUTE_LAUNCH(route_kernel, VV, logits, bias, sel, n_groups, topk_groups, T, E, K, score, renorm, \
               topk_ids, topk_w)
  if (V <= 1) RF(1);
  else if (V <= 2) RF(2);
  else if (V <= 4) RF(4);
  else if (V <= 8) RF(8);
  else RF(16);
#undef RF
  return launch_status();
}

template <typename TO>
static void route_bwd_launch(const float* logits, const float* bias, const int32_t* topk_ids,
                             const float* d_topk_w, int64_t T, int E, int K, int score,
                             int renorm, TO* d_logits, hipStream_t st) {
  const int V = (E + 63) / 64;
#define RB(VV)                                                                              \
  hipLaunchKernelGGL((route_bwd_kernel<VV, TO>),                                            \
                     dim3(static_cast<unsigned>((T + kWaves - 1) / kWaves)), dim3(256), 0, st, \
                     logits, bias, topk_ids, d_topk_w, T, E, K, score, renorm, d_logits)
  if (V <= 1) RB(1);
  else if (V <= 2) RB(2);
  else if (V <= 4) RB(4);
  else if (V <= 8) RB(8);
  else RB(16);
#undef RB
}

MOE_API int moe_route_bwd(const float* logits, const float* bias, int bias_mode,
                          const int32_t* topk_ids, const float* d_topk_w, int64_t T, int E, int K,
                          int score, int renorm, void* d_logits, int dlogits_dtype, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || K < 1 || K > E || K > 64) return MOE_ERR_ARG;
  if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_ERR_ARG;
  if (bias_mode != MOE_BIAS_LOGIT && bias_mode != MOE_BIAS_SELECT) return MOE_ERR_ARG;
  // a selection-only bias does not enter the weights
  if (bias_mode == MOE_BIAS_SELECT) bias = nullptr;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !d_topk_w || !d_logits) return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dlogits_dtype == MOE_F32)
    route_bwd_launch(logits, bias, topk_ids, d_topk_w, T, E, K, score, renorm,
                     static_cast<float*>(d_logits), st);
  else if (dlogits_dtype == MOE_BF16)
    route_bwd_launch(logits, bias, topk_ids, d_topk_w, T, E, K, score, renorm,
                     static_cast<bf16_t*>(d_logits), st);
  else
    return MOE_ERR_DTYPE;
  return launch_status();
}

MOE_API size_t moe_aux_loss_workspace(int64_t T, int E) {
  if (T < 0 || E < 1) return 0;
  const int64_t nb = (T + kAuxTok - 1) / kAuxTok;
  const size_t bytes = static_cast<size_t>(nb > 0 ? nb : 1) * E * (sizeof(float) + sizeof(int32_t));
  return (bytes + 255) & ~static_cast<size_t>(255);
}

MOE_API int moe_aux_loss(const float* logits, const int32_t* topk_ids, int64_t T, int E, int K,
                         int score, float alpha, float* loss, int32_t* expert_counts,
                         float* expert_probs, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 1 || E < 1 || E > 1024 || K < 1 || K > E || K > 64) return MOE_ERR_ARG;
  if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_ERR_ARG;
  if (!logits || !topk_ids || !loss) return MOE_ERR_ARG;
  if (ws_bytes < moe_aux_loss_workspace(T, E) || !workspace ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nb = static_cast<int>((T + kAuxTok - 1) / kAuxTok);
  float* psum = static_cast<float*>(workspace);
  int32_t* pcnt = reinterpret_cast<int32_t*>(psum + static_cast<int64_t>(nb) * E);
  const int V = (E + 63) / 64;
#define AP(VV)                                                                              \
  hipLaunchKernelGGL((aux_partial_kernel<VV>), dim3(nb), dim3(256), 0, st, logits, topk_ids, T, \
                     E, K, score, psum, pcnt)
  if (V <= 1) AP(1);
  else if (V <= 2) AP(2);
  else if (V <= 4) AP(4);
  else if (V <= 8) AP(8);
  else AP(16);
#undef AP
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(1024), 0, st, psum, pcnt, nb, T, E, K, alpha,
                     loss, expert_counts, expert_probs);
  return launch_status();
}

template <typename TO>
static void aux_bwd_launch(const float* logits, const int32_t* counts, int64_t T, int E, int K,
                           int score, float alpha, TO* d, int accumulate, hipStream_t st) {
  const int V = (E + 63) / 64;
  const unsigned g = static_cast<unsigned>((T + kWaves - 1) / kWaves);
#define AB(VV)                                                                                \
  hipLaunchKernelGGL((aux_bwd_kernel<VV, TO>), dim3(g), dim3(256), 0, st, logits, counts, T, E, \
                     K, score, alpha, d, accumulate)
  if (V <= 1) AB(1);
  else if (V <= 2) AB(2);
  else if (V <= 4) AB(4);
  else if (V <= 8) AB(8);
  else AB(16);
#undef AB
}

MOE_API int moe_aux_loss_bwd(const float* logits, const int32_t* expert_counts, int64_t T, int E,
                             int K, int score, float alpha, void* d_logits, int dlogits_dtype,
                             int accumulate, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || K < 1 || K > E || K > 64) return MOE_ERR_ARG;
  if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !expert_counts || !d_logits) return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dlogits_dtype == MOE_F32)
    aux_bwd_launch(logits, expert_counts, T, E, K, score, alpha, static_cast<float*>(d_logits),
                   accumulate, st);
  else if (dlogits_dtype == MOE_BF16)
    aux_bwd_launch(logits, expert_counts, T, E, K, score, alpha, static_cast<bf16_t*>(d_logits),
                   accumulate, st);
  else
    return MOE_ERR_DTYPE;
  return launch_status();
}
