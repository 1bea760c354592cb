// Top-K routing and its backward, one 64-lane wavefront per token.
//
// Follows the fused router of the TransformerEngine MoE block pull request
// (Description / Changes: top-K with optional sigmoid scoring): experts are
// ranked on the float32 logit (plus an optional per-expert prior), the lower
// id winning a tie; weights are softmax over all experts or the logistic
// function, optionally renormalised over the K selected.
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

template <int V>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int64_t T,
                                                    int E, int K, int score, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  float z[V];
  load_z<V>(logits + t * E, bias, E, lane, z);
  // candidate id per register slot; INT_MAX = not a candidate (padding or taken)
  int cid[V];
#pragma unroll
  for (int i = 0; i < V; ++i) cid[i] = (i * 64 + lane < E) ? i * 64 + lane : INT_MAX;

  int my_id = 0;       // lane j < K keeps the j-th selection
  float my_z = 0.f;
  for (int j = 0; j < K; ++j) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (cid[i] != INT_MAX && better(z[i], cid[i], bv, bi)) { bv = z[i]; bi = cid[i]; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    // bi is now wave-uniform; retire it
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (cid[i] == bi) cid[i] = INT_MAX;
    if (lane == j) { my_id = bi; my_z = bv; }
  }

  float p = 0.f;
  if (score == MOE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) m = fmaxf(m, z[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) s += (i * 64 + lane < E) ? expf(z[i] - m) : 0.f;
    s = wave_sum(s);
    p = (lane < K) ? expf(my_z - m) / s : 0.f;
  } else {
    p = (lane < K) ? 1.0f / (1.0f + expf(-my_z)) : 0.f;
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

}  // namespace
}  // namespace moe

using namespace moe;

#define ROUTE_LAUNCH(KERNEL, V, ...)                                                   \
  hipLaunchKernelGGL(KERNEL<V>, dim3(static_cast<unsigned>((T + kWaves - 1) / kWaves)), \
                     dim3(256), 0, st, __VA_ARGS__)

MOE_API int moe_route(const float* logits, const float* bias, int64_t T, int E, int K, int score,
                      int renorm, int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || K < 1 || K > E || K > 64) return MOE_ERR_ARG;
  if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int V = (E + 63) / 64;
  if (V <= 1) ROUTE_LAUNCH(route_kernel, 1, logits, bias, T, E, K, score, renorm, topk_ids, topk_w);
  else if (V <= 2) ROUTE_LAUNCH(route_kernel, 2, logits, bias, T, E, K, score, renorm, topk_ids, topk_w);
  else if (V <= 4) ROUTE_LAUNCH(route_kernel, 4, logits, bias, T, E, K, score, renorm, topk_ids, topk_w);
  else if (V <= 8) ROUTE_LAUNCH(route_kernel, 8, logits, bias, T, E, K, score, renorm, topk_ids, topk_w);
  else ROUTE_LAUNCH(route_kernel, 16, logits, bias, T, E, K, score, renorm, topk_ids, topk_w);
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

MOE_API int moe_route_bwd(const float* logits, const float* bias, const int32_t* topk_ids,
                          const float* d_topk_w, int64_t T, int E, int K, int score, int renorm,
                          void* d_logits, int dlogits_dtype, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || K < 1 || K > E || K > 64) return MOE_ERR_ARG;
  if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return MOE_ERR_ARG;
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
