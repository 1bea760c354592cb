// Backward of the router GEMM (logits = x . Wg, the gate projection of the
// TransformerEngine MoE block's sequence diagram; its backward is the
// gate-kernel gradient of the same diagram) with float32 d_logits:
//
//   d_Wg = x^T . d_logits            [D, E] float32
//   dx  (+)= d_logits . Wg^T         [T, D]
//
// x and Wg are bf16, d_logits is float32.  The products run on the bf16
// MFMA grouped GEMMs without losing d_logits' precision: each float32 value
// v is split into three bf16 values hi = bf16(v), mid = bf16(v - hi),
// lo = bf16(v - hi - mid) with v = hi + mid + lo exactly (v has 24
// significant bits; hi takes the leading 8 with round-to-nearest, the exact
// float32 residual has at most 16, mid takes 8 of those and the residual
// left, at most 8 bits, is lo; only values below ~2^-110 can lose bits to
// bf16 underflow).  A bf16 x bf16 product is exact in float32, so
//   x^T . [hi | mid | lo]  summed over the three planes, and
//   [hi | mid | lo] . [Wg | Wg | Wg]^T   (one contraction over 3 E)
// equal the float32 products up to the order of the float32 additions.
//
// Steps (all on `stream`):
//   1. prep: the split planes G3 [T, 3 Ep] (Ep = E rounded up to 8, zero
//      padding columns), the replicated weight W3 [D, 3 Ep] and the int32
//      group sizes of step 3 (token blocks, and T).
//   2. moe_gmm:  dx (+)= G3 . W3^T  (one group of T rows, Kdim = 3 Ep).
//   3. moe_tgmm: part[s] = x[block s]^T . G3[block s] -> [S, D, 3 Ep] float32
//      (the tokens split into S blocks so that the narrow [D, 3 Ep] output
//      still spreads over the chip).
//   4. reduce: d_Wg[d, e] = sum over s, then over the three planes, of
//      part[s, d, p Ep + e], in that fixed order (deterministic).
#include "common.h"

namespace moe {
namespace {

constexpr int kRbThreads = 256;
constexpr int kMaxSplit = 16;
constexpr int64_t kPartBudget = int64_t(64) << 20;   // bytes of float32 partials at most

int64_t round_up8(int64_t v) { return (v + 7) / 8 * 8; }

// Token blocks of the weight-gradient contraction: T / 512 of them, at most
// 16, fewer when their float32 partials would pass 64 MiB.
int split_count(int64_t T, int64_t D, int64_t Ep) {
  int64_t s = T / 512;
  if (s < 1) s = 1;
  if (s > kMaxSplit) s = kMaxSplit;
  while (s > 1 && s * D * 3 * Ep * 4 > kPartBudget) --s;
  return static_cast<int>(s);
}

struct RbLayout {
  int64_t Ep, S;
  size_t off_gs, off_g3, off_w3, off_part, total;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

RbLayout rb_layout(int64_t T, int64_t D, int E) {
  RbLayout l;
  l.Ep = round_up8(E);
  l.S = split_count(T, D, l.Ep);
  l.off_gs = 0;                                           // [kMaxSplit] split sizes, then T
  l.off_g3 = 256;
  l.off_w3 = l.off_g3 + align256(static_cast<size_t>(T * 3 * l.Ep) * 2);
  l.off_part = l.off_w3 + align256(static_cast<size_t>(D * 3 * l.Ep) * 2);
  l.total = l.off_part + align256(static_cast<size_t>(l.S * D * 3 * l.Ep) * 4);
  return l;
}

// Step 1: G3 planes from d_logits, W3 copies of Wg, and the group sizes.
__global__ __launch_bounds__(kRbThreads) void router_bwd_prep_kernel(
    const float* __restrict__ dl, const bf16_t* __restrict__ wg, int64_t T, int64_t D, int E,
    int64_t Ep, int S, bf16_t* __restrict__ g3, bf16_t* __restrict__ w3, int32_t* __restrict__ gs) {
  const int64_t n_g = T * Ep, n_w = D * Ep;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_g + n_w;
       i += stride) {
    if (i < n_g) {
      const int64_t t = i / Ep, e = i - t * Ep;
      const float v = e < E ? dl[t * E + e] : 0.f;
      const bf16_t hi = f32_to_bf16(v);
      const float r1 = v - bf16_to_f32(hi);          // exact
      const bf16_t mid = f32_to_bf16(r1);
      const bf16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));   // exact, and representable
      bf16_t* row = g3 + t * 3 * Ep;
      row[e] = hi;
      row[Ep + e] = mid;
      row[2 * Ep + e] = lo;
    } else {
      const int64_t j = i - n_g;
      const int64_t d = j / Ep, e = j - d * Ep;
      const bf16_t w = e < E ? wg[d * E + e] : bf16_t(0);
      bf16_t* row = w3 + d * 3 * Ep;
      row[e] = w;
      row[Ep + e] = w;
      row[2 * Ep + e] = w;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x <= kMaxSplit) {
    const int s = threadIdx.x;
    const int64_t per = T / S;
    int32_t v = 0;
    if (s < S) v = static_cast<int32_t>(s == S - 1 ? T - per * (S - 1) : per);
    if (s == kMaxSplit) v = static_cast<int32_t>(T);
    gs[s] = v;
  }
}

// Step 4: d_Wg[d, e] = sum_s sum_p part[s, d, p Ep + e].
__global__ __launch_bounds__(kRbThreads) void router_bwd_reduce_kernel(
    const float* __restrict__ part, int64_t D, int E, int64_t Ep, int S, float* __restrict__ out) {
  const int64_t n = D * E;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t d = i / E, e = i - d * E;
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* row = part + (static_cast<int64_t>(s) * D + d) * 3 * Ep;
      acc += row[e];
      acc += row[Ep + e];
      acc += row[2 * Ep + e];
    }
    out[i] = acc;
  }
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + kRbThreads - 1) / kRbThreads;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  if (b > cap) b = cap;
  return static_cast<unsigned>(b < 1 ? 1 : b);
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API size_t moe_router_bwd_workspace(int64_t T, int64_t D, int E) {
  if (T < 0 || D < 0 || E < 1) return 0;
  return rb_layout(T, D, E).total;
}

MOE_API int moe_router_bwd(const void* x, const void* Wg, const float* d_logits, int64_t T,
                           int64_t D, int E, float* d_Wg, void* dx, int dx_dtype,
                           int accumulate_dx, void* workspace, size_t ws_bytes, int32_t* err,
                           void* stream) {
  if (T < 0 || T > INT32_MAX || D < 1 || E < 1 || E > 1024 || D % 8) return MOE_ERR_ARG;
  if (dx_dtype != MOE_BF16 && dx_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (!Wg || !d_Wg || (T > 0 && (!x || !d_logits || !dx))) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(Wg) || (dx && !aligned16(dx))) return MOE_ERR_ARG;
  const RbLayout l = rb_layout(T, D, E);
  if (!workspace || ws_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {   // no tokens: d_Wg = 0 (no partial sums to add), dx is empty
    hipLaunchKernelGGL(router_bwd_reduce_kernel, dim3(grid_for(D * E)), dim3(kRbThreads), 0, st,
                       static_cast<const float*>(nullptr), D, E, round_up8(E), 0, d_Wg);
    return launch_status();
  }
  char* ws = static_cast<char*>(workspace);
  int32_t* gs = reinterpret_cast<int32_t*>(ws + l.off_gs);
  bf16_t* g3 = reinterpret_cast<bf16_t*>(ws + l.off_g3);
  bf16_t* w3 = reinterpret_cast<bf16_t*>(ws + l.off_w3);
  float* part = reinterpret_cast<float*>(ws + l.off_part);
  const int S = static_cast<int>(l.S);
  const int64_t K3 = 3 * l.Ep;
  hipLaunchKernelGGL(router_bwd_prep_kernel, dim3(grid_for((T + D) * l.Ep)), dim3(kRbThreads), 0,
                     st, d_logits, static_cast<const bf16_t*>(Wg), T, D, E, l.Ep, S, g3, w3, gs);
  int rc = launch_status();
  if (rc != MOE_OK) return rc;
  // dx (+)= G3 . W3^T: one group of T rows contracting over the 3 planes
  rc = moe_gmm(g3, T, K3, w3, K3, D * K3, 1, gs + kMaxSplit, nullptr, 1, K3, D, MOE_BF16, nullptr,
               dx, T, D, dx_dtype, accumulate_dx, err, stream);
  if (rc != MOE_OK) return rc;
  // part[s] = x[block s]^T . G3[block s]
  rc = moe_tgmm(x, D, g3, K3, gs, nullptr, S, T, D, K3, MOE_BF16, part, K3, D * K3, MOE_F32, 0,
                err, stream);
  if (rc != MOE_OK) return rc;
  hipLaunchKernelGGL(router_bwd_reduce_kernel, dim3(grid_for(D * E)), dim3(kRbThreads), 0, st, part,
                     D, E, l.Ep, S, d_Wg);
  return launch_status();
}
