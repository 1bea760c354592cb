// SwiGLU gating of the expert FFN and its backward, elementwise over
// [rows, F], four groups of 8 elements per thread per step (HBM-bound).  The two inputs
// are the gate and up projection outputs named in the TransformerEngine MoE
// block pull request's commit notes (gate_proj_out, up_proj_out).
#include "common.h"

namespace moe {
namespace {

// Grid-stride over groups of kU x 8 elements per thread: all loads of a
// group are issued (streaming hint) before any is used.
constexpr int kU = 4;

// Element group i (8 elements) of a [rows, F] matrix with row stride ld
// (cpr = F / 8 groups per row; i < 2^31 is checked on the host).
__device__ __forceinline__ int64_t strided8(uint32_t i, uint32_t cpr, int64_t ld) {
  const uint32_t r = i / cpr;
  return static_cast<int64_t>(r) * ld + static_cast<int64_t>(i - r * cpr) * 8;
}

template <typename TH, typename TA>
__global__ __launch_bounds__(256) void swiglu_kernel(const TH* __restrict__ h0,
                                                     const TH* __restrict__ h1, int64_t n8,
                                                     uint32_t cpr, int64_t ld_h,
                                                     TA* __restrict__ act) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * kU;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 * kU + threadIdx.x; i0 < n8;
       i0 += stride) {
    Raw8<TH> ra[kU], rb[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i < n8) {
        const int64_t o = strided8(static_cast<uint32_t>(i), cpr, ld_h);
        ra[u].load(h0 + o);
        rb[u].load(h1 + o);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i >= n8) break;
      float a[8], b[8], o[8];
      ra[u].get(a);
      rb[u].get(b);
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = swiglu_f32(a[q], b[q]);
      store8_nt(act + i * 8, o);
    }
  }
}

template <typename TH, typename TD>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const TH* __restrict__ h0,
                                                         const TH* __restrict__ h1,
                                                         int64_t ld_h,
                                                         const TD* __restrict__ da, int64_t n8,
                                                         uint32_t cpr, TD* __restrict__ d0,
                                                         TD* __restrict__ d1, int64_t ld_d) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * kU;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 * kU + threadIdx.x; i0 < n8;
       i0 += stride) {
    Raw8<TH> ra[kU], rb[kU];
    Raw8<TD> rg[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i < n8) {
        const int64_t o = strided8(static_cast<uint32_t>(i), cpr, ld_h);
        ra[u].load(h0 + o);
        rb[u].load(h1 + o);
        rg[u].load(da + i * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i >= n8) break;
      float a[8], b[8], g[8], o0[8], o1[8];
      ra[u].get(a);
      rb[u].get(b);
      rg[u].get(g);
#pragma unroll
      for (int q = 0; q < 8; ++q) swiglu_bwd_f32(a[q], b[q], g[q], o0[q], o1[q]);
      const int64_t od = strided8(static_cast<uint32_t>(i), cpr, ld_d);
      store8_nt(d0 + od, o0);
      store8_nt(d1 + od, o1);
    }
  }
}

unsigned grid_for(int64_t n8) {
  int64_t g = (n8 + 256 * kU - 1) / (256 * kU);
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 16;
  if (g > cap) g = cap;
  return static_cast<unsigned>(g < 1 ? 1 : g);
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API int moe_swiglu(const void* h0, const void* h1, int h_dtype, int64_t rows, int64_t F,
                       int64_t ld_h, void* act, int act_dtype, void* stream) {
  if (rows < 0 || F < 0 || ld_h < F) return MOE_ERR_ARG;
  if (!elem_bytes(h_dtype) || !elem_bytes(act_dtype)) return MOE_ERR_DTYPE;
  const int64_t n = rows * F;
  if (n == 0) return MOE_OK;
  if (!h0 || !h1 || !act || F % 8 || ld_h % 8 || !aligned16(h0) || !aligned16(h1) ||
      !aligned16(act))
    return MOE_ERR_ARG;
  const int64_t n8 = n / 8;
  if (n8 > INT32_MAX) return MOE_ERR_ARG;
  const uint32_t cpr = static_cast<uint32_t>(F / 8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned g = grid_for(n8);
#define SW(TH, TA)                                                                   \
  hipLaunchKernelGGL((swiglu_kernel<TH, TA>), dim3(g), dim3(256), 0, st,            \
                     static_cast<const TH*>(h0), static_cast<const TH*>(h1), n8, cpr, \
                     ld_h, static_cast<TA*>(act))
  if (h_dtype == MOE_BF16 && act_dtype == MOE_BF16) SW(bf16_t, bf16_t);
  else if (h_dtype == MOE_BF16) SW(bf16_t, float);
  else if (act_dtype == MOE_BF16) SW(float, bf16_t);
  else SW(float, float);
#undef SW
  return launch_status();
}

MOE_API int moe_swiglu_bwd(const void* h0, const void* h1, int h_dtype, int64_t ld_h,
                           const void* d_act, int64_t rows, int64_t F, void* d_h0, void* d_h1,
                           int64_t ld_dh, int d_dtype, void* stream) {
  if (rows < 0 || F < 0 || ld_h < F || ld_dh < F) return MOE_ERR_ARG;
  if (!elem_bytes(h_dtype) || !elem_bytes(d_dtype)) return MOE_ERR_DTYPE;
  const int64_t n = rows * F;
  if (n == 0) return MOE_OK;
  if (!h0 || !h1 || !d_act || !d_h0 || !d_h1 || F % 8 || ld_h % 8 || ld_dh % 8 ||
      !aligned16(h0) || !aligned16(h1) || !aligned16(d_act) || !aligned16(d_h0) ||
      !aligned16(d_h1))
    return MOE_ERR_ARG;
  const int64_t n8 = n / 8;
  if (n8 > INT32_MAX) return MOE_ERR_ARG;
  const uint32_t cpr = static_cast<uint32_t>(F / 8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned g = grid_for(n8);
#define SWB(TH, TD)                                                                          \
  hipLaunchKernelGGL((swiglu_bwd_kernel<TH, TD>), dim3(g), dim3(256), 0, st,                \
                     static_cast<const TH*>(h0), static_cast<const TH*>(h1), ld_h,           \
                     static_cast<const TD*>(d_act), n8, cpr, static_cast<TD*>(d_h0),         \
                     static_cast<TD*>(d_h1), ld_dh)
  if (h_dtype == MOE_BF16 && d_dtype == MOE_BF16) SWB(bf16_t, bf16_t);
  else if (h_dtype == MOE_BF16) SWB(bf16_t, float);
  else if (d_dtype == MOE_BF16) SWB(float, bf16_t);
  else SWB(float, float);
#undef SWB
  return launch_status();
}
