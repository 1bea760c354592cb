// FP8 current scaling of the expert-GEMM operands (the quantization=fp8
// recipe of the MaxText pull request "[Draft] Integrate TE/JAX GroupedGEMM
// for MoE": current-tensor scaling, e4m3 forward / e5m2 backward, two
// quantized copies; the per-expert amax of the expert weights named in the
// TransformerEngine MoE block pull request's commit notes).
//
//   moe_fp8_amax_scale  amax = max |x| per scaling unit (the whole tensor, or
//                       each of G equal row blocks: one expert's weight), then
//                       scale = fmax / amax (1 if amax is 0) and
//                       scale_inv = 1 / scale, correctly rounded float32.
//   moe_fp8_quantize    q = fp8(x * scale): the float32 product rounded to
//                       the nearest FP8 value (ties to even), saturated at
//                       fmax, sign kept.  Writes a row-wise copy and/or a
//                       transposed copy; both feed GEMMs whose operands are
//                       contraction-contiguous.
// HBM-bound.  OCP formats: E4M3FN (bias 7, 3 mantissa bits, fmax 448) and
// E5M2 (bias 15, 2 mantissa bits, fmax 57344).
#include "common.h"

namespace moe {
namespace {

constexpr int kAmaxPerBlock = 16384;   // elements per amax block (target)
constexpr int kMaxGroups = 1024;

// Code of the FP8 value nearest to v (ties to even), saturating; sign kept.
template <int FMT>
__device__ __forceinline__ uint32_t f32_to_fp8(float v) {
  constexpr int MB = FMT == MOE_FP8_E4M3 ? 3 : 2;
  constexpr int BIAS = FMT == MOE_FP8_E4M3 ? 7 : 15;
  constexpr uint32_t MAXC = FMT == MOE_FP8_E4M3 ? 0x7Eu : 0x7Bu;
  constexpr float FMAX = FMT == MOE_FP8_E4M3 ? 448.f : 57344.f;
  // smallest normal 2^(1 - BIAS); subnormal spacing 2^(1 - BIAS - MB)
  constexpr float MIN_NORMAL = FMT == MOE_FP8_E4M3 ? 0x1p-6f : 0x1p-14f;
  constexpr float INV_SUB_STEP = FMT == MOE_FP8_E4M3 ? 0x1p9f : 0x1p16f;
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7FFFFFFFu;
  const float a = __uint_as_float(ua);
  uint32_t code;
  if (!(a < FMAX)) {
    code = MAXC;
  } else if (a < MIN_NORMAL) {
    // exact power-of-two scaling, then round half to even (v_rndne_f32)
    code = static_cast<uint32_t>(__builtin_rintf(a * INV_SUB_STEP));
  } else {
    const int e = static_cast<int>(ua >> 23) - 127;
    const uint32_t m = ua & 0x7FFFFFu;
    uint32_t q = m >> (23 - MB);
    const uint32_t rem = m & ((1u << (23 - MB)) - 1u);
    const uint32_t half = 1u << (22 - MB);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    code = (static_cast<uint32_t>(e + BIAS) << MB) + q;   // a carry moves to the exponent
    if (code > MAXC) code = MAXC;
  }
  return sign | code;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// grid (nb, G): block b of unit g takes a grid-strided share of the unit's
// rows x cols elements (8 per thread per access) and writes its max |x|.
template <typename T>
__global__ __launch_bounds__(256) void amax_partial_kernel(const T* __restrict__ x, int64_t ld,
                                                           int64_t rows_per_unit, int64_t cols,
                                                           float* __restrict__ part) {
  const int g = blockIdx.y, nb = gridDim.x;
  const int64_t cpr = cols / 8;                      // 8-element chunks per row
  const int64_t n = rows_per_unit * cpr;
  const T* base = x + static_cast<int64_t>(g) * rows_per_unit * ld;
  float m = 0.f;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(nb) * 256) {
    const int64_t r = i / cpr, c = (i - r * cpr) * 8;
    Raw8<T> raw;
    raw.load(base + r * ld + c);
    float v[8];
    raw.get(v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    part[static_cast<int64_t>(g) * nb + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One block per unit: amax over its partials, then the scales.
template <int FMT>
__global__ __launch_bounds__(256) void scale_final_kernel(const float* __restrict__ part, int nb,
                                                          float* __restrict__ out, int G) {
  const int g = blockIdx.x;
  float m = 0.f;
  for (int b = threadIdx.x; b < nb; b += 256) m = fmaxf(m, part[static_cast<int64_t>(g) * nb + b]);
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float fmaxv = FMT == MOE_FP8_E4M3 ? 448.f : 57344.f;
    const float s = amax > 0.f ? __fdiv_rn(fmaxv, amax) : 1.f;
    out[g] = amax;
    out[G + g] = s;
    out[2 * G + g] = __fdiv_rn(1.f, s);
  }
}

int amax_blocks(int64_t elems, int G) {
  int64_t nb = (elems + kAmaxPerBlock - 1) / kAmaxPerBlock;
  const int64_t cap = G >= 2048 ? 1 : 2048 / G;
  if (nb > cap) nb = cap;
  return static_cast<int>(nb < 1 ? 1 : nb);
}

// Quantize tiles of 64 rows x 64 columns of a row-grouped matrix.  The tile
// schedule follows the 64-row tiles of each group (tile_base from the group
// sizes), times the column tiles.  Each thread converts 16 elements of one
// row (two 16-byte loads); the row-wise copy gets them as one 16-byte store,
// the transposed copy through an LDS transpose as 16-byte runs of rows.
// Transposed layouts:
//   qt_gs == 0: one [cols, P] matrix, group g's rows at columns
//               64 * (64-row tiles of the groups before g), the rows between
//               a group's end and its next multiple of 64 written as zero;
//   qt_gs > 0:  group g at qt + g * qt_gs as [cols, n_g] (row stride ld_qt),
//               only the group's own rows written.
template <typename T, int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(
    const T* __restrict__ x, int64_t ld, int64_t rows, int64_t cols,
    const int32_t* __restrict__ gsz, int G, const float* __restrict__ scale, int per_group,
    uint8_t* __restrict__ q, int64_t ld_q, uint8_t* __restrict__ qt, int64_t ld_qt, int64_t qt_gs,
    int32_t* err) {
  __shared__ int row_base[kMaxGroups + 1];
  __shared__ int tile_base[kMaxGroups + 1];
  __shared__ __attribute__((aligned(16))) uint8_t tr[64][64 + 16];
  const int ntc = static_cast<int>((cols + 63) / 64);
  scan_groups(gsz, G, rows, 64, 1, row_base, tile_base, blockIdx.x == 0 ? err : nullptr);
  __syncthreads();
  const int64_t total = static_cast<int64_t>(tile_base[G]) * ntc;
  const int tid = threadIdx.x;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int rt = static_cast<int>(t / ntc), ct = static_cast<int>(t - static_cast<int64_t>(rt) * ntc);
    int lo = 0, hi = G - 1;   // largest g with tile_base[g] <= rt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= rt) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int lr = rt - tile_base[g];                 // row tile inside the group
    const int n_g = row_base[g + 1] - row_base[g];
    const int r_in = 64 * lr;                         // first group row of the tile
    const int rv = min(64, n_g - r_in);
    const float s = scale[per_group ? g : 0];
    // thread: row tid / 4, columns 16 (tid % 4) .. + 15 of the tile
    const int r = tid >> 2, c16 = (tid & 3) * 16;
    const int64_t col = static_cast<int64_t>(ct) * 64 + c16;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (r < rv && col < cols) {
      const T* p = x + (static_cast<int64_t>(row_base[g]) + r_in + r) * ld + col;
      float v[16];
      Raw8<T> a, b;
      a.load(p);
      const bool two = col + 8 < cols;
      if (two) b.load(p + 8);
      a.get(v);
      if (two) b.get(v + 8);
      else
#pragma unroll
        for (int e = 8; e < 16; ++e) v[e] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) w[e >> 2] |= f32_to_fp8<FMT>(__fmul_rn(v[e], s)) << (8 * (e & 3));
      if (q) {
        uint8_t* d = q + (static_cast<int64_t>(row_base[g]) + r_in + r) * ld_q + col;
        // rows are 16-byte aligned when ld_q is a multiple of 16, else 8-byte
        if (two && !(ld_q & 15)) {
          *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          *reinterpret_cast<uint2*>(d) = make_uint2(w[0], w[1]);
          if (two) *reinterpret_cast<uint2*>(d + 8) = make_uint2(w[2], w[3]);
        }
      }
    }
    if (qt) {
      // rows past rv (group end, zero padding) carry zeros
#pragma unroll
      for (int e = 0; e < 16; ++e) tr[c16 + e][r] = static_cast<uint8_t>(w[e >> 2] >> (8 * (e & 3)));
      __syncthreads();
      // thread: tile column tid / 4, rows 16 (tid % 4) .. + 15
      const int cc = tid >> 2, r16 = (tid & 3) * 16;
      const int64_t gc = static_cast<int64_t>(ct) * 64 + cc;
      const int rows_out = qt_gs ? rv : 64;           // the global layout pads to 64
      if (gc < cols && r16 < rows_out) {
        uint8_t* d;
        if (qt_gs) d = qt + static_cast<int64_t>(g) * qt_gs + gc * ld_qt + r_in + r16;
        else d = qt + gc * ld_qt + static_cast<int64_t>(rt) * 64 + r16;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(&tr[cc][r16]);
        if (r16 + 16 <= rows_out) {
          *reinterpret_cast<uint4*>(d) = make_uint4(src[0], src[1], src[2], src[3]);
        } else {
          for (int e = 0; e < rows_out - r16; ++e) d[e] = tr[cc][r16 + e];
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API size_t moe_fp8_scale_workspace(int64_t rows, int64_t cols, int G) {
  if (rows < 0 || cols < 0 || G < 1) return 0;
  return static_cast<size_t>(G) * amax_blocks(rows / G * cols, G) * sizeof(float);
}

MOE_API int moe_fp8_amax_scale(const void* x, int64_t ld, int dtype, int64_t rows, int64_t cols,
                               int G, int fmt, float* scales, void* workspace, size_t ws_bytes,
                               void* stream) {
  if (rows < 0 || cols < 0 || G < 1 || ld < cols || rows % G) return MOE_ERR_ARG;
  if (!elem_bytes(dtype)) return MOE_ERR_DTYPE;
  if (fmt != MOE_FP8_E4M3 && fmt != MOE_FP8_E5M2) return MOE_ERR_ARG;
  if (cols % 8 || ld % 8 || !scales) return MOE_ERR_ARG;
  if (rows > 0 && cols > 0 && (!x || !aligned16(x))) return MOE_ERR_ARG;
  const int64_t per = rows / G;
  const int nb = amax_blocks(per * cols, G);
  if (!workspace || ws_bytes < static_cast<size_t>(G) * nb * sizeof(float) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15))
    return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  const dim3 grid(static_cast<unsigned>(nb), static_cast<unsigned>(G));
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(amax_partial_kernel<bf16_t>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(x), ld, per, cols, part);
  else
    hipLaunchKernelGGL(amax_partial_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(x), ld, per, cols, part);
  if (fmt == MOE_FP8_E4M3)
    hipLaunchKernelGGL(scale_final_kernel<MOE_FP8_E4M3>, dim3(G), dim3(256), 0, st, part, nb, scales, G);
  else
    hipLaunchKernelGGL(scale_final_kernel<MOE_FP8_E5M2>, dim3(G), dim3(256), 0, st, part, nb, scales, G);
  return launch_status();
}

MOE_API int moe_fp8_quantize(const void* x, int64_t ld, int dtype, int64_t rows, int64_t cols,
                             const int32_t* group_sizes, int G, const float* scale, int per_group,
                             int fmt, void* q, int64_t ld_q, void* qt, int64_t ld_qt,
                             int64_t qt_group_stride, int32_t* err, void* stream) {
  if (rows < 0 || cols < 0 || G < 1 || G > kMaxGroups || ld < cols) return MOE_ERR_ARG;
  if (rows > INT32_MAX) return MOE_ERR_ARG;
  if (!elem_bytes(dtype)) return MOE_ERR_DTYPE;
  if (fmt != MOE_FP8_E4M3 && fmt != MOE_FP8_E5M2) return MOE_ERR_ARG;
  if (cols % 8 || ld % 8 || !group_sizes || !scale || (!q && !qt)) return MOE_ERR_ARG;
  if (q && (ld_q < cols || ld_q % 8 || !aligned16(q))) return MOE_ERR_ARG;
  if (qt && (ld_qt % 16 || !aligned16(qt) || qt_group_stride < 0 || qt_group_stride % 16))
    return MOE_ERR_ARG;
  if (qt && qt_group_stride == 0 && ld_qt < moe_fp8_padded_rows(rows, G)) return MOE_ERR_ARG;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!x || !aligned16(x)) return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t tiles = ((rows + 63) / 64 + G) * ((cols + 63) / 64);
  int64_t grid = static_cast<int64_t>(device_cu_count()) * 8;
  if (tiles < grid) grid = tiles;
  if (grid < 1) grid = 1;
#define QZ(T, F)                                                                              \
  hipLaunchKernelGGL((quantize_kernel<T, F>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, \
                     st, static_cast<const T*>(x), ld, rows, cols, group_sizes, G, scale,       \
                     per_group, static_cast<uint8_t*>(q), ld_q, static_cast<uint8_t*>(qt),     \
                     ld_qt, qt_group_stride, err)
  if (dtype == MOE_BF16) {
    if (fmt == MOE_FP8_E4M3) QZ(bf16_t, MOE_FP8_E4M3); else QZ(bf16_t, MOE_FP8_E5M2);
  } else {
    if (fmt == MOE_FP8_E4M3) QZ(float, MOE_FP8_E4M3); else QZ(float, MOE_FP8_E5M2);
  }
#undef QZ
  return launch_status();
}
