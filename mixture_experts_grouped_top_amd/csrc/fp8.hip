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

// Codes of the FP8 values nearest to a, b, c, d (ties to even), saturating,
// sign kept, packed a in the low byte: each value is clamped to +-fmax
// (v_med3_f32) and converted by v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32, two per
// instruction.  The clamp makes the hardware rounding saturate; for every
// finite float32 this gives the same code as rounding the exact value to
// nearest-even and saturating (compared over all 2^32 bit patterns).
template <int FMT>
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  constexpr float FMAX = FMT == MOE_FP8_E4M3 ? 448.f : 57344.f;
  a = __builtin_amdgcn_fmed3f(a, -FMAX, FMAX);
  b = __builtin_amdgcn_fmed3f(b, -FMAX, FMAX);
  c = __builtin_amdgcn_fmed3f(c, -FMAX, FMAX);
  d = __builtin_amdgcn_fmed3f(d, -FMAX, FMAX);
  int r;
  if constexpr (FMT == MOE_FP8_E4M3) {
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  } else {
    r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  }
  return static_cast<uint32_t>(r);
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
  // four chunks per thread in flight per iteration
  constexpr int U = 4;
  const int64_t stride = static_cast<int64_t>(nb) * 256;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i0 < n; i0 += U * stride) {
    Raw8<T> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n) {
        const int64_t r = i / cpr, c = (i - r * cpr) * 8;
        raw[u].load(base + r * ld + c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * stride >= n) break;
      float v[8];
      raw[u].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    }
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

// Quantize tiles of 128 rows x 128 columns of a row-grouped matrix.  The
// rows of a tile are two 64-row tiles of the groups' 64-row tiling (which
// may belong to two groups), so every row segment of both copies a tile
// writes is a whole 128-byte line, written by one workgroup at one time.
// Each thread converts 8 consecutive rows x 8 columns (one 16-byte bf16
// load per row, eight in flight); the 16 lanes that share its rows read
// whole lines of each row (256 contiguous bytes of bf16) and write one
// whole 128-byte line of the row-wise copy.  A thread writes its 8 rows of
// each of its columns (two dwords) into an LDS tile that is read back
// along columns for the transposed copy.
// Transposed layouts:
//   qt_gs == 0: one [cols, P] matrix, the 64-row tile rt of the groups'
//               tiling at columns 64 rt (a group's rows, then zeros up to
//               its next multiple of 64);
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
  __shared__ __attribute__((aligned(16))) uint32_t tr[128][32 + 4];   // [column][rows / 4]
  const int ntc = static_cast<int>((cols + 127) / 128);
  scan_groups(gsz, G, rows, 64, 1, row_base, tile_base, blockIdx.x == 0 ? err : nullptr);
  __syncthreads();
  const int nrt = tile_base[G];                       // 64-row tiles
  const int64_t total = static_cast<int64_t>((nrt + 1) / 2) * ntc;
  const int tid = threadIdx.x;
  const int rg = tid >> 4, cg = tid & 15;              // rows 8 rg .. + 7, columns 8 cg .. + 7
  const int half = rg >> 3;                            // which 64-row tile of the pair
  auto group_of = [&](int rt) {
    int lo = 0, hi = G - 1;   // largest g with tile_base[g] <= rt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= rt) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int pr = static_cast<int>(t / ntc), ct = static_cast<int>(t - static_cast<int64_t>(pr) * ntc);
    // this thread's 64-row tile
    const int rt = 2 * pr + half;
    const bool tile_ok = rt < nrt;
    const int g = tile_ok ? group_of(rt) : 0;
    const int r_in = tile_ok ? 64 * (rt - tile_base[g]) : 0;     // first group row of the tile
    const int rv = tile_ok ? min(64, row_base[g + 1] - row_base[g] - r_in) : 0;
    const int lr = 8 * (rg & 7);                       // first of the thread's rows in its tile
    const int64_t col = static_cast<int64_t>(ct) * 128 + 8 * cg;
    const bool col_ok = col < cols;                    // cols is a multiple of 8
    const float s = scale[per_group ? g : 0];
    // eight loads, one per row; a lane with nothing to load reads x[0..7]
    Raw8<T> raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = col_ok && lr + i < rv;
      const T* p = x + (static_cast<int64_t>(row_base[g]) + r_in + lr + i) * ld + col;
      raw[i].load(ok ? p : x);
    }
    uint32_t w[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = col_ok && lr + i < rv;
      float v[8];
      raw[i].get(v);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t c = pack4_fp8<FMT>(__fmul_rn(v[4 * k], s), __fmul_rn(v[4 * k + 1], s),
                                          __fmul_rn(v[4 * k + 2], s), __fmul_rn(v[4 * k + 3], s));
        w[i][k] = ok ? c : 0u;
      }
      if (q && ok) {
        // 8-byte aligned: col and ld_q are multiples of 8
        uint8_t* d = q + (static_cast<int64_t>(row_base[g]) + r_in + lr + i) * ld_q + col;
        *reinterpret_cast<uint2*>(d) = make_uint2(w[i][0], w[i][1]);
      }
    }
    if (qt) {
      // column 8 cg + e, rows 8 rg .. + 7 as two dwords (row 8 rg in the low byte)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 8 * (e & 3);
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo |= ((w[i][e >> 2] >> sh) & 0xFFu) << (8 * i);
          hi |= ((w[i + 4][e >> 2] >> sh) & 0xFFu) << (8 * i);
        }
        *reinterpret_cast<uint2*>(&tr[8 * cg + e][2 * rg]) = make_uint2(lo, hi);
      }
      __syncthreads();
      // thread: tile column tid / 2, the 64 rows of tile 2 pr + (tid & 1)
      const int cc = tid >> 1, h = tid & 1;
      const int rt2 = 2 * pr + h;
      const int64_t gc = static_cast<int64_t>(ct) * 128 + cc;
      if (rt2 < nrt && gc < cols) {
        const uint32_t* sv = &tr[cc][16 * h];
        if (qt_gs == 0) {
          uint8_t* d = qt + gc * ld_qt + static_cast<int64_t>(rt2) * 64;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            *reinterpret_cast<uint4*>(d + 16 * k) = make_uint4(sv[4 * k], sv[4 * k + 1], sv[4 * k + 2], sv[4 * k + 3]);
        } else {
          const int g2 = group_of(rt2);
          const int r2 = 64 * (rt2 - tile_base[g2]);
          const int rv2 = min(64, row_base[g2 + 1] - row_base[g2] - r2);
          uint8_t* d = qt + static_cast<int64_t>(g2) * qt_gs + gc * ld_qt + r2;
          if (rv2 == 64) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              *reinterpret_cast<uint4*>(d + 16 * k) = make_uint4(sv[4 * k], sv[4 * k + 1], sv[4 * k + 2], sv[4 * k + 3]);
          } else {
            const uint8_t* sb = reinterpret_cast<const uint8_t*>(sv);
            for (int e = 0; e < rv2; ++e) d[e] = sb[e];
          }
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
  const int64_t tiles = ((rows + 63) / 128 + G) * ((cols + 127) / 128);
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
