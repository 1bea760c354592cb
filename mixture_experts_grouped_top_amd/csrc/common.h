// Internal helpers shared by the HIP sources of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

typedef uint16_t bf16_t;  // bf16 storage: the upper 16 bits of an IEEE float32

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two packed bf16 in one dword (lo = a, hi = b): round to
// nearest, ties to even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// float32 -> bf16, round to nearest, ties to even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.f));
}

// SwiGLU of one element, float32: silu(g) * u with silu(g) = g / (1 + e^-g).
// One definition for the SwiGLU pass and the fused up-projection epilogue,
// so that both give the same bits.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Gradients of SwiGLU for an upstream gradient d: d_g = d u s (1 + g (1 - s)),
// d_u = d g s with s = sigmoid(g).  One definition for the backward pass and
// the fused d_act epilogue.
__device__ __forceinline__ void swiglu_bwd_f32(float g, float u, float d, float& dg, float& du) {
  const float s = 1.0f / (1.0f + expf(-g));
  dg = d * u * s * (1.0f + g * (1.0f - s));
  du = d * g * s;
}

// Wave 0 scans the group sizes: row_base[g] (rows clipped to max_rows) and,
// if tile_base != nullptr, tile_base[g] = tiles of groups < g, where a group
// of n rows owns ceil(n / BM) * ntn tiles when cls_lo <= n <= cls_hi, else
// none.
__device__ inline void scan_groups(const int32_t* __restrict__ gsz, int G, int64_t max_rows, int BMv,
                            int ntn, int* row_base, int* tile_base, int32_t* err,
                            int cls_lo = 0, int cls_hi = 0x7fffffff) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int64_t rows_run = 0;
  int tiles_run = 0;
  bool bad = false;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int n = (g < G) ? gsz[g] : 0;
    if (n < 0) { n = 0; bad = true; }
    int64_t incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    int64_t start = rows_run + incl - n;
    int64_t end = rows_run + incl;
    if (end > max_rows) bad = true;
    if (start > max_rows) start = max_rows;
    if (end > max_rows) end = max_rows;
    const int neff = static_cast<int>(end - start);
    // only groups of cls_lo .. cls_hi rows own tiles (a launch for one size class)
    int t = tile_base && neff >= cls_lo && neff <= cls_hi ? ((neff + BMv - 1) / BMv) * ntn : 0;
    int tincl = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(tincl, o, 64);
      if (lane >= o) tincl += u;
    }
    if (g < G) {
      row_base[g] = static_cast<int>(start);
      if (tile_base) tile_base[g] = tiles_run + tincl - t;
    }
    rows_run += __shfl(incl, 63, 64);
    tiles_run += __shfl(tincl, 63, 64);
  }
  if (lane == 0) {
    row_base[G] = static_cast<int>(rows_run > max_rows ? max_rows : rows_run);
    if (tile_base) tile_base[G] = tiles_run;
  }
  if (bad && lane == 0 && err) atomicOr(err, MOE_DERR_GROUP_SIZES);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Load/store 8 consecutive elements (16 B for bf16, 32 B for f32) as floats.
__device__ __forceinline__ void load8(const bf16_t* p, float v[8]) {
  uint4 q = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const float v[8]) {
  uint4 q;
  q.x = pack_bf16x2(v[0], v[1]);
  q.y = pack_bf16x2(v[2], v[3]);
  q.z = pack_bf16x2(v[4], v[5]);
  q.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = q;
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Streaming (non-temporal) 16-byte accesses for data touched once: they
// leave L2 capacity to data that is reused.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4* p, uint4 v) {
  const u32x4 q = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void unpack8(const uint4& q, float v[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8_nt(const bf16_t* p, float v[8]) {
  unpack8(ld_nt(reinterpret_cast<const uint4*>(p)), v);
}
__device__ __forceinline__ void load8_nt(const float* p, float v[8]) {
  const uint4 a = ld_nt(reinterpret_cast<const uint4*>(p));
  const uint4 b = ld_nt(reinterpret_cast<const uint4*>(p + 4));
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
  v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
  v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ void store8_nt(bf16_t* p, const float v[8]) {
  st_nt(reinterpret_cast<uint4*>(p),
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])));
}
__device__ __forceinline__ void store8_nt(float* p, const float v[8]) {
  st_nt(reinterpret_cast<uint4*>(p), make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                __float_as_uint(v[2]), __float_as_uint(v[3])));
  st_nt(reinterpret_cast<uint4*>(p + 4), make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]),
                                                    __float_as_uint(v[6]), __float_as_uint(v[7])));
}

// Eight elements as raw bits (one 16-byte chunk for bf16, two for float32),
// loaded with a streaming hint; unpacked to float32 only after a batch of
// loads has been issued.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 q;
  __device__ __forceinline__ void load(const bf16_t* p) { q = ld_nt(reinterpret_cast<const uint4*>(p)); }
  __device__ __forceinline__ void get(float v[8]) const { unpack8(q, v); }
};
template <> struct Raw8<float> {
  uint4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = ld_nt(reinterpret_cast<const uint4*>(p));
    b = ld_nt(reinterpret_cast<const uint4*>(p + 4));
  }
  __device__ __forceinline__ void get(float v[8]) const {
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : (dtype == MOE_F32 ? 4 : 0); }

inline int launch_status() {
  if (hipPeekAtLastError() == hipSuccess) return MOE_OK;
  (void)hipGetLastError();  // clear the sticky launch error
  return MOE_ERR_LAUNCH;
}

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe
