// Grouped GEMM (gmm) and transposed grouped GEMM (tgmm) for gfx950.
//
// Semantics follow the MaxText pull request "Overlap moe comms with collective
// matmul" (gmm with an in-place partial sum whose row count may be below the
// padded lhs row count; tgmm with zero-initialised empty groups and output
// shape (groups, in_size, out_size)) and the grouped_gemm calls of the
// TransformerEngine MoE block.
//
// bf16 path: v_mfma_f32_32x32x16_bf16, float32 accumulators.  A workgroup of
// 4 waves (2 x 2) computes a BM x BN output tile; each wave a (BM/2) x (BN/2)
// block of 32 x 32 MFMA tiles.  Both operands sit in LDS as [x][BK] rows of
// the contraction index (128 B per row, 16-byte chunks XOR-swizzled by the
// row so that the 32 rows one MFMA operand read touches spread over all
// banks).  Operands whose contraction index is contiguous in memory (lhs
// rows; a transposed rhs) are copied as 16-byte chunks; operands whose
// contraction index is the row (a plain [K, N] rhs; both tgmm operands) are
// loaded as 4 rows x 8 columns per thread and transposed in registers into
// 8-byte LDS writes.  Global loads for step k+1 are issued before the MFMAs
// of step k (two LDS buffers, one barrier per step).
//
// Tile schedule: the per-group row counts stay on the device.  Each
// persistent workgroup scans group_sizes once into LDS (prefix of rows and of
// tiles), then walks the linear tile index; tiles of one group and one
// column block are consecutive, and consecutive tile indices are given to
// workgroups on the same XCD (workgroup b runs on XCD b % 8) so that they
// share operand blocks in that XCD's L2.  Empty groups own no gmm tiles;
// padded rows of a group's last row tile are masked.
#include <type_traits>

#include "common.h"

namespace moe {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;      // contraction elements per step

__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }
constexpr int NT = 256;     // threads per workgroup
constexpr int kMaxG = 1024;

__device__ __forceinline__ int lds_off(int x, int c) {
  return x * (BK * 2) + ((c ^ (x & 7) ^ ((x >> 3) & 7)) << 4);
}

// Element (x, k) at src[x * ld + k]: contraction contiguous.
template <int X>
struct RowK {
  static constexpr int N = X * (BK / 8) / NT;
  uint4 r[N];
  __device__ __forceinline__ void load(const bf16_t* src, int64_t ld, int xv, int kv) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * NT, x = q >> 3, c = q & 7;
      if (x < xv && c * 8 < kv) r[i] = *reinterpret_cast<const uint4*>(src + x * ld + c * 8);
      else r[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * NT, x = q >> 3, c = q & 7;
      *reinterpret_cast<uint4*>(lds + lds_off(x, c)) = r[i];
    }
  }
};

// Element (x, k) at src[k * ld + x]: contraction is the row index.
template <int X>
struct ColK {
  static constexpr int XQ = X / 8;
  static constexpr int N = (BK / 4) * XQ / NT;
  uint4 r[N][4];
  __device__ __forceinline__ void load(const bf16_t* src, int64_t ld, int xv, int kv) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = threadIdx.x + i * NT, xq = u % XQ, kq = u / XQ;
#pragma unroll
      for (int kr = 0; kr < 4; ++kr) {
        const int k = 4 * kq + kr;
        if (k < kv && xq * 8 < xv)
          r[i][kr] = *reinterpret_cast<const uint4*>(src + k * ld + xq * 8);
        else
          r[i][kr] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = threadIdx.x + i * NT, xq = u % XQ, kq = u / XQ;
      const uint32_t a[4] = {r[i][0].x, r[i][0].y, r[i][0].z, r[i][0].w};
      const uint32_t b[4] = {r[i][1].x, r[i][1].y, r[i][1].z, r[i][1].w};
      const uint32_t c[4] = {r[i][2].x, r[i][2].y, r[i][2].z, r[i][2].w};
      const uint32_t d[4] = {r[i][3].x, r[i][3].y, r[i][3].z, r[i][3].w};
#pragma unroll
      for (int xi = 0; xi < 8; ++xi) {
        const int dw = xi >> 1;
        uint32_t lo, hi;
        if (xi & 1) {
          lo = (a[dw] >> 16) | (b[dw] & 0xFFFF0000u);
          hi = (c[dw] >> 16) | (d[dw] & 0xFFFF0000u);
        } else {
          lo = (a[dw] & 0xFFFFu) | (b[dw] << 16);
          hi = (c[dw] & 0xFFFFu) | (d[dw] << 16);
        }
        const int x = xq * 8 + xi;
        *reinterpret_cast<uint2*>(lds + lds_off(x, kq >> 1) + ((kq & 1) << 3)) = make_uint2(lo, hi);
      }
    }
  }
};

template <int BM, int BN>
struct Mfma {
  static constexpr int FM = BM / 64, FN = BN / 64;  // 32x32 tiles per wave
  f32x16 acc[FM][FN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }
  __device__ __forceinline__ void step(const char* As, const char* Bs) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int xa = (w >> 1) * (BM / 2) + (lane & 31);
    const int xb = (w & 1) * (BN / 2) + (lane & 31);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = 2 * s + (lane >> 5);
      bf16x8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(xa + 32 * i, c));
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(xb + 32 * j, c));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // Visit every accumulator element with its (row, col) inside the tile.
  template <typename F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r0 = (w >> 1) * (BM / 2) + 4 * (lane >> 5);
    const int c0 = (w & 1) * (BN / 2) + (lane & 31);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          f(r0 + 32 * i + 8 * (r >> 2) + (r & 3), c0 + 32 * j, acc[i][j][r]);
  }
};

// Wave 0 scans the group sizes: row_base[g] (rows clipped to max_rows) and,
// if tile_base != nullptr, tile_base[g] = tiles of groups < g, where a group
// of n rows owns ceil(n / BM) * ntn tiles.
__device__ void scan_groups(const int32_t* __restrict__ gsz, int G, int64_t max_rows, int BMv,
                            int ntn, int* row_base, int* tile_base, int32_t* err) {
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
    int t = tile_base ? ((neff + BMv - 1) / BMv) * ntn : 0;
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

// Linear tile index of a persistent workgroup's it-th tile: the grid's
// workgroups on XCD x (b % 8 == x) take a contiguous run of indices.
__device__ __forceinline__ int64_t xcd_tile(int it) {
  const int b = blockIdx.x, g = gridDim.x;
  return static_cast<int64_t>(it) * g + (b & 7) * (g >> 3) + (b >> 3);
}

template <typename TO>
__device__ __forceinline__ void store_out(TO* p, float v, int accumulate) {
  if (accumulate) v += Elem<TO>::load(p);
  Elem<TO>::store(p, v);
}

// Zero rows [r0, r1) of out (row stride ld, N columns), grid-strided.
template <typename TO>
__device__ void zero_rows(TO* out, int64_t ld, int64_t N, int64_t r0, int64_t r1) {
  for (int64_t r = r0 + blockIdx.x; r < r1; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < N; c += NT) out[r * ld + c] = TO(0);
}

template <int BM, int BN, bool TRANS, typename TO>
__global__ __launch_bounds__(NT) void gmm_bf16_kernel(
    const bf16_t* __restrict__ lhs, int64_t ld_lhs, const bf16_t* __restrict__ rhs, int64_t ld_rhs,
    int64_t rhs_gs, const int32_t* __restrict__ gsz, int G, int64_t Kdim, int64_t N,
    TO* __restrict__ out, int64_t M_out, int64_t ld_out, int accumulate, int32_t* err) {
  __shared__ __attribute__((aligned(16))) char smem[2][(BM + BN) * BK * 2];
  __shared__ int row_base[kMaxG + 1];
  __shared__ int tile_base[kMaxG + 1];
  const int ntn = static_cast<int>((N + BN - 1) / BN);
  scan_groups(gsz, G, M_out, BM, ntn, row_base, tile_base, blockIdx.x == 0 ? err : nullptr);
  __syncthreads();
  const int total = tile_base[G];
  const int nk = static_cast<int>((Kdim + BK - 1) / BK);

  RowK<BM> la;
  typename std::conditional<TRANS, RowK<BN>, ColK<BN>>::type lb;
  Mfma<BM, BN> mm;

  for (int it = 0;; ++it) {
    const int64_t tile = xcd_tile(it);
    if (tile >= total) break;
    int lo = 0, hi = G - 1;  // largest g with tile_base[g] <= tile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int rows_g = row_base[g + 1] - row_base[g];
    const int mtiles = (rows_g + BM - 1) / BM;
    const int local = static_cast<int>(tile - tile_base[g]);
    const int nt = local / mtiles, mt = local % mtiles;
    const int64_t row0 = row_base[g] + static_cast<int64_t>(mt) * BM;
    const int rv = min(BM, rows_g - mt * BM);
    const int64_t col0 = static_cast<int64_t>(nt) * BN;
    const int cv = static_cast<int>(lmin(BN, N - col0));

    const bf16_t* a_src = lhs + row0 * ld_lhs;
    const bf16_t* b_src = TRANS ? rhs + g * rhs_gs + col0 * ld_rhs : rhs + g * rhs_gs + col0;
    auto load_step = [&](int kt) {
      const int64_t k0 = static_cast<int64_t>(kt) * BK;
      const int kv = static_cast<int>(lmin(BK, Kdim - k0));
      la.load(a_src + k0, ld_lhs, rv, kv);
      if (TRANS) lb.load(b_src + k0, ld_rhs, cv, kv);
      else lb.load(b_src + k0 * ld_rhs, ld_rhs, cv, kv);
    };
    mm.zero();
    if (nk > 0) {
      load_step(0);
      la.store(smem[0]);
      lb.store(smem[0] + BM * BK * 2);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_step(kt + 1);
        const char* buf = smem[kt & 1];
        mm.step(buf, buf + BM * BK * 2);
        if (kt + 1 < nk) {
          char* nb = smem[(kt + 1) & 1];
          la.store(nb);
          lb.store(nb + BM * BK * 2);
        }
        __syncthreads();
      }
    }
    TO* o = out + row0 * ld_out + col0;
    mm.for_each([&](int r, int c, float v) {
      if (r < rv && c < cv) store_out(o + static_cast<int64_t>(r) * ld_out + c, v, accumulate);
    });
  }
  if (!accumulate) zero_rows(out, ld_out, N, row_base[G], M_out);
}

template <int BM, int BN, typename TO>
__global__ __launch_bounds__(NT) void tgmm_bf16_kernel(
    const bf16_t* __restrict__ lhs, int64_t ld_lhs, const bf16_t* __restrict__ rhs, int64_t ld_rhs,
    const int32_t* __restrict__ gsz, int G, int64_t M, int64_t Kdim, int64_t N,
    TO* __restrict__ out, int64_t ld_out, int64_t out_gs, int accumulate, int32_t* err) {
  __shared__ __attribute__((aligned(16))) char smem[2][(BM + BN) * BK * 2];
  __shared__ int row_base[kMaxG + 1];
  scan_groups(gsz, G, M, BM, 1, row_base, nullptr, blockIdx.x == 0 ? err : nullptr);
  __syncthreads();
  const int mtn = static_cast<int>((Kdim + BM - 1) / BM);
  const int ntn = static_cast<int>((N + BN - 1) / BN);
  const int64_t per_group = static_cast<int64_t>(mtn) * ntn;
  const int64_t total = per_group * G;

  ColK<BM> la;
  ColK<BN> lb;
  Mfma<BM, BN> mm;

  for (int it = 0;; ++it) {
    const int64_t tile = xcd_tile(it);
    if (tile >= total) break;
    const int g = static_cast<int>(tile / per_group);
    const int local = static_cast<int>(tile - g * per_group);
    const int nt = local / mtn, mt = local % mtn;
    const int64_t r0 = row_base[g];
    const int rows_g = row_base[g + 1] - row_base[g];
    const int64_t m0 = static_cast<int64_t>(mt) * BM;
    const int64_t n0 = static_cast<int64_t>(nt) * BN;
    const int mv = static_cast<int>(lmin(BM, Kdim - m0));
    const int nv = static_cast<int>(lmin(BN, N - n0));
    TO* o = out + g * out_gs + m0 * ld_out + n0;
    if (rows_g == 0 && accumulate) continue;   // partial sum unchanged
    const int nk = (rows_g + BK - 1) / BK;
    const bf16_t* a_src = lhs + r0 * ld_lhs + m0;
    const bf16_t* b_src = rhs + r0 * ld_rhs + n0;
    auto load_step = [&](int kt) {
      const int k0 = kt * BK;
      const int kv = min(BK, rows_g - k0);
      la.load(a_src + static_cast<int64_t>(k0) * ld_lhs, ld_lhs, mv, kv);
      lb.load(b_src + static_cast<int64_t>(k0) * ld_rhs, ld_rhs, nv, kv);
    };
    mm.zero();
    if (nk > 0) {
      load_step(0);
      la.store(smem[0]);
      lb.store(smem[0] + BM * BK * 2);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_step(kt + 1);
        const char* buf = smem[kt & 1];
        mm.step(buf, buf + BM * BK * 2);
        if (kt + 1 < nk) {
          char* nb = smem[(kt + 1) & 1];
          la.store(nb);
          lb.store(nb + BM * BK * 2);
        }
        __syncthreads();
      }
    }
    mm.for_each([&](int r, int c, float v) {
      if (r < mv && c < nv) store_out(o + static_cast<int64_t>(r) * ld_out + c, v, accumulate);
    });
  }
}

// ---------------------------------------------------------------- float32
// Plain float32 FMA kernels (64 x 64 tiles, 4 x 4 outputs per thread) for
// float32 workloads; same schedule and semantics as the bf16 kernels.
constexpr int FB = 64, FK = 16;

template <bool TRANS>
__global__ __launch_bounds__(NT) void gmm_f32_kernel(
    const float* __restrict__ lhs, int64_t ld_lhs, const float* __restrict__ rhs, int64_t ld_rhs,
    int64_t rhs_gs, const int32_t* __restrict__ gsz, int G, int64_t Kdim, int64_t N,
    float* __restrict__ out_f, bf16_t* __restrict__ out_h, int64_t M_out, int64_t ld_out,
    int accumulate, int32_t* err) {
  __shared__ float As[FK][FB + 4];
  __shared__ float Bs[FK][FB + 4];
  __shared__ int row_base[kMaxG + 1];
  __shared__ int tile_base[kMaxG + 1];
  const int ntn = static_cast<int>((N + FB - 1) / FB);
  scan_groups(gsz, G, M_out, FB, ntn, row_base, tile_base, blockIdx.x == 0 ? err : nullptr);
  __syncthreads();
  const int total = tile_base[G];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int rows_g = row_base[g + 1] - row_base[g];
    const int mtiles = (rows_g + FB - 1) / FB;
    const int local = static_cast<int>(tile - tile_base[g]);
    const int nt = local / mtiles, mt = local % mtiles;
    const int64_t row0 = row_base[g] + static_cast<int64_t>(mt) * FB;
    const int rv = min(FB, rows_g - mt * FB);
    const int64_t col0 = static_cast<int64_t>(nt) * FB;
    const float* B = rhs + g * rhs_gs;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < Kdim; k0 += FK) {
      for (int i = threadIdx.x; i < FK * FB; i += NT) {
        const int m = i / FK, k = i % FK;   // A: k fastest (contiguous in lhs rows)
        As[k][m] = (m < rv && k0 + k < Kdim) ? lhs[(row0 + m) * ld_lhs + k0 + k] : 0.f;
        int n, kk;
        if (TRANS) { n = i / FK; kk = i % FK; } else { kk = i / FB; n = i % FB; }
        const bool ok = col0 + n < N && k0 + kk < Kdim;
        Bs[kk][n] = ok ? (TRANS ? B[(col0 + n) * ld_rhs + k0 + kk] : B[(k0 + kk) * ld_rhs + col0 + n]) : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < FK; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = As[k][ty * 4 + i]; b[i] = Bs[k][tx * 4 + i]; }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = ty * 4 + i;
        const int64_t c = col0 + tx * 4 + j;
        if (r < rv && c < N) {
          const int64_t off = (row0 + r) * ld_out + c;
          if (out_f) store_out(out_f + off, acc[i][j], accumulate);
          else store_out(out_h + off, acc[i][j], accumulate);
        }
      }
  }
  if (!accumulate) {
    if (out_f) zero_rows(out_f, ld_out, N, row_base[G], M_out);
    else zero_rows(out_h, ld_out, N, row_base[G], M_out);
  }
}

__global__ __launch_bounds__(NT) void tgmm_f32_kernel(
    const float* __restrict__ lhs, int64_t ld_lhs, const float* __restrict__ rhs, int64_t ld_rhs,
    const int32_t* __restrict__ gsz, int G, int64_t M, int64_t Kdim, int64_t N,
    float* __restrict__ out_f, bf16_t* __restrict__ out_h, int64_t ld_out, int64_t out_gs,
    int accumulate, int32_t* err) {
  __shared__ float As[FK][FB + 4];
  __shared__ float Bs[FK][FB + 4];
  __shared__ int row_base[kMaxG + 1];
  scan_groups(gsz, G, M, FB, 1, row_base, nullptr, blockIdx.x == 0 ? err : nullptr);
  __syncthreads();
  const int mtn = static_cast<int>((Kdim + FB - 1) / FB);
  const int ntn = static_cast<int>((N + FB - 1) / FB);
  const int64_t per_group = static_cast<int64_t>(mtn) * ntn;
  const int64_t total = per_group * G;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int g = static_cast<int>(tile / per_group);
    const int local = static_cast<int>(tile - g * per_group);
    const int nt = local / mtn, mt = local % mtn;
    const int64_t r0 = row_base[g];
    const int rows_g = row_base[g + 1] - row_base[g];
    if (rows_g == 0 && accumulate) continue;
    const int64_t m0 = static_cast<int64_t>(mt) * FB, n0 = static_cast<int64_t>(nt) * FB;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < rows_g; k0 += FK) {
      for (int i = threadIdx.x; i < FK * FB; i += NT) {
        const int k = i / FB, x = i % FB;
        const bool kin = k0 + k < rows_g;
        As[k][x] = (kin && m0 + x < Kdim) ? lhs[(r0 + k0 + k) * ld_lhs + m0 + x] : 0.f;
        Bs[k][x] = (kin && n0 + x < N) ? rhs[(r0 + k0 + k) * ld_rhs + n0 + x] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < FK; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = As[k][ty * 4 + i]; b[i] = Bs[k][tx * 4 + i]; }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t r = m0 + ty * 4 + i, c = n0 + tx * 4 + j;
        if (r < Kdim && c < N) {
          const int64_t off = g * out_gs + r * ld_out + c;
          if (out_f) store_out(out_f + off, acc[i][j], accumulate);
          else store_out(out_h + off, acc[i][j], accumulate);
        }
      }
  }
}

constexpr int kBM = 128, kBN = 128;

unsigned persistent_grid(int64_t upper_tiles, int per_cu) {
  int64_t g = static_cast<int64_t>(device_cu_count()) * per_cu;
  if (upper_tiles < g) g = upper_tiles;
  g = ((g + 7) / 8) * 8;
  return static_cast<unsigned>(g < 8 ? 8 : g);
}

bool mult8(int64_t v) { return v >= 0 && (v & 7) == 0; }

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API int moe_gmm(const void* lhs, int64_t M_lhs, int64_t ld_lhs, const void* rhs,
                    int64_t ld_rhs, int64_t rhs_group_stride, int trans_rhs,
                    const int32_t* group_sizes, int G, int64_t Kdim, int64_t N, int in_dtype,
                    void* out, int64_t M_out, int64_t ld_out, int out_dtype, int accumulate,
                    int32_t* err, void* stream) {
  if (G < 1 || G > kMaxG || M_lhs < 0 || M_out < 0 || M_out > M_lhs || Kdim < 0 || N < 0)
    return MOE_ERR_ARG;
  if (M_out > INT32_MAX) return MOE_ERR_ARG;
  if (in_dtype != MOE_BF16 && in_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (!mult8(Kdim) || !mult8(N) || !mult8(ld_lhs) || !mult8(ld_rhs) || !mult8(ld_out) ||
      !mult8(rhs_group_stride))
    return MOE_ERR_ARG;
  if (ld_lhs < Kdim || ld_out < N || ld_rhs < (trans_rhs ? Kdim : N)) return MOE_ERR_ARG;
  if (M_out == 0 || N == 0) return MOE_OK;
  if (!lhs || !rhs || !group_sizes || !out || !aligned16(lhs) || !aligned16(rhs) || !aligned16(out))
    return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == MOE_BF16) {
    const bf16_t* A = static_cast<const bf16_t*>(lhs);
    const bf16_t* B = static_cast<const bf16_t*>(rhs);
#define GMM(BMV, TR, TO)                                                                        \
  hipLaunchKernelGGL((gmm_bf16_kernel<BMV, kBN, TR, TO>), dim3(grid), dim3(NT), 0, st, A, ld_lhs, \
                     B, ld_rhs, rhs_group_stride, group_sizes, G, Kdim, N, static_cast<TO*>(out), \
                     M_out, ld_out, accumulate, err)
    if (Kdim <= BK) {
      // one contraction step: a taller row tile amortises the rhs tile
      constexpr int kTall = 256;
      const int64_t upper = ((M_out + kTall - 1) / kTall + G) * ((N + kBN - 1) / kBN);
      const unsigned grid = persistent_grid(upper, 1);
      if (trans_rhs) {
        if (out_dtype == MOE_BF16) GMM(kTall, true, bf16_t); else GMM(kTall, true, float);
      } else {
        if (out_dtype == MOE_BF16) GMM(kTall, false, bf16_t); else GMM(kTall, false, float);
      }
    } else {
      const int64_t upper = ((M_out + kBM - 1) / kBM + G) * ((N + kBN - 1) / kBN);
      const unsigned grid = persistent_grid(upper, 2);
      if (trans_rhs) {
        if (out_dtype == MOE_BF16) GMM(kBM, true, bf16_t); else GMM(kBM, true, float);
      } else {
        if (out_dtype == MOE_BF16) GMM(kBM, false, bf16_t); else GMM(kBM, false, float);
      }
    }
#undef GMM
  } else {
    const int64_t upper = ((M_out + FB - 1) / FB + G) * ((N + FB - 1) / FB);
    const unsigned grid = persistent_grid(upper, 4);
    float* of = out_dtype == MOE_F32 ? static_cast<float*>(out) : nullptr;
    bf16_t* oh = out_dtype == MOE_BF16 ? static_cast<bf16_t*>(out) : nullptr;
    if (trans_rhs)
      hipLaunchKernelGGL(gmm_f32_kernel<true>, dim3(grid), dim3(NT), 0, st,
                         static_cast<const float*>(lhs), ld_lhs, static_cast<const float*>(rhs),
                         ld_rhs, rhs_group_stride, group_sizes, G, Kdim, N, of, oh, M_out, ld_out,
                         accumulate, err);
    else
      hipLaunchKernelGGL(gmm_f32_kernel<false>, dim3(grid), dim3(NT), 0, st,
                         static_cast<const float*>(lhs), ld_lhs, static_cast<const float*>(rhs),
                         ld_rhs, rhs_group_stride, group_sizes, G, Kdim, N, of, oh, M_out, ld_out,
                         accumulate, err);
  }
  return launch_status();
}

MOE_API int moe_tgmm(const void* lhs, int64_t ld_lhs, const void* rhs, int64_t ld_rhs,
                     const int32_t* group_sizes, int G, int64_t M, int64_t Kdim, int64_t N,
                     int in_dtype, void* out, int64_t ld_out, int64_t out_group_stride,
                     int out_dtype, int accumulate, int32_t* err, void* stream) {
  if (G < 1 || G > kMaxG || M < 0 || Kdim < 0 || N < 0) return MOE_ERR_ARG;
  if (M > INT32_MAX) return MOE_ERR_ARG;
  if (in_dtype != MOE_BF16 && in_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (!mult8(Kdim) || !mult8(N) || !mult8(ld_lhs) || !mult8(ld_rhs) || !mult8(ld_out) ||
      !mult8(out_group_stride))
    return MOE_ERR_ARG;
  if (ld_lhs < Kdim || ld_rhs < N || ld_out < N || out_group_stride < Kdim * ld_out)
    return MOE_ERR_ARG;
  if (Kdim == 0 || N == 0) return MOE_OK;
  if (!lhs || !rhs || !group_sizes || !out || !aligned16(lhs) || !aligned16(rhs) || !aligned16(out))
    return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == MOE_BF16) {
    const int64_t upper = static_cast<int64_t>(G) * ((Kdim + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const unsigned grid = persistent_grid(upper, 2);
    const bf16_t* A = static_cast<const bf16_t*>(lhs);
    const bf16_t* B = static_cast<const bf16_t*>(rhs);
    if (out_dtype == MOE_BF16)
      hipLaunchKernelGGL((tgmm_bf16_kernel<kBM, kBN, bf16_t>), dim3(grid), dim3(NT), 0, st, A,
                         ld_lhs, B, ld_rhs, group_sizes, G, M, Kdim, N, static_cast<bf16_t*>(out),
                         ld_out, out_group_stride, accumulate, err);
    else
      hipLaunchKernelGGL((tgmm_bf16_kernel<kBM, kBN, float>), dim3(grid), dim3(NT), 0, st, A,
                         ld_lhs, B, ld_rhs, group_sizes, G, M, Kdim, N, static_cast<float*>(out),
                         ld_out, out_group_stride, accumulate, err);
  } else {
    const int64_t upper = static_cast<int64_t>(G) * ((Kdim + FB - 1) / FB) * ((N + FB - 1) / FB);
    const unsigned grid = persistent_grid(upper, 4);
    float* of = out_dtype == MOE_F32 ? static_cast<float*>(out) : nullptr;
    bf16_t* oh = out_dtype == MOE_BF16 ? static_cast<bf16_t*>(out) : nullptr;
    hipLaunchKernelGGL(tgmm_f32_kernel, dim3(grid), dim3(NT), 0, st, static_cast<const float*>(lhs),
                       ld_lhs, static_cast<const float*>(rhs), ld_rhs, group_sizes, G, M, Kdim, N,
                       of, oh, ld_out, out_group_stride, accumulate, err);
  }
  return launch_status();
}
