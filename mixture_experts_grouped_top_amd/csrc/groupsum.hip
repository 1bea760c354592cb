// Per-group column sums: out[g, :] = sum of the rows of group g of a
// [M, N] matrix whose rows are grouped as by the grouped GEMM (group g owns
// the rows following the groups before it).  This is the gradient of a
// per-expert bias added to every row of its group: the MLP biases of the
// chunked expert layer in the MaxText pull request "Overlap moe comms with
// collective matmul" (Testing: MLP bias with the chunked layer; the chunked
// layer's w0/w1/wo bias arguments).
//
// HBM-bound (reads M x N once).  Deterministic, no float atomics: pass 1
// gives every 256-row tile of every group and every 512-column strip to one
// workgroup, which sums the tile's rows into a float32 partial row; pass 2
// adds a group's partial rows in tile order.  Tiles never straddle groups,
// so a large group spreads over many workgroups and a small one costs one.
#include "common.h"

namespace moe {
namespace {

constexpr int kRowsPerTile = 256;
constexpr int kStripCols = 512;   // 64 lanes x 8 columns
constexpr int kMaxGroups = 1024;
constexpr int kLoadsInFlight = 4;

int64_t tiles_bound(int64_t M, int G) { return (M + kRowsPerTile - 1) / kRowsPerTile + G; }

__device__ __forceinline__ int group_of_tile(const int* tile_base, int G, int tile) {
  int lo = 0, hi = G - 1;   // largest g with tile_base[g] <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_base[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// grid (tiles bound, strips), 256 threads.  Wave w sums rows w, w + 4, ...
// of the tile (kLoadsInFlight rows loaded before they are added), then the
// four waves' sums are added in wave order through LDS.
template <typename TI>
__global__ __launch_bounds__(256) void group_sum_partial_kernel(
    const TI* __restrict__ in, int64_t ld, const int32_t* __restrict__ gsz,
    const int32_t* __restrict__ valid, int G, int64_t M, int64_t N, float* __restrict__ part,
    int32_t* err) {
  __shared__ int row_base[kMaxGroups + 1];
  __shared__ int tile_base[kMaxGroups + 1];
  __shared__ float red[4][kStripCols];
  scan_groups(gsz, G, M, kRowsPerTile, 1, row_base, tile_base,
              blockIdx.x == 0 && blockIdx.y == 0 ? err : nullptr);
  __syncthreads();
  const int tile = static_cast<int>(blockIdx.x);
  if (tile >= tile_base[G]) return;   // uniform over the workgroup
  const int g = group_of_tile(tile_base, G, tile);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = (tile - tile_base[g]) * kRowsPerTile;
  int rows_g = row_base[g + 1] - row_base[g];
  if (valid) rows_g = min(rows_g, max(valid[g], 0));   // the rest is zero
  const int nr = max(0, min(kRowsPerTile, rows_g - t0));
  const int64_t col = static_cast<int64_t>(blockIdx.y) * kStripCols + lane * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col < N) {
    const TI* base = in + (static_cast<int64_t>(row_base[g]) + t0) * ld + col;
    for (int r0 = w; r0 < nr; r0 += 4 * kLoadsInFlight) {
      Raw8<TI> raw[kLoadsInFlight];
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u) {
        const int r = r0 + 4 * u;
        if (r < nr) raw[u].load(base + static_cast<int64_t>(r) * ld);
      }
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u) {
        if (r0 + 4 * u >= nr) break;
        float v[8];
        raw[u].get(v);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += v[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[w][lane * 8 + e] = s[e];
  __syncthreads();
  // 256 threads x 2 columns: the strip's 512 sums, waves added in order
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x + 256 * h;
    const int64_t gc = static_cast<int64_t>(blockIdx.y) * kStripCols + c;
    if (gc < N)
      part[static_cast<int64_t>(tile) * N + gc] =
          ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
  }
}

// grid (G, ceil(N / 2048)), 256 threads of 8 columns: group g's partial rows
// added in tile order; an empty group gives zero (or leaves out unchanged
// when accumulating).
template <typename TO>
__global__ __launch_bounds__(256) void group_sum_final_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ gsz, int G, int64_t M, int64_t N,
    TO* __restrict__ out, int accumulate) {
  __shared__ int row_base[kMaxGroups + 1];
  __shared__ int tile_base[kMaxGroups + 1];
  scan_groups(gsz, G, M, kRowsPerTile, 1, row_base, tile_base, nullptr);
  __syncthreads();
  const int g = static_cast<int>(blockIdx.x);
  const int64_t col = (static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x) * 8;
  if (col >= N) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int t = tile_base[g]; t < tile_base[g + 1]; ++t) {
    float v[8];
    load8(part + static_cast<int64_t>(t) * N + col, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += v[e];
  }
  TO* o = out + static_cast<int64_t>(g) * N + col;
  if (accumulate) {
    float old[8];
    load8(o, old);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += old[e];
  }
  store8(o, s);
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API size_t moe_group_sum_workspace(int64_t M, int G, int64_t N) {
  if (M < 0 || G < 1 || N < 0) return 0;
  return static_cast<size_t>(tiles_bound(M, G) * N) * sizeof(float);
}

MOE_API int moe_group_sum(const void* in, int64_t ld_in, int in_dtype, const int32_t* group_sizes,
                          const int32_t* valid_rows, int G, int64_t M, int64_t N, void* out,
                          int out_dtype, int accumulate, void* workspace, size_t ws_bytes,
                          int32_t* err, void* stream) {
  if (G < 1 || G > kMaxGroups || M < 0 || N < 0 || ld_in < N) return MOE_ERR_ARG;
  if (M > INT32_MAX) return MOE_ERR_ARG;
  if (!elem_bytes(in_dtype) || !elem_bytes(out_dtype)) return MOE_ERR_DTYPE;
  if (N % 8 || ld_in % 8) return MOE_ERR_ARG;
  if (N == 0) return MOE_OK;
  if (!group_sizes || !out || !aligned16(out) || (M > 0 && (!in || !aligned16(in))))
    return MOE_ERR_ARG;
  const int64_t tiles = tiles_bound(M, G);
  if (tiles > INT32_MAX) return MOE_ERR_ARG;
  if (!workspace || ws_bytes < moe_group_sum_workspace(M, G, N) ||
      (reinterpret_cast<uintptr_t>(workspace) & 15))
    return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  const dim3 g1(static_cast<unsigned>(tiles), static_cast<unsigned>((N + kStripCols - 1) / kStripCols));
  if (in_dtype == MOE_BF16)
    hipLaunchKernelGGL(group_sum_partial_kernel<bf16_t>, g1, dim3(256), 0, st,
                       static_cast<const bf16_t*>(in), ld_in, group_sizes, valid_rows, G, M, N,
                       part, err);
  else
    hipLaunchKernelGGL(group_sum_partial_kernel<float>, g1, dim3(256), 0, st,
                       static_cast<const float*>(in), ld_in, group_sizes, valid_rows, G, M, N,
                       part, err);
  const dim3 g2(static_cast<unsigned>(G), static_cast<unsigned>((N + 2047) / 2048));
  if (out_dtype == MOE_BF16)
    hipLaunchKernelGGL(group_sum_final_kernel<bf16_t>, g2, dim3(256), 0, st, part, group_sizes, G,
                       M, N, static_cast<bf16_t*>(out), accumulate);
  else
    hipLaunchKernelGGL(group_sum_final_kernel<float>, g2, dim3(256), 0, st, part, group_sizes, G,
                       M, N, static_cast<float*>(out), accumulate);
  return launch_status();
}
