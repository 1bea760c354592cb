// Dispatch (permute) and combine (unpermute) with their backward passes.
//
// Permute is a two-level, deterministic counting sort of the routed slots by
// expert (the "global permute" of the TransformerEngine MoE block with
// group_sizes and align_size padding; token dropping in router order from the
// MaxText grouped-GEMM pull request's Tests):
//   1. hist    per block of kSlots slots: per-expert counts (LDS atomics on
//              integers, so order-free and exact); also marks every row of
//              slot_of_row as padding (-1).
//   2. scan    one workgroup: per expert, exclusive scan of the block counts
//              over blocks (each block's base rank), capacity clip, align,
//              exclusive scan over experts -> group offsets.
//   3. rank    per block: stable rank of each slot among same-expert slots,
//              from wave ballots over the bits of the expert id (peer mask,
//              popcount below the lane) plus per-wave counts in LDS; writes
//              row_of_slot and slot_of_row.
//   4. scatter one wave per token: read x[token] once, write it to the row
//              of each kept slot; padding rows are zeroed.
#include <mutex>

#include "common.h"

// Scratch of moe_permute_noalloc: the per-block expert counts (int32) that
// moe_permute keeps in its caller's workspace.  One copy per GPU, held until
// the process ends.  Host code never passes this name to a kernel: it is a
// host-side stand-in, and the device address comes from hipGetSymbolAddress
// (scratch_address below).
static __device__ __align__(256) int32_t scratch[MOE_PERMUTE_NOALLOC_SCRATCH_WORDS];

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kSlots = 1024;          // slots per block in hist/rank
constexpr int kMaxE = 1024;

__device__ __forceinline__ void flag_error(int32_t* err, int bit) {
  if (err) atomicOr(err, bit);
}

__global__ __launch_bounds__(kThreads) void permute_hist_kernel(
    const int32_t* __restrict__ ids, int64_t TK, int E, int32_t* __restrict__ blockcounts,
    int32_t* __restrict__ slot_of_row, int64_t rows, int32_t* err) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kSlots;
  for (int i = threadIdx.x; i < kSlots; i += kThreads) {
    const int64_t s = s0 + i;
    if (s < TK) {
      const int e = ids[s];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
      else flag_error(err, MOE_DERR_EXPERT_ID);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads)
    blockcounts[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
  // every row starts as padding; the rank pass overwrites the real ones
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; r < rows;
       r += static_cast<int64_t>(gridDim.x) * kThreads)
    slot_of_row[r] = -1;
}

// Inclusive scan over the 1024 threads of a block.
__device__ int block_scan_incl(int v, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = (lane < 16) ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_up(t, o, 64);
      if (lane >= o) t += u;
    }
    if (lane < 16) wsum[lane] = t;
  }
  __syncthreads();
  if (w > 0) v += wsum[w - 1];
  return v;
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(
    int32_t* __restrict__ blockcounts, int nblocks, int E, int align, int capacity,
    int capacity_layout, int64_t rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ group_sizes, int32_t* __restrict__ group_offsets, int32_t* err) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  int kept = 0, gs = 0;
  if (e < E) {
    int run = 0;
    for (int b = 0; b < nblocks; ++b) {
      int32_t* p = blockcounts + static_cast<int64_t>(b) * E + e;
      const int c = *p;
      *p = run;  // becomes this block's base rank for expert e
      run += c;
    }
    kept = (capacity > 0 && run > capacity) ? capacity : run;
    if (capacity_layout) gs = capacity;
    else if (align > 0) gs = ((kept + align - 1) / align) * align;
    else gs = kept;
  }
  const int incl = block_scan_incl(gs, wsum);
  if (e < E) {
    counts[e] = kept;
    group_sizes[e] = gs;
    group_offsets[e] = incl - gs;
    if (e == E - 1) {
      group_offsets[E] = incl;
      if (incl > rows) flag_error(err, MOE_DERR_ROWS);
    }
  }
}

__global__ __launch_bounds__(kThreads) void permute_rank_kernel(
    const int32_t* __restrict__ ids, int64_t TK, int E, int nbits, int capacity,
    const int32_t* __restrict__ blockbase, const int32_t* __restrict__ group_offsets,
    int64_t rows, int32_t* __restrict__ row_of_slot, int32_t* __restrict__ slot_of_row) {
  __shared__ int base[kMaxE];                     // running rank per expert
  __shared__ int wcnt[kThreads / 64][kMaxE];      // this chunk's per-wave counts
  __shared__ int goff[kMaxE];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    base[e] = blockbase[static_cast<int64_t>(blockIdx.x) * E + e];
    goff[e] = group_offsets[e];
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kSlots;
  for (int c0 = 0; c0 < kSlots; c0 += kThreads) {
    for (int i = threadIdx.x; i < (kThreads / 64) * E; i += kThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int64_t s = s0 + c0 + threadIdx.x;
    int e = (s < TK) ? ids[s] : -1;
    const bool valid = e >= 0 && e < E;
    if (!valid) e = 0;
    // lanes holding the same expert id: AND of per-bit ballots
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const int below = __popcll(peers & lt_mask);
    const int cnt = __popcll(peers);
    if (valid && below == cnt - 1) wcnt[w][e] = cnt;   // highest lane of each peer set
    __syncthreads();
    if (valid) {
      int rank = base[e] + below;
      for (int v = 0; v < w; ++v) rank += wcnt[v][e];
      int64_t row = -1;
      if (capacity == 0 || rank < capacity) {
        row = static_cast<int64_t>(goff[e]) + rank;
        if (row >= rows) row = -1;
      }
      row_of_slot[s] = static_cast<int32_t>(row);
      if (row >= 0) slot_of_row[row] = static_cast<int32_t>(s);
    } else if (s < TK) {
      row_of_slot[s] = -1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += kThreads) {
      int add = 0;
#pragma unroll
      for (int v = 0; v < kThreads / 64; ++v) add += wcnt[v][i];
      base[i] += add;
    }
    __syncthreads();
  }
}

// Rows r of a row-major matrix (nvec 16-byte chunks per row) whose
// slot_of_row is negative are padding: zero them, one wave per row.
__device__ __forceinline__ void zero_padding_row(const int32_t* __restrict__ sor, int64_t r,
                                                 int64_t rows, int64_t nvec, uint4* __restrict__ m) {
  if (r >= rows || sor[r] >= 0) return;
  uint4* d = m + r * nvec;
  for (int64_t i = threadIdx.x & 63; i < nvec; i += 64) st_nt(d + i, make_uint4(0, 0, 0, 0));
}

// A token's K (<= 64) slot rows, one per lane (lane j holds row_of_slot of
// slot j, -1 past K); readlane(v, j) then yields slot j's row as a
// wave-uniform value.
__device__ __forceinline__ int slot_rows(const int32_t* __restrict__ rt, int K) {
  const int lane = threadIdx.x & 63;
  return lane < K ? rt[lane] : -1;
}
__device__ __forceinline__ int lane_value(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ __forceinline__ float lane_value(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// x -> x_sorted: one wave per token reads x[t] once (kU chunks of 16 bytes
// per lane at a time) and writes it to the row of each of its kept slots;
// workgroups past the token range zero the padding rows.
constexpr int kU = 4;
__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    const uint4* __restrict__ x, int64_t nvec, int64_t T, int K, const int32_t* __restrict__ ros,
    const int32_t* __restrict__ sor, int64_t rows, uint4* __restrict__ xs, int64_t token_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (static_cast<int64_t>(blockIdx.x) >= token_blocks) {
    zero_padding_row(sor, wid - token_blocks * (kThreads / 64), rows, nvec, xs);
    return;
  }
  const int64_t t = wid;
  if (t >= T) return;
  const uint4* src = x + t * nvec;
  const int rl = slot_rows(ros + t * K, K);
  for (int64_t i0 = lane; i0 < nvec; i0 += 64 * kU) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i0 + 64 * u < nvec) v[u] = ld_nt(src + i0 + 64 * u);
    for (int j = 0; j < K; ++j) {
      const int r = lane_value(rl, j);
      if (r < 0) continue;
      uint4* dst = xs + static_cast<int64_t>(r) * nvec;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (i0 + 64 * u < nvec) st_nt(dst + i0 + 64 * u, v[u]);
    }
  }
}

// y[t] (+)= sum_j wt(t,j) * src[row_of_slot[t*K+j]]: one wave per token,
// 8 elements per lane per chunk, float32 sums in slot order.  Source rows
// are taken in batches of kJB whose loads are all issued before they are
// summed; a dropped slot adds 0 (it loads row 0 when src has rows).
// kJB (1, 2, 4 or 8) is the smallest of these that is >= min(K, 8).
template <typename T, bool WEIGHTED, int kJB>
__global__ __launch_bounds__(kThreads) void gather_sum_kernel(
    const T* __restrict__ src, int64_t rows, int64_t T_, int64_t D, int K,
    const int32_t* __restrict__ ros, const float* __restrict__ wts, T* __restrict__ dst,
    int accumulate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int rl = slot_rows(ros + t * K, K);
  const float wl = WEIGHTED ? (lane < K ? wts[t * K + lane] : 0.f) : 1.f;
  if (K <= kJB && rows > 0 && !accumulate) {
    // One batch holds every slot: software-pipelined over the lane's
    // chunks, the loads of chunk i + 1 are issued before chunk i is summed
    // and stored.  Every issue is unconditional (past the last chunk a lane
    // re-reads the first 16 bytes of row 0, an L2-resident line), so the
    // wait before each sum leaves the next chunk's loads in flight.
    const T* pr[kJB];
    float wv[kJB];
#pragma unroll
    for (int q = 0; q < kJB; ++q) {
      const int r = q < K ? lane_value(rl, q) : -1;
      wv[q] = r < 0 ? 0.f : (WEIGHTED ? lane_value(wl, q) : 1.f);
      pr[q] = src + static_cast<int64_t>(r < 0 ? 0 : r) * D;
    }
    T* out = dst + t * D;
    const int64_t c0 = static_cast<int64_t>(lane) * 8;
    const int nch = c0 < D ? static_cast<int>((D - c0 + 511) / 512) : 0;
    Raw8<T> ra[kJB], rb[kJB];
    auto issue = [&](Raw8<T>(&raw)[kJB], int i) {
      const bool real = i < nch;
      const int64_t c = c0 + 512 * static_cast<int64_t>(i);
#pragma unroll
      for (int q = 0; q < kJB; ++q) raw[q].load(real ? pr[q] + c : src + c0 % 512);
    };
    auto finish = [&](Raw8<T>(&raw)[kJB], int i) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int q = 0; q < kJB; ++q) {
        float v[8];
        raw[q].get(v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wv[q], v[e], acc[e]);
      }
      store8_nt(out + c0 + 512 * static_cast<int64_t>(i), acc);
    };
    if (nch == 0) return;
    issue(ra, 0);
    int i = 0;
    // scheduling barriers keep the issue order (the compiler would
    // otherwise move the next loads behind the sums)
    for (; i + 2 <= nch; i += 2) {
      issue(rb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      finish(ra, i);
      __builtin_amdgcn_sched_barrier(0);
      issue(ra, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      finish(rb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i < nch) finish(ra, i);
    return;
  }
  for (int64_t c = static_cast<int64_t>(lane) * 8; c < D; c += 64 * 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    if (accumulate) load8(dst + t * D + c, acc);
    // with no source rows every slot is dropped and the sum is empty
    for (int j0 = 0; rows > 0 && j0 < K; j0 += kJB) {
      Raw8<T> raw[kJB];
      float wv[kJB];
#pragma unroll
      for (int q = 0; q < kJB; ++q) {
        const int j = j0 + q;
        const int r = j < K ? lane_value(rl, j) : -1;
        wv[q] = r < 0 ? 0.f : (WEIGHTED ? lane_value(wl, j) : 1.f);
        raw[q].load(src + static_cast<int64_t>(r < 0 ? 0 : r) * D + c);
      }
#pragma unroll
      for (int q = 0; q < kJB; ++q) {
        float v[8];
        raw[q].get(v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wv[q], v[e], acc[e]);
      }
    }
    store8_nt(dst + t * D + c, acc);
  }
}

// Combine backward, one wave per token: for each batch of kJB slots, dy[t]
// is read once per chunk, d_y_sorted[row] = w dy[t] is written and
// d_w = <dy[t], y_sorted[row]> accumulated (per lane in chunk order, then
// summed over the wave); dropped slots get d_w = 0 and write nothing
// (their loads read row 0, which exists whenever rows > 0).
// Workgroups past the token range zero the padding rows of d_y_sorted.
template <typename T, int kJB>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ ys, int64_t T_, int64_t D, int K,
    const int32_t* __restrict__ ros, const int32_t* __restrict__ sor, int64_t rows,
    const float* __restrict__ wts, T* __restrict__ d_ys, float* __restrict__ d_w,
    int64_t token_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (static_cast<int64_t>(blockIdx.x) >= token_blocks) {
    zero_padding_row(sor, wid - token_blocks * (kThreads / 64), rows,
                     D * static_cast<int64_t>(sizeof(T)) / 16, reinterpret_cast<uint4*>(d_ys));
    return;
  }
  const int64_t t = wid;
  if (t >= T_) return;
  const int rl = slot_rows(ros + t * K, K);
  const float wl = lane < K ? wts[t * K + lane] : 0.f;
  const T* g = dy + t * D;
  if (K <= kJB && rows > 0) {
    // One batch holds every slot: software-pipelined over the lane's chunks
    // (the loads of chunk i + 1 are in flight while chunk i is scaled,
    // stored and dotted).  Past the lane's last chunk the issues re-read
    // its first chunk (dy row t and row 0 of y_sorted), so every wait
    // leaves the next chunk's loads in flight.
    int r[kJB];
    float wv[kJB], dot[kJB];
    const T* pr[kJB];
#pragma unroll
    for (int q = 0; q < kJB; ++q) {
      r[q] = q < K ? lane_value(rl, q) : -1;
      wv[q] = r[q] >= 0 ? lane_value(wl, q) : 0.f;
      dot[q] = 0.f;
      pr[q] = ys + static_cast<int64_t>(r[q] < 0 ? 0 : r[q]) * D;
    }
    const int64_t c0 = static_cast<int64_t>(lane) * 8;
    const int nch = c0 < D ? static_cast<int>((D - c0 + 511) / 512) : 0;
    Raw8<T> ga, gb, ra[kJB], rb[kJB];
    auto issue = [&](Raw8<T>& gv, Raw8<T>(&raw)[kJB], int i) {
      const int64_t c = i < nch ? c0 + 512 * static_cast<int64_t>(i) : c0;
      gv.load(g + c);
#pragma unroll
      for (int q = 0; q < kJB; ++q) raw[q].load(pr[q] + c);
    };
    auto finish = [&](const Raw8<T>& gv, const Raw8<T>(&raw)[kJB], int i) {
      const int64_t c = c0 + 512 * static_cast<int64_t>(i);
      float a[8];
      gv.get(a);
#pragma unroll
      for (int q = 0; q < kJB; ++q) {
        if (r[q] < 0) continue;
        float b[8], o[8];
        raw[q].get(b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = wv[q] * a[e];
          dot[q] = fmaf(a[e], b[e], dot[q]);
        }
        store8_nt(d_ys + static_cast<int64_t>(r[q]) * D + c, o);
      }
    };
    if (nch > 0) {
      issue(ga, ra, 0);
      int i = 0;
      for (; i + 2 <= nch; i += 2) {
        issue(gb, rb, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        finish(ga, ra, i);
        __builtin_amdgcn_sched_barrier(0);
        issue(ga, ra, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        finish(gb, rb, i + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i < nch) finish(ga, ra, i);
    }
#pragma unroll
    for (int q = 0; q < kJB; ++q) {
      if (q >= K) break;
      const float sdot = wave_sum(dot[q]);
      if (lane == 0) d_w[t * K + q] = r[q] >= 0 ? sdot : 0.f;
    }
    return;
  }
  for (int j0 = 0; j0 < K; j0 += kJB) {
    int r[kJB];
    float wv[kJB], dot[kJB];
#pragma unroll
    for (int q = 0; q < kJB; ++q) {
      const int j = j0 + q;
      r[q] = j < K ? lane_value(rl, j) : -1;
      wv[q] = r[q] >= 0 ? lane_value(wl, j) : 0.f;
      dot[q] = 0.f;
    }
    // with no rows every slot is dropped: only d_w = 0 is written
    for (int64_t c = static_cast<int64_t>(lane) * 8; rows > 0 && c < D; c += 512) {
      float a[8];
      Raw8<T> raw[kJB];
      load8(g + c, a);
#pragma unroll
      for (int q = 0; q < kJB; ++q)
        raw[q].load(ys + static_cast<int64_t>(r[q] < 0 ? 0 : r[q]) * D + c);
#pragma unroll
      for (int q = 0; q < kJB; ++q) {
        if (r[q] < 0) continue;
        float b[8], o[8];
        raw[q].get(b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = wv[q] * a[e];
          dot[q] = fmaf(a[e], b[e], dot[q]);
        }
        store8_nt(d_ys + static_cast<int64_t>(r[q]) * D + c, o);
      }
    }
#pragma unroll
    for (int q = 0; q < kJB; ++q) {
      if (j0 + q >= K) break;
      const float sdot = wave_sum(dot[q]);
      if (lane == 0) d_w[t * K + j0 + q] = r[q] >= 0 ? sdot : 0.f;
    }
  }
}

}  // namespace

static int64_t rows_bound(int64_t T, int K, int E, int align, int capacity, int capacity_layout) {
  if (T < 0 || K < 1 || E < 1 || align < 0 || capacity < 0) return -1;
  if (capacity_layout) return capacity > 0 ? static_cast<int64_t>(E) * capacity : -1;
  return T * K + (align > 0 ? static_cast<int64_t>(E) * (align - 1) : 0);
}

}  // namespace moe

using namespace moe;

MOE_API int64_t moe_rows_bound(int64_t T, int K, int E, int align, int capacity,
                               int capacity_layout) {
  return moe::rows_bound(T, K, E, align, capacity, capacity_layout);
}

MOE_API size_t moe_permute_workspace(int64_t T, int K, int E) {
  if (T < 0 || K < 1 || E < 1) return 0;
  const int64_t nb = (T * K + kSlots - 1) / kSlots;
  const size_t bytes = static_cast<size_t>(nb > 0 ? nb : 1) * E * sizeof(int32_t);
  return (bytes + 255) & ~static_cast<size_t>(255);
}

namespace moe {
namespace {

// Argument checks shared by both permute entry points (the workspace is
// checked by each).
int permute_check(const void* x, int dtype, int64_t T, int64_t D, const int32_t* topk_ids, int K,
                  int E, int align, int capacity, int capacity_layout, const void* x_sorted,
                  int64_t rows, const int32_t* counts, const int32_t* group_sizes,
                  const int32_t* group_offsets, const int32_t* row_of_slot,
                  const int32_t* slot_of_row) {
  if (T < 0 || D < 0 || K < 1 || K > 64 || E < 1 || E > kMaxE || align < 0 || capacity < 0)
    return MOE_ERR_ARG;
  if (capacity_layout && capacity <= 0) return MOE_ERR_ARG;
  const int64_t bound = moe::rows_bound(T, K, E, align, capacity, capacity_layout);
  if (rows < bound) return MOE_ERR_CAPACITY;
  if (!counts || !group_sizes || !group_offsets) return MOE_ERR_ARG;
  if (T * K > 0 && (!topk_ids || !row_of_slot)) return MOE_ERR_ARG;
  if (rows > 0 && !slot_of_row) return MOE_ERR_ARG;
  if (rows > INT32_MAX || T * K > INT32_MAX) return MOE_ERR_ARG;
  const int eb = elem_bytes(dtype);
  if (x_sorted) {
    if (!eb) return MOE_ERR_DTYPE;
    if ((T > 0 && !x) || (D * eb) % 16 || !aligned16(x) || !aligned16(x_sorted))
      return MOE_ERR_ARG;
  }
  return MOE_OK;
}

// The four permute launches; blockcounts holds ceil(T K / kSlots) x E int32
// (every entry is written by the hist pass before it is read).
int permute_launch(const void* x, int dtype, int64_t T, int64_t D, const int32_t* topk_ids, int K,
                   int E, int align, int capacity, int capacity_layout, void* x_sorted,
                   int64_t rows, int32_t* counts, int32_t* group_sizes, int32_t* group_offsets,
                   int32_t* row_of_slot, int32_t* slot_of_row, int32_t* blockcounts,
                   int32_t* err, hipStream_t st) {
  const int eb = elem_bytes(dtype);
  const int64_t TK = T * K;
  const int nb = static_cast<int>((TK + kSlots - 1) / kSlots);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  // at least one block, so that counts are zeroed and padding rows marked
  // even when there are no slots
  const int nbh = nb > 0 ? nb : 1;
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nbh), dim3(kThreads), 0, st, topk_ids, TK, E,
                     blockcounts, slot_of_row, rows, err);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, st, blockcounts, nbh, E, align,
                     capacity, capacity_layout, rows, counts, group_sizes, group_offsets, err);
  if (nb > 0)
    hipLaunchKernelGGL(permute_rank_kernel, dim3(nb), dim3(kThreads), 0, st, topk_ids, TK, E,
                       nbits, capacity, blockcounts, group_offsets, rows, row_of_slot,
                       slot_of_row);
  if (x_sorted && rows > 0 && D > 0) {
    const int64_t nvec = D * eb / 16;
    const int64_t token_blocks = (T + 3) / 4;
    const int64_t blocks = token_blocks + (rows + 3) / 4;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, st, static_cast<const uint4*>(x), nvec, T, K,
                       row_of_slot, slot_of_row, rows, static_cast<uint4*>(x_sorted),
                       token_blocks);
  }
  return launch_status();
}

// Device address of `scratch` on the current device, taken once per device
// (the same array lives at a different address on every GPU).
std::mutex g_scratch_mu;
void* g_scratch_addr[64] = {};

int scratch_address(int32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return MOE_ERR_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_ERR_LAUNCH;
    }
    g_scratch_addr[dev] = p;
  }
  *out = static_cast<int32_t*>(g_scratch_addr[dev]);
  return MOE_OK;
}

}  // namespace
}  // namespace moe

MOE_API int moe_permute(const void* x, int dtype, int64_t T, int64_t D, const int32_t* topk_ids,
                        int K, int E, int align, int capacity, int capacity_layout,
                        void* x_sorted, int64_t rows, int32_t* counts, int32_t* group_sizes,
                        int32_t* group_offsets, int32_t* row_of_slot, int32_t* slot_of_row,
                        void* workspace, size_t ws_bytes, int32_t* err, void* stream) {
  const int rc = permute_check(x, dtype, T, D, topk_ids, K, E, align, capacity, capacity_layout,
                               x_sorted, rows, counts, group_sizes, group_offsets, row_of_slot,
                               slot_of_row);
  if (rc != MOE_OK) return rc;
  if (ws_bytes < moe_permute_workspace(T, K, E) || !workspace ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return MOE_ERR_WORKSPACE;
  return permute_launch(x, dtype, T, D, topk_ids, K, E, align, capacity, capacity_layout,
                        x_sorted, rows, counts, group_sizes, group_offsets, row_of_slot,
                        slot_of_row, static_cast<int32_t*>(workspace), err,
                        static_cast<hipStream_t>(stream));
}

MOE_API int moe_permute_noalloc(const void* x, int dtype, int64_t T, int64_t D,
                                const int32_t* topk_ids, int K, int E, int align, int capacity,
                                int capacity_layout, void* x_sorted, int64_t rows,
                                int32_t* counts, int32_t* group_sizes, int32_t* group_offsets,
                                int32_t* row_of_slot, int32_t* slot_of_row, int32_t* err,
                                void* stream) {
  int rc = permute_check(x, dtype, T, D, topk_ids, K, E, align, capacity, capacity_layout,
                         x_sorted, rows, counts, group_sizes, group_offsets, row_of_slot,
                         slot_of_row);
  if (rc != MOE_OK) return rc;
  if (moe_permute_workspace(T, K, E) > sizeof(int32_t) * MOE_PERMUTE_NOALLOC_SCRATCH_WORDS)
    return MOE_ERR_WORKSPACE;
  int32_t* blockcounts = nullptr;
  rc = scratch_address(&blockcounts);
  if (rc != MOE_OK) return rc;
  return permute_launch(x, dtype, T, D, topk_ids, K, E, align, capacity, capacity_layout,
                        x_sorted, rows, counts, group_sizes, group_offsets, row_of_slot,
                        slot_of_row, blockcounts, err, static_cast<hipStream_t>(stream));
}

// Slot batch of the token-centric kernels for top-K routing.
static int slot_batch(int K) { return K <= 1 ? 1 : K <= 2 ? 2 : K <= 4 ? 4 : 8; }

template <typename T, bool W>
static void launch_gather_sum(int jb, unsigned blocks, hipStream_t st, const void* src,
                              int64_t rows, int64_t T_, int64_t D, int K, const int32_t* ros,
                              const float* w, void* dst, int accumulate) {
  const T* s = static_cast<const T*>(src);
  T* d = static_cast<T*>(dst);
#define GS(JB)                                                                             \
  hipLaunchKernelGGL((gather_sum_kernel<T, W, JB>), dim3(blocks), dim3(kThreads), 0, st, s, \
                     rows, T_, D, K, ros, w, d, accumulate)
  switch (jb) {
    case 1: GS(1); break;
    case 2: GS(2); break;
    case 4: GS(4); break;
    default: GS(8); break;
  }
#undef GS
}

template <bool W>
static int gather_sum(const void* src, int dtype, int64_t rows, int64_t T, int64_t D, int K,
                      const int32_t* ros, const float* w, void* dst, int accumulate,
                      hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>((T + 3) / 4);
  if (dtype == MOE_BF16)
    launch_gather_sum<bf16_t, W>(slot_batch(K), blocks, st, src, rows, T, D, K, ros, w, dst,
                                 accumulate);
  else
    launch_gather_sum<float, W>(slot_batch(K), blocks, st, src, rows, T, D, K, ros, w, dst,
                                accumulate);
  return launch_status();
}

template <typename T>
static void launch_combine_bwd(int jb, unsigned grid, hipStream_t st, const void* d_y,
                               const void* y_sorted, int64_t T_, int64_t D, int K,
                               const int32_t* ros, const int32_t* sor, int64_t rows,
                               const float* w, void* d_ys, float* d_w, int64_t token_blocks) {
  const T* a = static_cast<const T*>(d_y);
  const T* b = static_cast<const T*>(y_sorted);
  T* o = static_cast<T*>(d_ys);
#define CB(JB)                                                                            \
  hipLaunchKernelGGL((combine_bwd_kernel<T, JB>), dim3(grid), dim3(kThreads), 0, st, a, b, \
                     T_, D, K, ros, sor, rows, w, o, d_w, token_blocks)
  switch (jb) {
    case 1: CB(1); break;
    case 2: CB(2); break;
    case 4: CB(4); break;
    default: CB(8); break;
  }
#undef CB
}

MOE_API int moe_permute_bwd(const void* d_x_sorted, int dtype, int64_t T, int64_t D, int K,
                            int64_t rows, const int32_t* row_of_slot, void* d_x, int accumulate,
                            void* stream) {
  if (T < 0 || D < 0 || K < 1 || rows < 0) return MOE_ERR_ARG;
  if (!elem_bytes(dtype)) return MOE_ERR_DTYPE;
  if (T == 0 || D == 0) return MOE_OK;
  if (!d_x_sorted || !row_of_slot || !d_x || D % 8 || !aligned16(d_x_sorted) || !aligned16(d_x))
    return MOE_ERR_ARG;
  return gather_sum<false>(d_x_sorted, dtype, rows, T, D, K, row_of_slot, nullptr, d_x,
                           accumulate, static_cast<hipStream_t>(stream));
}

MOE_API int moe_combine(const void* y_sorted, int dtype, int64_t T, int64_t D, int K,
                        int64_t rows, const int32_t* row_of_slot, const float* topk_w, void* y,
                        void* stream) {
  if (T < 0 || D < 0 || K < 1 || rows < 0) return MOE_ERR_ARG;
  if (!elem_bytes(dtype)) return MOE_ERR_DTYPE;
  if (T == 0 || D == 0) return MOE_OK;
  if (!y_sorted || !row_of_slot || !topk_w || !y || D % 8 || !aligned16(y_sorted) ||
      !aligned16(y))
    return MOE_ERR_ARG;
  return gather_sum<true>(y_sorted, dtype, rows, T, D, K, row_of_slot, topk_w, y, 0,
                          static_cast<hipStream_t>(stream));
}

MOE_API int moe_combine_bwd(const void* d_y, const void* y_sorted, int dtype, int64_t T,
                            int64_t D, int K, int64_t rows, const int32_t* row_of_slot,
                            const int32_t* slot_of_row, const float* topk_w, void* d_y_sorted,
                            float* d_topk_w, void* stream) {
  if (T < 0 || D < 0 || K < 1 || rows < 0) return MOE_ERR_ARG;
  if (!elem_bytes(dtype)) return MOE_ERR_DTYPE;
  if (!d_y || !y_sorted || !row_of_slot || !slot_of_row || !topk_w || !d_y_sorted || !d_topk_w)
    return (T == 0 && rows == 0) ? MOE_OK : MOE_ERR_ARG;
  if (D % 8 || !aligned16(d_y) || !aligned16(y_sorted) || !aligned16(d_y_sorted))
    return MOE_ERR_ARG;
  const int64_t token_blocks = (T + 3) / 4;
  const unsigned grid = static_cast<unsigned>(token_blocks + (rows + 3) / 4);
  if (grid == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == MOE_BF16)
    launch_combine_bwd<bf16_t>(slot_batch(K), grid, st, d_y, y_sorted, T, D, K, row_of_slot,
                               slot_of_row, rows, topk_w, d_y_sorted, d_topk_w, token_blocks);
  else
    launch_combine_bwd<float>(slot_batch(K), grid, st, d_y, y_sorted, T, D, K, row_of_slot,
                              slot_of_row, rows, topk_w, d_y_sorted, d_topk_w, token_blocks);
  return launch_status();
}
