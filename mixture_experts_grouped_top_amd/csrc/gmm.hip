// Grouped GEMM (gmm) and transposed grouped GEMM (tgmm) for gfx950.
//
// Semantics follow the MaxText pull request "Overlap moe comms with collective
// matmul" (gmm with an in-place partial sum whose row count may be below the
// padded lhs row count; tgmm with zero-initialised empty groups and output
// shape (groups, in_size, out_size)) and the grouped_gemm calls of the
// TransformerEngine MoE block.
//
// bf16 path: v_mfma_f32_32x32x16_bf16, float32 accumulators in AGPRs.  A
// workgroup of 4 waves (2 x 2) computes a TM x TN output tile (256 x 256,
// 128 x 256 for small groups, 256 x 128 for narrow outputs); operands reach
// LDS by direct global->LDS loads through a ring of contraction steps, and
// the loads of later steps and the fragment reads of the next substep are
// interleaved one by one with the MFMAs of the current one.  The LDS
// layouts, the two-step (128-byte) loading of contraction-contiguous
// operands and the pipelines are described where they are defined below.
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
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;     // threads per workgroup (4 waves)
constexpr int kMaxG = 1024;

__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

// Position of a group's local tile l among mt x nt tiles: column blocks of
// kNB tiles, row-major inside a block (consecutive indices cover about
// 32 / kNB row tiles x kNB column tiles, so the tiles that run together on
// one XCD share both operand blocks in its L2).
constexpr int kNB = 4;
__device__ __forceinline__ void blocked_tile(int l, int mtiles, int ntiles, int& mt, int& nt) {
  const int per = mtiles * kNB;
  const int nb = l / per, rem = l - nb * per;
  const int width = min(kNB, ntiles - nb * kNB);
  mt = rem / width;
  nt = nb * kNB + rem % width;
}

// Linear tile index of a persistent workgroup's it-th tile: the grid's
// workgroups on XCD x (b % 8 == x) take a contiguous run of indices.
__device__ __forceinline__ int64_t xcd_index(int it, int b, int g) {
  return static_cast<int64_t>(it) * g + (b & 7) * (g >> 3) + (b >> 3);
}
__device__ __forceinline__ int64_t xcd_tile(int it) { return xcd_index(it, blockIdx.x, gridDim.x); }

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

// ---------------------------------------------------------------- bf16 MFMA
//
// Workgroup tile TM x TN (TN = 256, or 128 for narrow or single-step
// problems), contraction step TK = 32, a ring of three or four LDS stages
// (Stages below).  Waves are arranged
// 2 x 2, each owning a (TM/2) x (TN/2) block of 32 x 32 accumulators.
//
// LDS layouts (per stage, per operand), 16-byte chunks XOR-swizzled:
//   contraction-contiguous operand ("row" tile): [x][TK], 64-byte rows;
//     chunk c of row x sits at c ^ ((x >> 2) & 3).  A ds_read_b128 is
//     served 16 lanes (256 bytes, all 64 banks) per cycle; a fragment read
//     gives those lanes 16 consecutive rows, whose 64-byte rows start on 4
//     bank offsets, and the swizzle spreads the 4 rows of each offset over
//     the 4 chunk positions, so the read is conflict-free (measured with
//     the LDS bank-conflict counter; the (x >> 1) swizzle conflicts 2-way).
//     The swizzle repeats every 16 rows (fragment i of a wave is fragment 0
//     plus a constant offset).
//   contraction-major operand ("col" tile): [TK][BX], BX*2-byte rows;
//     chunk c of row k sits at c ^ 4 (k & 3), so the four rows x four chunks
//     that a transposing read (ds_read_b64_tr_b16) touches in one half-wave
//     are distinct banks.
// Full contraction steps are copied global -> LDS by global_load_lds_dwordx4
// (16 bytes per lane; each wave instruction fills 1 KB of LDS in lane order,
// so a lane fetches the global chunk that the swizzle places at its slot).
// These are issued through inline asm so that the only waits on them are
// the explicit ones at the top of each step.  Rows/columns past the valid
// extent are clamped to a valid address (their products land in output rows
// or columns that are never stored).  A ragged last contraction step is
// loaded through registers with zero fill.
//
// MFMA operand fragment for 32 x (k16 substep s): lane l holds x = x0 + l%32,
// k = 16 s + 8 (l / 32) + 0..7.  From a row tile that is one 16-byte read;
// from a col tile, two transposing reads: within each 16-lane group, lane
// 4 r + q addresses row k + r, columns 4 q .. 4 q + 3 of the group's 16
// columns, and receives its own column for the four rows.

constexpr int TK = 32;
constexpr int kCPR = TK / 8;                // 16-byte chunks per row of a row tile

__device__ __forceinline__ int row_swz(int x) { return (x >> 2) & 3; }
__device__ __forceinline__ int row_off(int x, int c) { return x * (TK * 2) + ((c ^ row_swz(x)) << 4); }

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ int col_swz(int k) { return (k & 3) << 2; }
template <int BX>
__device__ __forceinline__ int col_off(int k, int c) { return k * (BX * 2) + ((c ^ col_swz(k)) << 4); }

// threadIdx.x hidden from the optimiser: per-tile index arithmetic derived
// from it is recomputed inside the persistent tile loop instead of being
// hoisted out of it and kept live in registers across every tile.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// One global_load_lds_dwordx4: lane i's 16 bytes from sbase + voff land at
// LDS byte lds + 16 i.  sbase and lds are wave-uniform.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// An operand tile of BX x TK.  COLK: element (x, k) at base[k * ld + x];
// otherwise at base[x * ld + k].
template <bool COLK, int BX>
struct Operand {
  static constexpr int kBytes = BX * TK * 2;
  static constexpr int NJ = kBytes / 1024 / 4;   // DMA instructions per wave per stage
  static constexpr bool kPair = false;           // one DMA unit = one step
  static constexpr int kUnit = kBytes;
  static constexpr int NJU = NJ;
  static constexpr int NR = kBytes / 16 / NT;    // 16-byte chunks per thread (register path)
  const bf16_t* base;
  int64_t ld;
  int xv;                 // valid x extent (>= 1)
  // col tile: 0, or the distance of a second column range: the tile's columns
  // then come in 64-wide blocks alternating between the two ranges (block
  // 2 p: columns 64 p .. of the first, block 2 p + 1: the same of the second)
  int64_t split;
  uint32_t voff[NJ];      // byte offsets of this lane's DMA chunks

  __device__ __forceinline__ void setup(const bf16_t* b, int64_t ld_, int xv_, int64_t split_ = 0) {
    base = b;
    ld = ld_;
    xv = xv_;
    split = split_;
    const int tid = opaque_tid();
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int byte = (w * NJ + j) * 1024 + lane * 16;
      if (!COLK) {
        const int x = byte / (TK * 2);
        const int c = ((byte % (TK * 2)) >> 4) ^ row_swz(x);
        const int xx = x < xv ? x : xv - 1;
        voff[j] = static_cast<uint32_t>((xx * ld + c * 8) * 2);
      } else {
        const int k = byte / (BX * 2);
        int c = ((byte % (BX * 2)) >> 4) ^ col_swz(k);
        const int cmax = (xv - 1) >> 3;
        if (c > cmax) c = cmax;
        voff[j] = static_cast<uint32_t>((k * ld + col_of(c)) * 2);
      }
    }
  }
  __device__ __forceinline__ const bf16_t* step_base(int kt) const {
    return COLK ? base + static_cast<int64_t>(kt) * TK * ld : base + static_cast<int64_t>(kt) * TK;
  }
  // col tile: source column (elements from base) of the tile's 8-column chunk c
  __device__ __forceinline__ int64_t col_of(int c) const {
    const int b = c >> 3;   // 64-column block
    return c * 8 + (split ? (b & 1) * split - 64 * ((b + 1) >> 1) : 0);
  }
  // DMA instruction j (< NJ) of step kt; sb = uniform_ptr(step_base(kt)).
  __device__ __forceinline__ void dma_one(const void* sb, int j, uint32_t lds) const {
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    dma16(sb, voff[j], lds + (w * NJ + j) * 1024);
  }
  __device__ __forceinline__ void dma(int kt, uint32_t lds) const {
    const void* sb = uniform_ptr(step_base(kt));
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < NJ; ++j) dma16(sb, voff[j], lds + (w * NJ + j) * 1024);
  }
  // Register path for a partial step of kv < TK contraction elements.
  __device__ __forceinline__ void tail_load(int kt, int kv, uint4 (&r)[NR]) const {
    const bf16_t* b = step_base(kt);
    const int tid = opaque_tid();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = tid + i * NT;
      bool ok;
      const bf16_t* p;
      if (!COLK) {
        const int x = q / kCPR, c = q % kCPR;
        ok = x < xv && c * 8 < kv;
        p = b + x * ld + c * 8;
      } else {
        const int k = q / (BX / 8), c = q % (BX / 8);
        ok = k < kv && c * 8 < xv;
        p = b + k * ld + col_of(c);
      }
      r[i] = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void tail_store(char* lds, const uint4 (&r)[NR]) const {
    const int tid = opaque_tid();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = tid + i * NT;
      int off;
      if (!COLK) off = row_off(q / kCPR, q % kCPR);
      else off = col_off<BX>(q / (BX / 8), q % (BX / 8));
      *reinterpret_cast<uint4*>(lds + off) = r[i];
    }
  }
  // Per-lane byte offsets of this wave's MFMA fragments inside a stage tile.
  // Fragment (i, s) covers x = xw + 32 i + lane % 32 and
  // k = 16 s + 8 (lane / 32) + 0..7, where xw is the wave's first x.
  //   row tile: at fb[s] + i * 32 * 128 (one 16-byte read)
  //   col tile: at fb[i] + s * 16 * ROWB and + 4 * ROWB (two transposing
  //             reads; within each 16-lane group lane 4 r + q addresses row
  //             r, columns 4 q .. 4 q + 3, and receives its own column)
  static constexpr int ROWB = BX * 2;
  __device__ __forceinline__ static void frag_base(int xw, uint32_t (&fb)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (!COLK) {
        fb[t] = t < TK / 16 ? static_cast<uint32_t>(row_off(xw + (lane & 31), 2 * t + (lane >> 5))) : 0u;
      } else {
        const int g = lane >> 4, j = lane & 15;
        const int k = 8 * (g >> 1) + (j >> 2);
        const int xc = xw + 32 * t + 16 * (g & 1) + 4 * (j & 3);
        fb[t] = static_cast<uint32_t>(col_off<BX>(k, xc >> 3) + ((xc & 7) << 1));
      }
    }
  }
  __device__ __forceinline__ static bf16x8 frag(const char* lds, const uint32_t (&fb)[4], int i, int s) {
    if (!COLK) {
      return *reinterpret_cast<const bf16x8*>(lds + fb[s] + i * 32 * (TK * 2));
    } else {
      typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
      const char* p = lds + fb[i] + s * 16 * ROWB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * ROWB));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8, v);
    }
  }
};

// A contraction-contiguous ("row") operand of BX rows loaded in units of two
// steps: each DMA lane copies 16 bytes of a 128-byte row segment (two
// steps of 32 elements), so every request is a whole 128-byte line instead
// of half of one.  LDS unit layout [x][64]: row x at 128 x bytes, 16-byte
// chunk c at (c ^ ((x >> 1) & 7)): the 16 rows that one ds_read_b128 cycle
// serves start on 2 bank offsets and the swizzle gives the 8 rows of each
// offset 8 distinct chunk positions, so all 64 banks are hit once.  Substep sub (0..3) of a unit covers
// contraction elements 16 sub .. 16 sub + 15.
template <int BX>
struct PairRow {
  static constexpr int kBytes = BX * TK * 2;     // one step
  static constexpr int NJ = kBytes / 1024 / 4;
  static constexpr bool kPair = true;
  static constexpr int kUnit = 2 * kBytes;
  static constexpr int NJU = 2 * NJ;             // DMA instructions per wave per unit
  static constexpr int NR = kBytes / 16 / NT;    // register path: 16-byte chunks per thread
  const bf16_t* base;
  int64_t ld;
  int xv;
  uint32_t voff[NJU];

  __device__ __forceinline__ static int off(int x, int c) { return x * 128 + ((c ^ ((x >> 1) & 7)) << 4); }
  __device__ __forceinline__ void setup(const bf16_t* b, int64_t ld_, int xv_) {
    base = b;
    ld = ld_;
    xv = xv_;
    const int tid = opaque_tid();
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int j = 0; j < NJU; ++j) {
      const int byte = (w * NJU + j) * 1024 + lane * 16;
      const int x = byte >> 7;
      const int c = ((byte & 127) >> 4) ^ ((x >> 1) & 7);
      const int xx = x < xv ? x : xv - 1;
      voff[j] = static_cast<uint32_t>((xx * ld + c * 8) * 2);
    }
  }
  __device__ __forceinline__ const bf16_t* step_base(int kt) const {
    return base + static_cast<int64_t>(kt) * TK;
  }
  // DMA instruction j (< NJU) of the unit starting at step kt (even);
  // sb = uniform_ptr(step_base(kt)).
  __device__ __forceinline__ void dma_one(const void* sb, int j, uint32_t lds) const {
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    dma16(sb, voff[j], lds + (w * NJU + j) * 1024);
  }
  // Ragged last step (kv < TK elements) into the first half of a unit.
  __device__ __forceinline__ void tail_load(int kt, int kv, uint4 (&r)[NR]) const {
    const bf16_t* b = step_base(kt);
    const int tid = opaque_tid();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = tid + i * NT;
      const int x = q / kCPR, c = q % kCPR;
      const bool ok = x < xv && c * 8 < kv;
      r[i] = ok ? *reinterpret_cast<const uint4*>(b + x * ld + c * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void tail_store(char* lds, const uint4 (&r)[NR]) const {
    const int tid = opaque_tid();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = tid + i * NT;
      *reinterpret_cast<uint4*>(lds + off(q / kCPR, q % kCPR)) = r[i];
    }
  }
  // Fragment (i, sub): x = xw + 32 i + lane % 32, chunk 2 sub + lane / 32;
  // the swizzle term ((x >> 1) & 7) does not depend on i.
  __device__ __forceinline__ static void frag_base(int xw, uint32_t (&fb)[4]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < 4; ++t) fb[t] = static_cast<uint32_t>(off(xw + (lane & 31), 2 * t + (lane >> 5)));
  }
  __device__ __forceinline__ static bf16x8 frag(const char* lds, const uint32_t (&fb)[4], int i, int sub) {
    return *reinterpret_cast<const bf16x8*>(lds + fb[sub] + i * 32 * 128);
  }
};

template <int TM, int TN>
struct Acc {
  static constexpr int FM = TM / 64, FN = TN / 64;
  f32x16 v[FM][FN];
  // Fragment rows i < live take MFMAs; the rest hold only zero rows of lhs
  // (rows past a group's valid rows, or past its last row), so their
  // products are zero and are skipped.  Wave-uniform; FM unless a gmm tile
  // sets it.  Only 128-row tiles skip (they serve small, padded groups; in
  // the 256-row kernels the branches cost registers).
  static constexpr bool kSkip = TM <= 128;
  int live = FM;
  // live for a tile whose first vrows rows (of TM) may be non-zero, for
  // this wave's row block
  __device__ __forceinline__ void set_live_rows(int vrows) {
    const int wr = static_cast<int>(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >> 1) * (TM / 2);
    live = __builtin_amdgcn_readfirstlane(min(FM, max(0, (vrows - wr + 31) >> 5)));
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
  }
  // Fragments of one k16 substep.
  struct Frags {
    bf16x8 a[FM], b[FN];
  };
  template <class OA, class OB>
  __device__ __forceinline__ static void load(Frags& f, const char* As, const char* Bs,
                                              const uint32_t (&fa)[4], const uint32_t (&fb)[4],
                                              int sub) {
#pragma unroll
    for (int i = 0; i < FM; ++i) f.a[i] = OA::frag(As, fa, i, sub);
#pragma unroll
    for (int j = 0; j < FN; ++j) f.b[j] = OB::frag(Bs, fb, j, sub);
  }
  template <class OA>
  __device__ __forceinline__ static void load_a(Frags& f, const char* As, const uint32_t (&fa)[4],
                                                int i, int sub) {
    f.a[i] = OA::frag(As, fa, i, sub);
  }
  template <class OB>
  __device__ __forceinline__ static void load_b(Frags& f, const char* Bs, const uint32_t (&fb)[4],
                                                int j, int sub) {
    f.b[j] = OB::frag(Bs, fb, j, sub);
  }
  // Fragment read o (0 .. FM + FN - 1) of a substep, in the order the MFMAs
  // q = i FN + j consume them: a0, b0 .. b(FN-1), a1 .. a(FM-1).
  template <class OA, class OB>
  __device__ __forceinline__ static void load_one(Frags& f, const char* As, const char* Bs,
                                                  const uint32_t (&fa)[4], const uint32_t (&fb)[4],
                                                  int o, int suba, int subb) {
    if (o == 0) f.a[0] = OA::frag(As, fa, 0, suba);
    else if (o <= FN) f.b[o - 1] = OB::frag(Bs, fb, o - 1, subb);
    else f.a[o - FN] = OA::frag(As, fa, o - FN, suba);
  }
  __device__ __forceinline__ void mma_one(const Frags& f, int q) {
    const int i = q / FN, j = q % FN;
    if (!kSkip || i < live) v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], v[i][j], 0, 0, 0);
  }
  __device__ __forceinline__ void mma(const Frags& f) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (!kSkip || i < live)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], v[i][j], 0, 0, 0);
  }
  // f(row, col, value) for every accumulator element (row/col inside the tile)
  template <typename F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r0 = (w >> 1) * (TM / 2) + 4 * (lane >> 5);
    const int c0 = (w & 1) * (TN / 2) + (lane & 31);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          f(r0 + 32 * i + 8 * (r >> 2) + (r & 3), c0 + 32 * j, v[i][j][r]);
  }
};

struct MfmaArgs {
  const bf16_t* lhs;
  int64_t ld_lhs;
  const bf16_t* rhs;
  int64_t ld_rhs;
  int64_t rhs_gs;        // gmm: rhs group stride
  const int32_t* gsz;
  int G;
  int64_t M;             // gmm: output rows; tgmm: lhs/rhs rows
  int64_t Kdim;
  int64_t N;
  void* out;
  int64_t ld_out;
  int64_t out_gs;        // tgmm: output group stride
  int accumulate;
  int32_t* err;
  const int32_t* valid = nullptr;   // tgmm: leading rows of each group that may be non-zero
  const bf16_t* bias = nullptr;      // gmm: per-group bias rows [G, N], added to the output
  bf16_t* act = nullptr;             // gmm with the SwiGLU epilogue: act [M, F]
  int64_t ld_act = 0;
  int cls_lo = 0, cls_hi = 0x7fffffff;   // gmm: only groups of cls_lo .. cls_hi rows own tiles
  // gmm with the SwiGLU-backward epilogue: h0/h1 [M, N] (row stride ld_h) are
  // read, out is d_h0 and dh1 d_h1 (row stride ld_out)
  const bf16_t* h0 = nullptr;
  const bf16_t* h1 = nullptr;
  int64_t ld_h = 0;
  bf16_t* dh1 = nullptr;
};

// MFMAs of one substep (q = 0 .. NM-1) with NO other operations between
// them in order, pinned there with scheduling barriers: the operations are
// front-loaded, ceil(NO / NM) after each MFMA, so that fragment reads issued
// first have the whole substep to land.
template <int NM, int NO, class M, class O>
__device__ __forceinline__ void interleave(M&& mma, O&& op) {
  constexpr int K = (NO + NM - 1) / NM;
#pragma unroll
  for (int q = 0; q < NM; ++q) {
    mma(q);
#pragma unroll
    for (int o = q * K; o < (q + 1) * K && o < NO; ++o) op(o);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Contraction over one tile: nfull DMA steps, then an optional ragged step.
// LDS holds NS stages, each the A tile followed by the B tile.
//
// Software pipeline (TK = 32: two k16 substeps per stage):
//   prologue: DMA stages 0..NS-1; wait for stage 0; barrier; load frags(0, 0)
//   step s:   load frags(s, 1); MFMAs(s, 0);
//             wait for stage s + 1; barrier (also: all waves hold their
//             frags of stage s, so its buffer is free); DMA stage s + NS
//             into it; load frags(s + 1, 0);
//             MFMAs(s, 1)
// so MFMAs are queued whenever a wave waits at the barrier or on LDS.
template <int NS, class OA, class OB, class ACC>
__device__ __forceinline__ void contract(char* lds, const OA& A, const OB& B, int64_t Kc,
                                         ACC& acc, const uint32_t (&fa)[4],
                                         const uint32_t (&fb)[4]) {
  static_assert(TK == 32 && NS >= 2 && NS <= 4, "pipeline written for 2..4 stages of two substeps");
  constexpr int SB = OA::kBytes + OB::kBytes;
  const int nfull = static_cast<int>(Kc / TK);
  const int kv = static_cast<int>(Kc - static_cast<int64_t>(nfull) * TK);
  constexpr int PER = OA::NJ + OB::NJ;      // DMA instructions per thread per stage
  typename ACC::Frags f0, f1;
  acc.zero();
#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < nfull) {
      A.dma(p, lds_addr(lds + p * SB));
      B.dma(p, lds_addr(lds + p * SB + OA::kBytes));
    }
  if (nfull > 0) {
    // stage 0 has landed once at most the later prologue stages are in flight
    const int later = min(NS - 1, nfull - 1);
    if (later >= 3) wait_vmcnt<3 * PER>();
    else if (later == 2) wait_vmcnt<2 * PER>();
    else if (later == 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
    __syncthreads();
    ACC::template load<OA, OB>(f0, lds, lds + OA::kBytes, fa, fb, 0);
  }
  for (int s = 0; s < nfull; ++s) {
    const int cur = s % NS;
    char* cs = lds + cur * SB;
    {
      // MFMAs(s, 0) with the fragment reads of (s, 1) between them
      constexpr int NM = ACC::FM * ACC::FN;
      interleave<NM, ACC::FM + ACC::FN>(
          [&](int q) { acc.mma_one(f0, q); },
          [&](int o) { ACC::template load_one<OA, OB>(f1, cs, cs + OA::kBytes, fa, fb, o, 1, 1); });
    }
    if (s + 1 < nfull) {
      // stages s + 2 .. s + NS - 1 may still be in flight; s + 1 must have landed
      const int later = min(NS - 2, nfull - 2 - s);
      if (later >= 2) wait_vmcnt<2 * PER>();
      else if (later == 1) wait_vmcnt<PER>();
      else wait_vmcnt<0>();
      __syncthreads();
      char* ns = lds + ((s + 1) % NS) * SB;
      if (s + NS < nfull) {
        // MFMAs(s, 1) with the DMA of stage s + NS and the fragment reads of
        // (s + 1, 0) spread between them, in this order: each DMA issue,
        // which can wait for room in the load queue, then sits behind a
        // running MFMA instead of idling the matrix unit
        const void* sa = uniform_ptr(A.step_base(s + NS));
        const void* sb = uniform_ptr(B.step_base(s + NS));
        const uint32_t la = lds_addr(cs), lb = lds_addr(cs + OA::kBytes);
        constexpr int NM = ACC::FM * ACC::FN;
        constexpr int NF = ACC::FM + ACC::FN;
        interleave<NM, NF + OA::NJ + OB::NJ>(
            [&](int q) { acc.mma_one(f1, q); },
            [&](int o) {
              if (o < NF) ACC::template load_one<OA, OB>(f0, ns, ns + OA::kBytes, fa, fb, o, 0, 0);
              else if (o < NF + OA::NJ) A.dma_one(sa, o - NF, la);
              else B.dma_one(sb, o - NF - OA::NJ, lb);
            });
        continue;
      }
      ACC::template load<OA, OB>(f0, ns, ns + OA::kBytes, fa, fb, 0);
    }
    acc.mma(f1);
  }
  if (kv > 0) {
    // stage nfull % NS was last read NS steps ago (or by the previous tile)
    // and no DMA targets it; other waves may still read stage nfull - 1
    char* ts = lds + (nfull % NS) * SB;
    {
      uint4 t[OA::NR];
      A.tail_load(nfull, kv, t);
      A.tail_store(ts, t);
    }
    {
      uint4 t[OB::NR];
      B.tail_load(nfull, kv, t);
      B.tail_store(ts + OA::kBytes, t);
    }
    __syncthreads();
    ACC::template load<OA, OB>(f0, ts, ts + OA::kBytes, fa, fb, 0);
    ACC::template load<OA, OB>(f1, ts, ts + OA::kBytes, fa, fb, 1);
    acc.mma(f0);
    acc.mma(f1);
  }
  __syncthreads();   // every wave is done with all stages before they are refilled
}

// s_waitcnt vmcnt(n) for a wave-uniform n <= N (a chain of constant waits).
template <int N>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) wait_vmcnt<N>();
    else wait_vmcnt_dyn<N - 1>(n);
  }
}

// Contraction with a pair-loaded lhs (PairRow) and an rhs that is either
// pair-loaded too or a per-step operand (row or col tile), over a four-step
// LDS ring:
// A holds two units of two steps, B two such units or four single steps.
// The unit of a pair operand is free once both of its steps are consumed,
// so the pair for steps t + 3, t + 4 is issued after the barrier of odd
// steps t; a single-step B unit gets step t + 4 after every step t.  Every
// block is issued, also past the last step (it then re-reads the last
// valid unit into a unit that is no longer read), so each wait count is a
// constant.  Requires an even number (>= 2) of full steps; a ragged rest
// goes through registers into the first half of the next unit.
template <class PA, class OB, class ACC>
__device__ __forceinline__ void contract2(char* lds, const PA& A, const OB& B, int64_t Kc,
                                          ACC& acc, const uint32_t (&fa)[4],
                                          const uint32_t (&fb)[4]) {
  constexpr bool BP = OB::kPair;
  constexpr int UA = PA::kUnit, UB = OB::kUnit;
  constexpr int JA = PA::NJU, JB = OB::NJU;
  constexpr int NM = ACC::FM * ACC::FN;
  // vmcnt entries a wave may leave in flight when it needs the next step:
  // after an even step the pair issued with the last odd block plus the
  // later single-step blocks; after an odd step only later blocks
  constexpr int W_EVEN = BP ? JA + JB : JA + 2 * JB;
  constexpr int W_ODD = BP ? 0 : 2 * JB;
  constexpr int W_PRO = BP ? JA + JB : JA + 3 * JB;
  static_assert(W_PRO < 64, "vmcnt range");
  char* const la = lds;
  char* const lb = lds + 2 * UA;
  const int nfull = static_cast<int>(Kc / TK);
  const int kv = static_cast<int>(Kc - static_cast<int64_t>(nfull) * TK);
  auto aU = [&](int st) { return la + ((st >> 1) & 1) * UA; };
  auto bU = [&](int st) { return BP ? lb + ((st >> 1) & 1) * UB : lb + (st & 3) * UB; };
  // source step of a DMA unit, clamped to the last valid unit
  auto pair_src = [&](int st) { return st < nfull ? st : nfull - 2; };
  auto step_src = [&](int st) { return st < nfull ? st : nfull - 1; };
  // the DMA block of (virtual) step t, all at once (prologue)
  auto block = [&](int t) {
    if (t & 1) {
      const void* sa = uniform_ptr(A.step_base(pair_src(t + 3)));
      const uint32_t l = lds_addr(aU(t + 3));
#pragma unroll
      for (int j = 0; j < JA; ++j) A.dma_one(sa, j, l);
      if constexpr (BP) {
        const void* sb = uniform_ptr(B.step_base(pair_src(t + 3)));
        const uint32_t m = lds_addr(bU(t + 3));
#pragma unroll
        for (int j = 0; j < JB; ++j) B.dma_one(sb, j, m);
      }
    }
    if constexpr (!BP) {
      const void* sb = uniform_ptr(B.step_base(step_src(t + 4)));
      const uint32_t m = lds_addr(bU(t + 4));
#pragma unroll
      for (int j = 0; j < JB; ++j) B.dma_one(sb, j, m);
    }
  };
  typename ACC::Frags f0, f1;
  acc.zero();
  if (nfull == 0) {
    // only a ragged step: nothing to pipeline
  } else {
    for (int t = -4; t < 0; ++t) block(t);
    wait_vmcnt<W_PRO>();                     // step 0 (A pair of block -3, B of block -4)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ACC::FM; ++i) ACC::template load_a<PA>(f0, aU(0), fa, i, 0);
#pragma unroll
    for (int j = 0; j < ACC::FN; ++j) ACC::template load_b<OB>(f0, bU(0), fb, j, 0);
    // MFMAs(s, 0) with the fragment reads of (s, 1); P is the parity of s
    auto first_half = [&](auto par, int s) {
      constexpr int P = decltype(par)::value;
      constexpr int sa1 = 2 * P + 1, sb1 = BP ? 2 * P + 1 : 1;
      char* const ua = aU(s);
      char* const ub = bU(s);
      interleave<NM, ACC::FM + ACC::FN>(
          [&](int q) { acc.mma_one(f0, q); },
          [&](int o) { ACC::template load_one<PA, OB>(f1, ua, ub, fa, fb, o, sa1, sb1); });
    };
    // wait for step s + 1, barrier, then MFMAs(s, 1) with the fragment reads
    // of (s + 1, 0) and the DMA block of step s (all waves are done with
    // step s: its units may refill)
    auto second_half = [&](auto par, int s) {
      constexpr int P = decltype(par)::value;
      constexpr int na0 = 2 * (1 - P), nb0 = BP ? 2 * (1 - P) : 0;
      if constexpr (P == 1) wait_vmcnt<W_ODD>(); else wait_vmcnt<W_EVEN>();
      __syncthreads();
      char* const na = aU(s + 1);
      char* const nb = bU(s + 1);
      if constexpr (P == 1) {
        const void* sa = uniform_ptr(A.step_base(pair_src(s + 3)));
        const uint32_t da = lds_addr(aU(s + 3));
        const void* sb = uniform_ptr(B.step_base(BP ? pair_src(s + 3) : step_src(s + 4)));
        const uint32_t db = lds_addr(bU(BP ? s + 3 : s + 4));
        constexpr int NO = ACC::FM + ACC::FN + JA + JB;
        constexpr int NF = ACC::FM + ACC::FN;
        interleave<NM, NO>([&](int q) { acc.mma_one(f1, q); },
                           [&](int o) {
                             if (o < NF) ACC::template load_one<PA, OB>(f0, na, nb, fa, fb, o, na0, nb0);
                             else if (o < NF + JA) A.dma_one(sa, o - NF, da);
                             else B.dma_one(sb, o - NF - JA, db);
                           });
      } else {
        const void* sb = uniform_ptr(B.step_base(BP ? 0 : step_src(s + 4)));
        const uint32_t db = lds_addr(bU(s + 4));
        constexpr int NO = ACC::FM + ACC::FN + (BP ? 0 : JB);
        constexpr int NF = ACC::FM + ACC::FN;
        interleave<NM, NO>([&](int q) { acc.mma_one(f1, q); },
                           [&](int o) {
                             if (o < NF) ACC::template load_one<PA, OB>(f0, na, nb, fa, fb, o, na0, nb0);
                             else if constexpr (!BP) B.dma_one(sb, o - NF, db);
                           });
      }
    };
    const std::integral_constant<int, 0> even;
    const std::integral_constant<int, 1> odd;
    for (int s = 0; s + 2 < nfull; s += 2) {
      first_half(even, s);
      second_half(even, s);
      first_half(odd, s + 1);
      second_half(odd, s + 1);
    }
    first_half(even, nfull - 2);
    second_half(even, nfull - 2);
    first_half(odd, nfull - 1);
    acc.mma(f1);
    wait_vmcnt<0>();   // the re-reads issued past the last step have landed
  }
  if (kv > 0) {
    // the units of step nfull held steps nfull - 4 (.. nfull - 3), long
    // consumed; nothing is in flight
    {
      uint4 t[PA::NR];
      A.tail_load(nfull, kv, t);
      A.tail_store(aU(nfull), t);
    }
    {
      uint4 t[OB::NR];
      B.tail_load(nfull, kv, t);
      B.tail_store(bU(nfull), t);
    }
    __syncthreads();
    // nfull is even: the tail sits at substeps 0 and 1 of its units
#pragma unroll
    for (int i = 0; i < ACC::FM; ++i) {
      ACC::template load_a<PA>(f0, aU(nfull), fa, i, 0);
      ACC::template load_a<PA>(f1, aU(nfull), fa, i, 1);
    }
#pragma unroll
    for (int j = 0; j < ACC::FN; ++j) {
      ACC::template load_b<OB>(f0, bU(nfull), fb, j, 0);
      ACC::template load_b<OB>(f1, bU(nfull), fb, j, 1);
    }
    acc.mma(f0);
    acc.mma(f1);
  }
  __syncthreads();   // every wave is done with all units before they are refilled
}

// Stages and LDS bytes of a TM x TN tile (128-row tiles keep three stages
// so that two workgroups fit in one CU's LDS).
template <int TM, int TN>
struct Stages {
  static constexpr int NS = (TN >= 384 || TM <= 128) ? 3 : 4;
  static constexpr int kBytes = NS * (TM + TN) * TK * 2;
};

// Write the accumulator tile: for each of its FM 32-row slabs a wave stages
// the slab (32 x TN/2 float32) in its own LDS region, then reads it back as
// 8-column row chunks (four of a lane's chunks at once, so the reads overlap)
// and stores them with 16-byte (bf16) or 32-byte (fp32) accesses; rows >= rv
// and columns >= cv are skipped.  A wave whose whole block is stored plainly
// (in bounds, no partial sum, bias or scale) takes a path without per-chunk
// tests.  The LDS is the operand stages, free once the contraction has ended
// with a barrier.
template <int TM, int TN, typename TO, bool PF = true>
__device__ __forceinline__ void store_tile(const Acc<TM, TN>& acc, char* lds, TO* o, int64_t ldo,
                                           int rv, int cv, int accumulate,
                                           const bf16_t* bias = nullptr, float scale = 1.f,
                                           int rz = 1 << 30) {
  constexpr int WC = TN / 2;
  constexpr int SROW = WC * 4 + 16;
  constexpr int CPR = WC / 8;                 // 8-column chunks per slab row
  constexpr int NQ = 32 * CPR / 64;           // chunks per lane per slab
  constexpr int QB = NQ < 4 ? NQ : 4;         // chunks whose reads are in flight together
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  static_assert(4 * 32 * SROW <= Stages<TM, TN>::kBytes, "epilogue slabs fit in the stage buffers");
  char* slab = lds + w * 32 * SROW;
  const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * WC;
  const bool plain = !accumulate && !bias && scale == 1.f && wr + TM / 2 <= min(rv, rz) &&
                     wc + WC <= cv;
#pragma unroll
  for (int i = 0; i < Acc<TM, TN>::FM; ++i) {
    // bf16 partial sums (PF): all of the slab's old values are requested
    // before the slab is staged (one load round trip per slab, overlapping
    // the staging, 32 registers); float32 partial sums (64 registers, which
    // the 256 x 256 epilogues would spill) and the FP8 tgmm, which is
    // slower with it, load them chunk by chunk
    constexpr bool kPre = PF && sizeof(TO) == 2;
    Raw8<TO> prev[kPre ? NQ : 1];
    if (kPre && accumulate) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int chunk = lane + 64 * q;
        const int grow = wr + 32 * i + chunk / CPR, gcol = wc + 8 * (chunk % CPR);
        const bool ok = grow < rv && gcol < cv;
        prev[q].load(ok ? o + static_cast<int64_t>(grow) * ldo + gcol : o);
      }
    }
#pragma unroll
    for (int j = 0; j < Acc<TM, TN>::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = 32 * j + (lane & 31);
        *reinterpret_cast<float*>(slab + row * SROW + col * 4) = acc.v[i][j][r];
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q0 = 0; q0 < NQ; q0 += QB) {
    float4 lo[QB], hi[QB];
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      const int chunk = lane + 64 * (q0 + u);
      const int row = chunk / CPR, c8 = chunk % CPR;
      lo[u] = *reinterpret_cast<const float4*>(slab + row * SROW + c8 * 32);
      hi[u] = *reinterpret_cast<const float4*>(slab + row * SROW + c8 * 32 + 16);
    }
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      const int q = q0 + u;
      const int chunk = lane + 64 * q;
      const int row = chunk / CPR, c8 = chunk % CPR;
      const int grow = wr + 32 * i + row, gcol = wc + 8 * c8;
      float v[8] = {lo[u].x, lo[u].y, lo[u].z, lo[u].w, hi[u].x, hi[u].y, hi[u].z, hi[u].w};
      TO* p = o + static_cast<int64_t>(grow) * ldo + gcol;
      if (plain) {
        store8_nt(p, v);
        continue;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = grow < rz ? v[e] * scale : 0.f;   // rows >= rz: zero lhs rows
      if (grow < rv && gcol < cv) {
        if (accumulate) {
          float old[8];
          if constexpr (kPre) prev[q].get(old);
          else load8(p, old);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += old[e];
        }
        if (bias) {
          float b[8];
          load8(bias + gcol, b);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += b[e];
        }
        if (accumulate) store8(p, v);
        else store8_nt(p, v);
      }
    }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();   // the stages are refilled by the next tile
}

// Epilogue of the fused up-projection with SwiGLU.  The tile's columns come
// in 64-wide blocks alternating gate and up columns of the same d_ff range
// (block 2 p: gate columns f0 + 64 p .., block 2 p + 1: the up columns of the
// same d_ff), so the 128 columns of each wave hold the gate and up values of
// 64 d_ff columns and no wave needs another's: per 32-row slab it stages its
// block in its own LDS region (as store_tile), writes its rows of h0 and h1
// (bias added, rows >= rz zero) and act = silu(g) * u on the bf16-rounded h
// values (as the SwiGLU pass over h does).
template <int TM, int TN>
__device__ __forceinline__ void store_tile_swiglu(const Acc<TM, TN>& acc, char* lds, bf16_t* h0,
                                                  bf16_t* h1, int64_t ld_h, bf16_t* act,
                                                  int64_t ld_act, int rv, const bf16_t* b0,
                                                  const bf16_t* b1, int rz) {
  constexpr int WC = TN / 2;                  // columns per wave: 64 gate, 64 up
  constexpr int HC = WC / 2;                  // d_ff columns per wave
  constexpr int SROW = WC * 4 + 16;
  constexpr int CPR = HC / 8;                 // 8-column chunks per row of one half
  constexpr int NQ = 32 * CPR / 64;           // chunks per lane per slab
  static_assert(4 * 32 * SROW <= Stages<TM, TN>::kBytes, "epilogue slabs fit in the stage buffers");
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* slab = lds + w * 32 * SROW;
  const int wr = (w >> 1) * (TM / 2);
  const int fw = (w & 1) * HC;                // the wave's first d_ff column in the tile
  auto value = [&](int row, int col, int grow, const bf16_t* bias, float v[8]) {
    const float4 lo = *reinterpret_cast<const float4*>(slab + row * SROW + col * 4);
    const float4 hi = *reinterpret_cast<const float4*>(slab + row * SROW + col * 4 + 16);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = grow < rz ? v[e] : 0.f;
    if (bias) {
      float b[8];
      load8(bias, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += b[e];
    }
  };
#pragma unroll
  for (int i = 0; i < Acc<TM, TN>::FM; ++i) {
#pragma unroll
    for (int j = 0; j < Acc<TM, TN>::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = 32 * j + (lane & 31);
        *reinterpret_cast<float*>(slab + row * SROW + col * 4) = acc.v[i][j][r];
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int chunk = lane + 64 * q;
      const int row = chunk / CPR, c8 = chunk % CPR;
      const int grow = wr + 32 * i + row;
      if (grow < rv) {
        const int f = fw + 8 * c8;
        float g[8], u[8], o[8];
        value(row, 8 * c8, grow, b0 ? b0 + f : nullptr, g);
        value(row, HC + 8 * c8, grow, b1 ? b1 + f : nullptr, u);
        if (h0) {
          store8_nt(h0 + static_cast<int64_t>(grow) * ld_h + f, g);
          store8_nt(h1 + static_cast<int64_t>(grow) * ld_h + f, u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[e] = swiglu_f32(bf16_to_f32(f32_to_bf16(g[e])), bf16_to_f32(f32_to_bf16(u[e])));
        store8_nt(act + static_cast<int64_t>(grow) * ld_act + f, o);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();   // the stages are refilled by the next tile
}

// Epilogue of the d_act GEMM with the SwiGLU backward: the tile's value is
// d_act (rounded to bf16, as the stored d_act the SwiGLU backward pass reads),
// combined with the forward's h0, h1 into d_h0, d_h1.  Staged per wave as in
// store_tile; rows >= rz have zero d_act; rows >= rv and columns >= cv are
// not written.
template <int TM, int TN>
__device__ __forceinline__ void store_tile_swiglu_bwd(const Acc<TM, TN>& acc, char* lds, bf16_t* d0,
                                                      bf16_t* d1, int64_t ld_d, const bf16_t* h0,
                                                      const bf16_t* h1, int64_t ld_h, int rv,
                                                      int cv, int rz) {
  constexpr int WC = TN / 2;
  constexpr int SROW = WC * 4 + 16;
  constexpr int CPR = WC / 8;
  constexpr int NQ = 32 * CPR / 64;            // chunks per lane per slab
  static_assert(4 * 32 * SROW <= Stages<TM, TN>::kBytes, "epilogue slabs fit in the stage buffers");
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* slab = lds + w * 32 * SROW;
  const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * WC;
#pragma unroll
  for (int i = 0; i < Acc<TM, TN>::FM; ++i) {
    // every h0, h1 chunk of the slab is requested before the slab is
    // staged, so their latency overlaps the staging (one wait per slab;
    // requesting the next slab's chunks during this slab's stores, in the
    // same registers, was 12% slower on the Mixtral-8x7B shape)
    Raw8<bf16_t> ra[NQ], rb[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int chunk = lane + 64 * q;
      const int row = chunk / CPR, c8 = chunk % CPR;
      const int grow = wr + 32 * i + row, gcol = wc + 8 * c8;
      const bool ok = grow < rv && gcol < cv;
      const int64_t hoff = static_cast<int64_t>(ok ? grow : 0) * ld_h + (ok ? gcol : 0);
      ra[q].load(h0 + hoff);
      rb[q].load(h1 + hoff);
    }
#pragma unroll
    for (int j = 0; j < Acc<TM, TN>::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = 32 * j + (lane & 31);
        *reinterpret_cast<float*>(slab + row * SROW + col * 4) = acc.v[i][j][r];
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int chunk = lane + 64 * q;
      const int row = chunk / CPR, c8 = chunk % CPR;
      const int grow = wr + 32 * i + row, gcol = wc + 8 * c8;
      if (grow < rv && gcol < cv) {
        const float4 lo = *reinterpret_cast<const float4*>(slab + row * SROW + c8 * 32);
        const float4 hi = *reinterpret_cast<const float4*>(slab + row * SROW + c8 * 32 + 16);
        const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        float ga[8], ha[8], hb[8], o0[8], o1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ga[e] = grow < rz ? bf16_to_f32(f32_to_bf16(v[e])) : 0.f;
        ra[q].get(ha);
        rb[q].get(hb);
#pragma unroll
        for (int e = 0; e < 8; ++e) swiglu_bwd_f32(ha[e], hb[e], ga[e], o0[e], o1[e]);
        const int64_t doff = static_cast<int64_t>(grow) * ld_d + gcol;
        store8_nt(d0 + doff, o0);
        store8_nt(d1 + doff, o1);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();   // the stages are refilled by the next tile
}

// Groups of more rows than this take 256-row tiles even when most groups are
// small (a launch of their own).  On a DeepSeek-V3-shaped skewed load this
// saves 9-11% on the launches whose contraction (7168) exceeds the output
// width (2048) and costs 4-6% on the reverse shapes, which keep one launch.
constexpr int kSplitRows = 384;

// Largest group count a gmm tile variant supports: the 128-row variant
// keeps its LDS (three stages + two group prefixes) within half a CU.
constexpr int kMaxGShort = 1000;
template <int TM>
struct MaxG {
  static constexpr int value = TM <= 128 ? kMaxGShort : kMaxG;
};

template <bool B_COLK, int TM, int TN, typename TO, bool PAIR, bool SWI = false, bool SWB = false>
__global__ __launch_bounds__(NT, TM <= 128 ? 2 : 1) void gmm_mfma_kernel(MfmaArgs a) {
  static_assert(!SWI || (B_COLK && TN == 256 && std::is_same<TO, bf16_t>::value),
                "the SwiGLU epilogue takes a [K, 2F] rhs and bf16 outputs");
  static_assert(!SWB || (!SWI && std::is_same<TO, bf16_t>::value),
                "the SwiGLU-backward epilogue writes bf16 d_h0, d_h1");
  static_assert(!PAIR || Stages<TM, TN>::NS == 4, "pair loading uses the four-step ring");
  using OA = std::conditional_t<PAIR, PairRow<TM>, Operand<false, TM>>;
  // the rhs keeps single-step units even in the pair pipeline: a transposed
  // rhs in 128-byte pair units ran 7% slower on the Mixtral-8x7B shape
  using OB = Operand<B_COLK, TN>;
  __shared__ __attribute__((aligned(1024))) char smem[Stages<TM, TN>::kBytes];
  __shared__ int row_base[MaxG<TM>::value + 1];
  __shared__ int tile_base[MaxG<TM>::value + 1];
  const int ntn = static_cast<int>((a.N + TN - 1) / TN);
  scan_groups(a.gsz, a.G, a.M, TM, ntn, row_base, tile_base, blockIdx.x == 0 ? a.err : nullptr,
              a.cls_lo, a.cls_hi);
  __syncthreads();
  const int total = tile_base[a.G];
  TO* out = static_cast<TO*>(a.out);
  OA A;
  OB B;
  Acc<TM, TN> acc;
  uint32_t fa[4], fb[4];
  OA::frag_base(((threadIdx.x >> 6) >> 1) * (TM / 2), fa);
  OB::frag_base(((threadIdx.x >> 6) & 1) * (TN / 2), fb);
  for (int it = 0;; ++it) {
    const int64_t tile = xcd_tile(it);
    if (tile >= total) break;
    int lo = 0, hi = a.G - 1;   // largest g with tile_base[g] <= tile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int rows_g = row_base[g + 1] - row_base[g];
    const int mtiles = (rows_g + TM - 1) / TM;
    const int local = static_cast<int>(tile - tile_base[g]);
    int mt, nt;
    blocked_tile(local, mtiles, ntn, mt, nt);
    const int64_t row0 = row_base[g] + static_cast<int64_t>(mt) * TM;
    const int rv = min(TM, rows_g - mt * TM);
    const int64_t col0 = static_cast<int64_t>(nt) * TN;
    const int cv = static_cast<int>(lmin(TN, a.N - col0));
    // rows past the group's valid rows are zero in lhs: not loaded (the
    // DMA re-reads the last loaded row), and their products written as zero
    const int vr = a.valid ? max(0, min(rv, min(rows_g, max(a.valid[g], 0)) - mt * TM)) : rv;
    acc.set_live_rows(vr);
    A.setup(a.lhs + row0 * a.ld_lhs, a.ld_lhs, max(vr, 1));
    const bf16_t* bg = a.rhs + g * a.rhs_gs;
    if constexpr (SWI) {
      // d_ff columns f0 .. f0 + TN/2 of wi's gate half and of its up half
      // (F further), in 64-wide blocks alternating gate and up
      const int64_t F = a.N / 2, f0 = static_cast<int64_t>(nt) * (TN / 2);
      B.setup(bg + f0, a.ld_rhs, TN, F);
      if constexpr (PAIR) contract2(smem, A, B, a.Kdim, acc, fa, fb);
      else contract<Stages<TM, TN>::NS>(smem, A, B, a.Kdim, acc, fa, fb);
      bf16_t* h = static_cast<bf16_t*>(a.out);
      const bf16_t* bb = a.bias ? a.bias + g * a.N : nullptr;
      store_tile_swiglu(acc, smem, h ? h + row0 * a.ld_out + f0 : nullptr,
                        h ? h + row0 * a.ld_out + F + f0 : nullptr, a.ld_out,
                        a.act + row0 * a.ld_act + f0, a.ld_act, rv, bb ? bb + f0 : nullptr,
                        bb ? bb + F + f0 : nullptr, vr);
    } else {
      B.setup(B_COLK ? bg + col0 : bg + col0 * a.ld_rhs, a.ld_rhs, cv);
      if constexpr (PAIR) contract2(smem, A, B, a.Kdim, acc, fa, fb);
      else contract<Stages<TM, TN>::NS>(smem, A, B, a.Kdim, acc, fa, fb);
      if constexpr (SWB)
        store_tile_swiglu_bwd(acc, smem, out + row0 * a.ld_out + col0,
                              a.dh1 + row0 * a.ld_out + col0, a.ld_out,
                              a.h0 + row0 * a.ld_h + col0, a.h1 + row0 * a.ld_h + col0, a.ld_h,
                              rv, cv, vr);
      else
        store_tile(acc, smem, out + row0 * a.ld_out + col0, a.ld_out, rv, cv, a.accumulate,
                   a.bias ? a.bias + g * a.N + col0 : nullptr, 1.f, vr);
    }
  }
  if (a.cls_lo > 0) return;   // the launch of the small-group class zeroes the rest
  if constexpr (SWI) {
    if (out) zero_rows(out, a.ld_out, a.N, row_base[a.G], a.M);
    zero_rows(a.act, a.ld_act, a.N / 2, row_base[a.G], a.M);
  } else if constexpr (SWB) {
    zero_rows(out, a.ld_out, a.N, row_base[a.G], a.M);
    zero_rows(a.dh1, a.ld_out, a.N, row_base[a.G], a.M);
  } else {
    if (!a.accumulate) zero_rows(out, a.ld_out, a.N, row_base[a.G], a.M);
  }
}

// Rows of group g that the weight-gradient contraction covers: its rows
// (clipped to the buffer), or the first valid[g] of them.
__device__ __forceinline__ int tgmm_rows(const MfmaArgs& a, const int* row_base, int g) {
  const int n = row_base[g + 1] - row_base[g];
  return a.valid ? min(n, max(a.valid[g], 0)) : n;
}

// After scan_groups has filled row_base: wave 0 writes unit_base[g] = units
// of the groups before g, where a group owns `per` units when its
// contraction rows (tgmm_rows) lie in [lo, hi], else none.
__device__ inline void scan_class_units(const MfmaArgs& a, const int* row_base, int lo, int hi,
                                        int per, int* unit_base) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int run = 0;
  for (int g0 = 0; g0 < a.G; g0 += 64) {
    const int g = g0 + lane;
    int u = 0;
    if (g < a.G) {
      const int v = tgmm_rows(a, row_base, g);
      u = (v >= lo && v <= hi) ? per : 0;
    }
    int incl = u;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (g < a.G) unit_base[g] = run + incl - u;
    run += __shfl(incl, 63, 64);
  }
  if (lane == 0) unit_base[a.G] = run;
}

// Largest g with unit_base[g] <= u (unit_base non-decreasing, u < unit_base[G]).
__device__ __forceinline__ int find_group(const int* unit_base, int G, int64_t u) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (unit_base[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The tiles listed in tile_base (the groups' tiles one after another, TM x
// TN tiles of [Kdim, N] in column blocks) for workgroup b of nwg:
// out[g] tile = lhs[rows of g, tile rows]^T . rhs[rows of g, tile columns].
template <int TM, int TN, typename TO>
__device__ __forceinline__ void tgmm_tile_loop(const MfmaArgs& a, char* smem, const int* row_base,
                                               const int* tile_base, int b, int nwg) {
  const int mtn = static_cast<int>((a.Kdim + TM - 1) / TM);
  const int ntn = static_cast<int>((a.N + TN - 1) / TN);
  const int64_t total = tile_base[a.G];
  TO* out = static_cast<TO*>(a.out);
  Operand<true, TM> A;
  Operand<true, TN> B;
  Acc<TM, TN> acc;
  uint32_t fa[4], fb[4];
  Operand<true, TM>::frag_base(((threadIdx.x >> 6) >> 1) * (TM / 2), fa);
  Operand<true, TN>::frag_base(((threadIdx.x >> 6) & 1) * (TN / 2), fb);
  for (int it = 0;; ++it) {
    const int64_t tile = xcd_index(it, b, nwg);
    if (tile >= total) break;
    const int g = find_group(tile_base, a.G, tile);
    const int local = static_cast<int>(tile - tile_base[g]);
    int mt, nt;
    blocked_tile(local, mtn, ntn, mt, nt);
    const int64_t r0 = row_base[g];
    const int rows_g = tgmm_rows(a, row_base, g);   // the rest is zero
    if (rows_g == 0 && a.accumulate) continue;   // partial sum unchanged
    const int64_t m0 = static_cast<int64_t>(mt) * TM, n0 = static_cast<int64_t>(nt) * TN;
    const int mv = static_cast<int>(lmin(TM, a.Kdim - m0));
    const int nv = static_cast<int>(lmin(TN, a.N - n0));
    A.setup(a.lhs + r0 * a.ld_lhs + m0, a.ld_lhs, mv);
    B.setup(a.rhs + r0 * a.ld_rhs + n0, a.ld_rhs, nv);
    contract<Stages<TM, TN>::NS>(smem, A, B, rows_g, acc, fa, fb);
    store_tile(acc, smem, out + g * a.out_gs + m0 * a.ld_out + n0, a.ld_out, mv, nv,
               a.accumulate);
  }
}

// Transposed grouped GEMM over the groups whose contraction rows lie in
// [cls_lo, cls_hi] (all groups by default), every workgroup taking tiles.
template <int TM, int TN, typename TO>
__global__ __launch_bounds__(NT, TM <= 128 ? 2 : 1) void tgmm_mfma_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Stages<TM, TN>::kBytes];
  __shared__ int row_base[MaxG<TM>::value + 1];
  __shared__ int tile_base[MaxG<TM>::value + 1];
  scan_groups(a.gsz, a.G, a.M, TM, 1, row_base, nullptr, blockIdx.x == 0 ? a.err : nullptr);
  __syncthreads();
  const int per = static_cast<int>(((a.Kdim + TM - 1) / TM) * ((a.N + TN - 1) / TN));
  scan_class_units(a, row_base, a.cls_lo, a.cls_hi, per, tile_base);
  __syncthreads();
  tgmm_tile_loop<TM, TN, TO>(a, smem, row_base, tile_base, blockIdx.x, gridDim.x);
}

// Write a 128 x 256 accumulator tile as store_tile does, staging 16-row
// halves of each wave's 32-row slabs (half the LDS of store_tile: 4 x 16 x
// 528 bytes), so that the staging area fits beside the short loop's
// resident operand strip.  rows >= rv and columns >= cv are skipped.  Each
// wave stages in its own region; SYNC ends with a workgroup barrier.
template <typename TO, bool SYNC = true>
__device__ __forceinline__ void store_tile_halves(const Acc<128, 256>& acc, char* lds, TO* o,
                                                  int64_t ldo, int rv, int cv, int accumulate) {
  constexpr int TM = 128, TN = 256;
  constexpr int WC = TN / 2;
  constexpr int SROW = WC * 4 + 16;
  constexpr int CPR = WC / 8;                 // 8-column chunks per staged row
  constexpr int NQ = 16 * CPR / 64;           // chunks per lane per half slab
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* slab = lds + w * 16 * SROW;
  const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * WC;
  const bool plain = !accumulate && wr + TM / 2 <= rv && wc + WC <= cv;
#pragma unroll
  for (int i = 0; i < Acc<TM, TN>::FM; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // accumulator entries r of this half: rows 8 (r >> 2) + 4 (lane / 32) + (r & 3) - 16 h
#pragma unroll
      for (int j = 0; j < Acc<TM, TN>::FN; ++j)
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r) {
          const int row = 8 * ((r >> 2) & 1) + 4 * (lane >> 5) + (r & 3);
          const int col = 32 * j + (lane & 31);
          *reinterpret_cast<float*>(slab + row * SROW + col * 4) = acc.v[i][j][r];
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float4 lo[NQ], hi[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int chunk = lane + 64 * q;
        const int row = chunk / CPR, c8 = chunk % CPR;
        lo[q] = *reinterpret_cast<const float4*>(slab + row * SROW + c8 * 32);
        hi[q] = *reinterpret_cast<const float4*>(slab + row * SROW + c8 * 32 + 16);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int chunk = lane + 64 * q;
        const int row = chunk / CPR, c8 = chunk % CPR;
        const int grow = wr + 32 * i + 16 * h + row, gcol = wc + 8 * c8;
        float v[8] = {lo[q].x, lo[q].y, lo[q].z, lo[q].w, hi[q].x, hi[q].y, hi[q].z, hi[q].w};
        TO* p = o + static_cast<int64_t>(grow) * ldo + gcol;
        if (plain) {
          store8_nt(p, v);
        } else if (grow < rv && gcol < cv) {
          if (accumulate) {
            float old[8];
            load8(p, old);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += old[e];
            store8(p, v);
          } else {
            store8_nt(p, v);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  if (SYNC) __syncthreads();   // the staging area may be refilled by the next tile's operand
}

// Weight gradients of groups whose contraction is short (at most
// kShortRows = one step of rows): such a tile holds one MFMA step and 64 KB
// of output, so tile by tile its time is the operand load latency plus the
// output stores, and on gfx9 a wait for a load also waits for the stores
// issued before it.  Here a workgroup takes a unit = (group g, 256-column
// strip of N), or one of up to four runs of its consecutive tiles:
//   * the strip of rhs (the group's rows x 256 columns, zero past them) is
//     loaded into LDS once and stays there for the whole unit (run);
//   * the unit's 128-row tiles of Kdim run in order; the lhs block of tile
//     t + 1 (32 rows x 128) is copied global -> LDS into the other half of a
//     double buffer while tile t is contracted and stored, and tile t + 1
//     waits only for that copy: the wait leaves tile t's stores (issued
//     after the copy) in flight, so the stores of one tile overlap the next;
//   * the output leaves through half-slab staging in its own LDS region.
// Operand traffic is one rhs strip per unit and one lhs block per tile
// instead of both per tile.  lhs rows past the group's rows are not zeroed
// in LDS: the copy repeats the last row there, and the zero rhs rows cancel
// them.  Groups with no rows write zero blocks (or keep the partial sum).
// Units are listed in unit_base (ntn per group).
// Runs a unit's mtn tiles are taken in, by different workgroups of the
// persistent grid of nwg: with units a few times the grid, whole units leave
// the last round part-empty (1264 units on 512 workgroups: three rounds of
// work for 2.47).  The run count (1 .. 4, at most mtn) minimises rounds /
// runs, a unit's length in rounds, with 2% of a unit charged per extra run
// for its second rhs strip load and pipeline start.
__device__ __forceinline__ int unit_runs(int64_t units, int nwg, int mtn) {
  int parts = 1;
  int64_t best = (units + nwg - 1) / nwg * 100;
  for (int p = 2; p <= 4 && p <= mtn; ++p) {
    const int64_t c = (units * p + nwg - 1) / nwg * 100 / p + 2 * (p - 1);
    if (c < best) {
      best = c;
      parts = p;
    }
  }
  return parts;
}

constexpr int kShortRows = TK;
constexpr int kShortB = 256 * TK * 2;                        // resident rhs strip
constexpr int kShortA = 128 * TK * 2;                        // one lhs block
constexpr int kShortStage = 4 * 16 * (128 * 4 + 16);         // half-slab output staging
constexpr int kShortBytes = kShortB + 2 * kShortA + kShortStage;

// global_load_lds offsets of one 32-row x 128-column lhs block (a col tile
// of Operand<true, 128>'s layout) whose rows past kv repeat row kv - 1.
struct ShortLhs {
  static constexpr int BX = 128;
  static constexpr int NJ = Operand<true, BX>::NJ;
  uint32_t voff[NJ];
  __device__ __forceinline__ void setup(int64_t ld, int xv, int kv) {
    const int tid = opaque_tid();
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int byte = (w * NJ + j) * 1024 + lane * 16;
      const int k = byte / (BX * 2);
      int c = ((byte % (BX * 2)) >> 4) ^ col_swz(k);
      const int cmax = (xv - 1) >> 3;
      if (c > cmax) c = cmax;
      voff[j] = static_cast<uint32_t>(((k < kv ? k : kv - 1) * ld + c * 8) * 2);
    }
  }
  __device__ __forceinline__ void dma(const bf16_t* base, uint32_t lds) const {
    const void* sb = uniform_ptr(base);
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < NJ; ++j) dma16(sb, voff[j], lds + (w * NJ + j) * 1024);
  }
};

template <typename TO>
__device__ __forceinline__ void tgmm_short_loop(const MfmaArgs& a, char* smem, const int* row_base,
                                                const int* unit_base, int b, int nwg) {
  constexpr int TM = 128, TN = 256;
  using OA = Operand<true, TM>;
  using OB = Operand<true, TN>;
  // vector-memory instructions per wave of a plain (in-bounds, no partial
  // sum) output tile: 16 eight-element chunks per lane, one 16-byte store
  // each for bf16, two for float32
  constexpr int kStores = 16 * (sizeof(TO) == 2 ? 1 : 2);
  char* const Bs = smem;
  char* const As = smem + kShortB;                // two lhs blocks
  char* const Ss = smem + kShortB + 2 * kShortA;  // output staging
  const int mtn = static_cast<int>((a.Kdim + TM - 1) / TM);
  const int ntn = static_cast<int>((a.N + TN - 1) / TN);
  const int64_t units = unit_base[a.G];
  const int parts = unit_runs(units, nwg, mtn);
  const int64_t total = units * parts;
  TO* out = static_cast<TO*>(a.out);
  OB B;
  ShortLhs A;
  Acc<TM, TN> acc;
  uint32_t fa[4], fb[4];
  OA::frag_base(((threadIdx.x >> 6) >> 1) * (TM / 2), fa);
  OB::frag_base(((threadIdx.x >> 6) & 1) * (TN / 2), fb);
  for (int it = 0;; ++it) {
    const int64_t vunit = xcd_index(it, b, nwg);
    if (vunit >= total) break;
    const int64_t unit = vunit / parts;   // the parts of a unit are adjacent: one XCD
    const int part = static_cast<int>(vunit - unit * parts);
    const int mt_lo = part * mtn / parts, mt_hi = (part + 1) * mtn / parts;
    const int g = find_group(unit_base, a.G, unit);
    const int nt = static_cast<int>(unit - unit_base[g]);
    const int64_t r0 = row_base[g];
    const int rows_g = min(tgmm_rows(a, row_base, g), kShortRows);
    if (rows_g == 0 && a.accumulate) continue;   // partial sums unchanged
    const int64_t n0 = static_cast<int64_t>(nt) * TN;
    const int nv = static_cast<int>(lmin(TN, a.N - n0));
    const bf16_t* lhs_g = a.lhs + r0 * a.ld_lhs;
    // every wave is done with the previous unit's LDS (its last tile ended
    // with a barrier before the epilogue); the copies of the previous unit
    // have all landed (each tile waited for its own)
    if (rows_g > 0) {
      B.setup(a.rhs + r0 * a.ld_rhs + n0, a.ld_rhs, nv);
      uint4 t[OB::NR];
      B.tail_load(0, rows_g, t);
      B.tail_store(Bs, t);
      const int64_t mlo = static_cast<int64_t>(mt_lo) * TM;
      A.setup(a.ld_lhs, static_cast<int>(lmin(TM, a.Kdim - mlo)), rows_g);
      A.dma(lhs_g + mlo, lds_addr(As));
    }
    bool drain = true;   // the wait below must also cover the previous stores
    for (int mt = mt_lo; mt < mt_hi; ++mt) {
      const int64_t m0 = static_cast<int64_t>(mt) * TM;
      const int mv = static_cast<int>(lmin(TM, a.Kdim - m0));
      char* const cur = As + ((mt - mt_lo) & 1) * kShortA;
      if (rows_g > 0) {
        // this tile's lhs block: everything issued after its copy is the
        // previous tile's stores, which may stay in flight
        if (drain) wait_vmcnt<0>(); else wait_vmcnt<kStores>();
      }
      __syncthreads();
      if (rows_g > 0 && mt + 1 < mt_hi) {
        // the next block into the other half (read by tile mt - 1, whose
        // fragment reads all waves finished before its epilogue)
        A.setup(a.ld_lhs, static_cast<int>(lmin(TM, a.Kdim - m0 - TM)), rows_g);
        A.dma(lhs_g + m0 + TM, lds_addr(As + ((mt + 1 - mt_lo) & 1) * kShortA));
      }
      acc.zero();
      if (rows_g > 0) {
        typename Acc<TM, TN>::Frags f;
        Acc<TM, TN>::template load<OA, OB>(f, cur, Bs, fa, fb, 0);
        acc.mma(f);
        Acc<TM, TN>::template load<OA, OB>(f, cur, Bs, fa, fb, 1);
        acc.mma(f);
      }
      // a plain epilogue issues exactly kStores vector-memory instructions
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      drain = a.accumulate || (w >> 1) * (TM / 2) + TM / 2 > mv || (w & 1) * (TN / 2) + TN / 2 > nv;
      store_tile_halves<TO, false>(acc, Ss, out + g * a.out_gs + m0 * a.ld_out + n0, a.ld_out, mv,
                                   nv, a.accumulate);
    }
    __syncthreads();   // the unit's LDS is refilled by the next unit
  }
}

// Weight gradients of the groups with at most kShortRows contraction rows
// (cls_lo .. cls_hi), every workgroup taking units (tgmm_short_loop).
template <typename TO>
__global__ __launch_bounds__(NT, 2) void tgmm_short_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kShortBytes];
  __shared__ int row_base[kMaxGShort + 1];
  __shared__ int unit_base[kMaxGShort + 1];
  scan_groups(a.gsz, a.G, a.M, 128, 1, row_base, nullptr, blockIdx.x == 0 ? a.err : nullptr);
  __syncthreads();
  scan_class_units(a, row_base, a.cls_lo, min(a.cls_hi, kShortRows),
                   static_cast<int>((a.N + 255) / 256), unit_base);
  __syncthreads();
  tgmm_short_loop<TO>(a, smem, row_base, unit_base, blockIdx.x, gridDim.x);
}

// Weight gradients of groups whose contraction takes S steps (S = 2: 33 ..
// 64 rows, S = 4: 65 .. 128 rows): the short kernel's scheme with a
// resident rhs strip of S steps, where the output staging has no LDS of its
// own.  Per unit (group, 256-column strip, or a run of its tiles):
//   * the rhs strip (the group's rows x 256, zero past them) goes into LDS
//     through registers once;
//   * the lhs block of each 128-row tile of Kdim (S steps of 32 rows x 128,
//     rows past the group's repeating its last row, which the zero strip
//     rows cancel) is copied global -> LDS one tile ahead, into the other
//     half of a double buffer;
//   * once every wave has read its fragments of a tile's block, the block is
//     free and the tile's epilogue stages its output there, each wave in
//     its own quarter; the next tile's block is already in the other half,
//     so its wait leaves the stores of this tile in flight (they are the
//     youngest vector-memory instructions of the wave).
// LDS: S = 2: 32 KB strip + 2 x 16 KB blocks, two workgroups per CU;
// S = 4: 64 KB + 2 x 32 KB, one workgroup per CU.
template <int S>
struct Strip {
  static constexpr int kStepB = 256 * TK * 2;     // one strip step (32 rows x 256)
  static constexpr int kStepA = 128 * TK * 2;     // one lhs block step (32 rows x 128)
  static constexpr int kB = S * kStepB;
  static constexpr int kA = S * kStepA;
  static constexpr int kBytes = kB + 2 * kA;
  static constexpr int kWaveStage = kA / 4;       // a wave's staging bytes in a free block
  static constexpr int kRows = kWaveStage / 512;  // float32 rows of 128 columns per staging round
};

// Write a 128 x 256 accumulator tile through a wave's own staging region of
// ROWS x 128 float32 (unpadded 512-byte rows; in rows with bit 2 set the
// 8-column chunks are swapped with the ones 32 columns away, so the two
// half-waves of a write, 4 rows apart, hit different banks).  rows >= rv
// and columns >= cv are skipped.  No workgroup barrier: the region is the
// wave's alone until the caller's next barrier.
template <typename TO, int ROWS>
__device__ __forceinline__ void store_tile_staged(const Acc<128, 256>& acc, char* region, TO* o,
                                                  int64_t ldo, int rv, int cv, int accumulate) {
  constexpr int TM = 128, WC = 128;
  constexpr int CPR = WC / 8;                 // 8-column chunks per staged row
  constexpr int NQ = ROWS * CPR / 64;         // chunks per lane per round
  constexpr int RPS = 32 / ROWS;              // rounds per 32-row slab
  static_assert(ROWS == 8 || ROWS == 16, "staging rounds of 8 or 16 rows");
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * WC;
  const bool plain = !accumulate && wr + TM / 2 <= rv && wc + WC <= cv;
#pragma unroll
  for (int i = 0; i < Acc<TM, 256>::FM; ++i)
#pragma unroll
    for (int h = 0; h < RPS; ++h) {
      // entries r of this round: rows 8 (r >> 2) + 4 (lane / 32) + (r & 3) - ROWS h
#pragma unroll
      for (int j = 0; j < Acc<TM, 256>::FN; ++j)
#pragma unroll
        for (int r = ROWS / 2 * h; r < ROWS / 2 * (h + 1); ++r) {
          const int row = 8 * ((r >> 2) - ROWS / 8 * h) + 4 * (lane >> 5) + (r & 3);
          const int col = (32 * j + (lane & 31)) ^ (row & 4 ? 32 : 0);
          *reinterpret_cast<float*>(region + row * 512 + col * 4) = acc.v[i][j][r];
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float4 lo[NQ], hi[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int chunk = lane + 64 * q;
        const int row = chunk / CPR, c8 = (chunk % CPR) ^ (row & 4 ? 4 : 0);
        lo[q] = *reinterpret_cast<const float4*>(region + row * 512 + c8 * 32);
        hi[q] = *reinterpret_cast<const float4*>(region + row * 512 + c8 * 32 + 16);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int chunk = lane + 64 * q;
        const int row = chunk / CPR, c8 = chunk % CPR;
        const int grow = wr + 32 * i + ROWS * h + row, gcol = wc + 8 * c8;
        float v[8] = {lo[q].x, lo[q].y, lo[q].z, lo[q].w, hi[q].x, hi[q].y, hi[q].z, hi[q].w};
        TO* p = o + static_cast<int64_t>(grow) * ldo + gcol;
        if (plain) {
          store8_nt(p, v);
        } else if (grow < rv && gcol < cv) {
          if (accumulate) {
            float old[8];
            load8(p, old);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += old[e];
            store8(p, v);
          } else {
            store8_nt(p, v);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

template <int S, typename TO>
__device__ __forceinline__ void tgmm_strip_loop(const MfmaArgs& a, char* smem, const int* row_base,
                                                const int* unit_base, int b, int nwg) {
  constexpr int TM = 128, TN = 256;
  using OA = Operand<true, TM>;
  using OB = Operand<true, TN>;
  using C = Strip<S>;
  // vector-memory instructions per wave of a plain output tile (as in the
  // short kernel)
  constexpr int kStores = 16 * (sizeof(TO) == 2 ? 1 : 2);
  char* const Bs = smem;
  char* const As = smem + C::kB;                  // two lhs blocks
  const int mtn = static_cast<int>((a.Kdim + TM - 1) / TM);
  const int ntn = static_cast<int>((a.N + TN - 1) / TN);
  const int64_t units = unit_base[a.G];
  const int parts = unit_runs(units, nwg, mtn);
  const int64_t total = units * parts;
  TO* out = static_cast<TO*>(a.out);
  OB B;
  ShortLhs A;
  Acc<TM, TN> acc;
  uint32_t fa[4], fb[4];
  OA::frag_base(((threadIdx.x >> 6) >> 1) * (TM / 2), fa);
  OB::frag_base(((threadIdx.x >> 6) & 1) * (TN / 2), fb);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int it = 0;; ++it) {
    const int64_t vunit = xcd_index(it, b, nwg);
    if (vunit >= total) break;
    const int64_t unit = vunit / parts;
    const int part = static_cast<int>(vunit - unit * parts);
    const int mt_lo = part * mtn / parts, mt_hi = (part + 1) * mtn / parts;
    const int g = find_group(unit_base, a.G, unit);
    const int nt = static_cast<int>(unit - unit_base[g]);
    const int64_t r0 = row_base[g];
    // the class holds groups of more than 32 (S / 2) rows: every step up
    // to ns has rows, and steps past ns are neither loaded nor multiplied
    const int rows_g = min(tgmm_rows(a, row_base, g), TK * S);
    const int ns = (rows_g + TK - 1) / TK;
    const int64_t n0 = static_cast<int64_t>(nt) * TN;
    const int nv = static_cast<int>(lmin(TN, a.N - n0));
    const bf16_t* lhs_g = a.lhs + r0 * a.ld_lhs;
    // every wave is done with the previous unit's LDS (barrier at its end)
    B.setup(a.rhs + r0 * a.ld_rhs + n0, a.ld_rhs, nv);
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < ns) {
        uint4 t[OB::NR];
        B.tail_load(s, rows_g - TK * s, t);
        B.tail_store(Bs + s * C::kStepB, t);
      }
    auto copy_block = [&](int mt, char* dst) {
      const int64_t m0 = static_cast<int64_t>(mt) * TM;
      const int mv = static_cast<int>(lmin(TM, a.Kdim - m0));
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (s < ns) {
          A.setup(a.ld_lhs, mv, min(TK, rows_g - TK * s));
          A.dma(lhs_g + static_cast<int64_t>(TK) * s * a.ld_lhs + m0,
                lds_addr(dst + s * C::kStepA));
        }
    };
    copy_block(mt_lo, As);
    bool drain = true;   // the wait below must also cover the previous stores
    for (int mt = mt_lo; mt < mt_hi; ++mt) {
      const int64_t m0 = static_cast<int64_t>(mt) * TM;
      const int mv = static_cast<int>(lmin(TM, a.Kdim - m0));
      char* const cur = As + ((mt - mt_lo) & 1) * C::kA;
      // this tile's block: everything issued after its copy is the previous
      // tile's stores, which may stay in flight
      if (drain) wait_vmcnt<0>(); else wait_vmcnt<kStores>();
      __syncthreads();   // the block (and strip) visible; the other half's staging done
      if (mt + 1 < mt_hi) copy_block(mt + 1, As + ((mt + 1 - mt_lo) & 1) * C::kA);
      acc.zero();
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (s < ns) {
          typename Acc<TM, TN>::Frags f;
          Acc<TM, TN>::template load<OA, OB>(f, cur + s * C::kStepA, Bs + s * C::kStepB, fa, fb, 0);
          acc.mma(f);
          Acc<TM, TN>::template load<OA, OB>(f, cur + s * C::kStepA, Bs + s * C::kStepB, fa, fb, 1);
          acc.mma(f);
        }
      __syncthreads();   // every wave has its fragments: the block becomes staging
      // a plain epilogue issues exactly kStores vector-memory instructions
      drain = a.accumulate || (w >> 1) * (TM / 2) + TM / 2 > mv || (w & 1) * (TN / 2) + TN / 2 > nv;
      store_tile_staged<TO, C::kRows>(acc, cur + w * C::kWaveStage,
                                      out + g * a.out_gs + m0 * a.ld_out + n0, a.ld_out, mv, nv,
                                      a.accumulate);
    }
    __syncthreads();   // the unit's LDS is refilled by the next unit
  }
}

// Weight gradients of the groups with 32 S / 2 + 1 .. 32 S contraction rows
// (cls_lo .. cls_hi), every workgroup taking units (tgmm_strip_loop).
template <int S, typename TO>
__global__ __launch_bounds__(NT, S <= 2 ? 2 : 1) void tgmm_strip_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[Strip<S>::kBytes];
  __shared__ int row_base[kMaxGShort + 1];
  __shared__ int unit_base[kMaxGShort + 1];
  scan_groups(a.gsz, a.G, a.M, 128, 1, row_base, nullptr, nullptr);
  __syncthreads();
  scan_class_units(a, row_base, max(a.cls_lo, TK * S / 2 + 1), min(a.cls_hi, TK * S),
                   static_cast<int>((a.N + 255) / 256), unit_base);
  __syncthreads();
  tgmm_strip_loop<S, TO>(a, smem, row_base, unit_base, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- fp8 MFMA
//
// FP8 operands (the quantization=fp8 run of the MaxText grouped-GEMM pull
// request: e4m3 forward, e5m2 backward, current scaling) on
// v_mfma_f32_32x32x64_f8f6f4: both operands contraction-contiguous (the
// quantizer writes the transposed copy each GEMM needs), so both are "row"
// tiles.  A contraction step is the same 64-byte row segment as a bf16 step
// and reuses its LDS layout, DMA and fragment reads: the 64 FP8 values of a
// step are viewed as 32 two-byte units.  One MFMA consumes both 16-byte
// fragments (substeps 0 and 1) of a step; A and B use the same byte-to-k
// assignment, so the products pair up correctly.  Each step waits for its
// data, reads all fragments, then runs its MFMAs with the DMA of a later
// step spread between them.  Two tile shapes, chosen per launch like the
// bf16 ones: 256 x 256 with a four-step ring and one workgroup per CU when groups
// hold 512 rows or more on average (contraction rows for the tgmm), else
// 128 x 256 with a three-step ring and two workgroups per CU.  The epilogue
// multiplies by the two operands' scale_inv (per tensor, or per expert for
// the weights).
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4v __attribute__((ext_vector_type(4)));

template <int TM, int TN, int FA, int FB>
struct Acc8 : Acc<TM, TN> {
  using Base = Acc<TM, TN>;
  struct Frags8 {
    i32x8 a[Base::FM], b[Base::FN];
  };
  template <class O>
  __device__ __forceinline__ static i32x8 frag8(const char* lds, const uint32_t (&fb)[4], int i) {
    const i32x4v lo = __builtin_bit_cast(i32x4v, O::frag(lds, fb, i, 0));
    const i32x4v hi = __builtin_bit_cast(i32x4v, O::frag(lds, fb, i, 1));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ __forceinline__ void mma8(const Frags8& f, int q) {
    const int i = q / Base::FN, j = q % Base::FN;
    if (!Base::kSkip || i < this->live)
      this->v[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], this->v[i][j],
                                                                     FA, FB, 0, 0, 0, 0);
  }
};

struct Fp8Args {
  const bf16_t* lhs;     // FP8 bytes viewed as two-byte units
  int64_t ld_lhs;        // in units
  const bf16_t* rhs;
  int64_t ld_rhs;
  int64_t rhs_gs;        // gmm: rhs group stride (units)
  const int32_t* gsz;
  const int32_t* valid;  // tgmm: rows of each group that may be non-zero (or null)
  int G;
  int64_t M;             // gmm: output rows; tgmm: rows of the grouped buffers
  int64_t Kdim;          // gmm: contraction (units); tgmm: output rows per group
  int64_t N;
  void* out;
  int64_t ld_out;
  int64_t out_gs;
  int accumulate;
  int32_t* err;
  const float* sinv_a;   // [1]
  const float* sinv_b;   // gmm: [G] (per expert); tgmm: [1]
  const bf16_t* bias;    // gmm: [G, N] or null
};

// A contraction-major FP8 operand of BX = 256 columns: element (x, k) at
// byte k * ld + x of the source (a [K, N] weight as stored), one step = 64
// contraction rows.  LDS rows of 256 bytes; the 16-byte chunk c of row k sits
// at position c ^ 2 (k & 7).  A transposing read (ds_read_b64_tr_b8) lets
// each 16-lane group address an 8-row x 16-byte block (lane 2 r + q: row r,
// bytes 8 q .. 8 q + 7) and gives lane j the bytes of column j for rows
// 0..7, in row order.  The 32 lanes of a half-wave read the same 8 rows of
// 32 columns, two chunks per row, which the swizzle places on 16 distinct
// chunk positions (all 64 banks).  Fragment (i, s) of lane l: column
// xw + 32 i + l % 32, contraction rows 32 s + 16 (l / 32) + 0..15 in order,
// the bytes a row-tile fragment holds for the same k, so the two layouts
// feed one MFMA.  Columns past the valid extent are clamped to the last
// valid chunk (their products land in columns that are never stored); the
// chunk holding column xv - 1 is read whole, which stays inside the row's
// ld bytes because ld is a multiple of 16.
template <int BX>
struct F8Col {
  static_assert(BX == 256, "the swizzle spans 16 chunk positions");
  static constexpr int kBytes = BX * TK * 2;      // 64 rows x BX bytes
  static constexpr int NJ = kBytes / 1024 / 4;    // DMA instructions per wave per stage
  static constexpr int NR = kBytes / 16 / NT;     // register path: chunks per thread
  static constexpr int CPR = BX / 16;             // chunks per row
  const bf16_t* base;     // FP8 bytes in two-byte units
  int64_t ld;             // row stride in units
  int xv;                 // valid columns (>= 1)
  uint32_t voff[NJ];

  __device__ __forceinline__ static int swz(int k) { return (k & 7) << 1; }
  __device__ __forceinline__ void setup(const bf16_t* b, int64_t ld_, int xv_) {
    base = b;
    ld = ld_;
    xv = xv_;
    const int tid = opaque_tid();
    const int lane = tid & 63, w = tid >> 6;
    const int cmax = (xv - 1) >> 4;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int byte = (w * NJ + j) * 1024 + lane * 16;
      const int k = byte / BX;
      int c = ((byte % BX) >> 4) ^ swz(k);
      if (c > cmax) c = cmax;
      voff[j] = static_cast<uint32_t>(k * ld * 2 + c * 16);
    }
  }
  __device__ __forceinline__ const bf16_t* step_base(int kt) const {
    return base + static_cast<int64_t>(kt) * (2 * TK) * ld;
  }
  __device__ __forceinline__ void dma_one(const void* sb, int j, uint32_t lds) const {
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    dma16(sb, voff[j], lds + (w * NJ + j) * 1024);
  }
  __device__ __forceinline__ void dma(int kt, uint32_t lds) const {
    const void* sb = uniform_ptr(step_base(kt));
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < NJ; ++j) dma16(sb, voff[j], lds + (w * NJ + j) * 1024);
  }
  // Register path for a partial step of kv < TK units (2 kv contraction rows).
  __device__ __forceinline__ void tail_load(int kt, int kv, uint4 (&r)[NR]) const {
    const char* b = reinterpret_cast<const char*>(step_base(kt));
    const int tid = opaque_tid();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = tid + i * NT;
      const int k = q / CPR, c = q % CPR;
      const bool ok = k < 2 * kv && c * 16 < xv;
      const char* p = b + static_cast<int64_t>(k) * ld * 2 + c * 16;
      r[i] = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void tail_store(char* lds, const uint4 (&r)[NR]) const {
    const int tid = opaque_tid();
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = tid + i * NT;
      const int k = q / CPR, c = q % CPR;
      *reinterpret_cast<uint4*>(lds + k * BX + ((c ^ swz(k)) << 4)) = r[i];
    }
  }
  __device__ __forceinline__ static void frag_base(int xw, uint32_t (&fb)[4]) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j = lane & 15;
    const int r = j >> 1, q = j & 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = (xw + 32 * t + 16 * (g & 1)) >> 4;
      fb[t] = static_cast<uint32_t>((16 * (g >> 1) + r) * BX + ((c ^ (2 * r)) << 4) + 8 * q);
    }
  }
  __device__ __forceinline__ static bf16x8 frag(const char* lds, const uint32_t (&fb)[4], int i, int s) {
    typedef int i32x2v __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) i32x2v lds_i32x2;
    const char* p = lds + fb[i] + s * 32 * BX;
    const i32x2v lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
    const i32x2v hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 8 * BX));
    const i32x4v v = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Contraction over nfull full steps and kv trailing units (< TK) of A and B
// (both row operands), NS-stage ring.  Every step issues one DMA block, the
// source clamped to the last full step past the end, so the wait before
// each step is a constant.
template <int NS, class OA, class OB, class ACC>
__device__ __forceinline__ void contract_f8(char* lds, const OA& A, const OB& B, int64_t Kc,
                                            ACC& acc, const uint32_t (&fa)[4],
                                            const uint32_t (&fb)[4]) {
  constexpr int SB = OA::kBytes + OB::kBytes;
  constexpr int PER = OA::NJ + OB::NJ;
  constexpr int NM = ACC::FM * ACC::FN;
  static_assert((NS - 2) * PER < 64, "vmcnt range");
  const int nfull = static_cast<int>(Kc / TK);
  const int kv = static_cast<int>(Kc - static_cast<int64_t>(nfull) * TK);
  typename ACC::Frags8 f;
  acc.zero();
  if (nfull > 0) {
    auto src = [&](int st) { return st < nfull ? st : nfull - 1; };
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) {
      A.dma(src(p), lds_addr(lds + p * SB));
      B.dma(src(p), lds_addr(lds + p * SB + OA::kBytes));
    }
    for (int s = 0; s < nfull; ++s) {
      wait_vmcnt<(NS - 2) * PER>();          // step s has landed
      __syncthreads();                        // ... for every wave; step s - 1 is consumed
      const char* cs = lds + (s % NS) * SB;
#pragma unroll
      for (int i = 0; i < ACC::FM; ++i) f.a[i] = ACC::template frag8<OA>(cs, fa, i);
#pragma unroll
      for (int j = 0; j < ACC::FN; ++j) f.b[j] = ACC::template frag8<OB>(cs + OA::kBytes, fb, j);
      // step s + NS - 1 into the stage of step s - 1
      const int nx = src(s + NS - 1);
      const void* sa = uniform_ptr(A.step_base(nx));
      const void* sb = uniform_ptr(B.step_base(nx));
      char* ds = lds + ((s + NS - 1) % NS) * SB;
      const uint32_t la = lds_addr(ds), lb = lds_addr(ds + OA::kBytes);
      interleave<NM, PER>([&](int q) { acc.mma8(f, q); },
                          [&](int o) {
                            if (o < OA::NJ) A.dma_one(sa, o, la);
                            else B.dma_one(sb, o - OA::NJ, lb);
                          });
    }
    wait_vmcnt<0>();
  }
  if (kv > 0) {
    __syncthreads();   // every wave's DMA has landed and no wave reads the stages
    char* ts = lds + (nfull % NS) * SB;
    {
      uint4 t[OA::NR];
      A.tail_load(nfull, kv, t);
      A.tail_store(ts, t);
    }
    {
      uint4 t[OB::NR];
      B.tail_load(nfull, kv, t);
      B.tail_store(ts + OA::kBytes, t);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ACC::FM; ++i) f.a[i] = ACC::template frag8<OA>(ts, fa, i);
#pragma unroll
    for (int j = 0; j < ACC::FN; ++j) f.b[j] = ACC::template frag8<OB>(ts + OA::kBytes, fb, j);
#pragma unroll
    for (int q = 0; q < NM; ++q) acc.mma8(f, q);
  }
  __syncthreads();   // every wave is done with all stages before they are refilled
}

// Four-stage variant with two fragment sets: the fragments of step s + 1
// are read between the MFMAs of step s (the bf16 pipeline's overlap), so no
// step starts with exposed LDS reads.  Used by the 256-row gmm (3-4% faster
// on the Mixtral-8x7B shape); in the 256-row tgmm the second fragment set
// makes the epilogue spill and the launch 16% slower, so it keeps
// contract_f8.  A stage is free once every wave has
// passed the barrier of the step it holds (its fragments were read during
// the step before), so step s refills the stage of step s with step s + NS.
template <int NS, class OA, class OB, class ACC>
__device__ __forceinline__ void contract_f8_db(char* lds, const OA& A, const OB& B, int64_t Kc,
                                               ACC& acc, const uint32_t (&fa)[4],
                                               const uint32_t (&fb)[4]) {
  constexpr int SB = OA::kBytes + OB::kBytes;
  constexpr int PER = OA::NJ + OB::NJ;
  constexpr int NM = ACC::FM * ACC::FN;
  constexpr int NF = ACC::FM + ACC::FN;
  static_assert((NS - 1) * PER < 64, "vmcnt range");
  const int nfull = static_cast<int>(Kc / TK);
  const int kv = static_cast<int>(Kc - static_cast<int64_t>(nfull) * TK);
  typename ACC::Frags8 f0, f1;
  acc.zero();
  if (nfull > 0) {
    // DMA sources past the last full step re-read it, so every wait below
    // is a constant
    auto src = [&](int st) { return st < nfull ? st : nfull - 1; };
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      A.dma(src(p), lds_addr(lds + p * SB));
      B.dma(src(p), lds_addr(lds + p * SB + OA::kBytes));
    }
    wait_vmcnt<(NS - 1) * PER>();   // step 0 has landed
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ACC::FM; ++i) f0.a[i] = ACC::template frag8<OA>(lds, fa, i);
#pragma unroll
    for (int j = 0; j < ACC::FN; ++j) f0.b[j] = ACC::template frag8<OB>(lds + OA::kBytes, fb, j);
    // MFMAs of step s on fc; fragments of step s + 1 into fn and the DMA of
    // step s + NS between them
    auto step = [&](typename ACC::Frags8& fc, typename ACC::Frags8& fn, int s) {
      wait_vmcnt<(NS - 2) * PER>();   // step s + 1 has landed
      __syncthreads();                // ... for every wave, and stage s is read
      const char* ns = lds + ((s + 1) % NS) * SB;
      const int nx = src(s + NS);
      const void* sa = uniform_ptr(A.step_base(nx));
      const void* sb = uniform_ptr(B.step_base(nx));
      char* ds = lds + (s % NS) * SB;
      const uint32_t la = lds_addr(ds), lb = lds_addr(ds + OA::kBytes);
      interleave<NM, NF + PER>(
          [&](int q) { acc.mma8(fc, q); },
          [&](int o) {
            if (o < ACC::FM) fn.a[o] = ACC::template frag8<OA>(ns, fa, o);
            else if (o < NF) fn.b[o - ACC::FM] = ACC::template frag8<OB>(ns + OA::kBytes, fb, o - ACC::FM);
            else if (o < NF + OA::NJ) A.dma_one(sa, o - NF, la);
            else B.dma_one(sb, o - NF - OA::NJ, lb);
          });
    };
    int s = 0;
    for (; s + 2 <= nfull; s += 2) {
      step(f0, f1, s);
      step(f1, f0, s + 1);
    }
    if (s < nfull) step(f0, f1, s);
    wait_vmcnt<0>();
  }
  if (kv > 0) {
    __syncthreads();   // every wave's DMA has landed and no wave reads the stages
    char* ts = lds + (nfull % NS) * SB;
    {
      uint4 t[OA::NR];
      A.tail_load(nfull, kv, t);
      A.tail_store(ts, t);
    }
    {
      uint4 t[OB::NR];
      B.tail_load(nfull, kv, t);
      B.tail_store(ts + OA::kBytes, t);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ACC::FM; ++i) f0.a[i] = ACC::template frag8<OA>(ts, fa, i);
#pragma unroll
    for (int j = 0; j < ACC::FN; ++j) f0.b[j] = ACC::template frag8<OB>(ts + OA::kBytes, fb, j);
#pragma unroll
    for (int q = 0; q < NM; ++q) acc.mma8(f0, q);
  }
  __syncthreads();   // every wave is done with all stages before they are refilled
}

constexpr int kF8TN = 256;
template <int TM>
struct F8Tile {
  static constexpr int NS = TM >= 256 ? 4 : 3;
  static constexpr int kBytes = NS * (TM + kF8TN) * TK * 2;
};

// Grouped GEMM, ragged rows: out[rows of g] (+)= sa sb[g] A[rows of g] B_g^T
// (+ bias[g]), B_g = rhs + g rhs_gs as [N, K], or with B_KN as [K, N] read
// through transposing LDS reads.
template <int FA, int FB, typename TO, int TM, bool B_KN = false>
__global__ __launch_bounds__(NT, TM >= 256 ? 1 : 2) void gmm_fp8_kernel(Fp8Args a) {
  constexpr int TN = kF8TN;
  using OB = std::conditional_t<B_KN, F8Col<TN>, Operand<false, TN>>;
  __shared__ __attribute__((aligned(1024))) char smem[F8Tile<TM>::kBytes];
  __shared__ int row_base[kMaxGShort + 1];
  __shared__ int tile_base[kMaxGShort + 1];
  const int ntn = static_cast<int>((a.N + TN - 1) / TN);
  scan_groups(a.gsz, a.G, a.M, TM, ntn, row_base, tile_base, blockIdx.x == 0 ? a.err : nullptr);
  __syncthreads();
  const int total = tile_base[a.G];
  TO* out = static_cast<TO*>(a.out);
  Operand<false, TM> A;
  OB B;
  Acc8<TM, TN, FA, FB> acc;
  uint32_t fa[4], fb[4];
  Operand<false, TM>::frag_base(((threadIdx.x >> 6) >> 1) * (TM / 2), fa);
  OB::frag_base(((threadIdx.x >> 6) & 1) * (TN / 2), fb);
  const float sa = a.sinv_a[0];
  for (int it = 0;; ++it) {
    const int64_t tile = xcd_tile(it);
    if (tile >= total) break;
    int lo = 0, hi = a.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int rows_g = row_base[g + 1] - row_base[g];
    const int mtiles = (rows_g + TM - 1) / TM;
    const int local = static_cast<int>(tile - tile_base[g]);
    int mt, nt;
    blocked_tile(local, mtiles, ntn, mt, nt);
    const int64_t row0 = row_base[g] + static_cast<int64_t>(mt) * TM;
    const int rv = min(TM, rows_g - mt * TM);
    const int64_t col0 = static_cast<int64_t>(nt) * TN;
    const int cv = static_cast<int>(lmin(TN, a.N - col0));
    const int vr = a.valid ? max(0, min(rv, min(rows_g, max(a.valid[g], 0)) - mt * TM)) : rv;
    acc.set_live_rows(vr);
    A.setup(a.lhs + row0 * a.ld_lhs, a.ld_lhs, max(vr, 1));
    if constexpr (B_KN) B.setup(a.rhs + g * a.rhs_gs + col0 / 2, a.ld_rhs, cv);
    else B.setup(a.rhs + g * a.rhs_gs + col0 * a.ld_rhs, a.ld_rhs, cv);
    if constexpr (F8Tile<TM>::NS == 4) contract_f8_db<4>(smem, A, B, a.Kdim, acc, fa, fb);
    else contract_f8<F8Tile<TM>::NS>(smem, A, B, a.Kdim, acc, fa, fb);
    store_tile(static_cast<const Acc<TM, TN>&>(acc), smem, out + row0 * a.ld_out + col0, a.ld_out,
               rv, cv, a.accumulate, a.bias ? a.bias + g * a.N + col0 : nullptr, sa * a.sinv_b[g],
               vr);
  }
  if (!a.accumulate) zero_rows(out, a.ld_out, a.N, row_base[a.G], a.M);
}

// Transposed grouped GEMM over transposed copies: lhs_t [Kdim, P] and
// rhs_t [N, P], group g at columns 64 * (64-row tiles of the groups before
// g); out[g] (+)= sa sb lhs_t[:, cols of g] rhs_t[:, cols of g]^T.  The
// contraction covers the group's rows rounded up to 64 (the quantizer wrote
// zeros there), or its valid rows rounded up.
template <int FA, int FB, typename TO, int TM>
__global__ __launch_bounds__(NT, TM >= 256 ? 1 : 2) void tgmm_fp8_kernel(Fp8Args a) {
  constexpr int TN = kF8TN;
  __shared__ __attribute__((aligned(1024))) char smem[F8Tile<TM>::kBytes];
  __shared__ int row_base[kMaxGShort + 1];
  __shared__ int tile_base[kMaxGShort + 1];
  scan_groups(a.gsz, a.G, a.M, 64, 1, row_base, tile_base, blockIdx.x == 0 ? a.err : nullptr);
  __syncthreads();
  const int mtn = static_cast<int>((a.Kdim + TM - 1) / TM);
  const int ntn = static_cast<int>((a.N + TN - 1) / TN);
  const int64_t per_group = static_cast<int64_t>(mtn) * ntn;
  const int64_t total = per_group * a.G;
  TO* out = static_cast<TO*>(a.out);
  Operand<false, TM> A;
  Operand<false, TN> B;
  Acc8<TM, TN, FA, FB> acc;
  uint32_t fa[4], fb[4];
  Operand<false, TM>::frag_base(((threadIdx.x >> 6) >> 1) * (TM / 2), fa);
  Operand<false, TN>::frag_base(((threadIdx.x >> 6) & 1) * (TN / 2), fb);
  const float scale = a.sinv_a[0] * a.sinv_b[0];
  for (int it = 0;; ++it) {
    const int64_t tile = xcd_tile(it);
    if (tile >= total) break;
    const int g = static_cast<int>(tile / per_group);
    const int local = static_cast<int>(tile - g * per_group);
    int mt, nt;
    blocked_tile(local, mtn, ntn, mt, nt);
    int rows_g = row_base[g + 1] - row_base[g];
    if (a.valid) rows_g = min(rows_g, max(a.valid[g], 0));
    if (rows_g == 0 && a.accumulate) continue;
    const int64_t kc = static_cast<int64_t>((rows_g + 63) / 64) * 32;    // units
    const int64_t c0 = static_cast<int64_t>(tile_base[g]) * 32;           // units
    const int64_t m0 = static_cast<int64_t>(mt) * TM, n0 = static_cast<int64_t>(nt) * TN;
    const int mv = static_cast<int>(lmin(TM, a.Kdim - m0));
    const int nv = static_cast<int>(lmin(TN, a.N - n0));
    A.setup(a.lhs + m0 * a.ld_lhs + c0, a.ld_lhs, mv);
    B.setup(a.rhs + n0 * a.ld_rhs + c0, a.ld_rhs, nv);
    contract_f8<F8Tile<TM>::NS>(smem, A, B, kc, acc, fa, fb);
    store_tile<TM, TN, TO, false>(static_cast<const Acc<TM, TN>&>(acc), smem,
                                  out + g * a.out_gs + m0 * a.ld_out + n0, a.ld_out, mv, nv,
                                  a.accumulate, nullptr, scale);
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
    int accumulate, int32_t* err, const float* __restrict__ bias) {
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
          const float v = bias ? acc[i][j] + bias[g * N + c] : acc[i][j];
          if (out_f) store_out(out_f + off, v, accumulate);
          else store_out(out_h + off, v, accumulate);
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
    const int32_t* __restrict__ gsz, const int32_t* __restrict__ valid, int G, int64_t M,
    int64_t Kdim, int64_t N, float* __restrict__ out_f, bf16_t* __restrict__ out_h,
    int64_t ld_out, int64_t out_gs, int accumulate, int32_t* err) {
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
    int rows_g = row_base[g + 1] - row_base[g];
    if (valid) rows_g = min(rows_g, max(valid[g], 0));
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

unsigned persistent_grid(int64_t upper_tiles, int per_cu) {
  int64_t g = static_cast<int64_t>(device_cu_count()) * per_cu;
  if (upper_tiles < g) g = upper_tiles;
  g = ((g + 7) / 8) * 8;
  return static_cast<unsigned>(g < 8 ? 8 : g);
}

bool mult8(int64_t v) { return v >= 0 && (v & 7) == 0; }

constexpr int64_t kMaxLd = int64_t(1) << 22;   // keeps per-lane DMA byte offsets in 32 bits

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API int moe_gmm(const void* lhs, int64_t M_lhs, int64_t ld_lhs, const void* rhs,
                    int64_t ld_rhs, int64_t rhs_group_stride, int trans_rhs,
                    const int32_t* group_sizes, const int32_t* valid_rows, int G, int64_t Kdim,
                    int64_t N, int in_dtype,
                    const void* bias, void* out, int64_t M_out, int64_t ld_out, int out_dtype,
                    int accumulate, int32_t* err, void* stream) {
  if (G < 1 || G > kMaxG || M_lhs < 0 || M_out < 0 || M_out > M_lhs || Kdim < 0 || N < 0)
    return MOE_ERR_ARG;
  if (M_out > INT32_MAX) return MOE_ERR_ARG;
  if (in_dtype != MOE_BF16 && in_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (!mult8(Kdim) || !mult8(N) || !mult8(ld_lhs) || !mult8(ld_rhs) || !mult8(ld_out) ||
      !mult8(rhs_group_stride))
    return MOE_ERR_ARG;
  if (ld_lhs < Kdim || ld_out < N || ld_rhs < (trans_rhs ? Kdim : N)) return MOE_ERR_ARG;
  if (ld_lhs > kMaxLd || ld_rhs > kMaxLd) return MOE_ERR_ARG;
  if (M_out == 0 || N == 0) return MOE_OK;
  if (!lhs || !rhs || !group_sizes || !out || !aligned16(lhs) || !aligned16(rhs) || !aligned16(out))
    return MOE_ERR_ARG;
  if (bias && !aligned16(bias)) return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == MOE_BF16) {
    MfmaArgs a{static_cast<const bf16_t*>(lhs), ld_lhs, static_cast<const bf16_t*>(rhs), ld_rhs,
               rhs_group_stride, group_sizes, G, M_out, Kdim, N, out, ld_out, 0, accumulate, err,
               valid_rows};
    a.bias = static_cast<const bf16_t*>(bias);
    // narrow outputs and single-step contractions use a 256 x 128 tile;
    // small groups (fewer than 512 rows per group on average) use 128-row
    // tiles, two workgroups per CU
    const bool narrow = N <= 128 || Kdim <= TK;
    const bool short_m = !narrow && G <= kMaxGShort && M_out < 512 * static_cast<int64_t>(G);
    const int TMv = short_m ? 128 : 256;
    const int TNv = narrow ? 128 : 256;
    const int64_t upper = ((M_out + TMv - 1) / TMv + G) * ((N + TNv - 1) / TNv);
    const unsigned grid = persistent_grid(upper, short_m ? 2 : 1);
    // 256-row tiles load row operands as 128-byte segments (two steps per
    // DMA unit) when the number of full contraction steps is even
    const int64_t nsteps = Kdim / TK;
    const bool pair = !short_m && nsteps >= 2 && nsteps % 2 == 0;
#define GMM(BC, TMV, TNV, TO, P) \
  hipLaunchKernelGGL((gmm_mfma_kernel<BC, TMV, TNV, TO, P>), dim3(grid), dim3(NT), 0, st, a)
#define GMM2(BC, TMV, TNV, TO)          \
  do {                                  \
    if (pair) GMM(BC, TMV, TNV, TO, true); \
    else GMM(BC, TMV, TNV, TO, false);  \
  } while (0)
    if (narrow) {
      if (trans_rhs) {
        if (out_dtype == MOE_BF16) GMM2(false, 256, 128, bf16_t); else GMM2(false, 256, 128, float);
      } else {
        if (out_dtype == MOE_BF16) GMM2(true, 256, 128, bf16_t); else GMM2(true, 256, 128, float);
      }
    } else if (short_m) {
      // for contractions at least as long as the output is wide, groups
      // above kSplitRows rows take 256-row tiles in a launch of their own
      // (their weight blocks are read once per 256 rows, and the launch runs
      // at the large-tile MFMA rate); the rest take 128-row tiles
      if (G > 1 && Kdim >= N) {
        MfmaArgs b = a;
        b.cls_lo = kSplitRows + 1;
        const unsigned grid_big = persistent_grid(((M_out + 255) / 256 + G) * ((N + 255) / 256), 1);
        const bool pair_big = nsteps >= 2 && nsteps % 2 == 0;
#define GMMB(BC, TO, P) \
  hipLaunchKernelGGL((gmm_mfma_kernel<BC, 256, 256, TO, P>), dim3(grid_big), dim3(NT), 0, st, b)
        if (trans_rhs) {
          if (out_dtype == MOE_BF16) { if (pair_big) GMMB(false, bf16_t, true); else GMMB(false, bf16_t, false); }
          else { if (pair_big) GMMB(false, float, true); else GMMB(false, float, false); }
        } else {
          if (out_dtype == MOE_BF16) { if (pair_big) GMMB(true, bf16_t, true); else GMMB(true, bf16_t, false); }
          else { if (pair_big) GMMB(true, float, true); else GMMB(true, float, false); }
        }
#undef GMMB
        a.cls_hi = kSplitRows;
      }
      if (trans_rhs) {
        if (out_dtype == MOE_BF16) GMM(false, 128, 256, bf16_t, false); else GMM(false, 128, 256, float, false);
      } else {
        if (out_dtype == MOE_BF16) GMM(true, 128, 256, bf16_t, false); else GMM(true, 128, 256, float, false);
      }
    } else {
      if (trans_rhs) {
        if (out_dtype == MOE_BF16) GMM2(false, 256, 256, bf16_t); else GMM2(false, 256, 256, float);
      } else {
        if (out_dtype == MOE_BF16) GMM2(true, 256, 256, bf16_t); else GMM2(true, 256, 256, float);
      }
    }
#undef GMM2
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
                         accumulate, err, static_cast<const float*>(bias));
    else
      hipLaunchKernelGGL(gmm_f32_kernel<false>, dim3(grid), dim3(NT), 0, st,
                         static_cast<const float*>(lhs), ld_lhs, static_cast<const float*>(rhs),
                         ld_rhs, rhs_group_stride, group_sizes, G, Kdim, N, of, oh, M_out, ld_out,
                         accumulate, err, static_cast<const float*>(bias));
  }
  return launch_status();
}

MOE_API int moe_gmm_swiglu(const void* lhs, int64_t M_lhs, int64_t ld_lhs, const void* rhs,
                           int64_t ld_rhs, int64_t rhs_group_stride, const int32_t* group_sizes,
                           const int32_t* valid_rows, int G, int64_t Kdim, int64_t F, int in_dtype,
                           const void* bias, void* h, int64_t ld_h, void* act, int64_t ld_act,
                           int64_t M_out, int32_t* err, void* stream) {
  if (G < 1 || G > kMaxG || M_lhs < 0 || M_out < 0 || M_out > M_lhs || Kdim < 0 || F < 0)
    return MOE_ERR_ARG;
  if (M_out > INT32_MAX) return MOE_ERR_ARG;
  if (in_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (F % 128 || !mult8(Kdim) || !mult8(ld_lhs) || !mult8(ld_rhs) || !mult8(rhs_group_stride) ||
      !mult8(ld_act) || (h && !mult8(ld_h)))
    return MOE_ERR_ARG;
  if (ld_lhs < Kdim || ld_rhs < 2 * F || ld_act < F || (h && ld_h < 2 * F)) return MOE_ERR_ARG;
  if (ld_lhs > kMaxLd || ld_rhs > kMaxLd) return MOE_ERR_ARG;
  if (M_out == 0 || F == 0) return MOE_OK;
  if (!lhs || !rhs || !group_sizes || !act || !aligned16(lhs) || !aligned16(rhs) ||
      !aligned16(act) || (h && !aligned16(h)) || (bias && !aligned16(bias)))
    return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t N = 2 * F;
  MfmaArgs a{static_cast<const bf16_t*>(lhs), ld_lhs, static_cast<const bf16_t*>(rhs), ld_rhs,
             rhs_group_stride, group_sizes, G, M_out, Kdim, N, h, ld_h, 0, 0, err, valid_rows};
  a.bias = static_cast<const bf16_t*>(bias);
  a.act = static_cast<bf16_t*>(act);
  a.ld_act = ld_act;
  // tiles as moe_gmm's: 128-row tiles for small groups, else 256 x 256
  const bool short_m = G <= kMaxGShort && M_out < 512 * static_cast<int64_t>(G);
  const int TMv = short_m ? 128 : 256;
  const int64_t upper = ((M_out + TMv - 1) / TMv + G) * (N / 256);
  const unsigned grid = persistent_grid(upper, short_m ? 2 : 1);
  const int64_t nsteps = Kdim / TK;
  const bool pair = !short_m && nsteps >= 2 && nsteps % 2 == 0;
  if (short_m) {
    if (G > 1 && Kdim >= N) {   // large groups in 256-row tiles, as in moe_gmm
      MfmaArgs b = a;
      b.cls_lo = kSplitRows + 1;
      const unsigned grid_big = persistent_grid(((M_out + 255) / 256 + G) * (N / 256), 1);
      if (nsteps >= 2 && nsteps % 2 == 0)
        hipLaunchKernelGGL((gmm_mfma_kernel<true, 256, 256, bf16_t, true, true>), dim3(grid_big), dim3(NT), 0, st, b);
      else
        hipLaunchKernelGGL((gmm_mfma_kernel<true, 256, 256, bf16_t, false, true>), dim3(grid_big), dim3(NT), 0, st, b);
      a.cls_hi = kSplitRows;
    }
    hipLaunchKernelGGL((gmm_mfma_kernel<true, 128, 256, bf16_t, false, true>), dim3(grid), dim3(NT), 0, st, a);
  } else if (pair)
    hipLaunchKernelGGL((gmm_mfma_kernel<true, 256, 256, bf16_t, true, true>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((gmm_mfma_kernel<true, 256, 256, bf16_t, false, true>), dim3(grid), dim3(NT), 0, st, a);
  return launch_status();
}

MOE_API int moe_gmm_swiglu_bwd(const void* lhs, int64_t M_lhs, int64_t ld_lhs, const void* rhs,
                               int64_t ld_rhs, int64_t rhs_group_stride,
                               const int32_t* group_sizes, const int32_t* valid_rows, int G,
                               int64_t Kdim, int64_t F, int in_dtype, const void* h0,
                               const void* h1, int64_t ld_h, void* d_h0, void* d_h1,
                               int64_t ld_dh, int64_t M_out, int32_t* err, void* stream) {
  if (G < 1 || G > kMaxG || M_lhs < 0 || M_out < 0 || M_out > M_lhs || Kdim < 0 || F < 0)
    return MOE_ERR_ARG;
  if (M_out > INT32_MAX) return MOE_ERR_ARG;
  if (in_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (!mult8(Kdim) || !mult8(F) || !mult8(ld_lhs) || !mult8(ld_rhs) || !mult8(rhs_group_stride) ||
      !mult8(ld_h) || !mult8(ld_dh))
    return MOE_ERR_ARG;
  if (F <= 128 || Kdim <= TK) return MOE_ERR_ARG;   // the narrow tile shapes are not offered
  if (ld_lhs < Kdim || ld_rhs < Kdim || ld_h < F || ld_dh < F) return MOE_ERR_ARG;
  if (ld_lhs > kMaxLd || ld_rhs > kMaxLd) return MOE_ERR_ARG;
  if (M_out == 0) return MOE_OK;
  if (!lhs || !rhs || !group_sizes || !h0 || !h1 || !d_h0 || !d_h1 || !aligned16(lhs) ||
      !aligned16(rhs) || !aligned16(h0) || !aligned16(h1) || !aligned16(d_h0) || !aligned16(d_h1))
    return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MfmaArgs a{static_cast<const bf16_t*>(lhs), ld_lhs, static_cast<const bf16_t*>(rhs), ld_rhs,
             rhs_group_stride, group_sizes, G, M_out, Kdim, F, d_h0, ld_dh, 0, 0, err, valid_rows};
  a.h0 = static_cast<const bf16_t*>(h0);
  a.h1 = static_cast<const bf16_t*>(h1);
  a.ld_h = ld_h;
  a.dh1 = static_cast<bf16_t*>(d_h1);
  // tiles as moe_gmm's with a transposed rhs
  const bool short_m = G <= kMaxGShort && M_out < 512 * static_cast<int64_t>(G);
  const int64_t nsteps = Kdim / TK;
  const bool pair = nsteps >= 2 && nsteps % 2 == 0;
  if (short_m) {
    const int64_t upper = ((M_out + 127) / 128 + G) * ((F + 255) / 256);
    const unsigned grid = persistent_grid(upper, 2);
    if (G > 1 && Kdim >= F) {
      MfmaArgs b = a;
      b.cls_lo = kSplitRows + 1;
      const unsigned grid_big = persistent_grid(((M_out + 255) / 256 + G) * ((F + 255) / 256), 1);
      if (pair)
        hipLaunchKernelGGL((gmm_mfma_kernel<false, 256, 256, bf16_t, true, false, true>), dim3(grid_big), dim3(NT), 0, st, b);
      else
        hipLaunchKernelGGL((gmm_mfma_kernel<false, 256, 256, bf16_t, false, false, true>), dim3(grid_big), dim3(NT), 0, st, b);
      a.cls_hi = kSplitRows;
    }
    hipLaunchKernelGGL((gmm_mfma_kernel<false, 128, 256, bf16_t, false, false, true>), dim3(grid), dim3(NT), 0, st, a);
  } else {
    const int64_t upper = ((M_out + 255) / 256 + G) * ((F + 255) / 256);
    const unsigned grid = persistent_grid(upper, 1);
    if (pair)
      hipLaunchKernelGGL((gmm_mfma_kernel<false, 256, 256, bf16_t, true, false, true>), dim3(grid), dim3(NT), 0, st, a);
    else
      hipLaunchKernelGGL((gmm_mfma_kernel<false, 256, 256, bf16_t, false, false, true>), dim3(grid), dim3(NT), 0, st, a);
  }
  return launch_status();
}

MOE_API int moe_tgmm(const void* lhs, int64_t ld_lhs, const void* rhs, int64_t ld_rhs,
                     const int32_t* group_sizes, const int32_t* valid_rows, int G, int64_t M,
                     int64_t Kdim, int64_t N, int in_dtype, void* out, int64_t ld_out,
                     int64_t out_group_stride, int out_dtype, int accumulate, int32_t* err,
                     void* stream) {
  if (G < 1 || G > kMaxG || M < 0 || Kdim < 0 || N < 0) return MOE_ERR_ARG;
  if (M > INT32_MAX) return MOE_ERR_ARG;
  if (in_dtype != MOE_BF16 && in_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (!mult8(Kdim) || !mult8(N) || !mult8(ld_lhs) || !mult8(ld_rhs) || !mult8(ld_out) ||
      !mult8(out_group_stride))
    return MOE_ERR_ARG;
  if (ld_lhs < Kdim || ld_rhs < N || ld_out < N || out_group_stride < Kdim * ld_out)
    return MOE_ERR_ARG;
  if (ld_lhs > kMaxLd || ld_rhs > kMaxLd) return MOE_ERR_ARG;
  if (Kdim == 0 || N == 0) return MOE_OK;
  if (!lhs || !rhs || !group_sizes || !out || !aligned16(lhs) || !aligned16(rhs) || !aligned16(out))
    return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (in_dtype == MOE_BF16) {
    MfmaArgs a{static_cast<const bf16_t*>(lhs), ld_lhs, static_cast<const bf16_t*>(rhs), ld_rhs,
               0, group_sizes, G, M, Kdim, N, out, ld_out, out_group_stride, accumulate, err,
               valid_rows};
    // short contractions (under 512 rows per group on average) leave each
    // tile's latency and stores exposed.  There the groups are split by the
    // rows their contraction covers (valid_rows, else the group size) into
    // five launches: at most kShortRows rows in the short kernel (resident
    // rhs strip, lhs blocks copied ahead, stores of one tile overlapping
    // the next), 33..64 and 65..128 rows in the strip kernels (the same
    // scheme over two and four steps), up to kSplitRows in 128 x 256 tiles
    // (two workgroups per CU), the rest in 256 x 256 tiles (half the operand
    // traffic per flop).  On the DeepSeek-V3 shape: 2.7 ms per launch in one
    // 128-row launch -> 2.4 ms.  (256-row tiles for the mid-sized groups took
    // 0.9 ms more.)  Otherwise one launch of 256 x 256 tiles does every group.
    const bool short_k = M < 512 * static_cast<int64_t>(G) && G <= kMaxGShort;
    auto grid_for = [&](int TMv, int per_cu) {
      return persistent_grid(static_cast<int64_t>(G) * ((Kdim + TMv - 1) / TMv) * ((N + 255) / 256),
                             per_cu);
    };
#define TGMM(TMc, TOc, ARGS, GRID) \
  hipLaunchKernelGGL((tgmm_mfma_kernel<TMc, 256, TOc>), dim3(GRID), dim3(NT), 0, st, ARGS)
#define TGMMS(TOc, ARGS, GRID) \
  hipLaunchKernelGGL((tgmm_short_kernel<TOc>), dim3(GRID), dim3(NT), 0, st, ARGS)
#define TGMMR(Sc, TOc, ARGS, GRID) \
  hipLaunchKernelGGL((tgmm_strip_kernel<Sc, TOc>), dim3(GRID), dim3(NT), 0, st, ARGS)
    if (short_k) {
      MfmaArgs s_ = a, r2_ = a, r4_ = a, m_ = a, b_ = a;
      s_.cls_hi = kShortRows;
      r2_.cls_lo = kShortRows + 1;
      r2_.cls_hi = 2 * kShortRows;
      r4_.cls_lo = 2 * kShortRows + 1;
      r4_.cls_hi = 4 * kShortRows;
      m_.cls_lo = 4 * kShortRows + 1;
      m_.cls_hi = kSplitRows;
      b_.cls_lo = kSplitRows + 1;
      r2_.err = r4_.err = m_.err = b_.err = nullptr;   // the first launch checks the group sizes
      const int64_t units = static_cast<int64_t>(G) * ((N + 255) / 256);
      const unsigned gs_ = persistent_grid(units, 2), g4_ = persistent_grid(units, 1);
      const unsigned gm_ = grid_for(128, 2), gb_ = grid_for(256, 1);
      if (out_dtype == MOE_BF16) {
        TGMMS(bf16_t, s_, gs_);
        TGMMR(2, bf16_t, r2_, gs_);
        TGMMR(4, bf16_t, r4_, g4_);
        TGMM(128, bf16_t, m_, gm_);
        TGMM(256, bf16_t, b_, gb_);
      } else {
        TGMMS(float, s_, gs_);
        TGMMR(2, float, r2_, gs_);
        TGMMR(4, float, r4_, g4_);
        TGMM(128, float, m_, gm_);
        TGMM(256, float, b_, gb_);
      }
    } else {
      const unsigned grid = grid_for(256, 1);
      if (out_dtype == MOE_BF16) TGMM(256, bf16_t, a, grid); else TGMM(256, float, a, grid);
    }
#undef TGMMR
#undef TGMMS
#undef TGMM
  } else {
    const int64_t upper = static_cast<int64_t>(G) * ((Kdim + FB - 1) / FB) * ((N + FB - 1) / FB);
    const unsigned grid = persistent_grid(upper, 4);
    float* of = out_dtype == MOE_F32 ? static_cast<float*>(out) : nullptr;
    bf16_t* oh = out_dtype == MOE_BF16 ? static_cast<bf16_t*>(out) : nullptr;
    hipLaunchKernelGGL(tgmm_f32_kernel, dim3(grid), dim3(NT), 0, st, static_cast<const float*>(lhs),
                       ld_lhs, static_cast<const float*>(rhs), ld_rhs, group_sizes, valid_rows, G,
                       M, Kdim, N, of, oh, ld_out, out_group_stride, accumulate, err);
  }
  return launch_status();
}

MOE_API int moe_gmm_fp8(const void* lhs, int64_t M_lhs, int64_t ld_lhs, int lhs_fmt,
                        const float* lhs_scale_inv, const void* rhs, int64_t ld_rhs,
                        int64_t rhs_group_stride, int trans_rhs, int rhs_fmt,
                        const float* rhs_scale_inv,
                        const int32_t* group_sizes, const int32_t* valid_rows, int G, int64_t Kdim,
                        int64_t N,
                        const void* bias, void* out, int64_t M_out, int64_t ld_out, int out_dtype,
                        int accumulate, int32_t* err, void* stream) {
  if (G < 1 || G > kMaxGShort || M_lhs < 0 || M_out < 0 || M_out > M_lhs || Kdim < 0 || N < 0)
    return MOE_ERR_ARG;
  if (M_out > INT32_MAX) return MOE_ERR_ARG;
  if ((lhs_fmt != MOE_FP8_E4M3 && lhs_fmt != MOE_FP8_E5M2) ||
      (rhs_fmt != MOE_FP8_E4M3 && rhs_fmt != MOE_FP8_E5M2))
    return MOE_ERR_ARG;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (Kdim % 16 || ld_lhs % 16 || ld_rhs % 16 || rhs_group_stride % 16 || !mult8(N) ||
      !mult8(ld_out))
    return MOE_ERR_ARG;
  if (ld_lhs < Kdim || ld_rhs < (trans_rhs ? Kdim : N) || ld_out < N) return MOE_ERR_ARG;
  if (ld_lhs / 2 > kMaxLd || ld_rhs / 2 > kMaxLd) return MOE_ERR_ARG;
  if (M_out == 0 || N == 0) return MOE_OK;
  if (!lhs || !rhs || !group_sizes || !out || !lhs_scale_inv || !rhs_scale_inv ||
      !aligned16(lhs) || !aligned16(rhs) || !aligned16(out) || (bias && !aligned16(bias)))
    return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Fp8Args a{static_cast<const bf16_t*>(lhs), ld_lhs / 2, static_cast<const bf16_t*>(rhs),
            ld_rhs / 2, rhs_group_stride / 2, group_sizes, valid_rows, G, M_out, Kdim / 2, N, out,
            ld_out, 0, accumulate, err, lhs_scale_inv, rhs_scale_inv,
            static_cast<const bf16_t*>(bias)};
  // 256-row tiles when groups hold 512 rows or more on average
  const bool big = M_out >= 512 * static_cast<int64_t>(G);
  const int TMv = big ? 256 : 128;
  const int64_t upper = ((M_out + TMv - 1) / TMv + G) * ((N + kF8TN - 1) / kF8TN);
  const unsigned grid = persistent_grid(upper, big ? 1 : 2);
#define G8T(FA, FB, TO, TMV)                                                                   \
  do {                                                                                         \
    if (trans_rhs)                                                                             \
      hipLaunchKernelGGL((gmm_fp8_kernel<FA, FB, TO, TMV>), dim3(grid), dim3(NT), 0, st, a);    \
    else                                                                                       \
      hipLaunchKernelGGL((gmm_fp8_kernel<FA, FB, TO, TMV, true>), dim3(grid), dim3(NT), 0, st, a); \
  } while (0)
#define G8(FA, FB, TO) do { if (big) G8T(FA, FB, TO, 256); else G8T(FA, FB, TO, 128); } while (0)
#define G8O(FA, FB) \
  do { if (out_dtype == MOE_BF16) G8(FA, FB, bf16_t); else G8(FA, FB, float); } while (0)
  if (lhs_fmt == MOE_FP8_E4M3 && rhs_fmt == MOE_FP8_E4M3) G8O(MOE_FP8_E4M3, MOE_FP8_E4M3);
  else if (lhs_fmt == MOE_FP8_E5M2 && rhs_fmt == MOE_FP8_E4M3) G8O(MOE_FP8_E5M2, MOE_FP8_E4M3);
  else if (lhs_fmt == MOE_FP8_E4M3) G8O(MOE_FP8_E4M3, MOE_FP8_E5M2);
  else G8O(MOE_FP8_E5M2, MOE_FP8_E5M2);
#undef G8O
#undef G8
#undef G8T
  return launch_status();
}

MOE_API int64_t moe_fp8_padded_rows(int64_t rows, int G) {
  if (rows < 0 || G < 1) return -1;
  return 64 * ((rows + 63) / 64 + G - 1);
}

MOE_API int moe_tgmm_fp8(const void* lhs_t, int64_t ld_lhs, int lhs_fmt, const float* lhs_scale_inv,
                         const void* rhs_t, int64_t ld_rhs, int rhs_fmt,
                         const float* rhs_scale_inv, const int32_t* group_sizes,
                         const int32_t* valid_rows, int G, int64_t M, int64_t Kdim, int64_t N,
                         void* out, int64_t ld_out, int64_t out_group_stride, int out_dtype,
                         int accumulate, int32_t* err, void* stream) {
  if (G < 1 || G > kMaxGShort || M < 0 || M > INT32_MAX || Kdim < 0 || N < 0) return MOE_ERR_ARG;
  if ((lhs_fmt != MOE_FP8_E4M3 && lhs_fmt != MOE_FP8_E5M2) ||
      (rhs_fmt != MOE_FP8_E4M3 && rhs_fmt != MOE_FP8_E5M2))
    return MOE_ERR_ARG;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  const int64_t P = moe_fp8_padded_rows(M, G);
  if (ld_lhs % 16 || ld_rhs % 16 || ld_lhs < P || ld_rhs < P || !mult8(N) || !mult8(ld_out) ||
      ld_out < N || out_group_stride < Kdim * ld_out)
    return MOE_ERR_ARG;
  if (ld_lhs / 2 > kMaxLd || ld_rhs / 2 > kMaxLd) return MOE_ERR_ARG;
  if (Kdim == 0 || N == 0) return MOE_OK;
  if (!lhs_t || !rhs_t || !group_sizes || !out || !lhs_scale_inv || !rhs_scale_inv ||
      !aligned16(lhs_t) || !aligned16(rhs_t) || !aligned16(out))
    return MOE_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Fp8Args a{static_cast<const bf16_t*>(lhs_t), ld_lhs / 2, static_cast<const bf16_t*>(rhs_t),
            ld_rhs / 2, 0, group_sizes, valid_rows, G, M, Kdim, N, out, ld_out, out_group_stride,
            accumulate, err, lhs_scale_inv, rhs_scale_inv, nullptr};
  // 256-row tiles when groups contract over 512 rows or more on average
  const bool big = M >= 512 * static_cast<int64_t>(G);
  const int TMv = big ? 256 : 128;
  const int64_t upper = ((Kdim + TMv - 1) / TMv) * ((N + kF8TN - 1) / kF8TN) * G;
  const unsigned grid = persistent_grid(upper, big ? 1 : 2);
#define T8T(FA, FB, TO, TMV) \
  hipLaunchKernelGGL((tgmm_fp8_kernel<FA, FB, TO, TMV>), dim3(grid), dim3(NT), 0, st, a)
#define T8(FA, FB, TO) do { if (big) T8T(FA, FB, TO, 256); else T8T(FA, FB, TO, 128); } while (0)
#define T8O(FA, FB) \
  do { if (out_dtype == MOE_BF16) T8(FA, FB, bf16_t); else T8(FA, FB, float); } while (0)
  if (lhs_fmt == MOE_FP8_E4M3 && rhs_fmt == MOE_FP8_E5M2) T8O(MOE_FP8_E4M3, MOE_FP8_E5M2);
  else if (lhs_fmt == MOE_FP8_E4M3) T8O(MOE_FP8_E4M3, MOE_FP8_E4M3);
  else if (rhs_fmt == MOE_FP8_E5M2) T8O(MOE_FP8_E5M2, MOE_FP8_E5M2);
  else T8O(MOE_FP8_E5M2, MOE_FP8_E4M3);
#undef T8O
#undef T8
#undef T8T
  return launch_status();
}
