// Definitions shared by the grouped GEMM kernels (forward and backward):
// launch arguments, the tile table of slot-grouped products and the raw
// buffer resources of the operands.  Internal to the library.
#pragma once
#include "occ_internal.h"

namespace occ {
namespace {

struct GemmArgs {
  const int32_t *row_offset;  // [G+1] on the device (slots); nullptr: one dense group
  int G;
  int dense_rows;
  const void *A;
  int64_t lda;
  const void *B;
  int64_t ldb;
  int64_t b_group_stride;  // elements between the weights of consecutive experts
  int64_t a_bytes;         // bytes of the whole A operand (< 4 GiB: buffer loads)
  int64_t b_bytes;         // bytes of the whole weight operand (< 4 GiB)
  int64_t up_offset;       // SwiGLU: elements from a gate row to its up row
  int nseg;                // output columns per weight segment
  int64_t nseg_stride;     // elements between weight segments along the output
  int kseg;                // K per weight segment
  int64_t kseg_stride;     // elements between weight segments along K
  int K;
  int N;                   // output columns
  void *C;
  int64_t ldc;
  // SwiGLU forward with the pre-activations kept: [G | U] rows (bf16, row
  // stride ldgu, G in columns [0, N), U in [N, 2N)), else nullptr
  void *gu;
  int64_t ldgu;
  // backward GEMMs only
  int M;                   // output rows when K is grouped (fixed)
  int64_t c_group_stride;  // elements between the outputs of consecutive experts
  const void *aux;         // SwiGLU backward: the recomputed [G | U] rows
  int64_t ldaux;
  // tile order inside a group: 0 = m-tiles fastest (the n-tiles' weight
  // panels read once, the rows re-read per pass over the n-tiles),
  // 1 = n-tiles fastest (the rows read once, the panels re-read per m-tile)
  int n_inner;
  int32_t expert_of_group[OCC_MAX_E];
};

constexpr int kThreads = 256;  // fp32 kernel
constexpr int kBK = 64;
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
constexpr int kLdsK = kBK + 8;

// Raw buffer resource over a whole operand.  Built from kernel arguments
// only, so it is wave-uniform and lives in SGPRs; tile and lane positions go
// into the 32-bit per-lane offset, the k position into the scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)(uint32_t)bytes,
                                           kBufferFlags);
}

__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Wave 0 writes cumulative m-tile counts of the groups into ts[0..G].
__device__ __forceinline__ void group_tile_scan(const int32_t *row_offset, int G, int BM,
                                                int32_t *ts) {
  const int lane = threadIdx.x;
  int carry = 0;
  if (lane == 0) ts[0] = 0;
  for (int g0 = 0; g0 < G; g0 += kWave) {
    const int g = g0 + lane;
    int v = 0;
    if (g < G) v = (row_offset[g + 1] - row_offset[g] + BM - 1) / BM;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int u = __shfl_up(v, off);
      if (lane >= off) v += u;
    }
    if (g < G) ts[g + 1] = carry + v;
    carry += __shfl(v, kWave - 1);
  }
}

struct TileCoord {
  int group, row_begin, rows, n0;
};

// The tile table of a launch: cumulative m-tiles per group (ts[0..G]) and the
// group row offsets (ro[0..G]) in LDS; returns the number of tiles.
template <int BM, int BNO>
__device__ __forceinline__ int tile_table(const GemmArgs &a, int32_t *ts, int32_t *ro) {
  const int ntn = (a.N + BNO - 1) / BNO;
  if (a.row_offset == nullptr) return ((a.dense_rows + BM - 1) / BM) * ntn;
  if (threadIdx.x < kWave) group_tile_scan(a.row_offset, a.G, BM, ts);
  for (int g = threadIdx.x; g <= a.G; g += blockDim.x) ro[g] = a.row_offset[g];
  __syncthreads();
  return ts[a.G] * ntn;
}

// Tile number `logical`: group-major, then n-tile with the m-tile fastest,
// or (n_inner) m-tile with the n-tile fastest.
template <int BM, int BNO>
__device__ __forceinline__ TileCoord tile_coord(const GemmArgs &a, const int32_t *ts,
                                                const int32_t *ro, int logical) {
  const int ntn = (a.N + BNO - 1) / BNO;
  TileCoord tc;
  if (a.row_offset != nullptr) {
    int lo = 0, hi = a.G - 1;  // last group whose first tile is <= logical
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ts[mid] * ntn <= logical) lo = mid;
      else hi = mid - 1;
    }
    const int mtg = ts[lo + 1] - ts[lo];
    const int local = logical - ts[lo] * ntn;
    const int nt = a.n_inner ? local % ntn : local / mtg;
    const int mt = a.n_inner ? local / ntn : local - nt * mtg;
    tc.group = lo;
    tc.row_begin = ro[lo] + mt * BM;
    tc.rows = min(BM, ro[lo + 1] - tc.row_begin);
    tc.n0 = nt * BNO;
  } else {
    const int total_mt = (a.dense_rows + BM - 1) / BM;
    const int nt = a.n_inner ? logical % ntn : logical / total_mt;
    const int mt = a.n_inner ? logical / ntn : logical - nt * total_mt;
    tc.group = 0;
    tc.row_begin = mt * BM;
    tc.rows = min(BM, a.dense_rows - tc.row_begin);
    tc.n0 = nt * BNO;
  }
  return tc;
}

// Arguments with the slot -> expert map of a placement filled in.
inline GemmArgs base_args(const Placement &pl) {
  GemmArgs a{};
  for (int g = 0; g < OCC_MAX_E; ++g) a.expert_of_group[g] = pl.expert_at[g];
  return a;
}

// Tile order of a grouped product from its shapes (the host does not know
// the groups' row counts, so their mean stands in): the 32 CUs of an XCD run
// neighbouring tiles together.  With the m-tiles fastest a group's rows are
// re-read once per pass over the n-tiles and each weight panel is read once;
// with the n-tiles fastest the reverse.  The n-tiles go fastest when a
// group's weights are at most half the size of its rows (stress layer
// gate/up GEMM: 12.6 MB of rows against 6.3 MB of weights per slot, 2242 ->
// 2130 us; the same order on its down GEMM, 4.7 against 3.1 MB, measured 3%
// slower, and 23% slower on the Mixtral-shaped gate/up GEMM).
inline void choose_tile_order(GemmArgs &a, int64_t rows_per_group, int64_t weight_rows) {
  // both operands have K columns: compare rows
  a.n_inner = 2 * weight_rows <= rows_per_group ? 1 : 0;
}

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

}  // namespace
}  // namespace occ
