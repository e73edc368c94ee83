// Grouped expert GEMMs on the EPD layout.
//
// Expert Coupling in MoE Pretraining, Abstract: tokens are dispatched to
// "expert networks"; Occult, Figure 4 caption: expert computing runs on the
// EPD state.  The experts are SwiGLU FFNs without biases:
//   up:   h   = silu(A W_gate^T) * (A W_up^T)    (SwiGLU fused in the epilogue)
//   down: out = h W_down^T
// EPD rows of slot g are contiguous ([slot_offset[g], slot_offset[g+1])), so
// each slot is one dense GEMM with a data-dependent row count.  The tile table
// (cumulative m-tiles per slot) is built on the device from slot_offset, so
// no host synchronisation is needed.
//
// bf16: persistent blocks, one per CU, each walking a contiguous range of
// tiles of its XCD.  A block works on a 256 x 256 x 64 tile with 2 x 4 waves
// (wave tile 128 x 64, two waves per SIMD) of v_mfma_f32_32x32x16_bf16, fp32
// accumulators.  Global tiles go through registers (raw buffer loads, one
// k-tile ahead) into double-buffered, padded LDS (row stride 72 elements =
// 144 bytes, so the 16 rows read by one MFMA operand load fall in distinct
// banks); one barrier per k-tile, placed before the last k step so that the
// next k-tile's first fragments load under that step's MFMAs.  The next
// tile's first k-tile is loaded during the epilogue.  The epilogue applies
// SwiGLU, rounds to bf16 in hardware and stages the tile in LDS, which is
// written out as 16-byte row segments.  For training steps the SwiGLU GEMM
// can also keep its pre-activations [G | U] (KEEP), staged and written the
// same way before h, so the backward need not recompute them.
#include <atomic>
#include <type_traits>

#include "occ_gemm_common.h"

namespace occ {
namespace {

// bf16 grouped GEMM.  2 x NWN waves, wave tile (BM/2) x (BN/NWN) made of
// 32x32 output blocks of v_mfma_f32_32x32x16_bf16.  Operand layout of that
// instruction: lane l supplies row (or column) l % 32 and the eight k values
// 8*(l/32) .. 8*(l/32)+7 of a 16-deep k step; output element i of lane l is
// row 8*(i/4) + 4*(l/32) + i%4, column l % 32.
template <int BM, int BN, int PF, bool SWIGLU, int NWN, bool KEEP = false>
__global__ __launch_bounds__(2 * NWN * kWave) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NT = 2 * NWN * kWave;               // 2 x NWN waves
  constexpr int WM = BM / 2, WN = BN / NWN;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int BNO = SWIGLU ? BN / 2 : BN;        // output columns per tile
  constexpr int A_CH = BM * (kBK / 8) / NT;        // 16-byte chunks per thread
  constexpr int B_CH = BN * (kBK / 8) / NT;
  static_assert(A_CH * NT == BM * (kBK / 8) && B_CH * NT == BN * (kBK / 8), "whole chunks");
  constexpr int STAGE = (BM + BN) * kLdsK;          // elements per LDS stage
  constexpr int KSTEPS = kBK / 16;
  constexpr int CLD = BNO + 8;  // staged output row stride
  static_assert(BM * CLD <= 2 * STAGE, "output staging must fit in the tile buffers");
  constexpr int GLD = BN + 8;  // staged [G | U] row stride (KEEP)
  static_assert(!KEEP || (SWIGLU && BM * GLD <= 2 * STAGE), "[G | U] staging");
  static_assert(!SWIGLU || NI % 2 == 0, "gate and up halves");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  __shared__ int32_t ts[OCC_MAX_E + 1];
  __shared__ int32_t ro[OCC_MAX_E + 1];

  // Persistent blocks (one per CU).  Blocks are dealt round-robin to the 8
  // XCDs; the blocks of XCD x walk a contiguous range of tiles, so the tiles
  // that share a weight panel run together on one XCD and share its L2.
  const int ntiles = tile_table<BM, BNO>(a, ts, ro);
  const int xcd = blockIdx.x % kXcds;
  const int nbx = gridDim.x / kXcds + (xcd < (int)(gridDim.x % kXcds) ? 1 : 0);
  const int x0 = xcd * (ntiles / kXcds) + min(xcd, ntiles % kXcds);
  const int x1 = x0 + ntiles / kXcds + (xcd < ntiles % kXcds ? 1 : 0);
  static_assert(PF == 1, "one k-tile in registers");
  // Global loads are buffer loads: one resource per operand, a per-thread
  // 32-bit byte offset fixed for the whole tile (set_offsets), and a scalar k
  // offset, so the k loop does no vector address arithmetic.  Rows are
  // clamped inside the tile, so every access is in bounds.
  const __amdgpu_buffer_rsrc_t a_rsrc = operand_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t b_rsrc = operand_rsrc(a.B, a.b_bytes);
  uint32_t a_off[A_CH], b_off[B_CH];
  auto set_offsets = [&](const TileCoord &t) {
    // the thread index is re-read (opaque to the compiler) so that per-thread
    // index arithmetic is recomputed here instead of staying live
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int ex = a.expert_of_group[t.group];
    const uint32_t a_base = (uint32_t)((int64_t)t.row_begin * a.lda * 2);
    const uint32_t b_base = (uint32_t)((int64_t)ex * a.b_group_stride * 2);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + NT * i, r = c >> 3, cc = c & 7;
      a_off[i] = a_base + (uint32_t)(((int64_t)min(r, t.rows - 1) * a.lda + cc * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + NT * i, r = c >> 3, cc = c & 7;
      // output column n of this weight row; a tile may span weight segments
      const int rr = SWIGLU ? (r < BN / 2 ? r : r - BN / 2) : r;
      const int n = t.n0 + min(rr, a.N - 1 - t.n0);
      const int sg = n / a.nseg;
      int64_t off = (int64_t)sg * a.nseg_stride + (int64_t)(n - sg * a.nseg) * a.ldb;
      if (SWIGLU && r >= BN / 2) off += a.up_offset;
      b_off[i] = b_base + (uint32_t)((off + cc * 8) * 2);
    }
  };
  // PF k-tiles in flight: a ring of PF register sets; the k loop is unrolled by
  // PF so that every set index is a compile-time constant
  u32x4 ra[PF][A_CH], rb[PF][B_CH];
#define OCC_LOAD_REGS(kt_, set_)                                                    \
  do {                                                                              \
    const int k0_ = (kt_) * kBK;                                                    \
    const int ks_ = k0_ / a.kseg;                                                   \
    const int64_t bk_ = (int64_t)ks_ * a.kseg_stride + (k0_ - ks_ * a.kseg);        \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) ra[set_][i] = __builtin_bit_cast( \
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off[i], k0_ * 2, 0));  \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) rb[set_][i] = __builtin_bit_cast( \
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_off[i], (int)bk_ * 2, 0)); \
  } while (0)
  // The next tile's first k-tile is loaded into registers right after the k
  // loop, so its latency hides behind the epilogue, where those registers
  // are free.
  int logical = x0 + (int)(blockIdx.x / kXcds);
  TileCoord tc{};
  if (logical < x1) {
    tc = tile_coord<BM, BNO>(a, ts, ro, logical);
    set_offsets(tc);
    OCC_LOAD_REGS(0, 0);
  }
  for (; logical < x1; logical += nbx) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave / NWN, wn = wave % NWN;
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

  // LDS row of each B fragment: SwiGLU pairs gate block ni with up block ni + NI/2
  int brow[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    if (SWIGLU)
      brow[ni] = ni < NI / 2 ? wn * (WN / 2) + ni * 32 : BN / 2 + wn * (WN / 2) + (ni - NI / 2) * 32;
    else
      brow[ni] = wn * WN + ni * 32;
  }
  // LDS element offsets: one lane-dependent base for the stores of the
  // staged chunks and one per operand for the fragment reads.  The chunk,
  // fragment, k-step and stage parts are compile-time constants (the k loop
  // is unrolled over the two stages), so each LDS access is a base register
  // plus an immediate offset and the per-lane addresses take few registers.
  const int w_base = (tid >> 3) * kLdsK + (tid & 7) * 8;  // chunk 0 of this thread
  constexpr int W_CHUNK = (NT / 8) * kLdsK;               // chunk i: NT/8 * i rows on
  const int frag_r = lane & 31, frag_k = (lane >> 5) * 8;
  const int a_rd = (wm * WM + frag_r) * kLdsK + frag_k;
  const int b_rd = BM * kLdsK + ((SWIGLU ? wn * (WN / 2) : wn * WN) + frag_r) * kLdsK + frag_k;
  constexpr auto a_fo = [](int mi) { return mi * 32 * kLdsK; };
  constexpr auto b_fo = [](int ni) {
    return (SWIGLU ? (ni < NI / 2 ? ni * 32 : BN / 2 + (ni - NI / 2) * 32) : ni * 32) * kLdsK;
  };

#define OCC_STORE_LDS(buf_, set_)                                                   \
  do {                                                                              \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                \
        *reinterpret_cast<u32x4 *>(smem + w_base + ((buf_) * STAGE + i * W_CHUNK)) = \
            ra[set_][i];                                                            \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                                \
        *reinterpret_cast<u32x4 *>(smem + w_base +                                  \
                                   ((buf_) * STAGE + BM * kLdsK + i * W_CHUNK)) =   \
            rb[set_][i];                                                            \
  } while (0)

  // Loads past the last k-tile re-read the last one (in bounds, L2-resident),
  // which keeps the loop branch-free.  k-tile kt multiplies from LDS stage
  // kt % 2 while, during k steps 0..KSTEPS-2, it stores k-tile kt+1 (staged
  // in registers) into the other stage and refills those registers with
  // k-tile kt+2 (A and B chunks as one sequence, spread evenly).  The k-tile's
  // one barrier follows those stores, and the last k step's MFMAs then cover
  // the LDS latency of k-tile kt+1's first fragments.
  constexpr int WSTEPS = KSTEPS - 1;
  constexpr int C_PER = (A_CH + B_CH + WSTEPS - 1) / WSTEPS;  // chunks per k step
  const int nk = a.K / kBK;
  OCC_STORE_LDS(0, 0);  // k-tile 0
  __syncthreads();
  OCC_LOAD_REGS(min(PF, nk - 1), 0);
  bf16x8v af[2][MI], bfr[2][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    af[0][mi] = *reinterpret_cast<const bf16x8v *>(smem + a_rd + a_fo(mi));
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    bfr[0][ni] = *reinterpret_cast<const bf16x8v *>(smem + b_rd + b_fo(ni));
  __builtin_amdgcn_sched_barrier(0);
  auto k_tile = [&](auto stage, int kt) {
    constexpr int P = decltype(stage)::value;  // LDS stage of this k-tile
    const int kn = min(kt + 1 + PF, nk - 1);    // k-tile refilled in this one
    const int k0n = kn * kBK;
    const int ksn = k0n / a.kseg;
    const int64_t bkn = (int64_t)ksn * a.kseg_stride + (k0n - ksn * a.kseg);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int q = ks & 1;
      // fragments of the next k step (of the next k-tile in the last step:
      // after the barrier, from the other stage) while these multiply
      const int fo = ks + 1 < KSTEPS ? P * STAGE + (ks + 1) * 16 : (1 - P) * STAGE;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[q ^ 1][mi] = *reinterpret_cast<const bf16x8v *>(smem + a_rd + (fo + a_fo(mi)));
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bfr[q ^ 1][ni] = *reinterpret_cast<const bf16x8v *>(smem + b_rd + (fo + b_fo(ni)));
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[q][ni], af[q][mi],
                                                               acc[mi][ni], 0, 0, 0);
      if (ks < WSTEPS) {
#pragma unroll
        for (int j = 0; j < C_PER; ++j) {
          const int c = ks * C_PER + j;
          if (c < A_CH) {
            *reinterpret_cast<u32x4 *>(smem + w_base + ((1 - P) * STAGE + c * W_CHUNK)) =
                ra[0][c];
            ra[0][c] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off[c], k0n * 2, 0));
          } else if (c < A_CH + B_CH) {
            const int i = c - A_CH;
            *reinterpret_cast<u32x4 *>(smem + w_base +
                                       ((1 - P) * STAGE + BM * kLdsK + i * W_CHUNK)) = rb[0][i];
            rb[0][i] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_off[i], (int)bkn * 2, 0));
          }
        }
      }
      // issue order inside the k step: the next step's fragment reads first
      // (so their latency hides under this step's MFMAs), two MFMAs, the
      // staging stores and refill loads, then the remaining MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, MI + NI, 0);  // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);        // MFMA
      if (ks < WSTEPS) {
        __builtin_amdgcn_sched_group_barrier(0x200, C_PER, 0);  // DS writes
        __builtin_amdgcn_sched_group_barrier(0x020, C_PER, 0);  // buffer loads
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MI * NI - 2, 0);  // MFMA
      __builtin_amdgcn_sched_barrier(0);
      if (ks == WSTEPS - 1) __syncthreads();
    }
  };
  for (int kb = 0; kb < nk; kb += 2) {
    k_tile(std::integral_constant<int, 0>{}, kb);
    if (kb + 1 < nk) k_tile(std::integral_constant<int, 1>{}, kb + 1);
  }
  const TileCoord cur = tc;
  if (logical + nbx < x1) {  // the next tile's first k-tile, during this epilogue
    tc = tile_coord<BM, BNO>(a, ts, ro, logical + nbx);
    set_offsets(tc);
    OCC_LOAD_REGS(0, 0);
  }

  // ---- epilogue: (SwiGLU), round to bf16, store ---------------------------
  // The weight fragment is the MFMA's first operand, so a 32 x 32 accumulator
  // block holds (output column, token) pairs: lane l has token row l % 32 and
  // the output columns 8q + 4(l / 32) + j (j < 4) in registers 4q + j, i.e.
  // four runs of 4 adjacent columns.  Each run is rounded to bf16 in hardware
  // (round to nearest even), staged in LDS with one 8-byte store and the tile
  // is written as 16-byte row segments (8-byte stores straight from registers
  // measured 2% slower for SwiGLU tiles and 16% slower for full-width ones).
  uint16_t *Cg = static_cast<uint16_t *>(a.C) + (int64_t)cur.row_begin * a.ldc + cur.n0;
  uint16_t *Cs = smem;
  const int crow = lane & 31, ccol = (lane >> 5) * 4;
  if (KEEP) {
    // [G | U] of the tile, rounded to bf16 like h's inputs, staged as 256
    // columns (gate columns, then up columns) and written to the G and U
    // halves of the kept rows
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * WM + mi * 32 + crow;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = brow[ni] + ccol;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x2v lo = {acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]};
          const f32x2v hi = {acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]};
          const u32x2 packed = {
              __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2v)),
              __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2v))};
          *reinterpret_cast<u32x2 *>(Cs + row * GLD + col + 8 * q) = packed;
        }
      }
    }
    __syncthreads();
    uint16_t *Gg = static_cast<uint16_t *>(a.gu) + (int64_t)cur.row_begin * a.ldgu + cur.n0;
    constexpr int GCH = BN / 8, HALF = GCH / 2;  // 16-byte chunks per staged row
    for (int c = tid; c < BM * GCH; c += NT) {
      const int r = c / GCH, cc = c - r * GCH;
      const int hc = cc < HALF ? cc : cc - HALF;  // chunk inside its half
      if (r < cur.rows && cur.n0 + hc * 8 < a.N)
        *reinterpret_cast<u32x4 *>(Gg + (int64_t)r * a.ldgu + (cc < HALF ? 0 : a.N) + hc * 8) =
            *reinterpret_cast<const u32x4 *>(Cs + r * GLD + cc * 8);
    }
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int row = wm * WM + mi * 32 + crow;
#pragma unroll
    for (int ni = 0; ni < (SWIGLU ? NI / 2 : NI); ++ni) {
      const int col = (SWIGLU ? wn * (WN / 2) : wn * WN) + ni * 32 + ccol;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (SWIGLU) v[j] = silu(acc[mi][ni][4 * q + j]) * acc[mi][ni + NI / 2][4 * q + j];
          else v[j] = acc[mi][ni][4 * q + j];
        }
        const f32x2v lo = {v[0], v[1]}, hi = {v[2], v[3]};
        const u32x2 packed = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2v)),
                              __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2v))};
        *reinterpret_cast<u32x2 *>(Cs + row * CLD + col + 8 * q) = packed;
      }
    }
  }
  // (every read of real data in the last k-tile came before its barrier, and
  // the last k step's reads of the other buffer are dead, so the staging
  // stores overwrite nothing still needed)
  __syncthreads();
  constexpr int RCH = BNO / 8;  // 16-byte chunks per output row
  for (int c = tid; c < BM * RCH; c += NT) {
    const int r = c / RCH, cc = c - r * RCH;
    if (r < cur.rows && cur.n0 + cc * 8 < a.N)
      *reinterpret_cast<u32x4 *>(Cg + (int64_t)r * a.ldc + cc * 8) =
          *reinterpret_cast<const u32x4 *>(Cs + r * CLD + cc * 8);
  }
  __syncthreads();  // the staging area is the next tile's first LDS stage
  }
#undef OCC_LOAD_REGS
#undef OCC_STORE_LDS
}

// fp32 layers: one thread per output element, fp32 FMAs in K order.
template <bool SWIGLU>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs a, int max_rows) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int row = (int)(gid / a.N), col = (int)(gid % a.N);
  if (row >= max_rows) return;
  int g = 0;
  if (a.row_offset != nullptr) {
    if (row >= a.row_offset[a.G]) return;
    int lo = 0, hi = a.G - 1;  // last group whose start is <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.row_offset[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    g = lo;
  } else if (row >= a.dense_rows) {
    return;
  }
  const float *A = static_cast<const float *>(a.A) + (int64_t)row * a.lda;
  const int nsg = col / a.nseg;
  const float *Bn = static_cast<const float *>(a.B) + (int64_t)a.expert_of_group[g] * a.b_group_stride +
                    (int64_t)nsg * a.nseg_stride + (int64_t)(col - nsg * a.nseg) * a.ldb;
  float s0 = 0.0f, s1 = 0.0f;
  for (int k = 0; k < a.K; ++k) {
    const int ks = k / a.kseg;
    const int64_t bk = (int64_t)ks * a.kseg_stride + (k - ks * a.kseg);
    s0 = __builtin_fmaf(A[k], Bn[bk], s0);
    if (SWIGLU) s1 = __builtin_fmaf(A[k], Bn[a.up_offset + bk], s1);
  }
  const float v = SWIGLU ? silu(s0) * s1 : s0;
  static_cast<float *>(a.C)[(int64_t)row * a.ldc + col] = v;
}

template <int BM, int BN, int PF, bool SWIGLU, int NWN, bool KEEP = false>
void launch_bf16(const GemmArgs &a, int max_rows, int n_cu, hipStream_t st) {
  constexpr int BNO = SWIGLU ? BN / 2 : BN;
  // worst case over all splits of max_rows rows into the groups
  const int64_t groups = a.row_offset != nullptr ? a.G : 1;
  const int64_t mt = (max_rows + groups * (BM - 1)) / BM;
  const int64_t tiles = mt * ((a.N + BNO - 1) / BNO);
  // one persistent block per CU (a block fills a CU's LDS)
  const int64_t grid = tiles < n_cu ? tiles : n_cu;
  gemm_bf16_kernel<BM, BN, PF, SWIGLU, NWN, KEEP><<<(unsigned)grid, 2 * NWN * kWave, 0, st>>>(a);
}

template <bool SWIGLU>
hipError_t run_gemm(const GemmArgs &a, int dtype, int max_rows, hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  if (dtype == OCC_F32) {
    const int64_t n = (int64_t)max_rows * a.N;
    gemm_f32_kernel<SWIGLU><<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        a, max_rows);
    return hipGetLastError();
  }
  const int n_cu = device_cu_count();
  if (n_cu <= 0) return hipGetLastError();
  // 8 waves (2 x 4, two per SIMD, 128 x 64 wave tiles): against 4 waves of
  // 128 x 128 the LDS serves about 1.7 times the fragment bandwidth, which
  // bounds the k loop (same-process A/B on the OLMoE-shaped layer: gate/up
  // 325 -> 297 us with the barrier before the last k step; 4 waves with the
  // barrier at the end of the k-tile measured faster than 8).
  if (SWIGLU && a.gu != nullptr) launch_bf16<256, 256, 1, true, 4, true>(a, max_rows, n_cu, st);
  else if (SWIGLU) launch_bf16<256, 256, 1, true, 4>(a, max_rows, n_cu, st);
  else launch_bf16<256, 256, 1, false, 4>(a, max_rows, n_cu, st);
  return hipGetLastError();
}

}  // namespace

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxDevices) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess
               ? n : 0;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 0;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_expert_up(const occ_layer_desc &L, const void *epd, const int32_t *slot_offset,
                            const Placement &pl, const void *w_gate_up, void *h, const void *x,
                            const void *w_gate_up_sh, void *h_sh, hipStream_t st, void *gu) {
  const int64_t d = L.d, I = L.I;
  GemmArgs a = base_args(pl);
  a.row_offset = slot_offset;
  a.G = L.E;
  a.A = epd;
  a.lda = d;
  a.B = w_gate_up;
  a.ldb = d;
  a.b_group_stride = 2 * I * d;
  a.a_bytes = (int64_t)L.T * L.k * d * 2;
  a.b_bytes = (int64_t)L.E * 2 * I * d * 2;
  a.up_offset = I * d;
  a.nseg = (int)I;
  a.nseg_stride = 0;
  a.kseg = (int)d;
  a.kseg_stride = 0;
  a.K = (int)d;
  a.N = (int)I;
  a.C = h;
  a.ldc = I;
  a.gu = gu;
  a.ldgu = 2 * I;
  choose_tile_order(a, (int64_t)L.T * L.k / L.E, 2 * I);
  hipError_t err = run_gemm<true>(a, L.dtype, L.T * L.k, st);
  if (err != hipSuccess || L.n_shared == 0) return err;
  const int64_t Is = L.I_shared;
  GemmArgs s{};
  s.row_offset = nullptr;
  s.G = 1;
  s.dense_rows = L.T;
  s.A = x;
  s.lda = d;
  s.B = w_gate_up_sh;
  s.ldb = d;
  s.b_group_stride = 0;
  s.a_bytes = (int64_t)L.T * d * 2;
  s.b_bytes = (int64_t)L.n_shared * 2 * Is * d * 2;
  s.up_offset = Is * d;
  s.nseg = (int)Is;
  s.nseg_stride = 2 * Is * d;
  s.kseg = (int)d;
  s.kseg_stride = 0;
  s.K = (int)d;
  s.N = (int)(L.n_shared * Is);
  s.C = h_sh;
  s.ldc = L.n_shared * Is;
  choose_tile_order(s, L.T, 2 * L.n_shared * Is);
  return run_gemm<true>(s, L.dtype, L.T, st);
}

hipError_t launch_expert_down(const occ_layer_desc &L, const int32_t *slot_offset,
                              const Placement &pl, const void *w_down, const void *h,
                              void *out_epd, const void *w_down_sh, const void *h_sh,
                              void *shared_out, hipStream_t st) {
  const int64_t d = L.d, I = L.I;
  GemmArgs a = base_args(pl);
  a.row_offset = slot_offset;
  a.G = L.E;
  a.A = h;
  a.lda = I;
  a.B = w_down;
  a.ldb = I;
  a.b_group_stride = d * I;
  a.a_bytes = (int64_t)L.T * L.k * I * 2;
  a.b_bytes = (int64_t)L.E * d * I * 2;
  a.up_offset = 0;
  a.nseg = (int)d;
  a.nseg_stride = 0;
  a.kseg = (int)I;
  a.kseg_stride = 0;
  a.K = (int)I;
  a.N = (int)d;
  a.C = out_epd;
  a.ldc = d;
  choose_tile_order(a, (int64_t)L.T * L.k / L.E, d);
  hipError_t err = run_gemm<false>(a, L.dtype, L.T * L.k, st);
  if (err != hipSuccess || L.n_shared == 0) return err;
  const int64_t Is = L.I_shared;
  GemmArgs s{};
  s.row_offset = nullptr;
  s.G = 1;
  s.dense_rows = L.T;
  s.A = h_sh;
  s.lda = L.n_shared * Is;
  s.B = w_down_sh;
  s.ldb = Is;
  s.b_group_stride = 0;
  s.a_bytes = (int64_t)L.T * L.n_shared * Is * 2;
  s.b_bytes = (int64_t)L.n_shared * d * Is * 2;
  s.up_offset = 0;
  s.nseg = (int)d;
  s.nseg_stride = 0;
  s.kseg = (int)Is;
  s.kseg_stride = d * Is;
  s.K = (int)(L.n_shared * Is);
  s.N = (int)d;
  s.C = shared_out;
  s.ldc = d;
  choose_tile_order(s, L.T, d);
  return run_gemm<false>(s, L.dtype, L.T, st);
}

}  // namespace occ
