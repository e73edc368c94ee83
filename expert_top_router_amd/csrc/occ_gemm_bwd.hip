// Grouped GEMMs of the expert backward (bf16).
//
// Expert Coupling in MoE Pretraining, Abstract: every MoE layer runs its
// all-to-alls in the forward and the backward pass; Occult, Figure 4 caption:
// expert computing runs on the EPD state.  For the SwiGLU experts
// (h = silu(G) U, out = h W_down^T) the backward of one slot needs
//   [G | U] = EPD W_gate_up^T                    (recomputed, as in the forward)
//   dh      = d_out W_down                       (W_down[e] stored [d][I])
//   dG = dh U silu'(G),  dU = dh silu(G)          (fused into dh's epilogue)
//   d_EPD   = [dG | dU] W_gate_up                 (W_gate_up[e] stored [2I][d])
//   dW_down[e]    = sum over the slot's rows of d_out^T h
//   dW_gate_up[e] = sum over the slot's rows of [dG | dU]^T EPD
// Three of them read an operand whose contiguous dimension is not K: the
// weights as stored, and both operands of the weight gradients, where K runs
// over the rows of a slot.
//
// gemm_bwd_kernel keeps the forward kernel's structure: persistent blocks
// dealt to the XCDs in contiguous tile ranges, 2 x NWN waves on a 256 x 256 x
// 64 tile of v_mfma_f32_32x32x16_bf16, global tiles through registers (one
// k-tile ahead) into double-buffered LDS, the stores of the next tile and the
// loads of the one after interleaved with the first three MFMA k steps, then
// the k-tile's one barrier, so the last k step covers the LDS latency of the
// next tile's first fragments.  The activation-gradient GEMMs run 8 waves
// (two per SIMD: 7-12% faster than 4 on the OLMoE-shaped layer); the weight
// gradients, whose fp32 output stores dominate their epilogue, keep 4.
// Per operand, the layout in memory decides the layout in LDS:
//   layout 0 (K-contiguous rows): LDS [row][K], row stride 72 elements; an
//     MFMA operand (8 consecutive k of one row) is one 16-byte LDS read.
//   layout 1 (rows of K, M or N contiguous): LDS [k][row], copied as stored,
//     row stride 288 elements (576 bytes: the four k rows that one 16-lane
//     group reads start 64 bytes apart modulo 256, so a half wave touches
//     every bank once); an MFMA operand is two ds_read_b64_tr_b16, the CDNA4
//     LDS transpose read (within 16 lanes, lane i receives element i % 4 of
//     the 8 bytes read by lane 4j + i / 4, j = 0..3).
// GK: K is grouped (rows [row_offset[g], row_offset[g+1]) of slot g); the
// operands' buffer resources end at the slot's last row, so rows past it in
// the last k-tile load as zero (the buffer unit's range check).
#include "occ_gemm_common.h"

namespace occ {
namespace {

enum { EPI_BF16 = 0, EPI_SWIGLU_BWD = 1, EPI_F32 = 2 };

constexpr int kLdsMN = 256 + 32;  // layout-1 LDS row stride (elements)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA operand (8 consecutive k of one row) from a layout-1 LDS tile: p is the
// lane's address for k rows 0..3 of the 8, computed by mn_frag_base.
__device__ __forceinline__ bf16x8v lds_tr8(const uint16_t *p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * kLdsMN));
  return __builtin_bit_cast(bf16x8v, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Lane offset (elements) of a layout-1 operand read for the 32 rows starting
// at row 0 of the tile: lane l needs row l % 32 and k 8(l/32) .. +7; in its
// group of 16 lanes, the lane with index r reads k row r / 4 (+4 for the
// second read) at rows 16 ((l / 16) % 2) + 4 (r % 4) .. +3.
__device__ __forceinline__ int mn_frag_base(int lane) {
  const int r = lane & 15;
  return (8 * (lane >> 5) + (r >> 2)) * kLdsMN + 16 * ((lane >> 4) & 1) + 4 * (r & 3);
}

__device__ __forceinline__ float silu_grad(float g, float sg) {  // d silu / dg, sg = sigmoid(g)
  return sg * (1.0f + g * (1.0f - sg));
}

template <int ALAY, int BLAY, bool GK, int EPI, int NWN>
__global__ __launch_bounds__(2 * NWN * kWave) void gemm_bwd_kernel(GemmArgs a) {
  constexpr int BM = 256, BN = 256, NT = 2 * NWN * kWave, WM = 128, WN = BN / NWN, MI = 4,
                NI = WN / 32;
  constexpr int CH = BM * (kBK / 8) / NT;  // 16-byte chunks per thread and operand per k-tile
  constexpr int A_SZ = ALAY == 0 ? BM * kLdsK : kBK * kLdsMN;
  constexpr int B_SZ = BLAY == 0 ? BN * kLdsK : kBK * kLdsMN;
  constexpr int STAGE = A_SZ + B_SZ;
  constexpr int CLD = BN + 8;
  constexpr int KSTEPS = kBK / 16;
  static_assert(BM * CLD <= 2 * STAGE, "output staging must fit in the tile buffers");
  static_assert(!GK || (ALAY == 1 && BLAY == 1), "grouped K reads rows of K");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  __shared__ int32_t ts[OCC_MAX_E + 1];
  __shared__ int32_t ro[OCC_MAX_E + 1];
  __shared__ int32_t byrank[OCC_MAX_E];

  const int ntn = (a.N + BN - 1) / BN;
  const int ntm = GK ? (a.M + BM - 1) / BM : 0;
  // Blocks are dealt round-robin to the XCDs (nx groups when the grid is
  // smaller); the blocks of group x walk its tiles with stride nbx.
  const int nx = min((int)gridDim.x, kXcds);
  const int xcd = blockIdx.x % nx;
  const int nbx = gridDim.x / nx + (xcd < (int)(gridDim.x % nx) ? 1 : 0);
  int x0, x1;
  if (GK) {
    // A slot's tiles all contract over its rows, so a tile costs about its
    // slot's row count.  Slots are ranked by rows (descending, lower slot on
    // ties) and dealt to the groups in snake order (0..nx-1, nx-1..0, ...):
    // the j-th slot of group x has rank nx j + (j even ? x : nx - 1 - x).
    // no row offsets: one group of dense_rows rows (the shared experts)
    for (int g = threadIdx.x; g <= a.G; g += blockDim.x)
      ro[g] = a.row_offset != nullptr ? a.row_offset[g] : (g == 0 ? 0 : a.dense_rows);
    __syncthreads();
    for (int g = threadIdx.x; g < a.G; g += blockDim.x) {
      const int rg = ro[g + 1] - ro[g];
      int r = 0;
      for (int h = 0; h < a.G; ++h) {
        const int rh = ro[h + 1] - ro[h];
        r += (rh > rg || (rh == rg && h < g)) ? 1 : 0;
      }
      byrank[r] = g;
    }
    __syncthreads();
    if (a.row_offset != nullptr) {
      int nslot = 0;
      for (int j = 0; nx * j + ((j & 1) ? nx - 1 - xcd : xcd) < a.G; ++j) ++nslot;
      x0 = 0;
      x1 = nslot * ntm * ntn;
    } else {
      // one group: its tiles in contiguous ranges per XCD group
      const int ntiles = ntm * ntn;
      x0 = xcd * (ntiles / nx) + min(xcd, ntiles % nx);
      x1 = x0 + ntiles / nx + (xcd < ntiles % nx ? 1 : 0);
    }
  } else {
    // tiles in slot order, contiguous ranges per group
    const int ntiles = tile_table<BM, BN>(a, ts, ro);
    x0 = xcd * (ntiles / nx) + min(xcd, ntiles % nx);
    x1 = x0 + ntiles / nx + (xcd < ntiles % nx ? 1 : 0);
  }
  const __amdgpu_buffer_rsrc_t a_rsrc = operand_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t b_rsrc = operand_rsrc(a.B, a.b_bytes);
  for (int logical = x0 + (int)(blockIdx.x / nx); logical < x1; logical += nbx) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave / NWN, wn = wave % NWN;
  // tile: output rows [m0, m0 + mrows), columns [n0, ...), K rows [k_lo, k_hi)
  int group, m0, mrows, n0, k_lo, k_hi;
  if (GK) {
    const int j = a.row_offset != nullptr ? logical / (ntm * ntn) : 0;
    group = a.row_offset != nullptr ? byrank[nx * j + ((j & 1) ? nx - 1 - xcd : xcd)] : 0;
    const int rem = logical - j * ntm * ntn;
    const int nt = rem / ntm, mt = rem - nt * ntm;
    m0 = mt * BM;
    mrows = min(BM, a.M - m0);
    n0 = nt * BN;
    k_lo = ro[group];
    k_hi = ro[group + 1];
  } else {
    const TileCoord tc = tile_coord<BM, BN>(a, ts, ro, logical);
    group = tc.group;
    m0 = tc.row_begin;
    mrows = tc.rows;
    n0 = tc.n0;
    k_lo = 0;
    k_hi = a.K;
  }
  // tile coordinates are uniform over the block: keep them in scalar registers
  group = __builtin_amdgcn_readfirstlane(group);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  mrows = __builtin_amdgcn_readfirstlane(mrows);
  n0 = __builtin_amdgcn_readfirstlane(n0);
  k_lo = __builtin_amdgcn_readfirstlane(k_lo);
  k_hi = __builtin_amdgcn_readfirstlane(k_hi);
  const int expert = a.expert_of_group[group];
  const int64_t b_base = GK ? 0 : (int64_t)expert * a.b_group_stride;

  // Per-thread chunk c = tid + NT * i.  Layout 0: tile row c / 8, k chunk c % 8
  // (voffset fixed per tile, k in the scalar offset).  Layout 1: k row
  // c / 32 = tid / 32 + 8 i, column chunk tid % 32 (the same for every i).
  uint32_t a_off[CH], b_off[CH];
  int a_dst[CH], b_dst[CH];
  const int mn_kr = tid >> 5, mn_col = (tid & 31) * 8;
  const int a_col = min(m0 + mn_col, (GK ? a.M : m0 + mrows) - 8);  // layout 1
  const int b_col = min(n0 + mn_col, a.N - 8);                       // layout 1
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + NT * i;
    if (ALAY == 0) {
      a_off[i] = (uint32_t)(((int64_t)(m0 + min(c >> 3, mrows - 1)) * a.lda + (c & 7) * 8) * 2);
      a_dst[i] = (c >> 3) * kLdsK + (c & 7) * 8;
    } else {
      a_off[i] = (uint32_t)(((int64_t)(k_lo + mn_kr + (NT / 32) * i) * a.lda + a_col) * 2);
      a_dst[i] = (mn_kr + (NT / 32) * i) * kLdsMN + mn_col;
    }
    if (BLAY == 0) {
      const int n = n0 + min(c >> 3, a.N - 1 - n0);
      b_off[i] = (uint32_t)((b_base + (int64_t)n * a.ldb + (c & 7) * 8) * 2);
      b_dst[i] = A_SZ + (c >> 3) * kLdsK + (c & 7) * 8;
    } else {
      b_off[i] = (uint32_t)((b_base + (int64_t)(k_lo + mn_kr + (NT / 32) * i) * a.ldb + b_col) * 2);
      b_dst[i] = A_SZ + (mn_kr + (NT / 32) * i) * kLdsMN + mn_col;
    }
  }

  // Loads of chunk i of the k-tile starting at K row k0 (relative to k_lo).
  // Layout 0: fixed per-lane offset, k in the scalar offset.  Layout 1 with a
  // fixed K: fixed per-lane offset, k row in the scalar offset.  Grouped K:
  // the operand's buffer resource ends at the slot's last row (k_hi), and the
  // whole offset goes into the per-lane offset, which the buffer unit checks
  // against that size: rows at or past k_hi in the last k-tile read as zero
  // and touch no memory.
  const __amdgpu_buffer_rsrc_t ga_rsrc =
      GK ? operand_rsrc(a.A, (int64_t)k_hi * a.lda * 2) : a_rsrc;
  const __amdgpu_buffer_rsrc_t gb_rsrc =
      GK ? operand_rsrc(a.B, (int64_t)k_hi * a.ldb * 2) : b_rsrc;
  auto load_a = [&](int i, int k0) -> u32x4 {
    if (ALAY == 0)
      return __builtin_bit_cast(u32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off[i], k0 * 2, 0));
    if (!GK)
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           a_rsrc, a_off[i], (int)((int64_t)k0 * a.lda * 2), 0));
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         ga_rsrc, a_off[i] + (uint32_t)(k0 * a.lda * 2), 0, 0));
  };
  auto load_b = [&](int i, int k0) -> u32x4 {
    if (BLAY == 0)
      return __builtin_bit_cast(u32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_off[i], k0 * 2, 0));
    if (!GK)
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           b_rsrc, b_off[i], (int)((int64_t)k0 * a.ldb * 2), 0));
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         gb_rsrc, b_off[i] + (uint32_t)(k0 * a.ldb * 2), 0, 0));
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;

  // fragment addresses (k step 0) of the wave's 32-row blocks
  const int frag_r = lane & 31, frag_k = (lane >> 5) * 8;
  const int mnb = mn_frag_base(lane);
  int a_frag[MI], b_frag[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    a_frag[mi] = ALAY == 0 ? (wm * WM + mi * 32 + frag_r) * kLdsK + frag_k
                           : mnb + wm * WM + mi * 32;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    b_frag[ni] = A_SZ + (BLAY == 0 ? (wn * WN + ni * 32 + frag_r) * kLdsK + frag_k
                                   : mnb + wn * WN + ni * 32);
  auto frag_a = [&](const uint16_t *S, int mi, int ks) -> bf16x8v {
    if (ALAY == 0) return *reinterpret_cast<const bf16x8v *>(S + a_frag[mi] + ks * 16);
    return lds_tr8(S + a_frag[mi] + ks * 16 * kLdsMN);
  };
  auto frag_b = [&](const uint16_t *S, int ni, int ks) -> bf16x8v {
    if (BLAY == 0) return *reinterpret_cast<const bf16x8v *>(S + b_frag[ni] + ks * 16);
    return lds_tr8(S + b_frag[ni] + ks * 16 * kLdsMN);
  };

  const int nk = k_hi > k_lo ? (k_hi - k_lo + kBK - 1) / kBK : 0;
  if (nk > 0) {
    u32x4 ra[CH], rb[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      ra[i] = load_a(i, 0);
      rb[i] = load_b(i, 0);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      *reinterpret_cast<u32x4 *>(smem + a_dst[i]) = ra[i];
      *reinterpret_cast<u32x4 *>(smem + b_dst[i]) = rb[i];
    }
    __syncthreads();
    {
      const int k1 = min(1, nk - 1) * kBK;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        ra[i] = load_a(i, k1);
        rb[i] = load_b(i, k1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Step kt multiplies tile kt while, during k steps 0..KSTEPS-2, it stores
    // tile kt + 1 (in registers) into the other buffer and refills the
    // registers with tile kt + 2 (clamped to the last tile: re-reads stay in
    // bounds and are unused).  The step's one barrier follows those stores,
    // and the last k step's MFMAs cover the LDS latency of tile kt + 1's first
    // fragments.
    constexpr int WSTEPS = KSTEPS - 1;
    constexpr int C_PER = (2 * CH + WSTEPS - 1) / WSTEPS;  // chunks stored per k step
    bf16x8v af[2][MI], bfr[2][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) af[0][mi] = frag_a(smem, mi, 0);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) bfr[0][ni] = frag_b(smem, ni, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const uint16_t *S = smem + (kt & 1) * STAGE;
      uint16_t *Wn = smem + ((kt + 1) & 1) * STAGE;
      const int kn = min(kt + 2, nk - 1) * kBK;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int q = ks & 1;
        // fragments of the next k step (of the next tile in the last step:
        // after the barrier, from the other buffer)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          af[q ^ 1][mi] = ks + 1 < KSTEPS ? frag_a(S, mi, ks + 1) : frag_a(Wn, mi, 0);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bfr[q ^ 1][ni] = ks + 1 < KSTEPS ? frag_b(S, ni, ks + 1) : frag_b(Wn, ni, 0);
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
            if (c < CH) {
              *reinterpret_cast<u32x4 *>(Wn + a_dst[c]) = ra[c];
              ra[c] = load_a(c, kn);
            } else if (c < 2 * CH) {
              *reinterpret_cast<u32x4 *>(Wn + b_dst[c - CH]) = rb[c - CH];
              rb[c - CH] = load_b(c - CH, kn);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ks == WSTEPS - 1) __syncthreads();
      }
    }
  }

  // ---- epilogue (lane l: output row l % 32, columns 8q + 4(l/32) + j) -------
  const int crow = lane & 31, ccol = (lane >> 5) * 4;
  if (EPI == EPI_F32) {
    // nseg > 0: output column n is column n % nseg of the matrix at
    // (n / nseg) * nseg_stride (a product over several matrices side by side;
    // nseg is a multiple of 4, so a lane's run of 4 columns stays in one)
    float *Cg = static_cast<float *>(a.C) + (int64_t)expert * a.c_group_stride;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * WM + mi * 32 + crow;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * WN + ni * 32 + ccol + 8 * q;
          const int n = n0 + col;
          const int64_t co = a.nseg > 0 ? (int64_t)(n / a.nseg) * a.nseg_stride + n % a.nseg : n;
          if (row < mrows && n < a.N)
            *reinterpret_cast<float4 *>(Cg + (int64_t)(m0 + row) * a.ldc + co) =
                make_float4(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                            acc[mi][ni][4 * q + 3]);
        }
    }
  } else {
    // bf16 rows staged in LDS and written with 16-byte stores; the SwiGLU
    // backward writes dG (columns [0, N)) and dU ([N, 2N)).  It reads G and U
    // once, in two halves of the tile's rows (each wave's 32-row blocks 0-1,
    // then 2-3): a half's dG and dU rows are staged side by side (2 x 128
    // rows) and written out before the next half.
    constexpr int RCH = BN / 8;
    const uint16_t *GU = static_cast<const uint16_t *>(a.aux);
    if (EPI == EPI_SWIGLU_BWD) {
      static_assert(MI == 4 && 2 * (BM / 2) * CLD <= 2 * STAGE, "two half tiles staged");
      uint16_t *CsG = smem, *CsU = smem + (BM / 2) * CLD;
      int prow = crow;
      asm volatile("" : "+v"(prow));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) {
          const int mi = 2 * half + mh;
          const int row = wm * WM + mi * 32 + prow;   // tile row
          const int srow = wm * (WM / 2) + mh * 32 + prow;  // staging row
          const int grow = m0 + min(row, mrows - 1);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int col = wn * WN + ni * 32 + ccol;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int gc = min(n0 + col + 8 * q, a.N - 4);
              const u32x2 gp = *reinterpret_cast<const u32x2 *>(GU + (int64_t)grow * a.ldaux + gc);
              const u32x2 up =
                  *reinterpret_cast<const u32x2 *>(GU + (int64_t)grow * a.ldaux + a.N + gc);
              const float gv[4] = {__uint_as_float(gp.x << 16), __uint_as_float(gp.x & 0xffff0000u),
                                   __uint_as_float(gp.y << 16), __uint_as_float(gp.y & 0xffff0000u)};
              const float uv[4] = {__uint_as_float(up.x << 16), __uint_as_float(up.x & 0xffff0000u),
                                   __uint_as_float(up.y << 16), __uint_as_float(up.y & 0xffff0000u)};
              float vg[4], vu[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float dh = acc[mi][ni][4 * q + j];
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[j]));
                vg[j] = dh * uv[j] * silu_grad(gv[j], sg);
                vu[j] = dh * gv[j] * sg;
              }
              const f32x2v glo = {vg[0], vg[1]}, ghi = {vg[2], vg[3]};
              const f32x2v ulo = {vu[0], vu[1]}, uhi = {vu[2], vu[3]};
              *reinterpret_cast<u32x2 *>(CsG + srow * CLD + col + 8 * q) = u32x2{
                  __builtin_bit_cast(uint32_t, __builtin_convertvector(glo, bf16x2v)),
                  __builtin_bit_cast(uint32_t, __builtin_convertvector(ghi, bf16x2v))};
              *reinterpret_cast<u32x2 *>(CsU + srow * CLD + col + 8 * q) = u32x2{
                  __builtin_bit_cast(uint32_t, __builtin_convertvector(ulo, bf16x2v)),
                  __builtin_bit_cast(uint32_t, __builtin_convertvector(uhi, bf16x2v))};
            }
          }
          // one 32-row block at a time: keeps the G / U loads from being
          // hoisted all together (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        uint16_t *Cg = static_cast<uint16_t *>(a.C) + (int64_t)m0 * a.ldc + n0;
        for (int c = tid; c < 2 * (BM / 2) * RCH; c += NT) {
          const int part = c / ((BM / 2) * RCH);        // 0: dG, 1: dU
          const int cr = c - part * (BM / 2) * RCH;
          const int sr = cr / RCH, cc = cr - sr * RCH;
          // staging row sr is tile row (sr / 64) * 128 + 64 half + sr % 64
          const int r = (sr / (WM / 2)) * WM + half * (WM / 2) + sr % (WM / 2);
          const uint16_t *src = (part ? CsU : CsG) + sr * CLD + cc * 8;
          if (r < mrows && n0 + cc * 8 < a.N)
            *reinterpret_cast<u32x4 *>(Cg + (int64_t)r * a.ldc + part * a.N + cc * 8) =
                *reinterpret_cast<const u32x4 *>(src);
        }
        __syncthreads();
      }
    } else {
    constexpr int PASSES = 1;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      uint16_t *Cs = smem;
      // opaque per pass: G and U are re-read in pass 1 rather than kept live
      int prow = crow;
      asm volatile("" : "+v"(prow));
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * WM + mi * 32 + prow;
        const int grow = m0 + min(row, mrows - 1);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = wn * WN + ni * 32 + ccol;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
            if (EPI == EPI_SWIGLU_BWD) {
              const int gc = min(n0 + col + 8 * q, a.N - 4);
              const u32x2 gp = *reinterpret_cast<const u32x2 *>(GU + (int64_t)grow * a.ldaux + gc);
              const u32x2 up =
                  *reinterpret_cast<const u32x2 *>(GU + (int64_t)grow * a.ldaux + a.N + gc);
              const float gv[4] = {__uint_as_float(gp.x << 16), __uint_as_float(gp.x & 0xffff0000u),
                                   __uint_as_float(gp.y << 16), __uint_as_float(gp.y & 0xffff0000u)};
              const float uv[4] = {__uint_as_float(up.x << 16), __uint_as_float(up.x & 0xffff0000u),
                                   __uint_as_float(up.y << 16), __uint_as_float(up.y & 0xffff0000u)};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float dh = acc[mi][ni][4 * q + j];
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[j]));
                v[j] = pass == 0 ? dh * uv[j] * silu_grad(gv[j], sg) : dh * gv[j] * sg;
              }
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) v[j] = acc[mi][ni][4 * q + j];
            }
            const f32x2v lo = {v[0], v[1]}, hi = {v[2], v[3]};
            const u32x2 packed = {
                __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2v)),
                __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2v))};
            *reinterpret_cast<u32x2 *>(Cs + row * CLD + col + 8 * q) = packed;
          }
        }
        // one 32-row block at a time: keeps the G / U loads from being
        // hoisted all together (register pressure)
        if (EPI == EPI_SWIGLU_BWD) __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      uint16_t *Cg = static_cast<uint16_t *>(a.C) + (int64_t)m0 * a.ldc + n0 + pass * a.N;
      for (int c = tid; c < BM * RCH; c += NT) {
        const int r = c / RCH, cc = c - r * RCH;
        if (r < mrows && n0 + cc * 8 < a.N)
          *reinterpret_cast<u32x4 *>(Cg + (int64_t)r * a.ldc + cc * 8) =
              *reinterpret_cast<const u32x4 *>(Cs + r * CLD + cc * 8);
      }
      __syncthreads();
    }
    }
  }
  __syncthreads();  // the staging area is the next tile's first LDS stage
  }
}

template <int ALAY, int BLAY, bool GK, int EPI, int NWN>
hipError_t launch_bwd(const GemmArgs &a, int64_t tiles, hipStream_t st) {
  if (tiles <= 0) return hipSuccess;
  const int n_cu = device_cu_count();
  if (n_cu <= 0) return hipGetLastError();
  const int64_t grid = tiles < n_cu ? tiles : n_cu;
  gemm_bwd_kernel<ALAY, BLAY, GK, EPI, NWN><<<(unsigned)grid, 2 * NWN * kWave, 0, st>>>(a);
  return hipGetLastError();
}

// upper bound of the tiles of a slot-grouped product with max_rows rows
int64_t grouped_tiles(int max_rows, int G, int N) {
  return ((int64_t)max_rows + (int64_t)G * 255) / 256 * ((N + 255) / 256);
}

}  // namespace

hipError_t launch_expert_backward(const occ_layer_desc &L, const int32_t *slot_offset,
                                  const Placement &pl, const void *epd, const void *w_gate_up,
                                  const void *w_down, const void *h, const void *d_out_epd,
                                  void *gu, void *dgu, void *d_epd, float *dw_gate_up,
                                  float *dw_down, hipStream_t st, bool recompute_gu) {
  if (L.dtype == OCC_F32)
    return launch_expert_backward_f32(L, slot_offset, pl, epd, w_gate_up, w_down, h, d_out_epd,
                                      gu, dgu, d_epd, dw_gate_up, dw_down, st);
  const int64_t d = L.d, I = L.I, R = (int64_t)L.T * L.k, E = L.E;
  hipError_t err;
  // 1. [G | U] = EPD W_gate_up^T, recomputed and stored in bf16
  GemmArgs a = base_args(pl);
  a.row_offset = slot_offset;
  a.G = L.E;
  a.A = epd;
  a.lda = d;
  a.a_bytes = R * d * 2;
  a.B = w_gate_up;
  a.ldb = d;
  a.b_group_stride = 2 * I * d;
  a.b_bytes = E * 2 * I * d * 2;
  a.K = (int)d;
  a.N = (int)(2 * I);
  a.C = gu;
  a.ldc = 2 * I;
  choose_tile_order(a, R / E, 2 * I);
  // (skipped when the forward kept them: the same products, same rounding)
  if (recompute_gu &&
      (err = launch_bwd<0, 0, false, EPI_BF16, 4>(a, grouped_tiles((int)R, L.E, a.N), st)) !=
          hipSuccess)
    return err;
  // 2. dh = d_out_EPD W_down (W_down[e] is [d][I]); SwiGLU backward -> [dG | dU]
  a = base_args(pl);
  a.row_offset = slot_offset;
  a.G = L.E;
  a.A = d_out_epd;
  a.lda = d;
  a.a_bytes = R * d * 2;
  a.B = w_down;
  a.ldb = I;
  a.b_group_stride = d * I;
  a.b_bytes = E * d * I * 2;
  a.K = (int)d;
  a.N = (int)I;
  a.aux = gu;
  a.ldaux = 2 * I;
  a.C = dgu;
  a.ldc = 2 * I;
  choose_tile_order(a, R / E, I);
  if ((err = launch_bwd<0, 1, false, EPI_SWIGLU_BWD, 4>(a, grouped_tiles((int)R, L.E, a.N), st)) !=
      hipSuccess)
    return err;
  // 3. dW_down[e] = sum over the slot's rows of d_out_EPD^T h   ([d][I], fp32)
  a = base_args(pl);
  a.row_offset = slot_offset;
  a.G = L.E;
  a.A = d_out_epd;
  a.lda = d;
  a.a_bytes = R * d * 2;
  a.M = (int)d;
  a.B = h;
  a.ldb = I;
  a.b_bytes = R * I * 2;
  a.N = (int)I;
  a.C = dw_down;
  a.ldc = I;
  a.c_group_stride = d * I;
  if ((err = launch_bwd<1, 1, true, EPI_F32, 2>(a, E * ((d + 255) / 256) * ((I + 255) / 256), st)) !=
      hipSuccess)
    return err;
  // 4. dW_gate_up[e] = sum over the slot's rows of [dG | dU]^T EPD   ([2I][d], fp32)
  a = base_args(pl);
  a.row_offset = slot_offset;
  a.G = L.E;
  a.A = dgu;
  a.lda = 2 * I;
  a.a_bytes = R * 2 * I * 2;
  a.M = (int)(2 * I);
  a.B = epd;
  a.ldb = d;
  a.b_bytes = R * d * 2;
  a.N = (int)d;
  a.C = dw_gate_up;
  a.ldc = d;
  a.c_group_stride = 2 * I * d;
  if ((err = launch_bwd<1, 1, true, EPI_F32, 2>(a, E * ((2 * I + 255) / 256) * ((d + 255) / 256),
                                               st)) != hipSuccess)
    return err;
  // 5. dEPD = [dG | dU] W_gate_up (W_gate_up[e] is [2I][d]).  Last, so that
  // the write-back of the weight gradients' fp32 tiles from the caches
  // overlaps this MFMA-bound GEMM rather than the memory-bound kernels that
  // follow the call (measured: the backward sequence 1830 -> 1783 us on the
  // OLMoE-shaped layer)
  a = base_args(pl);
  a.row_offset = slot_offset;
  a.G = L.E;
  a.A = dgu;
  a.lda = 2 * I;
  a.a_bytes = R * 2 * I * 2;
  a.B = w_gate_up;
  a.ldb = d;
  a.b_group_stride = 2 * I * d;
  a.b_bytes = E * 2 * I * d * 2;
  a.K = (int)(2 * I);
  a.N = (int)d;
  a.C = d_epd;
  a.ldc = d;
  choose_tile_order(a, R / E, d);
  return launch_bwd<0, 1, false, EPI_BF16, 4>(a, grouped_tiles((int)R, L.E, a.N), st);
}

// Backward of the shared experts (always active, weight 1, on the ORI rows
// X): per shared expert s, on its own columns of the [T][n_sh * 2 I_sh]
// buffers gu and dgu,
//   [G | U]_s = X W_gate_up_sh[s]^T                      (recomputed, bf16)
//   dh_s      = dY W_down_sh[s];  [dG | dU]_s by the SwiGLU backward (bf16)
//   dW_down_sh[s]    = dY^T h_s            (fp32 [d][I_sh]; h_s: the forward's)
//   dW_gate_up_sh[s] = [dG | dU]_s^T X     (fp32 [2 I_sh][d])
// then dx_shared = [dG | dU] W_gate_up_sh as one product over K = n_sh * 2 I_sh
// (bf16 [T][d]): the sum over the shared experts of their input gradients.
hipError_t launch_shared_backward(const occ_layer_desc &L, const void *x, const void *w_gate_up_sh,
                                  const void *w_down_sh, const void *h_sh, const void *dy,
                                  void *gu, void *dgu, void *dx_shared, float *dw_gate_up_sh,
                                  float *dw_down_sh, hipStream_t st) {
  if (L.dtype == OCC_F32)
    return launch_shared_backward_f32(L, x, w_gate_up_sh, w_down_sh, h_sh, dy, gu, dgu, dx_shared,
                                      dw_gate_up_sh, dw_down_sh, st);
  // (T = 0: the products over no rows launch no tiles; the weight gradients,
  // sums over no rows, are written as zeros)
  const int64_t T = L.T, d = L.d, Is = L.I_shared, ns = L.n_shared, W2 = ns * 2 * Is;
  const uint16_t *wdn = static_cast<const uint16_t *>(w_down_sh);
  uint16_t *gub = static_cast<uint16_t *>(gu);
  uint16_t *dgub = static_cast<uint16_t *>(dgu);
  hipError_t err;
  const Placement none{};
  auto dense = [&]() {
    GemmArgs a = base_args(none);
    a.row_offset = nullptr;
    a.G = 1;
    a.dense_rows = (int)T;
    return a;
  };
  // 1. [G | U] of every shared expert: X times the stacked W_gate_up_sh
  //    ([n_sh 2 I_sh][d]), one product
  GemmArgs a = dense();
  a.A = x;
  a.lda = d;
  a.a_bytes = T * d * 2;
  a.B = w_gate_up_sh;
  a.ldb = d;
  a.b_bytes = W2 * d * 2;
  a.K = (int)d;
  a.N = (int)W2;
  a.C = gub;
  a.ldc = W2;
  choose_tile_order(a, T, W2);
  if ((err = launch_bwd<0, 0, false, EPI_BF16, 4>(a, grouped_tiles((int)T, 1, a.N), st)) !=
      hipSuccess)
    return err;
  // 2. per shared expert: dh_s = dY W_down_sh[s] ([d][I_sh]); SwiGLU backward
  //    into its [dG | dU] columns
  for (int64_t s = 0; s < ns; ++s) {
    a = dense();
    a.A = dy;
    a.lda = d;
    a.a_bytes = T * d * 2;
    a.B = wdn + s * d * Is;
    a.ldb = Is;
    a.b_bytes = d * Is * 2;
    a.K = (int)d;
    a.N = (int)Is;
    a.aux = gub + s * 2 * Is;
    a.ldaux = W2;
    a.C = dgub + s * 2 * Is;
    a.ldc = W2;
    choose_tile_order(a, T, Is);
    if ((err = launch_bwd<0, 1, false, EPI_SWIGLU_BWD, 4>(a, grouped_tiles((int)T, 1, a.N), st)) !=
        hipSuccess)
      return err;
  }
  // 3. dW_down_sh[s] = dY^T h_s for every s at once: output columns of the
  //    [d][n_sh I_sh] product go to matrix s = column / I_sh (K: the T rows)
  a = dense();
  a.A = dy;
  a.lda = d;
  a.a_bytes = T * d * 2;
  a.M = (int)d;
  a.B = h_sh;
  a.ldb = ns * Is;
  a.b_bytes = T * ns * Is * 2;
  a.N = (int)(ns * Is);
  a.nseg = (int)Is;
  a.nseg_stride = d * Is;
  a.C = dw_down_sh;
  a.ldc = Is;
  if ((err = launch_bwd<1, 1, true, EPI_F32, 2>(a, ((d + 255) / 256) * ((a.N + 255) / 256), st)) !=
      hipSuccess)
    return err;
  // 4. dW_gate_up_sh = [dG | dU]^T X, the stacked [n_sh 2 I_sh][d] at once
  a = dense();
  a.A = dgub;
  a.lda = W2;
  a.a_bytes = T * W2 * 2;
  a.M = (int)W2;
  a.B = x;
  a.ldb = d;
  a.b_bytes = T * d * 2;
  a.N = (int)d;
  a.C = dw_gate_up_sh;
  a.ldc = d;
  if ((err = launch_bwd<1, 1, true, EPI_F32, 2>(a, ((W2 + 255) / 256) * ((d + 255) / 256), st)) !=
      hipSuccess)
    return err;
  // 5. dx_shared = [dG | dU] W_gate_up_sh over all shared experts at once
  a = dense();
  a.A = dgub;
  a.lda = W2;
  a.a_bytes = T * W2 * 2;
  a.B = w_gate_up_sh;
  a.ldb = d;
  a.b_bytes = W2 * d * 2;
  a.K = (int)W2;
  a.N = (int)d;
  a.C = dx_shared;
  a.ldc = d;
  choose_tile_order(a, T, d);
  return launch_bwd<0, 1, false, EPI_BF16, 4>(a, grouped_tiles((int)T, 1, a.N), st);
}

}  // namespace occ
