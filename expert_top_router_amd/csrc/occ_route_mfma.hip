// Routing on the matrix cores: the in-order logit chains as K = 1 fp32 MFMAs.
//
// Expert Coupling in MoE Pretraining, Abstract: each token is routed to k of
// the E experts; the gate is a softmax over the E logits and the selection is
// on the logits (descending, lower expert index first on equal logits).  A
// logit is the fp32 chain acc = fma(x[t][j], w[e][j], acc) over j = 0..d-1
// in order.
//
// v_mfma_f32_16x16x1f32 (K = 1) adds to each of its four 16 x 16 accumulator
// blocks the outer product of 16 A values and 16 B values, and rounds every
// element once: element by element it is fmaf(a, b, c), the same bits as the
// VALU's v_fma_f32 (checked on this chip over normal, subnormal, infinite,
// NaN and signed-zero operands).  A sequence of these MFMAs over ascending j
// therefore runs every chain of a tile in the definition's order, bit for
// bit, while each lane supplies one A and one B value per step instead of
// reading both operands of every FMA: 1024 chains advance per MFMA.
//
// Tile: a wave owns 16 tokens x 64 EACC experts.  A lane L supplies row L % 16
// of block L / 16 of A and column L % 16 of block L / 16 of B, so every block
// gets the wave's 16 tokens (lane L: token L % 16) and accumulator a covers
// experts 64 a + L; element i of lane l is token 4 (l / 16) + i % 4 and
// expert 64 a + 16 (i / 4) + l % 16.  A dependent MFMA issues every ≈52 cycles
// on one chain and every ≈36 on two, so throughput needs about one tile per
// SIMD; the chip fills from T ≈ 16 K tokens.
//
// Operands: X straight from global memory (one 16-byte load per lane and 8
// bf16 or 4 fp32 columns, a chunk ahead in registers); the fp32 router rows
// staged per block in LDS (row stride JC + 4 floats: a 16-byte read by 64
// lanes of 64 rows is conflict-free), two chunk buffers, one barrier per
// chunk.  Softmax and top-k: each 16-lane row holds four tokens, so the
// reductions are DPP row reductions.
#include <type_traits>

#include "occ_internal.h"

namespace occ {
namespace {

typedef float ff32x16 __attribute__((ext_vector_type(16)));

template <int DT, int EACC>
__global__ __launch_bounds__(256, 2) void route_mfma_kernel(
    int T, int d, int E, int k, int renorm, const typename Elem<DT>::T *__restrict__ x,
    const float *__restrict__ wr, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    float *__restrict__ logits) {
  using ET = typename Elem<DT>::T;
  constexpr int NW = 4, TB = 16 * NW;          // waves and tokens per block
  constexpr int EPAD = 64 * EACC;
  constexpr int JC = DT == OCC_BF16 ? 64 : 32;  // columns per chunk
  constexpr int LW = JC + 4;                    // router row stride in LDS (floats)
  constexpr int VPL = 16 / (int)sizeof(ET);     // X values per 16-byte load
  constexpr int XL = JC / VPL;                  // X loads per lane and chunk
  constexpr int WPR = JC / 4;                   // 16-byte router loads per row and chunk
  constexpr int WL = EPAD * WPR / 256;          // ... per thread and chunk
  static_assert(WL * 256 == EPAD * WPR, "whole router chunks");
  __shared__ __attribute__((aligned(16))) float ws[2][EPAD * LW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TB + 16 * wave;  // the wave's first token
  const ET *xr = x + (size_t)min(t0 + (lane & 15), T - 1) * d;
  const int nch = d / JC;

  // Loads are unconditional (chunks past the last re-read it, rows past E
  // the last row; nothing uses them), so the compiler's waits stay partial.
  u32x4 wb[WL];
  u32x4 xb[2][XL];
  auto load_w = [&](int c) __attribute__((always_inline)) {
    c = min(c, nch - 1);
#pragma unroll
    for (int u = 0; u < WL; ++u) {
      const int i = tid + 256 * u, r = min(i / WPR, E - 1), cc = (i % WPR) * 4;
      wb[u] = *reinterpret_cast<const u32x4 *>(wr + (size_t)r * d + c * JC + cc);
    }
  };
  auto store_w = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < WL; ++u) {
      const int i = tid + 256 * u, r = i / WPR, cc = (i % WPR) * 4;
      *reinterpret_cast<u32x4 *>(&ws[st][r * LW + cc]) = wb[u];
    }
  };
  auto load_x = [&](int c, u32x4 *dst) __attribute__((always_inline)) {
    c = min(c, nch - 1);
#pragma unroll
    for (int u = 0; u < XL; ++u)
      dst[u] = *reinterpret_cast<const u32x4 *>(xr + c * JC + u * VPL);
  };

  ff32x16 acc[EACC];
#pragma unroll
  for (int a = 0; a < EACC; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[a][i] = 0.0f;

  load_w(0);
  load_x(0, xb[0]);
  store_w(0);
  load_w(1);
  load_x(1, xb[1]);
  __syncthreads();
  // chunk c from LDS stage c & 1 and X set S; then chunk c + 1's router rows
  // go to the other stage and chunk c + 2 is loaded into the freed registers
  auto body = [&](int c, auto setc) __attribute__((always_inline)) {
    constexpr int S = decltype(setc)::value;
    const float *wl = &ws[c & 1][lane * LW];
    // the router reads of group g + 1 go out before the MFMAs of group g
    // (scheduling barriers keep the order), so their LDS latency hides
    // under those MFMAs
    float4 wv[2][EACC];
#pragma unroll
    for (int a = 0; a < EACC; ++a)
      wv[0][a] = *reinterpret_cast<const float4 *>(wl + a * 64 * LW);
#pragma unroll
    for (int g = 0; g < JC / 4; ++g) {  // 4-column groups, j ascending
      const int cu = g & 1;
      if (g + 1 < JC / 4) {
#pragma unroll
        for (int a = 0; a < EACC; ++a)
          wv[cu ^ 1][a] = *reinterpret_cast<const float4 *>(wl + a * 64 * LW + 4 * (g + 1));
      }
      float xf[VPL];
      widen<DT>(xb[S][4 * g / VPL], xf);
      const int o = (4 * g) % VPL;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
#pragma unroll
        for (int a = 0; a < EACC; ++a) {
          const float4 &w4 = wv[cu][a];
          const float b = c4 == 0 ? w4.x : c4 == 1 ? w4.y : c4 == 2 ? w4.z : w4.w;
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x1f32(xf[o + c4], b, acc[a], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_w((c + 1) & 1);
    load_w(c + 2);
    load_x(c + 2, xb[S]);
    __syncthreads();
  };
  for (int c = 0; c < nch; c += 2) {
    body(c, std::integral_constant<int, 0>{});
    if (c + 1 < nch) body(c + 1, std::integral_constant<int, 1>{});
  }

  // ---- softmax and top-k: row R of the wave holds tokens 4 R + s ----------
  const int q = lane & 15, R = lane >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int t = t0 + 4 * R + s;
    constexpr int NV = 4 * EACC;
    float v[NV], key[NV], p[NV];
    bool live[NV];
    float lm = -INFINITY;
#pragma unroll
    for (int a = 0; a < EACC; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int n = 4 * a + b, e = 64 * a + 16 * b + q;  // ascending e in n
        v[n] = acc[a][4 * b + s];
        live[n] = e < E;
        key[n] = live[n] ? (isnan(v[n]) ? -INFINITY : v[n]) : -INFINITY;
        lm = fmaxf(lm, key[n]);
      }
    const float mx = row_max(lm);
    float zl = 0.0f;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      p[n] = live[n] ? expf(v[n] - mx) : 0.0f;
      zl += p[n];
    }
    const float z = row_sum(zl);
    if (logits != nullptr && t < T) {
#pragma unroll
      for (int n = 0; n < NV; ++n)
        if (live[n]) logits[(size_t)t * E + 64 * (n / 4) + 16 * (n % 4) + q] = v[n];
    }
    int my_e = -1;
    float my_p = 0.0f, psum = 0.0f;
    for (int j = 0; j < k; ++j) {
      // the lane's best live entry (key descending, expert ascending), then
      // the row's: its largest key, and the lowest expert holding it
      float bk = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int n = 0; n < NV; ++n)
        if (live[n] && (key[n] > bk || be == 0x7fffffff)) {
          bk = key[n];
          be = 64 * (n / 4) + 16 * (n % 4) + q;
        }
      const float m = row_max(bk);
      const int ge = row_min_i(bk == m ? be : 0x7fffffff);
      float pw = 0.0f;
#pragma unroll
      for (int n = 0; n < NV; ++n)
        if (64 * (n / 4) + 16 * (n % 4) + q == ge) {
          live[n] = false;  // the owner retires the winner
          pw = p[n];
        }
      pw = row_sum(pw);  // the winner's p (the other lanes add zeros)
      psum += pw;
      if (q == j) {
        my_e = ge;
        my_p = pw;
      }
    }
    if (t < T && q < k) {
      idx_out[(size_t)t * k + q] = my_e;
      w_out[(size_t)t * k + q] = renorm ? my_p / psum : my_p / z;
    }
  }
}

template <int DT, int EACC>
hipError_t launch_e(const occ_layer_desc &L, const void *x, const float *wr, int32_t *idx,
                    float *w, float *logits, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  const dim3 grid((L.T + 63) / 64);
  route_mfma_kernel<DT, EACC><<<grid, 256, 0, st>>>(L.T, L.d, L.E, L.k, L.renorm,
                                                    static_cast<const ET *>(x), wr, idx, w,
                                                    logits);
  return hipGetLastError();
}

}  // namespace

bool route_mfma_applies(const occ_layer_desc &L) {
  const int jc = L.dtype == OCC_BF16 ? 64 : 32;
  return L.E > 32 && L.E <= 128 && L.k <= 16 && L.d % jc == 0;
}

hipError_t launch_route_mfma(const occ_layer_desc &L, const void *x, const float *wr,
                             int32_t *idx, float *w, float *logits, hipStream_t st) {
  if (L.T == 0) return hipSuccess;
  if (L.dtype == OCC_BF16)
    return L.E > 64 ? launch_e<OCC_BF16, 2>(L, x, wr, idx, w, logits, st)
                    : launch_e<OCC_BF16, 1>(L, x, wr, idx, w, logits, st);
  return L.E > 64 ? launch_e<OCC_F32, 2>(L, x, wr, idx, w, logits, st)
                  : launch_e<OCC_F32, 1>(L, x, wr, idx, w, logits, st);
}

}  // namespace occ
