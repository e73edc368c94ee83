// Routing: logits, softmax gate and top-k selection.
//
// Expert Coupling in MoE Pretraining, Abstract: each token is routed to k of
// the E experts.  The gate is a softmax over all E logits; selection is on
// the logits (descending, lower expert index first on equal logits).
//
// Each logit is the fp32 chain acc = fma(x[t][j], w[e][j], acc) over
// j = 0..d-1 in order.  v_fma_f32 rounds once, like C's fmaf, so the chain
// is bit-identical to any IEEE implementation of that definition; that is
// what makes the chosen indices reproducible bit for bit.  The chain cannot
// be split over j, so the contraction stays on the fp32 VALU (not MFMA) and
// the parallelism is over (token, expert) pairs.
//
// Mapping: a wave is cut into Q = 64/ESEG segments of ESEG lanes; the lanes
// of a segment hold the experts (lane el owns experts el + ESEG*i, i < EP)
// and a segment owns TPL tokens.  The token values of a d-chunk are read
// from LDS as broadcasts, the router rows as 16-byte per-lane reads, and the
// softmax/top-k reductions stay inside a segment (xor shuffles below ESEG).
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;
constexpr int kJC = 32;        // d-chunk staged in LDS
constexpr int kLds = kJC + 4;  // padded fp32 row stride (breaks bank aliasing)

struct Best {
  float key;
  int e;
  float p;
};

__device__ __forceinline__ bool better(float ka, int ea, float kb, int eb) {
  // (key descending, expert ascending); invalid entries carry e = INT_MAX
  return ka > kb || (ka == kb && ea < eb);
}

template <int DT, int ESEG, int EP, int TPL>
__global__ __launch_bounds__(kThreads) void route_topk_kernel(
    int T, int d, int E, int k, int renorm, const typename Elem<DT>::T *__restrict__ x,
    const typename Elem<DT>::T *__restrict__ wr, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out, float *__restrict__ logits) {
  using ET = typename Elem<DT>::T;
  constexpr int Q = kWave / ESEG;
  constexpr int TW = Q * TPL;                  // tokens per wave
  constexpr int TB = TW * (kThreads / kWave);  // tokens per block
  constexpr int EMAX = ESEG * EP;
  constexpr int VEC = 16 / sizeof(ET);         // elements per 16-byte load
  constexpr int TPR = kJC / VEC;               // threads per staged row
  __shared__ __attribute__((aligned(16))) float xs[TB * kLds];
  __shared__ __attribute__((aligned(16))) float ws[EMAX * kLds];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int q = lane / ESEG;   // segment
  const int el = lane % ESEG;  // lane in segment
  const int t0 = blockIdx.x * TB;

  float acc[TPL][EP];
#pragma unroll
  for (int m = 0; m < TPL; ++m)
#pragma unroll
    for (int i = 0; i < EP; ++i) acc[m][i] = 0.0f;

  for (int j0 = 0; j0 < d; j0 += kJC) {
    const int jn = min(kJC, d - j0);  // multiple of 8 (d % 8 == 0)
    // stage X[t0 .. t0+TB)[j0 .. j0+jn) and W[0 .. EMAX)[j0 .. j0+jn) as fp32
    for (int c = tid; c < TB * TPR; c += kThreads) {
      const int r = c / TPR, cv = (c % TPR) * VEC;
      const int t = t0 + r;
#pragma unroll
      for (int u = 0; u < VEC; ++u)
        xs[r * kLds + cv + u] =
            (t < T && cv + u < jn) ? Elem<DT>::load(x, (size_t)t * d + j0 + cv + u) : 0.0f;
    }
    for (int c = tid; c < EMAX * TPR; c += kThreads) {
      const int r = c / TPR, cv = (c % TPR) * VEC;
#pragma unroll
      for (int u = 0; u < VEC; ++u)
        ws[r * kLds + cv + u] =
            (r < E && cv + u < jn) ? Elem<DT>::load(wr, (size_t)r * d + j0 + cv + u) : 0.0f;
    }
    __syncthreads();
    if (jn == kJC) {
#pragma unroll
      for (int jj = 0; jj < kJC; jj += 4) {
        float4 wv[EP];
#pragma unroll
        for (int i = 0; i < EP; ++i)
          wv[i] = *reinterpret_cast<const float4 *>(&ws[(el + ESEG * i) * kLds + jj]);
#pragma unroll
        for (int m = 0; m < TPL; ++m) {
          const float4 xv =
              *reinterpret_cast<const float4 *>(&xs[(wave * TW + q + Q * m) * kLds + jj]);
#pragma unroll
          for (int i = 0; i < EP; ++i) {
            acc[m][i] = __builtin_fmaf(xv.x, wv[i].x, acc[m][i]);
            acc[m][i] = __builtin_fmaf(xv.y, wv[i].y, acc[m][i]);
            acc[m][i] = __builtin_fmaf(xv.z, wv[i].z, acc[m][i]);
            acc[m][i] = __builtin_fmaf(xv.w, wv[i].w, acc[m][i]);
          }
        }
      }
    } else {
      for (int jj = 0; jj < jn; ++jj) {
#pragma unroll
        for (int m = 0; m < TPL; ++m) {
          const float xv = xs[(wave * TW + q + Q * m) * kLds + jj];
#pragma unroll
          for (int i = 0; i < EP; ++i)
            acc[m][i] = __builtin_fmaf(xv, ws[(el + ESEG * i) * kLds + jj], acc[m][i]);
        }
      }
    }
    __syncthreads();
  }

  // ---- softmax and top-k per token, inside the segment --------------------
#pragma unroll
  for (int m = 0; m < TPL; ++m) {
    const int t = t0 + wave * TW + q + Q * m;  // uniform inside the segment
    float key[EP], p[EP];
    bool live[EP];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < EP; ++i) {
      const int e = el + ESEG * i;
      live[i] = e < E;
      key[i] = live[i] ? (isnan(acc[m][i]) ? -INFINITY : acc[m][i]) : -INFINITY;
      mx = fmaxf(mx, key[i]);
    }
#pragma unroll
    for (int off = ESEG / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < EP; ++i) {
      p[i] = live[i] ? expf(acc[m][i] - mx) : 0.0f;
      z += p[i];
    }
#pragma unroll
    for (int off = ESEG / 2; off > 0; off >>= 1) z += __shfl_xor(z, off);

    if (logits != nullptr && t < T) {
#pragma unroll
      for (int i = 0; i < EP; ++i)
        if (live[i]) logits[(size_t)t * E + el + ESEG * i] = acc[m][i];
    }

    int my_e = -1;
    float my_p = 0.0f, psum = 0.0f;
    for (int j = 0; j < k; ++j) {
      Best b{-INFINITY, INT_MAX, 0.0f};
#pragma unroll
      for (int i = 0; i < EP; ++i) {
        const int e = el + ESEG * i;
        if (live[i] && better(key[i], e, b.key, b.e)) b = Best{key[i], e, p[i]};
      }
#pragma unroll
      for (int off = ESEG / 2; off > 0; off >>= 1) {
        const float ok = __shfl_xor(b.key, off);
        const int oe = __shfl_xor(b.e, off);
        const float op = __shfl_xor(b.p, off);
        if (better(ok, oe, b.key, b.e)) b = Best{ok, oe, op};
      }
      // the owner retires the winner
#pragma unroll
      for (int i = 0; i < EP; ++i)
        if (el + ESEG * i == b.e) live[i] = false;
      psum += b.p;
      if (el == j) {
        my_e = b.e;
        my_p = b.p;
      }
    }
    if (t < T && el < k) {
      idx_out[(size_t)t * k + el] = my_e;
      w_out[(size_t)t * k + el] = renorm ? my_p / psum : my_p / z;
    }
  }
}

template <int DT, int ESEG, int EP>
hipError_t launch_tpl(const occ_layer_desc &L, const void *x, const void *wr, int32_t *idx,
                      float *w, float *logits, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  constexpr int Q = kWave / ESEG;
  // enough waves to keep four per SIMD busy, then longer per-lane token lists
  const long waves_tpl1 = ((long)L.T + Q - 1) / Q;
  int tpl = 1;
  if (waves_tpl1 >= 4L * 4096) tpl = 4;
  else if (waves_tpl1 >= 2L * 4096) tpl = 2;
  const int tb = Q * tpl * (kThreads / kWave);
  const dim3 grid((L.T + tb - 1) / tb);
  const ET *xp = static_cast<const ET *>(x);
  const ET *wp = static_cast<const ET *>(wr);
  if (tpl == 4)
    route_topk_kernel<DT, ESEG, EP, 4><<<grid, kThreads, 0, st>>>(L.T, L.d, L.E, L.k, L.renorm,
                                                                  xp, wp, idx, w, logits);
  else if (tpl == 2)
    route_topk_kernel<DT, ESEG, EP, 2><<<grid, kThreads, 0, st>>>(L.T, L.d, L.E, L.k, L.renorm,
                                                                  xp, wp, idx, w, logits);
  else
    route_topk_kernel<DT, ESEG, EP, 1><<<grid, kThreads, 0, st>>>(L.T, L.d, L.E, L.k, L.renorm,
                                                                  xp, wp, idx, w, logits);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const occ_layer_desc &L, const void *x, const void *wr, int32_t *idx,
                     float *w, float *logits, hipStream_t st) {
  if (L.E <= 4) return launch_tpl<DT, 4, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 8) return launch_tpl<DT, 8, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 16) return launch_tpl<DT, 16, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 32) return launch_tpl<DT, 32, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 64) return launch_tpl<DT, 64, 1>(L, x, wr, idx, w, logits, st);
  return launch_tpl<DT, 64, 2>(L, x, wr, idx, w, logits, st);
}

}  // namespace

hipError_t launch_route_topk(const occ_layer_desc &L, const void *x, const void *wr,
                             int32_t *idx, float *w, float *logits, hipStream_t st) {
  if (L.T == 0) return hipSuccess;
  return L.dtype == OCC_F32 ? launch_dt<OCC_F32>(L, x, wr, idx, w, logits, st)
                            : launch_dt<OCC_BF16>(L, x, wr, idx, w, logits, st);
}

}  // namespace occ
