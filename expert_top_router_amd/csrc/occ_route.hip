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
// Mapping: a wave is cut into Q = 64/ESEG segments of ESEG lanes; lane el of
// a segment owns experts el + ESEG*i (i < EP) and the segment owns TPL
// tokens, so a lane keeps TPL*EP independent chains.  The block's 4 waves
// share one staged d-chunk of X (as fp32) and of the router (fp32, each row
// read by one lane as 16-byte vectors, conflict-free with a 36-float row
// stride); X values are segment-wide LDS broadcasts.  Chunks are
// double-buffered: the next chunk is loaded into registers while the current
// one is consumed, with one barrier per chunk.  Softmax and top-k then run
// inside each segment with xor shuffles.
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;
constexpr int kJC = 32;        // d-chunk staged in LDS
constexpr int kLds = kJC + 4;  // padded fp32 row stride

struct Best {
  float key;
  int e;
  float p;
};

__device__ __forceinline__ bool better(float ka, int ea, float kb, int eb) {
  // (key descending, expert ascending); empty candidates carry e = INT_MAX
  return ka > kb || (ka == kb && ea < eb);
}

template <int DT, int ESEG, int EP, int TPL>
__global__ __launch_bounds__(kThreads) void route_topk_kernel(
    int T, int d, int E, int k, int renorm, const typename Elem<DT>::T *__restrict__ x,
    const float *__restrict__ wr, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    float *__restrict__ logits) {
  using ET = typename Elem<DT>::T;
  constexpr int Q = kWave / ESEG;
  constexpr int TW = Q * TPL;                  // tokens per wave
  constexpr int TB = TW * (kThreads / kWave);  // tokens per block
  constexpr int EMAX = ESEG * EP;
  constexpr int XV = 16 / sizeof(ET);          // x elements per 16-byte load
  constexpr int XLOADS = TB * kJC / XV;        // 16-byte loads of one X chunk
  constexpr int WLOADS = EMAX * kJC / 4;       // 16-byte loads of one router chunk
  constexpr int XPT = (XLOADS + kThreads - 1) / kThreads;
  constexpr int WPT = (WLOADS + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) float xs[2][TB * kLds];
  __shared__ __attribute__((aligned(16))) float ws[2][EMAX * kLds];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int q = lane / ESEG;
  const int el = lane % ESEG;
  const int t0 = blockIdx.x * TB;

  float acc[TPL][EP];
#pragma unroll
  for (int m = 0; m < TPL; ++m)
#pragma unroll
    for (int i = 0; i < EP; ++i) acc[m][i] = 0.0f;

  u32x4 xr[XPT];
  float4 wrg[WPT];
  // global -> registers for the chunk at j0 (rows past T / E and columns past
  // d are zero and never enter a chain: the compute loop stops at jn)
#define OCC_ROUTE_LOAD(j0_)                                                           \
  do {                                                                                \
    _Pragma("unroll") for (int u = 0; u < XPT; ++u) {                                 \
      const int c = tid + kThreads * u;                                               \
      const int r = c / (kJC / XV), cv = (c % (kJC / XV)) * XV;                       \
      const int t = t0 + r;                                                           \
      xr[u] = u32x4{0u, 0u, 0u, 0u};                                                  \
      if (c < XLOADS && t < T && (j0_) + cv < d)                                      \
        xr[u] = *reinterpret_cast<const u32x4 *>(x + (size_t)t * d + (j0_) + cv);     \
    }                                                                                 \
    _Pragma("unroll") for (int u = 0; u < WPT; ++u) {                                 \
      const int c = tid + kThreads * u;                                               \
      const int r = c / (kJC / 4), cv = (c % (kJC / 4)) * 4;                          \
      wrg[u] = make_float4(0.f, 0.f, 0.f, 0.f);                                       \
      if (c < WLOADS && r < E && (j0_) + cv < d)                                      \
        wrg[u] = *reinterpret_cast<const float4 *>(wr + (size_t)r * d + (j0_) + cv);  \
    }                                                                                 \
  } while (0)
#define OCC_ROUTE_STORE(buf_)                                                         \
  do {                                                                                \
    _Pragma("unroll") for (int u = 0; u < XPT; ++u) {                                 \
      const int c = tid + kThreads * u;                                               \
      if (c < XLOADS) {                                                               \
        const int r = c / (kJC / XV), cv = (c % (kJC / XV)) * XV;                     \
        float f[XV];                                                                  \
        widen<DT>(xr[u], f);                                                          \
        _Pragma("unroll") for (int v = 0; v < XV; v += 4)                             \
            *reinterpret_cast<float4 *>(&xs[buf_][r * kLds + cv + v]) =               \
            make_float4(f[v], f[v + 1], f[v + 2], f[v + 3]);                          \
      }                                                                               \
    }                                                                                 \
    _Pragma("unroll") for (int u = 0; u < WPT; ++u) {                                 \
      const int c = tid + kThreads * u;                                               \
      if (c < WLOADS) {                                                               \
        const int r = c / (kJC / 4), cv = (c % (kJC / 4)) * 4;                        \
        *reinterpret_cast<float4 *>(&ws[buf_][r * kLds + cv]) = wrg[u];               \
      }                                                                               \
    }                                                                                 \
  } while (0)

  const int nch = (d + kJC - 1) / kJC;
  OCC_ROUTE_LOAD(0);
  OCC_ROUTE_STORE(0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int cur = ch & 1;
    const int j0 = ch * kJC;
    const int jn = min(kJC, d - j0);  // multiple of 8 (d % 8 == 0)
    if (ch + 1 < nch) OCC_ROUTE_LOAD(j0 + kJC);
    const float *xsc = xs[cur];
    const float *wsc = ws[cur];
#pragma unroll
    for (int jj = 0; jj < kJC; jj += 4) {
      if (jj < jn) {
        float4 wv[EP], xv[TPL];
#pragma unroll
        for (int i = 0; i < EP; ++i)
          wv[i] = *reinterpret_cast<const float4 *>(&wsc[(el + ESEG * i) * kLds + jj]);
#pragma unroll
        for (int m = 0; m < TPL; ++m)
          xv[m] = *reinterpret_cast<const float4 *>(&xsc[(wave * TW + q + Q * m) * kLds + jj]);
        // j ascending inside every chain; the TPL*EP chains interleave
#pragma unroll
        for (int m = 0; m < TPL; ++m)
#pragma unroll
          for (int i = 0; i < EP; ++i) acc[m][i] = __builtin_fmaf(xv[m].x, wv[i].x, acc[m][i]);
#pragma unroll
        for (int m = 0; m < TPL; ++m)
#pragma unroll
          for (int i = 0; i < EP; ++i) acc[m][i] = __builtin_fmaf(xv[m].y, wv[i].y, acc[m][i]);
#pragma unroll
        for (int m = 0; m < TPL; ++m)
#pragma unroll
          for (int i = 0; i < EP; ++i) acc[m][i] = __builtin_fmaf(xv[m].z, wv[i].z, acc[m][i]);
#pragma unroll
        for (int m = 0; m < TPL; ++m)
#pragma unroll
          for (int i = 0; i < EP; ++i) acc[m][i] = __builtin_fmaf(xv[m].w, wv[i].w, acc[m][i]);
      }
    }
    if (ch + 1 < nch) OCC_ROUTE_STORE(cur ^ 1);
    __syncthreads();
  }
#undef OCC_ROUTE_LOAD
#undef OCC_ROUTE_STORE

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
      Best b{-INFINITY, 0x7fffffff, 0.0f};
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
#pragma unroll
      for (int i = 0; i < EP; ++i)
        if (el + ESEG * i == b.e) live[i] = false;  // the owner retires the winner
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
hipError_t launch_tpl(const occ_layer_desc &L, const void *x, const float *wr, int32_t *idx,
                      float *w, float *logits, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  constexpr int Q = kWave / ESEG;
  // about one wave per SIMD (1024) before lengthening the per-lane token list
  const long per = (long)L.T / ((long)Q * 1024);
  const int tpl = per >= 8 ? 8 : per >= 4 ? 4 : per >= 2 ? 2 : 1;
  const int tb = Q * tpl * (kThreads / kWave);
  const dim3 grid((L.T + tb - 1) / tb);
  const ET *xp = static_cast<const ET *>(x);
#define OCC_ROUTE_LAUNCH(TPL_)                                                    \
  route_topk_kernel<DT, ESEG, EP, TPL_><<<grid, kThreads, 0, st>>>(               \
      L.T, L.d, L.E, L.k, L.renorm, xp, wr, idx, w, logits)
  if (tpl == 8) OCC_ROUTE_LAUNCH(8);
  else if (tpl == 4) OCC_ROUTE_LAUNCH(4);
  else if (tpl == 2) OCC_ROUTE_LAUNCH(2);
  else OCC_ROUTE_LAUNCH(1);
#undef OCC_ROUTE_LAUNCH
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const occ_layer_desc &L, const void *x, const float *wr, int32_t *idx,
                     float *w, float *logits, hipStream_t st) {
  if (L.E <= 4) return launch_tpl<DT, 4, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 8) return launch_tpl<DT, 8, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 16) return launch_tpl<DT, 16, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 32) return launch_tpl<DT, 32, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 64) return launch_tpl<DT, 64, 1>(L, x, wr, idx, w, logits, st);
  return launch_tpl<DT, 64, 2>(L, x, wr, idx, w, logits, st);
}

}  // namespace

hipError_t launch_route_topk(const occ_layer_desc &L, const void *x, const float *wr,
                             int32_t *idx, float *w, float *logits, hipStream_t st) {
  if (L.T == 0) return hipSuccess;
  return L.dtype == OCC_F32 ? launch_dt<OCC_F32>(L, x, wr, idx, w, logits, st)
                            : launch_dt<OCC_BF16>(L, x, wr, idx, w, logits, st);
}

}  // namespace occ
