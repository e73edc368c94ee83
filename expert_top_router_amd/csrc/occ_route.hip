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
// be split over j, so the parallelism is over (token, expert) pairs.  This
// file runs the chains on the fp32 VALU; at batches that give every SIMD a
// 16-token tile, routers of 33..128 experts run them as K = 1 fp32 MFMAs
// instead, which round like fmaf (occ_route_mfma.hip).
//
// Mapping: a wave is cut into Q = 64/ESEG segments of ESEG lanes; lane el of
// a segment owns experts el + ESEG*i (i < EP) and the segment owns TPL
// tokens, so a lane keeps TPL*EP independent chains.  The block's 4 or 8
// waves share one staged d-chunk of X (as fp32) and of the router (fp32, each
// row read by one lane as 16-byte vectors; the row stride of JC + 4 floats
// puts the 16 rows of a quarter-wave in distinct banks); X values are
// segment-wide LDS broadcasts, or, when a whole wave serves one token with
// one or two tokens per lane, one LDS value per lane handed to the FMAs by
// DPP row broadcasts (chunk_bcast, software-pipelined over 16-column groups).
// Chunks of JC = 32..128 columns go through a
// two-deep register pipeline (chunk c + 2 loads while chunk c is multiplied
// from LDS and chunk c + 1 waits in registers), one barrier per chunk.
// Softmax and top-k then run inside each segment with xor shuffles.
#include "occ_internal.h"

namespace occ {
namespace {

// acc = fma(x of lane J of this lane's 16-lane row, w, acc): the FMA takes
// its first operand through DPP row_newbcast (CDNA3/4), which hands every
// lane of a row the value held by lane J of that row.  One v_fmac_f32_dpp,
// rounding once like fmaf.
template <int J> __device__ __forceinline__ void fmac_row_bcast(float &acc, float x, float w) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(x), "v"(w), "i"(J));
}

struct Best {
  float key;
  int e;
  float p;
};

__device__ __forceinline__ bool better(float ka, int ea, float kb, int eb) {
  // (key descending, expert ascending); empty candidates carry e = INT_MAX
  return ka > kb || (ka == kb && ea < eb);
}

template <int DT, int ESEG, int EP, int TPL, int JC, int THR>
__global__ __launch_bounds__(THR) void route_topk_kernel(
    int T, int d, int E, int k, int renorm, const typename Elem<DT>::T *__restrict__ x,
    const float *__restrict__ wr, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    float *__restrict__ logits) {
  using ET = typename Elem<DT>::T;
  constexpr int Q = kWave / ESEG;
  constexpr int TW = Q * TPL;                  // tokens per wave
  constexpr int kThreads = THR;
  constexpr int TB = TW * (kThreads / kWave);  // tokens per block
  constexpr int EMAX = ESEG * EP;
  constexpr int kJC = JC;                      // d-chunk staged in LDS
  constexpr int kLds = kJC + 4;                // padded fp32 row stride
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

  // Two register sets: the loads of chunk c go into set c % 2 two chunks
  // before it is stored to LDS, so each load has two chunks of compute to land.
  u32x4 xr0[XPT], xr1[XPT];
  float4 wr0[WPT], wr1[WPT];
  // global -> registers for the chunk at j0 (rows past T / E and columns past
  // d are zero and never enter a chain: the compute loop stops at jn)
#define OCC_ROUTE_LOAD(xr, wrg, j0_)                                                  \
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
#define OCC_ROUTE_STORE(xr, wrg, buf_)                                                \
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

  // Whole-wave segments (ESEG == 64, one token per segment) with few tokens
  // per lane: per 16 columns a lane reads its router values (4 x 16 bytes per
  // expert) and, per token, only the one X value of its position in its
  // 16-lane row; the FMAs take X through DPP row broadcasts.  X reads from LDS
  // drop 16-fold against the broadcast 16-byte reads of the general loop,
  // which matters when 1-2 tokens per lane leave the router reads little
  // reuse (OLMoE-shaped layer: 57 -> 48 us); with 8 tokens per lane the
  // general loop measured faster before this loop was software-pipelined.
  // On whole chunks the reads of the next 16 columns are issued before the
  // FMAs of these (scheduling barriers keep the compiler from sinking them):
  // OLMoE-shaped layer 48 -> 43 us.  A DPP-broadcast FMA issues at about
  // half the rate of a plain one, so routers with tokens enough for several
  // per lane take 16-lane segments instead (the launcher).  jn is a multiple
  // of 8.
  constexpr bool BC = ESEG == kWave && (TPL <= 2 || EP == 1);
  auto chunk_bcast = [&](const float *wsc, const float *xsc, int jn) {
    const int xl = lane & 15;
    if (jn == kJC && kJC % 16 == 0) {
      // whole chunk: the loads of column group g + 16 go out before the FMAs
      // of group g, so the LDS latency hides behind them (two register sets)
      float4 wv[2][EP][4];
      float xv[2][TPL];
      auto load_group = [&](int g, int set) {
#pragma unroll
        for (int i = 0; i < EP; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            wv[set][i][v] =
                *reinterpret_cast<const float4 *>(&wsc[(el + ESEG * i) * kLds + g + 4 * v]);
#pragma unroll
        for (int m = 0; m < TPL; ++m) xv[set][m] = xsc[(wave * TW + q + Q * m) * kLds + g + xl];
      };
      load_group(0, 0);
#pragma unroll
      for (int g = 0; g < kJC; g += 16) {
        const int cs = (g / 16) & 1;
        if (g + 16 < kJC) load_group(g + 16, cs ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#define OCC_ROUTE_BCP(J, C)                                                           \
  _Pragma("unroll") for (int m = 0; m < TPL; ++m)                                     \
  _Pragma("unroll") for (int i = 0; i < EP; ++i)                                      \
      fmac_row_bcast<J>(acc[m][i], xv[cs][m], wv[cs][i][(J) / 4].C);
        OCC_ROUTE_BCP(0, x) OCC_ROUTE_BCP(1, y) OCC_ROUTE_BCP(2, z) OCC_ROUTE_BCP(3, w)
        OCC_ROUTE_BCP(4, x) OCC_ROUTE_BCP(5, y) OCC_ROUTE_BCP(6, z) OCC_ROUTE_BCP(7, w)
        OCC_ROUTE_BCP(8, x) OCC_ROUTE_BCP(9, y) OCC_ROUTE_BCP(10, z) OCC_ROUTE_BCP(11, w)
        OCC_ROUTE_BCP(12, x) OCC_ROUTE_BCP(13, y) OCC_ROUTE_BCP(14, z) OCC_ROUTE_BCP(15, w)
#undef OCC_ROUTE_BCP
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    for (int g = 0; g < jn; g += 16) {
      float4 wv[EP][4];
#pragma unroll
      for (int i = 0; i < EP; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          wv[i][v] = *reinterpret_cast<const float4 *>(&wsc[(el + ESEG * i) * kLds + g + 4 * v]);
      float xv[TPL];
#pragma unroll
      for (int m = 0; m < TPL; ++m) xv[m] = xsc[(wave * TW + q + Q * m) * kLds + g + xl];
      // j ascending inside every chain; the TPL * EP chains interleave
#define OCC_ROUTE_BC(J, C)                                                            \
  _Pragma("unroll") for (int m = 0; m < TPL; ++m)                                     \
  _Pragma("unroll") for (int i = 0; i < EP; ++i)                                      \
      fmac_row_bcast<J>(acc[m][i], xv[m], wv[i][(J) / 4].C);
      OCC_ROUTE_BC(0, x) OCC_ROUTE_BC(1, y) OCC_ROUTE_BC(2, z) OCC_ROUTE_BC(3, w)
      OCC_ROUTE_BC(4, x) OCC_ROUTE_BC(5, y) OCC_ROUTE_BC(6, z) OCC_ROUTE_BC(7, w)
      if (g + 8 < jn) {
        OCC_ROUTE_BC(8, x) OCC_ROUTE_BC(9, y) OCC_ROUTE_BC(10, z) OCC_ROUTE_BC(11, w)
        OCC_ROUTE_BC(12, x) OCC_ROUTE_BC(13, y) OCC_ROUTE_BC(14, z) OCC_ROUTE_BC(15, w)
      }
#undef OCC_ROUTE_BC
    }
  };

  // General loop: per 4 columns, one 16-byte router read per expert and one
  // segment-broadcast 16-byte X read per token.  With few chains per lane
  // (TPL * EP <= 4) the loop is latency-bound, and on whole chunks the reads
  // of the 4-column groups up to kAhead ahead go out before the FMAs of this
  // one (a ring of kAhead + 1 register sets; scheduling barriers keep the
  // order): Mixtral-shaped layer 73 -> 46 us with one group ahead, 42 with
  // three (seven: 42).  With more chains per lane it is not used: on the
  // 128-expert layer 32 chains gain nothing with it and 64 spill.
  constexpr int kAhead = 3;
  auto fma4 = [&](const float4 *wv, const float4 *xv) {
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
  };
  auto chunk_general = [&](const float *wsc, const float *xsc, int jn) {
    auto load4 = [&](int jj, float4 *wv, float4 *xv) {
#pragma unroll
      for (int i = 0; i < EP; ++i)
        wv[i] = *reinterpret_cast<const float4 *>(&wsc[(el + ESEG * i) * kLds + jj]);
#pragma unroll
      for (int m = 0; m < TPL; ++m)
        xv[m] = *reinterpret_cast<const float4 *>(&xsc[(wave * TW + q + Q * m) * kLds + jj]);
    };
    if (TPL * EP <= 4 && jn == kJC) {
      constexpr int kSets = kAhead + 1;
      float4 wv[kSets][EP], xv[kSets][TPL];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) load4(4 * s, wv[s], xv[s]);
#pragma unroll
      for (int jj = 0; jj < kJC; jj += 4) {
        const int gi = jj / 4, nx = (gi + kAhead) % kSets;
        if (jj + 4 * kAhead < kJC) load4(jj + 4 * kAhead, wv[nx], xv[nx]);
        __builtin_amdgcn_sched_barrier(0);
        fma4(wv[gi % kSets], xv[gi % kSets]);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll 8
    for (int jj = 0; jj < kJC; jj += 4) {
      if (jj < jn) {
        float4 wv[EP], xv[TPL];
        load4(jj, wv, xv);
        fma4(wv, xv);
      }
    }
  };

  const int nch = (d + kJC - 1) / kJC;
  // chunk ch is multiplied from LDS buffer ch % 2, chunk ch + 1 waits in
  // register set (ch + 1) % 2, and chunk ch + 2 is loading into set ch % 2
  OCC_ROUTE_LOAD(xr0, wr0, 0);
  if (nch > 1) OCC_ROUTE_LOAD(xr1, wr1, kJC);
  OCC_ROUTE_STORE(xr0, wr0, 0);
  if (nch > 2) OCC_ROUTE_LOAD(xr0, wr0, 2 * kJC);
  __syncthreads();
#define OCC_ROUTE_CHUNK(ch_, cur_, xn, wn)                                            \
  do {                                                                                \
    const int j0 = (ch_) * kJC;                                                       \
    const int jn = min(kJC, d - j0); /* multiple of 8 (d % 8 == 0) */                 \
    const float *xsc = xs[cur_];                                                      \
    const float *wsc = ws[cur_];                                                      \
    if (BC) {                                                                         \
      chunk_bcast(wsc, xsc, jn);                                                      \
    } else {                                                                          \
      chunk_general(wsc, xsc, jn);                                                    \
    }                                                                                 \
    if ((ch_) + 1 < nch) OCC_ROUTE_STORE(xn, wn, (cur_) ^ 1);                         \
    if ((ch_) + 3 < nch) OCC_ROUTE_LOAD(xn, wn, ((ch_) + 3) * kJC);                   \
    __syncthreads();                                                                  \
  } while (0)
  for (int ch = 0; ch < nch; ch += 2) {
    OCC_ROUTE_CHUNK(ch, 0, xr1, wr1);
    if (ch + 1 < nch) OCC_ROUTE_CHUNK(ch + 1, 1, xr0, wr0);
  }
#undef OCC_ROUTE_CHUNK
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

// LDS bytes of one block: double-buffered X and router chunks.
constexpr int route_lds(int tb, int emax, int jc) { return 2 * (tb + emax) * (jc + 4) * 4; }

template <int DT, int ESEG, int EP, int TPL, int THR>
void launch_jc(const occ_layer_desc &L, const void *x, const float *wr, int32_t *idx, float *w,
               float *logits, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  constexpr int TB = kWave / ESEG * TPL * (THR / kWave);
  // The widest d-chunk that leaves room for two waves per SIMD (two 4-wave
  // blocks, or one 8-wave block, per CU): long chunks mean few barriers.
  constexpr int kBudget = THR == 512 ? 150 * 1024 : 80 * 1024;
  constexpr int JC = route_lds(TB, ESEG * EP, 128) <= kBudget  ? 128
                     : route_lds(TB, ESEG * EP, 64) <= kBudget ? 64
                                                               : 32;
  static_assert(route_lds(TB, ESEG * EP, JC) <= 160 * 1024, "LDS");
  const dim3 grid((L.T + TB - 1) / TB);
  route_topk_kernel<DT, ESEG, EP, TPL, JC, THR><<<grid, THR, 0, st>>>(
      L.T, L.d, L.E, L.k, L.renorm, static_cast<const ET *>(x), wr, idx, w, logits);
}

template <int DT, int ESEG, int EP>
hipError_t launch_tpl(const occ_layer_desc &L, const void *x, const float *wr, int32_t *idx,
                      float *w, float *logits, hipStream_t st) {
  constexpr int Q = kWave / ESEG;
  // About two waves per SIMD (2048) before lengthening the per-lane token
  // list.  Routers of 33..64 experts use 8-wave blocks: every block re-reads
  // the whole router, so more tokens per block means less router traffic
  // (wider routers already carry 8 tokens per lane).  (One 4-wave block per
  // CU with four tokens per lane measured slower: one wave per SIMD leaves
  // the LDS and FMA latencies exposed.)
  constexpr int THR = ESEG == 64 && EP == 1 ? 512 : 256;
  const long per = (long)L.T / ((long)Q * 2048);
  if (per >= 8) launch_jc<DT, ESEG, EP, 8, THR>(L, x, wr, idx, w, logits, st);
  else if (per >= 4) launch_jc<DT, ESEG, EP, 4, THR>(L, x, wr, idx, w, logits, st);
  else if (per >= 2) launch_jc<DT, ESEG, EP, 2, THR>(L, x, wr, idx, w, logits, st);
  else launch_jc<DT, ESEG, EP, 1, THR>(L, x, wr, idx, w, logits, st);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const occ_layer_desc &L, const void *x, const float *wr, int32_t *idx,
                     float *w, float *logits, hipStream_t st) {
  if (L.E <= 4) return launch_tpl<DT, 4, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 8) return launch_tpl<DT, 8, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 16) return launch_tpl<DT, 16, 1>(L, x, wr, idx, w, logits, st);
  if (L.E <= 32) return launch_tpl<DT, 32, 1>(L, x, wr, idx, w, logits, st);
  // Wider routers: each 16-byte LDS read (4 columns of one router row, or of
  // one token's X broadcast to a segment) feeds more FMAs when a lane holds
  // several experts and several tokens, and per CU the LDS serves about one
  // 16-byte wave read per ~5 cycles against one wave FMA per ~2 cycles.  So
  // 16-lane segments with 4 or 8 experts per lane when there are tokens
  // enough for two waves per SIMD (DeepSeek-V2-Lite-shaped layer, T = 16384:
  // 111 -> 95 us; stress layer, 128 experts: 537 -> 456 us, same-process
  // A/B; logits and indices identical, the gate weights within 3e-7, their
  // softmax sums taken in another order).  With fewer tokens (T = 4096) the
  // whole-wave segments with DPP broadcasts stay faster (42 against 48 us).
  if (L.E <= 64) {
    if (L.T >= 16384) return launch_tpl<DT, 16, 4>(L, x, wr, idx, w, logits, st);
    return launch_tpl<DT, 64, 1>(L, x, wr, idx, w, logits, st);
  }
  return launch_tpl<DT, 16, 8>(L, x, wr, idx, w, logits, st);
}

}  // namespace

hipError_t launch_route_topk(const occ_layer_desc &L, const void *x, const float *wr,
                             int32_t *idx, float *w, float *logits, hipStream_t st) {
  if (L.T == 0) return hipSuccess;
  // Wider routers at batches that give every SIMD a 16-token tile run their
  // chains on the matrix cores (same bits; occ_route_mfma.hip).
  if (route_mfma_applies(L) && L.T >= 16384)
    return launch_route_mfma(L, x, wr, idx, w, logits, st);
  return L.dtype == OCC_F32 ? launch_dt<OCC_F32>(L, x, wr, idx, w, logits, st)
                            : launch_dt<OCC_BF16>(L, x, wr, idx, w, logits, st);
}

}  // namespace occ
