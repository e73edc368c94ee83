// Routing through a certified candidate filter (bf16 tokens, no logits
// output).
//
// Expert Coupling in MoE Pretraining, Abstract: each token is routed to k of
// the E experts.  The selection is defined on the in-order fp32 FMA chain
// l[t][e] = fma(x[t][d-1], w[e][d-1], ... fma(x[t][0], w[e][0], 0)); only
// the experts that can be among a token's k largest chains need the chain.
//
//   prep:    router rows to bf16 (h = RNE(w), residual r = w - h) in the
//            workspace, and per expert the bound factor
//            B_e = 1.01 (2 d u |h_e| + 1.01 d u |w_e| + |r_e|), u = 2^-24
//   approx:  a[t][e] = sum_j x[t][j] h[e][j] with bf16 MFMA (exact products,
//            fp32 accumulation), and |x_t|
//   exact:   |a - l| <= |x_t| B_e: the MFMA sum and the chain each carry at
//            most 2 d u (resp. 1.01 d u) times sum_j |x_j h_j| (|x_j w_j|),
//            bounded by Cauchy-Schwarz, and the residual adds sum_j |x_j r_j|.
//            With delta_t = 1.01 |x_t| max_e B_e and a_(k) the k-th largest
//            a, every expert of the true top k has a >= a_(k) - 2 delta_t
//            (the true k-th largest chain is >= a_(k) - delta_t), and every
//            other expert has a chain strictly below it, so the top k of the
//            chains over those candidates is the top k over all experts, ties
//            included.  The candidates' chains run in order in fp32 like the
//            full kernel's, so logits and indices are the same bit for bit.
//            The softmax denominator takes the candidates' chains and the
//            other experts' approximate logits (a relative change of the
//            order of their rounding, as between two summation orders).
//            A block with a token of more than kCap candidates, or with a
//            non-finite approximate logit or norm, runs every chain of every
//            token instead (then identical to the full kernel up to the order
//            of the softmax sum), and so does every block when a router row is
//            not bf16-exact (the approximate logits then carry the rows'
//            rounding, too coarse for the other experts' share of the softmax
//            sum; correct, but slower than the full kernel).
#include <type_traits>

#include "occ_internal.h"

namespace occ {
namespace {

typedef __bf16 fbf16x8 __attribute__((ext_vector_type(8)));
typedef float ff32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t fu32x2 __attribute__((ext_vector_type(2)));

constexpr int kCap = 16;      // candidates per token
constexpr int kNT = 512;      // threads per block (8 waves)
constexpr float kU = 5.9604645e-8f;  // 2^-24

struct FilterWs {
  uint16_t *wh;  // [E][d] bf16 router
  float *bnd;    // [E] bound factor B_e
  int32_t *ex;   // [E] 1 when the row is bf16-exact
  float *ag;     // [T][E] approximate logits
  float *xn;     // [T] |x_t|
};

size_t a256(size_t n) { return (n + 255) / 256 * 256; }

FilterWs carve(const occ_layer_desc &L, void *ws) {
  char *p = static_cast<char *>(ws);
  FilterWs f;
  f.wh = reinterpret_cast<uint16_t *>(p);
  p += a256((size_t)L.E * L.d * 2);
  f.bnd = reinterpret_cast<float *>(p);
  p += a256((size_t)L.E * 4);
  f.ex = reinterpret_cast<int32_t *>(p);
  p += a256((size_t)L.E * 4);
  f.ag = reinterpret_cast<float *>(p);
  p += a256((size_t)L.T * L.E * 4);
  f.xn = reinterpret_cast<float *>(p);
  return f;
}

// ---- prep: one block per router row ---------------------------------------
__global__ __launch_bounds__(256) void route_prep_kernel(int d, const float *__restrict__ wr,
                                                         uint16_t *__restrict__ wh,
                                                         float *__restrict__ bnd,
                                                         int32_t *__restrict__ ex) {
  __shared__ float red[3][4];
  __shared__ int redx[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float sw = 0.0f, sh = 0.0f, sr = 0.0f;
  int exact = 1;
  const float4 *src = reinterpret_cast<const float4 *>(wr + (size_t)e * d);
  fu32x2 *dst = reinterpret_cast<fu32x2 *>(wh + (size_t)e * d);
  for (int i = tid; i < d / 4; i += 256) {
    const float4 v = src[i];
    const float w[4] = {v.x, v.y, v.z, v.w};
    uint32_t hb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      hb[c] = f32_to_bf16(w[c]);
      const float h = __uint_as_float(hb[c] << 16), r = w[c] - h;
      sw = __builtin_fmaf(w[c], w[c], sw);
      sh = __builtin_fmaf(h, h, sh);
      sr = __builtin_fmaf(r, r, sr);
      exact &= r == 0.0f ? 1 : 0;
    }
    dst[i] = fu32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sw += __shfl_xor(sw, off);
    sh += __shfl_xor(sh, off);
    sr += __shfl_xor(sr, off);
    exact &= __shfl_xor(exact, off);
  }
  if (lane == 0) {
    red[0][wave] = sw;
    red[1][wave] = sh;
    red[2][wave] = sr;
    redx[wave] = exact;
  }
  __syncthreads();
  if (tid == 0) {
    const float a = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const float b = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    const float c = red[2][0] + red[2][1] + red[2][2] + red[2][3];
    const float du = (float)d * kU;
    bnd[e] = 1.01f * (2.0f * du * sqrtf(b) + 1.01f * du * sqrtf(a) + sqrtf(c));
    ex[e] = redx[0] & redx[1] & redx[2] & redx[3];
  }
}

// ---- approx: 128 tokens x 32*EB experts per block, bf16 MFMA ---------------
// v_mfma_f32_32x32x16_bf16 with the token fragment first: lane l supplies
// row (token or expert) l % 32 and the 8 k values 8*(l/32)..+7 of a 16-deep
// step; output element r of lane l is token 8*(r/4) + 4*(l/32) + r%4 of the
// tile, expert l % 32.
template <int EB, int KT>
__global__ __launch_bounds__(kNT) void route_approx_kernel(int T, int d, int E,
                                                           const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ wh,
                                                           float *__restrict__ ag,
                                                           float *__restrict__ xn) {
  constexpr int kTok = KT;             // tokens per block
  constexpr int EPAD = 32 * EB;
  constexpr int JA = 64, LA = JA + 8;  // k-chunk and padded row stride (bf16)
  constexpr int XCT = kTok * JA / 8;   // 16-byte token chunks per k-chunk
  constexpr int XC = (XCT + kNT - 1) / kNT;
  constexpr int WCH = EPAD * JA / 8;   // 16-byte router chunks per k-chunk
  constexpr int WC = (WCH + kNT - 1) / kNT;
  static_assert(kTok % 32 == 0, "whole 32-token MFMA tiles");
  __shared__ __attribute__((aligned(16))) uint16_t xa[2][kTok * LA];
  __shared__ __attribute__((aligned(16))) uint16_t wa[2][EPAD * LA];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTok;
  const int nch = d / JA;
  constexpr int NTILE = kTok / 32 * EB;
  constexpr int TPW = NTILE >= 8 ? NTILE / 8 : 1;
  const int id0 = wave * TPW;
  const bool wact = id0 < NTILE;  // uniform
  const int tb = id0 / EB;

  // A ring of KP register sets: set c % KP holds k-chunk c from its load
  // until it is stored to LDS, so each chunk's loads have KP - 1 chunks of
  // compute to land.  128-token blocks: two sets keep the kernel at 110
  // registers, two blocks per CU (stress layer in the step: one set 250.5
  // us, four sets at one block per CU 243.3, two sets 238.7); 32-token
  // blocks have little compute per chunk, so eight sets keep enough bytes
  // in flight.
  constexpr int KP = kTok == 128 ? 2 : 8;
  u32x4 rx[KP][XC], rw[KP][WC];
  float sx[XC];
#pragma unroll
  for (int u = 0; u < XC; ++u) sx[u] = 0.0f;
  // Loads are unconditional (rows past T or E re-read the last one, chunks
  // past the last re-read it; no output takes them), so the compiler's waits
  // can count them.
  auto load = [&](int ch, int set) __attribute__((always_inline)) {
    const int j0 = min(ch, nch - 1) * JA;
#pragma unroll
    for (int u = 0; u < XC; ++u) {
      const int c = min(tid + kNT * u, XCT - 1), r = c >> 3, cc = (c & 7) * 8;
      const int t = min(t0 + r, T - 1);
      rx[set][u] = *reinterpret_cast<const u32x4 *>(x + (size_t)t * d + j0 + cc);
    }
#pragma unroll
    for (int u = 0; u < WC; ++u) {
      const int c = min(tid + kNT * u, WCH - 1), r = min(c >> 3, E - 1), cc = (c & 7) * 8;
      rw[set][u] = *reinterpret_cast<const u32x4 *>(wh + (size_t)r * d + j0 + cc);
    }
  };
  auto store = [&](int st, int set, bool norm) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < XC; ++u) {
      const int c = tid + kNT * u, r = c >> 3, cc = (c & 7) * 8;
      if (c >= XCT) continue;
      *reinterpret_cast<u32x4 *>(&xa[st][r * LA + cc]) = rx[set][u];
      if (norm) {  // not for the re-reads past the last chunk
        float f[8];
        widen<OCC_BF16>(rx[set][u], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) sx[u] = __builtin_fmaf(f[i], f[i], sx[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < WC; ++u) {
      const int c = tid + kNT * u, r = c >> 3, cc = (c & 7) * 8;
      if (c < WCH) *reinterpret_cast<u32x4 *>(&wa[st][r * LA + cc]) = rw[set][u];
    }
  };
  ff32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
#pragma unroll
  for (int c = 0; c < KP; ++c) load(c, c);
  store(0, 0, true);
  load(KP, 0);
  __syncthreads();
  // chunk ch from LDS stage ch & 1; then chunk ch + 1 (register set SET =
  // (ch + 1) % KP) goes to the other stage and SET is refilled with chunk
  // ch + 1 + KP
  auto body = [&](int ch, auto setc) __attribute__((always_inline)) {
    constexpr int SET = decltype(setc)::value;
    const int st = ch & 1;
    if (wact && ch < nch) {
#pragma unroll
      for (int s = 0; s < JA / 16; ++s) {
        const int ko = s * 16 + (lane >> 5) * 8;
        const fbf16x8 af =
            *reinterpret_cast<const fbf16x8 *>(&xa[st][(tb * 32 + (lane & 31)) * LA + ko]);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const int eb = (id0 + i) % EB;
          const fbf16x8 bv =
              *reinterpret_cast<const fbf16x8 *>(&wa[st][(eb * 32 + (lane & 31)) * LA + ko]);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bv, acc[i], 0, 0, 0);
        }
      }
    }
    store(st ^ 1, SET, ch + 1 < nch);
    load(ch + 1 + KP, SET);
    __syncthreads();
  };
  static_assert(8 % KP == 0, "the loop below is unrolled by eight");
  for (int ch = 0; ch < nch; ch += 8) {
    body(ch, std::integral_constant<int, 1 % KP>{});
    body(ch + 1, std::integral_constant<int, 2 % KP>{});
    body(ch + 2, std::integral_constant<int, 3 % KP>{});
    body(ch + 3, std::integral_constant<int, 4 % KP>{});
    body(ch + 4, std::integral_constant<int, 5 % KP>{});
    body(ch + 5, std::integral_constant<int, 6 % KP>{});
    body(ch + 6, std::integral_constant<int, 7 % KP>{});
    body(ch + 7, std::integral_constant<int, 0>{});
  }
  if (wact) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int e = ((id0 + i) % EB) * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + tb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T && e < E) ag[(size_t)t * E + e] = acc[i][r];
      }
    }
  }
  // |x_t|: the 8 threads of a token row are consecutive lanes
#pragma unroll
  for (int u = 0; u < XC; ++u) {
    float v = sx[u];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    const int c = tid + kNT * u, t = t0 + (c >> 3);
    if ((tid & 7) == 0 && c < XCT && t < T) xn[t] = sqrtf(v);
  }
}

// ---- exact: certify, run the candidates' chains, softmax and top-k ---------
// Chains, KT = 128 tokens per block: lane = token 64 (wave / 4) + lane,
// slots q = (wave % 4) + 4 i of that token's candidate list (i < 4); KT = 32:
// lane = token lane % 32, the one slot 2 wave + lane / 32.  X is staged as
// bf16 (widened when read, one 16-byte read per 8 columns), the router as
// bf16 when every row is bf16-exact (else fp32), four chunks of loads ahead
// in registers.  KT = 128: 69 KB of LDS and at most 128 registers, so two
// blocks (four waves per SIMD) share a CU; KT = 32: one block per CU.
template <int EB, int KT>
__global__ __launch_bounds__(kNT, KT == 128 ? 4 : 2) void route_exact_kernel(
    int T, int d, int E, int k, int renorm, const uint16_t *__restrict__ x,
    const float *__restrict__ wr, const uint16_t *__restrict__ wh, const float *__restrict__ bnd,
    const int32_t *__restrict__ ex, float *__restrict__ agg, const float *__restrict__ xng,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
  constexpr int kTok = KT;                   // tokens per block
  static_assert(kTok == 128 || kTok == 32, "the two lane mappings below");
  constexpr int EPAD = 32 * EB;
  // columns per chunk: 64 for 32-token blocks, whose chunks carry little
  // compute, so that more bytes are in flight
  constexpr int JB = kTok == 128 ? 32 : 64;
  constexpr int LX = JB + 8, LW = JB + 4;    // row strides: bf16 X, fp32 router
  constexpr int KPF = 4;                     // register sets of loads in flight
  // X staging rows for every thread's piece: threads past the block's
  // tokens store into spare rows that nothing reads, so the stores (and the
  // loads feeding them) stay unconditional; a guarded store lets the
  // compiler sink its load next to it, one full memory latency per chunk
  constexpr int XROWS = kNT / (JB / 8) > kTok ? kNT / (JB / 8) : kTok;
  // router rows likewise (bf16 rows of JB / 8 pieces or fp32 rows of JB / 4)
  constexpr int WPN_B = (EPAD * JB / 8 + kNT - 1) / kNT, WPN_F = (EPAD * JB / 4 + kNT - 1) / kNT;
  constexpr int WROWS_B = WPN_B * kNT / (JB / 8), WROWS_F = WPN_F * kNT / (JB / 4);
  constexpr int WROWS = WROWS_B > WROWS_F ? (WROWS_B > EPAD ? WROWS_B : EPAD)
                                          : (WROWS_F > EPAD ? WROWS_F : EPAD);
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][XROWS * LX];
  __shared__ __attribute__((aligned(16))) float ws[2][WROWS * LW];
  __shared__ __attribute__((aligned(16))) float exl[kTok][kCap];
  __shared__ __attribute__((aligned(16))) uint8_t cl[kTok][kCap];
  __shared__ int32_t nc[kTok];
  __shared__ float am[kTok], znc[kTok];
  __shared__ int all_flag;
  __shared__ uint8_t pos_s[kTok], perm_s[kTok];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTok;
  if (tid == 0) all_flag = 0;
  float bmax = 0.0f;
  int rexact = 1;
  for (int e = lane; e < E; e += 64) {
    bmax = fmaxf(bmax, bnd[e]);
    rexact &= ex[e];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    bmax = fmaxf(bmax, __shfl_xor(bmax, off));
    rexact &= __shfl_xor(rexact, off);
  }
  __syncthreads();

  // candidates: a 16-lane segment per token (four tokens per wave at a
  // time, tt = wave + 8 (4 it + segment)); lane q of a segment holds the
  // approximate logits of experts PL q .. PL q + PL - 1
  {
    constexpr int PL = EPAD / 16;
    const int sgm = lane >> 4, q = lane & 15;
    for (int it = 0; it < kTok / (kNT / 64) / 4; ++it) {
      const int tt = wave + 8 * (4 * it + sgm), t = t0 + tt;
      const bool tok = t < T;
      float a[PL];
#pragma unroll
      for (int c = 0; c < PL; ++c) {
        const int e = PL * q + c;
        a[c] = (tok && e < E) ? agg[(size_t)t * E + e] : -INFINITY;
      }
      bool bad = false;
      bool live[PL];
#pragma unroll
      for (int c = 0; c < PL; ++c) {
        live[c] = PL * q + c < E;
        bad |= live[c] && !isfinite(a[c]);
      }
      // the k-th largest: k rounds of (segment max, retire its lowest holder)
      float kth = -INFINITY, amax = -INFINITY;
      bool v[PL];
#pragma unroll
      for (int c = 0; c < PL; ++c) v[c] = live[c];
      for (int j = 0; j < k; ++j) {
        float lm = -INFINITY;
#pragma unroll
        for (int c = 0; c < PL; ++c) lm = fmaxf(lm, v[c] ? a[c] : -INFINITY);
        const float m = row_max(lm);
        if (j == 0) amax = m;
        kth = m;
        int le = 0x7fffffff;
#pragma unroll
        for (int c = PL - 1; c >= 0; --c)
          if (v[c] && a[c] == m) le = PL * q + c;
        const int ge = row_min_i(le);
#pragma unroll
        for (int c = 0; c < PL; ++c)
          if (PL * q + c == ge) v[c] = false;
      }
      const float delta = (tok ? xng[t] : 0.0f) * bmax * 1.01f;
      const float theta = kth - 2.0f * delta;
      int lc = 0;
#pragma unroll
      for (int c = 0; c < PL; ++c) lc += (live[c] && a[c] >= theta) ? 1 : 0;
      const int pos = row_scan_i(lc) - lc;  // candidates of the lower lanes
      const int cnt = row_sum_i(lc);
      const bool segbad = row_max(bad ? 1.0f : 0.0f) > 0.0f;
      const bool ok = tok && !segbad && isfinite(theta) && isfinite(amax) && cnt <= kCap;
      if (tok && !ok) {
        if (q == 0) nc[tt] = -1;
        all_flag = 1;  // every lane of the segment writes the same value
      }
      float zl = 0.0f;
      int w = pos;
#pragma unroll
      for (int c = 0; c < PL; ++c) {
        const bool cand = live[c] && a[c] >= theta;
        if (ok && cand) cl[tt][w] = (uint8_t)(PL * q + c);
        w += cand ? 1 : 0;
        if (live[c] && !cand) zl += expf(a[c] - amax);
      }
      // the other experts' share of the softmax sum, relative to amax
      const float z = row_sum(zl);
      if (q == 0 && ok) {
        nc[tt] = cnt;
        am[tt] = amax;
        znc[tt] = z;
      }
      if (q == 0 && !tok) nc[tt] = 0;
    }
  }
  __syncthreads();

  // every chain when a token could not be certified, or when the router rows
  // are not bf16-exact: then the approximate logits carry the rows' bf16
  // rounding, too coarse for the softmax sum of the other experts
  const bool full = all_flag != 0 || !rexact;  // uniform
  const int npass = full ? (E + kCap - 1) / kCap : 1;
  // Certified blocks order their tokens by candidate count (descending, then
  // token index) before the chains: a wave runs as many slots as the largest
  // count among its 64 tokens, and grouping similar counts cuts the idle
  // slots (the stress layer's padding 1.28 -> 1.15 times the chains).  Token
  // row r of X is staged at LDS row pos_s[r], so a lane still reads row tl.
  if (!full) {
    if (tid < kTok) {
      const int mine = nc[tid];
      int rank = 0;
      for (int u = 0; u < kTok; ++u) {
        const int o = nc[u];
        rank += (o > mine || (o == mine && u < tid)) ? 1 : 0;
      }
      pos_s[tid] = (uint8_t)rank;
      perm_s[rank] = (uint8_t)tid;
    }
    __syncthreads();
  }
  // chain slots: 128 tokens -> a lane keeps token 64 (wave / 4) + lane and
  // slots (wave % 4) + 4 i, i < 4; 32 tokens -> token lane % 32 and the one
  // slot 2 wave + lane / 32
  constexpr int SPL = kCap * kTok / kNT;     // slots per lane
  constexpr int NSG = kCap / SPL;            // slot groups
  const int tl = kTok == 128 ? 64 * (wave >> 2) + lane : (lane & 31);
  const int sg = kTok == 128 ? (wave & 3) : 2 * wave + (lane >> 5);
  const int tok = full ? tl : (int)perm_s[tl];  // the token of this lane's chains
  const int ntk = t0 + tok < T ? (full ? E : nc[tok]) : 0;
  constexpr int XCT = kTok * JB / 8;         // 16-byte X pieces per chunk (one per thread at most)
  static_assert(XCT <= kNT, "one X load per thread and chunk");
  const int xr0 = min(tid, XCT - 1) / (JB / 8);  // this thread's X row (token)
  const int xrow = tid >= XCT ? tid / (JB / 8)    // a spare row
                   : full ? xr0 : (int)pos_s[xr0];  // ... and its LDS row
  const int nchb = d / JB;
  // one pass over d for the chains of slots p * kCap + sg + 4 i.  The
  // certified path (one pass) writes only LDS, the every-chain path writes
  // the exact logits back to global memory: kept apart, so that the
  // barriers of the certified path need not wait for global stores (which
  // share the completion counter with the loads in flight)
  auto pass = [&](int p, auto fullc) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(fullc)::value;
    int ei[SPL];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int q = p * kCap + sg + NSG * i;
      const bool v = q < ntk;
      ei[i] = v ? (FULL ? q : (int)cl[tok][q]) : 0;
      mine += v ? 1 : 0;
    }
    int nmax = mine;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nmax = max(nmax, __shfl_xor(nmax, off));
    float acc[SPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i) acc[i] = 0.0f;
    // One pass over d.  RB: the router rows are bf16-exact and stream from the
    // workspace's bf16 copy (one 16-byte LDS read per chain and 8 columns,
    // widened in registers); otherwise fp32 rows (two reads).
    auto run = [&](auto rbc) __attribute__((always_inline)) {
      constexpr bool RB = decltype(rbc)::value;
      constexpr int WCN = RB ? EPAD * JB / 8 : EPAD * JB / 4;  // 16-byte router loads
      constexpr int WPN = (WCN + kNT - 1) / kNT;
      constexpr int WPR = RB ? JB / 8 : JB / 4;                // loads per router row
      // register ring: set (c % KP) holds chunk c until it is stored to LDS
      // (four sets for bf16 router rows, two for fp32 ones: registers)
      constexpr int KP = RB ? KPF : 2;
      u32x4 bx[KP];
      u32x4 bw[KP][WPN];
      // Loads are unconditional (rows past T or E re-read the last one, which
      // no chain or output uses), so the compiler's waits can count them.
      auto loadb = [&](int c, int set) __attribute__((always_inline)) {
        const int j0 = c * JB;
        {
          const int cc = (tid % (JB / 8)) * 8, t = min(t0 + xr0, T - 1);
          bx[set] = *reinterpret_cast<const u32x4 *>(x + (size_t)t * d + j0 + cc);
        }
#pragma unroll
        for (int u = 0; u < WPN; ++u) {
          const int cw = min(tid + kNT * u, WCN - 1), r = min(cw / WPR, E - 1);
          const int cc = (cw % WPR) * (RB ? 8 : 4);
          if (RB) bw[set][u] = *reinterpret_cast<const u32x4 *>(wh + (size_t)r * d + j0 + cc);
          else bw[set][u] = *reinterpret_cast<const u32x4 *>(wr + (size_t)r * d + j0 + cc);
        }
      };
      auto storeb = [&](int st, int set) __attribute__((always_inline)) {
        {
          const int cc = (tid % (JB / 8)) * 8;
          *reinterpret_cast<u32x4 *>(&xs[st][xrow * LX + cc]) = bx[set];
        }
#pragma unroll
        for (int u = 0; u < WPN; ++u) {  // pieces past the router go to spare rows
          const int cw = tid + kNT * u, r = cw / WPR, cc = (cw % WPR) * (RB ? 8 : 4);
          if (RB) *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(ws[st]) + r * LX + cc) = bw[set][u];
          else *reinterpret_cast<u32x4 *>(&ws[st][r * LW + cc]) = bw[set][u];
        }
      };
      __syncthreads();  // earlier readers of the staging buffers are done
      // KPF register sets: set s holds chunk c (c % KPF == s) until it is
      // stored.  The chunk count is padded to a multiple of KPF; loads and
      // stores past the last chunk re-read it (in bounds) and only the FMAs
      // skip it, so every iteration issues the same loads and the compiler's
      // waits stay partial.
#pragma unroll
      for (int c = 0; c < KP; ++c) loadb(min(c, nchb - 1), c);
      storeb(0, 0);
      loadb(min(KP, nchb - 1), 0);
      __syncthreads();
      auto body = [&](int ch, auto setc) __attribute__((always_inline)) {
        constexpr int SET = decltype(setc)::value;  // the register set of chunk ch + 1
        const int st = ch & 1;
        if (ch < nchb) {
          const uint16_t *xr = &xs[st][tl * LX];
#pragma unroll
          for (int jj = 0; jj < JB; jj += 8) {
            float xf[8];
            widen<OCC_BF16>(*reinterpret_cast<const u32x4 *>(xr + jj), xf);
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
              if (i < nmax) {
                float wf[8];
                if (RB) {
                  widen<OCC_BF16>(*reinterpret_cast<const u32x4 *>(
                                      reinterpret_cast<const uint16_t *>(ws[st]) + ei[i] * LX + jj),
                                  wf);
                } else {
                  const float4 wa = *reinterpret_cast<const float4 *>(&ws[st][ei[i] * LW + jj]);
                  const float4 wb =
                      *reinterpret_cast<const float4 *>(&ws[st][ei[i] * LW + jj + 4]);
                  wf[0] = wa.x; wf[1] = wa.y; wf[2] = wa.z; wf[3] = wa.w;
                  wf[4] = wb.x; wf[5] = wb.y; wf[6] = wb.z; wf[7] = wb.w;
                }
                // j ascending inside every chain
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[i] = __builtin_fmaf(xf[c], wf[c], acc[i]);
              }
            }
          }
        }
        // chunk ch + 1 to the other stage, its set refilled with chunk
        // ch + 1 + KP
        storeb(st ^ 1, SET);
        loadb(min(ch + 1 + KP, nchb - 1), SET);
        __syncthreads();
      };
      static_assert(KPF == 4 && 4 % KP == 0, "the loop below is unrolled by four");
      for (int ch = 0; ch < nchb; ch += 4) {
        body(ch, std::integral_constant<int, 1 % KP>{});
        body(ch + 1, std::integral_constant<int, 2 % KP>{});
        body(ch + 2, std::integral_constant<int, 3 % KP>{});
        body(ch + 3, std::integral_constant<int, 0>{});
      }
    };
    if (FULL) {
      if (rexact) run(std::true_type{});
      else run(std::false_type{});
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int q = p * kCap + sg + NSG * i;
        if (q < ntk) agg[(size_t)(t0 + tl) * E + q] = acc[i];  // exact, in place
      }
    } else {
      run(std::true_type{});  // certified blocks have a bf16-exact router
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int q = sg + NSG * i;
        if (q < ntk) exl[tok][q] = acc[i];
      }
    }
  };
  if (!full) {
    pass(0, std::false_type{});
  } else {
    for (int p = 0; p < npass; ++p) pass(p, std::true_type{});
  }
  __syncthreads();  // also orders the block's global writes of exact logits before the reads

  if (!full) {
    // certified blocks: a 16-lane segment per token (four per wave at a
    // time), lane q holding candidate q; softmax over the candidates plus the
    // other experts' precomputed share, and each candidate's rank in
    // (logit descending, expert ascending) order is its output position
    const int sgm = lane >> 4, q = lane & 15;
#pragma unroll
    for (int it = 0; it < kTok / (kNT / 64) / 4; ++it) {
      const int tt = wave + 8 * (4 * it + sgm), t = t0 + tt;
      const int n = t < T ? nc[tt] : 0;
      const bool valid = q < n;
      const int e = valid ? (int)cl[tt][q] : 0;
      const float val = valid ? exl[tt][q] : 0.0f;
      const float key = valid ? (isnan(val) ? -INFINITY : val) : -INFINITY;
      const float mx = row_max(key);
      const float p = valid ? expf(val - mx) : 0.0f;
      float z = row_sum(p);
      if (n > 0) z += znc[tt] * expf(am[tt] - mx);
      int rank = 0;
      const float4 *kv = reinterpret_cast<const float4 *>(&exl[tt][0]);
      const u32x4 ev = *reinterpret_cast<const u32x4 *>(&cl[tt][0]);
#pragma unroll
      for (int v = 0; v < kCap / 4; ++v) {
        const float4 f = kv[v];
        const float fk[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int q2 = 4 * v + c;
          const int e2 = (int)((ev[q2 >> 2] >> (8 * (q2 & 3))) & 0xffu);
          const float k2 = isnan(fk[c]) ? -INFINITY : fk[c];
          rank += (q2 < n && (k2 > key || (k2 == key && e2 < e))) ? 1 : 0;
        }
      }
      const bool sel = valid && rank < k;
      const float psum = row_sum(sel ? p : 0.0f);
      if (sel) {
        idx_out[(size_t)t * k + rank] = e;
        w_out[(size_t)t * k + rank] = renorm ? p / psum : p / z;
      }
    }
    return;
  }

  // every chain (uncertified block): softmax over all experts, top-k in k rounds
  for (int tt = wave; tt < kTok; tt += kNT / 64) {
    const int t = t0 + tt;
    if (t >= T) continue;
    const int n = full ? 0 : nc[tt];
    float val[2], key[2], pp[2];
    bool sel[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = lane + 64 * h;
      const bool live = (h == 0 || EPAD > 64) && e < E;
      val[h] = 0.0f;
      sel[h] = false;
      if (full && live) {
        val[h] = agg[(size_t)t * E + e];
        sel[h] = true;
      }
      for (int q = 0; q < n; ++q)
        if (live && (int)cl[tt][q] == e) {
          val[h] = exl[tt][q];
          sel[h] = true;
        }
      key[h] = sel[h] ? (isnan(val[h]) ? -INFINITY : val[h]) : -INFINITY;
    }
    float mx = fmaxf(key[0], key[1]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float z = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pp[h] = sel[h] ? expf(val[h] - mx) : 0.0f;
      z += pp[h];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    if (!full) z += znc[tt] * expf(am[tt] - mx);
    int my_e = -1;
    float my_p = 0.0f, psum = 0.0f;
    for (int j = 0; j < k; ++j) {
      float bk = -INFINITY, bp = 0.0f;
      int be = 0x7fffffff;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = lane + 64 * h;
        if (sel[h] && (key[h] > bk || (key[h] == bk && e < be))) {
          bk = key[h];
          be = e;
          bp = pp[h];
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ok = __shfl_xor(bk, off);
        const int oe = __shfl_xor(be, off);
        const float op = __shfl_xor(bp, off);
        if (ok > bk || (ok == bk && oe < be)) {
          bk = ok;
          be = oe;
          bp = op;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (lane + 64 * h == be) sel[h] = false;
      psum += bp;
      if (lane == j) {
        my_e = be;
        my_p = bp;
      }
    }
    if (lane < k) {
      idx_out[(size_t)t * k + lane] = my_e;
      w_out[(size_t)t * k + lane] = renorm ? my_p / psum : my_p / z;
    }
  }
}

template <int EB, int KT>
hipError_t launch_eb(const occ_layer_desc &L, const void *x, const float *wr, int32_t *idx,
                     float *w, const FilterWs &f, hipStream_t st) {
  const dim3 grid((L.T + KT - 1) / KT);
  route_approx_kernel<EB, KT><<<grid, kNT, 0, st>>>(
      L.T, L.d, L.E, static_cast<const uint16_t *>(x), f.wh, f.ag, f.xn);
  route_exact_kernel<EB, KT><<<grid, kNT, 0, st>>>(L.T, L.d, L.E, L.k, L.renorm,
                                                   static_cast<const uint16_t *>(x), wr, f.wh,
                                                   f.bnd, f.ex, f.ag, f.xn, idx, w);
  return hipGetLastError();
}

}  // namespace

bool route_filter_applies(const occ_layer_desc &L) {
  return L.dtype == OCC_BF16 && L.E >= 32 && L.E <= 128 && L.k <= kCap && L.d % 64 == 0;
}

size_t route_filter_workspace_bytes(const occ_layer_desc &L) {
  if (!route_filter_applies(L)) return 0;
  return a256((size_t)L.E * L.d * 2) + 2 * a256((size_t)L.E * 4) + a256((size_t)L.T * L.E * 4) +
         a256((size_t)L.T * 4);
}

hipError_t launch_route_filtered(const occ_layer_desc &L, const void *x, const float *wr,
                                 int32_t *idx, float *w, void *ws, hipStream_t st) {
  if (L.T == 0) return hipSuccess;
  const FilterWs f = carve(L, ws);
  route_prep_kernel<<<L.E, 256, 0, st>>>(L.d, wr, f.wh, f.bnd, f.ex);
  // 128-token blocks from 32768 tokens (one per CU and more), 32-token
  // blocks below, where 128-token blocks leave most CUs idle (OLMoE-shaped
  // layer, 4096 tokens: 119 -> 49 us; DeepSeek-V2-Lite-shaped, 16384: 123 ->
  // 87 us; the chains of a 32-token block are one per lane, so their
  // latency bounds it)
  const bool big = L.T >= 32768;
  if (L.E > 64) return big ? launch_eb<4, 128>(L, x, wr, idx, w, f, st)
                           : launch_eb<4, 32>(L, x, wr, idx, w, f, st);
  return big ? launch_eb<2, 128>(L, x, wr, idx, w, f, st)
             : launch_eb<2, 32>(L, x, wr, idx, w, f, st);
}

}  // namespace occ
