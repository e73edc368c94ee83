// Backward pass through the BRIMs: gradient of the combine and of the
// routing (bf16 and fp32 layers).
//
// Expert Coupling in MoE Pretraining, Abstract: every MoE layer runs its
// all-to-alls in the forward and in the backward pass; Occult, Figure 4
// caption: the token states and their moves are guided by the BRIMs, which
// the backward walks in the opposite direction.  With the upstream gradient
// dY [T][d]:
//   grad-combine (one wave per ORI token, rows found through BRIM_0/BRIM_1):
//     d_out_sfd[s] = dY[t]                       (the backward send buffer)
//     d_out_epd[r] = w[r] * dY[t]                (rounded to the layer dtype)
//     dw[r]        = sum_c dY[t][c] out_epd[r][c] (fp32, the weight's gradient)
//   router: for the token's picks, dp from dw (through the renormalisation
//     when the weights were renormalised), then the softmax backward
//     dlogit[e] = p[e] (dp[e] - sum_e' p[e'] dp[e']) over all E experts;
//     dx_router = dlogit W_r and dW_r = dlogit^T X (fp32).
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = kThreads / kWave;

__device__ __forceinline__ void unpack_bf16(const u32x4 &u, float *f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack_bf16(const float *f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return u32x4{w[0], w[1], w[2], w[3]};
}

// 16-byte chunks of the layer dtype <-> fp32
template <int DT> struct Vec;
template <> struct Vec<OCC_BF16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const u32x4 &u, float *f) { unpack_bf16(u, f); }
  static __device__ __forceinline__ u32x4 pack(const float *f) { return pack_bf16(f); }
};
template <> struct Vec<OCC_F32> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const u32x4 &u, float *f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ u32x4 pack(const float *f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};

template <int DT, int NCH>
__global__ __launch_bounds__(kThreads) void grad_combine_kernel(
    int T, int D, int L, int ld, int row16, const u32x4 *__restrict__ dy,
    const int32_t *__restrict__ brim0, const int32_t *__restrict__ brim1,
    const float *__restrict__ epd_w, const u32x4 *__restrict__ out_epd,
    u32x4 *__restrict__ d_out_sfd, u32x4 *__restrict__ d_out_epd, float *__restrict__ dw) {
  using V = Vec<DT>;
  constexpr int VE = V::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave leaves together
  u32x4 v[NCH];
  float g[NCH][VE];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = lane + kWave * c;
    v[c] = i < row16 ? dy[(size_t)t * row16 + i] : u32x4{0u, 0u, 0u, 0u};
    V::unpack(v[c], g[c]);
  }
  const int npairs = D * L;
  for (int p0 = 0; p0 < npairs; p0 += kWave) {
    const int p = p0 + lane;
    int32_t s = -1, r = -1;
    bool first = false;
    float wr = 0.0f;
    if (p < npairs) {
      const int dv = p / L, l = p - dv * L;
      s = brim0[(size_t)dv * T + t];
      first = l == 0;
      if (s >= 0) {
        r = brim1[(size_t)l * ld + s];
        if (r >= 0) wr = epd_w[r];
      }
    }
    uint64_t ms = d_out_sfd != nullptr ? __ballot(first && s >= 0) : 0;
    uint64_t mr = __ballot(r >= 0);
    while (ms) {
      const int b = __ffsll((long long)ms) - 1;
      ms &= ms - 1;
      const int32_t row = __builtin_amdgcn_readlane(s, b);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane + kWave * c;
        if (i < row16) d_out_sfd[(size_t)row * row16 + i] = v[c];
      }
    }
    while (mr) {
      const int b = __ffsll((long long)mr) - 1;
      mr &= mr - 1;
      // the row's loads go out before the weight is read from its lane, so
      // they do not wait for the weight's load
      const int32_t row = __builtin_amdgcn_readlane(r, b);
      u32x4 ov[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane + kWave * c;
        if (i < row16) ov[c] = out_epd[(size_t)row * row16 + i];
      }
      const float wb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(wr), b));
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane + kWave * c;
        if (i < row16) {
          float o[VE], d[VE];
          V::unpack(ov[c], o);
#pragma unroll
          for (int u = 0; u < VE; ++u) {
            dot = __builtin_fmaf(g[c][u], o[u], dot);
            d[u] = wb * g[c][u];
          }
          d_out_epd[(size_t)row * row16 + i] = V::pack(d);
        }
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
      if (lane == 0) dw[row] = dot;
    }
  }
}

// One wave per token: dlogit[t][e] for every expert (E <= 128: two per lane).
__global__ __launch_bounds__(kThreads) void router_grad_kernel(
    int T, int E, int k, int D, int L, int ld, int renorm, Placement pl,
    const float *__restrict__ logits, const int32_t *__restrict__ idx,
    const float *__restrict__ topk_w, const int32_t *__restrict__ brim0,
    const int32_t *__restrict__ brim1, const float *__restrict__ dw,
    float *__restrict__ dlogit) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  const float *lt = logits + (size_t)t * E;
  float l0 = lane < E ? lt[lane] : -INFINITY, l1 = lane + kWave < E ? lt[lane + kWave] : -INFINITY;
  float mx = fmaxf(l0, l1);
  for (int off = kWave / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float p0 = lane < E ? expf(l0 - mx) : 0.0f, p1 = lane + kWave < E ? expf(l1 - mx) : 0.0f;
  float z = p0 + p1;
  for (int off = kWave / 2; off > 0; off >>= 1) z += __shfl_xor(z, off);
  p0 /= z;
  p1 /= z;
  // the picks: lane j < k holds pick j, its weight and its weight's gradient
  int ej = -1;
  float wj = 0.0f, gj = 0.0f;
  if (lane < k) {
    ej = idx[(size_t)t * k + lane];
    wj = topk_w[(size_t)t * k + lane];
    if ((unsigned)ej < (unsigned)OCC_MAX_E && pl.slot_of[ej] >= 0) {
      const int g = pl.slot_of[ej];
      const int32_t s = brim0[(size_t)(g / L) * T + t];
      const int32_t r = s >= 0 ? brim1[(size_t)(g % L) * ld + s] : -1;
      gj = r >= 0 ? dw[r] : 0.0f;
    }
  }
  // dp of the picks: renormalised weights w_j = p_j / P give
  // dp_j = (dw_j - sum_i dw_i w_i) / P, P = sum over the picks of p
  float dpj = gj;
  if (renorm) {
    // p of pick j lives in lane e % 64 (first or second half): fetch both
    // halves from that lane in uniform control flow, then choose
    const int src = ej >= 0 ? ej % kWave : 0;
    const float pa = __shfl(p0, src), pb = __shfl(p1, src);
    const float pj = (lane < k && ej >= 0) ? (ej < kWave ? pa : pb) : 0.0f;
    float P = pj, gw = lane < k ? gj * wj : 0.0f;
    for (int off = kWave / 2; off > 0; off >>= 1) {
      P += __shfl_xor(P, off);
      gw += __shfl_xor(gw, off);
    }
    dpj = (gj - gw) / P;
  }
  // scatter dp to the experts, then the softmax backward
  float dp0 = 0.0f, dp1 = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int e = __shfl(ej, j);
    const float d = __shfl(dpj, j);
    if (e == lane) dp0 = d;
    if (e == lane + kWave) dp1 = d;
  }
  float sdp = p0 * dp0 + p1 * dp1;
  for (int off = kWave / 2; off > 0; off >>= 1) sdp += __shfl_xor(sdp, off);
  float *dl = dlogit + (size_t)t * E;
  if (lane < E) dl[lane] = p0 * (dp0 - sdp);
  if (lane + kWave < E) dl[lane + kWave] = p1 * (dp1 - sdp);
}

// The router's two products, dx_router = dlogit W_r and dW_r = dlogit^T x,
// on the matrix cores in fp32 (v_mfma_f32_16x16x4f32: products exact,
// fp32 sums; the contractions over E and over T take a different order than
// a plain loop, within fp32 rounding):
//   C[z][m][n] = sum over k in chunk z of A(m, k) B(k, n)
//   A(m, k) = a[k * lda + m] when A_KM (m contiguous), a[m * lda + k] otherwise
//   B(k, n) = b[k * ldb + n] (fp32 or bf16, n contiguous, ldb % 8 == 0)
// A block owns a 128 x 128 tile of C and one chunk of K; four waves of
// 64 x 64 (4 x 4 MFMA blocks of 16 x 16, 64 accumulators per lane).  The
// operands pass through LDS 32 k at a time, in registers one slab ahead, each
// stored as it lies in memory (16-byte stores): A as [m][k] (row stride 36
// floats) or [k][m], B as [k][n] (row stride 132 floats).  MFMA operand
// layout: lane l supplies row (column) l % 16 at k-slot l / 16.  Per 16 k a
// lane feeds 4 successive MFMAs with k = k0 + 4 (l / 16) + s (s < 4), the same
// on both operands: one 16-byte read from a [m][k] tile, four 4-byte reads
// from a k-major one (conflict-free: the four k rows of a read are 4 rows
// apart, 16 banks).  Output element i of lane l is row 4 (l / 16) + i,
// column l % 16.
constexpr int kRBM = 128, kRBN = 128, kRBK = 32;
constexpr int kRLK = kRBK + 4;    // [m][k] row stride
constexpr int kRLN = kRBN + 4;    // [k][m] / [k][n] row stride
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <bool A_KM, int DT>
__global__ __launch_bounds__(kThreads, 2) void router_gemm_kernel(
    int M, int N, int K, int kchunk, const float *__restrict__ a, int lda,
    const typename Elem<DT>::T *__restrict__ b, int ldb, float *__restrict__ c) {
  constexpr int AST = A_KM ? kRBK * kRLN : kRBM * kRLK;  // floats per A stage
  constexpr int BST = kRBK * kRLN;
  __shared__ __attribute__((aligned(16))) float As[2 * AST];
  __shared__ __attribute__((aligned(16))) float Bs[2 * BST];
  constexpr int BW = DT == OCC_BF16 ? 8 : 4;       // B elements per 16-byte load
  constexpr int ALOADS = kRBM * kRBK / 4 / kThreads;
  constexpr int BLOADS = kRBK * kRBN / BW / kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kRBM, n0 = blockIdx.x * kRBN;
  const int k_lo = blockIdx.z * kchunk;
  const int k_hi = min(K, k_lo + kchunk);
  f32x4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  float4 ar[ALOADS];
  u32x4 br[BLOADS];
  // element (r, cq) of a thread's j-th 16-byte piece: A_KM and B pieces are 4
  // (8) consecutive m (n) at one k, the others 4 consecutive k of one m
  auto a_piece = [&](int j, int &r, int &cq) {
    const int q = tid + kThreads * j;
    if (A_KM) {
      r = q / (kRBM / 4);
      cq = (q % (kRBM / 4)) * 4;
    } else {
      r = q / (kRBK / 4);
      cq = (q % (kRBK / 4)) * 4;
    }
  };
  // Rows past M or N and k past the chunk load zeros (their products are 0).
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < ALOADS; ++j) {
      int r, cq;
      a_piece(j, r, cq);
      const int k = k0 + (A_KM ? r : cq), m = m0 + (A_KM ? cq : r);
      ar[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      const int lim_c = A_KM ? M - m : k_hi - k;  // valid elements along the piece
      if (k < k_hi && m < M) {
        const float *src = A_KM ? a + (size_t)k * lda + m : a + (size_t)m * lda + k;
        if (lim_c >= 4 && (lda & 3) == 0) {
          ar[j] = *reinterpret_cast<const float4 *>(src);
        } else {
          ar[j].x = src[0];
          ar[j].y = lim_c > 1 ? src[1] : 0.f;
          ar[j].z = lim_c > 2 ? src[2] : 0.f;
          ar[j].w = lim_c > 3 ? src[3] : 0.f;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < BLOADS; ++j) {
      const int q = tid + kThreads * j;
      const int kk = q / (kRBN / BW), n = n0 + (q % (kRBN / BW)) * BW;
      const int k = k0 + kk;
      br[j] = (k < k_hi && n < N)
                  ? *reinterpret_cast<const u32x4 *>(b + (size_t)k * ldb + n)
                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int j = 0; j < ALOADS; ++j) {
      int r, cq;
      a_piece(j, r, cq);
      *reinterpret_cast<float4 *>(&As[st * AST + r * (A_KM ? kRLN : kRLK) + cq]) = ar[j];
    }
#pragma unroll
    for (int j = 0; j < BLOADS; ++j) {
      const int q = tid + kThreads * j;
      const int kk = q / (kRBN / BW), nn = (q % (kRBN / BW)) * BW;
      float f[BW];
      widen<DT>(br[j], f);
#pragma unroll
      for (int i = 0; i < BW; i += 4)
        *reinterpret_cast<float4 *>(&Bs[st * BST + kk * kRLN + nn + i]) =
            make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
    }
  };

  const int fr = lane & 15, fk = (lane >> 4) * 4;
  // fragment bases: [m][k] tiles at row m, column k; k-major tiles at row k
  const int a_rd = A_KM ? fk * kRLN + wm * 64 + fr : (wm * 64 + fr) * kRLK + fk;
  const int b_rd = fk * kRLN + wn * 64 + fr;
  int st = 0;
  if (k_lo < k_hi) {
    load(k_lo);
    store(0);
    __syncthreads();
  }
  for (int k0 = k_lo; k0 < k_hi; k0 += kRBK) {
    if (k0 + kRBK < k_hi) load(k0 + kRBK);
    const float *ab = As + st * AST + a_rd;
    const float *bb = Bs + st * BST + b_rd;
#pragma unroll
    for (int g = 0; g < kRBK / 16; ++g) {
      float af[4][4], bf[4][4];  // [block][step]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (A_KM) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) af[i][s4] = ab[(16 * g + s4) * kRLN + i * 16];
        } else {
          const float4 v = *reinterpret_cast<const float4 *>(ab + i * 16 * kRLK + 16 * g);
          af[i][0] = v.x; af[i][1] = v.y; af[i][2] = v.z; af[i][3] = v.w;
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) bf[i][s4] = bb[(16 * g + s4) * kRLN + i * 16];
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][s4], bf[j][s4], acc[i][j], 0, 0, 0);
    }
    if (k0 + kRBK < k_hi) {
      store(st ^ 1);  // the other stage: its last readers passed the barrier below
      __syncthreads();
      st ^= 1;
    }
  }
  float *cz = c + (size_t)blockIdx.z * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + fk + r;
        if (m < M && n < N) cz[(size_t)m * N + n] = acc[i][j][r];
      }
    }
}

// out[i] = sum over z ascending of part[z][i] (n4 float4 groups per part).
__global__ __launch_bounds__(kThreads) void chunk_sum_kernel(int64_t n4, int chunks,
                                                             const float4 *__restrict__ part,
                                                             float4 *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  float4 s = part[i];
  for (int z = 1; z < chunks; ++z) {
    const float4 v = part[z * n4 + i];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  out[i] = s;
}

// Split of dW_r's contraction over T: about two blocks per compute unit,
// chunks of at least 128 tokens.
int router_dw_kchunk(const occ_layer_desc &Ld) {
  const int tiles = ((Ld.E + kRBM - 1) / kRBM) * ((Ld.d + kRBN - 1) / kRBN);
  const int want = (512 + tiles - 1) / tiles;
  const int most = (Ld.T + 127) / 128;
  const int chunks = std::max(1, std::min(want, most));
  const int per = (Ld.T + chunks - 1) / chunks;
  return std::max(kRBK, (per + kRBK - 1) / kRBK * kRBK);
}

int chunks_per_lane(int row16) { return (row16 + kWave - 1) / kWave; }

}  // namespace

hipError_t launch_grad_combine(const occ_layer_desc &Ld, const void *dy, const occ_brim &b,
                               const void *out_epd, void *d_out_sfd, void *d_out_epd, float *dw,
                               hipStream_t st) {
  if (Ld.T == 0) return hipSuccess;
  const int row16 = Ld.d * (Ld.dtype == OCC_F32 ? 4 : 2) / 16;
  const int L = Ld.E / Ld.D;
  const int ld = Ld.T * (Ld.k < Ld.D ? Ld.k : Ld.D);
  const dim3 grid((Ld.T + kTokPerBlock - 1) / kTokPerBlock);
  const int nch = chunks_per_lane(row16);
#define OCC_GC(DT, N)                                                                        \
  grad_combine_kernel<DT, N><<<grid, kThreads, 0, st>>>(                                     \
      Ld.T, Ld.D, L, ld, row16, static_cast<const u32x4 *>(dy), b.brim0, b.brim1, b.epd_w,   \
      static_cast<const u32x4 *>(out_epd), static_cast<u32x4 *>(d_out_sfd),                  \
      static_cast<u32x4 *>(d_out_epd), dw)
  if (Ld.dtype == OCC_F32) {
    if (nch <= 1) OCC_GC(OCC_F32, 1);
    else if (nch <= 2) OCC_GC(OCC_F32, 2);
    else if (nch <= 4) OCC_GC(OCC_F32, 4);
    else OCC_GC(OCC_F32, 8);
  } else {
    if (nch <= 1) OCC_GC(OCC_BF16, 1);
    else if (nch <= 2) OCC_GC(OCC_BF16, 2);
    else if (nch <= 4) OCC_GC(OCC_BF16, 4);
    else OCC_GC(OCC_BF16, 8);
  }
#undef OCC_GC
  return hipGetLastError();
}

size_t router_backward_ws_bytes(const occ_layer_desc &Ld) {
  const int kc = router_dw_kchunk(Ld);
  const int chunks = Ld.T > 0 ? (Ld.T + kc - 1) / kc : 1;
  return chunks > 1 ? (size_t)chunks * Ld.E * Ld.d * sizeof(float) : 0;
}

hipError_t launch_router_backward(const occ_layer_desc &Ld, const Placement &pl, const void *x,
                                  const float *w_router, const float *logits,
                                  const int32_t *idx, const float *topk_w, const occ_brim &b,
                                  const float *dw, float *dlogit, float *dx_router,
                                  float *dw_router, void *ws, hipStream_t st) {
  const int T = Ld.T, E = Ld.E, d = Ld.d, L = Ld.E / Ld.D;
  const int ld = Ld.T * (Ld.k < Ld.D ? Ld.k : Ld.D);
  using BT = Elem<OCC_BF16>::T;
  if (T > 0) {
    router_grad_kernel<<<(T + kTokPerBlock - 1) / kTokPerBlock, kThreads, 0, st>>>(
        T, E, Ld.k, Ld.D, L, ld, Ld.renorm, pl, logits, idx, topk_w, b.brim0, b.brim1, dw,
        dlogit);
    const dim3 gx((d + kRBN - 1) / kRBN, (T + kRBM - 1) / kRBM, 1);
    router_gemm_kernel<false, OCC_F32><<<gx, kThreads, 0, st>>>(
        T, d, E, (E + kRBK - 1) / kRBK * kRBK, dlogit, E, w_router, d, dx_router);
  }
  const int kc = router_dw_kchunk(Ld);
  const int chunks = T > 0 ? (T + kc - 1) / kc : 1;
  const dim3 gw((d + kRBN - 1) / kRBN, (E + kRBM - 1) / kRBM, chunks);
  float *dst = chunks > 1 ? static_cast<float *>(ws) : dw_router;
  if (Ld.dtype == OCC_F32)
    router_gemm_kernel<true, OCC_F32><<<gw, kThreads, 0, st>>>(
        E, d, T, kc, dlogit, E, static_cast<const float *>(x), d, dst);
  else
    router_gemm_kernel<true, OCC_BF16><<<gw, kThreads, 0, st>>>(
        E, d, T, kc, dlogit, E, static_cast<const BT *>(x), d, dst);
  if (chunks > 1) {
    const int64_t n4 = (int64_t)E * d / 4;
    chunk_sum_kernel<<<(unsigned)((n4 + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        n4, chunks, static_cast<const float4 *>(ws), reinterpret_cast<float4 *>(dw_router));
  }
  return hipGetLastError();
}

}  // namespace occ
