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
// as one fp32 VALU tile kernel (contractions over E and over T in fp32;
// neither is large enough to pay for a split into bf16 MFMA operands).
//   C[z][m][n] = sum over k in chunk z of A(m, k) B(k, n)
//   A(m, k) = a[k * lda + m] when A_KM (m contiguous), a[m * lda + k] otherwise
//   B(k, n) = b[k * ldb + n] (fp32 or bf16, n contiguous, ldb % 8 == 0)
// A block owns a 64 x 128 tile of C and one chunk of K (kchunk % 32 == 0);
// each thread keeps 8 x 4 outputs in registers, both operands pass through
// LDS 32 k at a time with the next k-slab's loads in flight.
constexpr int kRBM = 64, kRBN = 128, kRBK = 32;

template <bool A_KM, int DT>
__global__ __launch_bounds__(kThreads) void router_gemm_kernel(
    int M, int N, int K, int kchunk, const float *__restrict__ a, int lda,
    const typename Elem<DT>::T *__restrict__ b, int ldb, float *__restrict__ c) {
  __shared__ float As[kRBK][kRBM + 4];
  __shared__ float Bs[kRBK][kRBN];
  constexpr int BW = DT == OCC_BF16 ? 8 : 4;  // B elements per 16-byte load
  constexpr int BLOADS = kRBK * kRBN / BW / kThreads;
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * kRBM, n0 = blockIdx.x * kRBN;
  const int k_lo = blockIdx.z * kchunk;
  const int k_hi = min(K, k_lo + kchunk);
  const int tx = tid % 32, ty = tid / 32;  // outputs: cols n0+4tx.., rows m0+8ty..
  float acc[8][4] = {};
  float ar[8];
  u32x4 br[BLOADS];

  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = tid + kThreads * j;
      const int kk = A_KM ? q / kRBM : q % kRBK, mm = A_KM ? q % kRBM : q / kRBK;
      const int k = k0 + kk, m = m0 + mm;
      ar[j] = (k < k_hi && m < M) ? (A_KM ? a[(size_t)k * lda + m] : a[(size_t)m * lda + k])
                                  : 0.0f;
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
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = tid + kThreads * j;
      As[A_KM ? q / kRBM : q % kRBK][A_KM ? q % kRBM : q / kRBK] = ar[j];
    }
#pragma unroll
    for (int j = 0; j < BLOADS; ++j) {
      const int q = tid + kThreads * j;
      float f[BW];
      widen<DT>(br[j], f);
      float *dst = &Bs[q / (kRBN / BW)][(q % (kRBN / BW)) * BW];
#pragma unroll
      for (int i = 0; i < BW; i += 4)
        *reinterpret_cast<float4 *>(dst + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
    }
  };

  if (k_lo < k_hi) load(k_lo);
  for (int k0 = k_lo; k0 < k_hi; k0 += kRBK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + kRBK < k_hi) load(k0 + kRBK);
#pragma unroll 8
    for (int kk = 0; kk < kRBK; ++kk) {
      const float4 a0 = *reinterpret_cast<const float4 *>(&As[kk][ty * 8]);
      const float4 a1 = *reinterpret_cast<const float4 *>(&As[kk][ty * 8 + 4]);
      const float4 bv = *reinterpret_cast<const float4 *>(&Bs[kk][tx * 4]);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bw[j], acc[i][j]);
    }
  }
  const int n = n0 + tx * 4;
  if (n >= N) return;
  float *cz = c + (size_t)blockIdx.z * M * N;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + ty * 8 + i;
    if (m < M)
      *reinterpret_cast<float4 *>(cz + (size_t)m * N + n) =
          make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
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
