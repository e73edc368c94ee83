// Backward pass through the BRIMs (bf16 layers): gradient of the combine and
// of the routing.
//
// Expert Coupling in MoE Pretraining, Abstract: every MoE layer runs its
// all-to-alls in the forward and in the backward pass; Occult, Figure 4
// caption: the token states and their moves are guided by the BRIMs, which
// the backward walks in the opposite direction.  With the upstream gradient
// dY [T][d]:
//   grad-combine (one wave per ORI token, rows found through BRIM_0/BRIM_1):
//     d_out_sfd[s] = dY[t]                       (the backward send buffer)
//     d_out_epd[r] = w[r] * dY[t]                (rounded to bf16)
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

template <int NCH>
__global__ __launch_bounds__(kThreads) void grad_combine_kernel(
    int T, int D, int L, int ld, int row16, const u32x4 *__restrict__ dy,
    const int32_t *__restrict__ brim0, const int32_t *__restrict__ brim1,
    const float *__restrict__ epd_w, const u32x4 *__restrict__ out_epd,
    u32x4 *__restrict__ d_out_sfd, u32x4 *__restrict__ d_out_epd, float *__restrict__ dw) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave leaves together
  u32x4 v[NCH];
  float g[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = lane + kWave * c;
    v[c] = i < row16 ? dy[(size_t)t * row16 + i] : u32x4{0u, 0u, 0u, 0u};
    unpack_bf16(v[c], g[c]);
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
      const int32_t row = __builtin_amdgcn_readlane(r, b);
      const float wb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(wr), b));
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane + kWave * c;
        if (i < row16) {
          float o[8], d[8];
          unpack_bf16(out_epd[(size_t)row * row16 + i], o);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            dot = __builtin_fmaf(g[c][u], o[u], dot);
            d[u] = wb * g[c][u];
          }
          d_out_epd[(size_t)row * row16 + i] = pack_bf16(d);
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

// dx_router[t][c] = sum_e dlogit[t][e] W_r[e][c]  (one thread per output)
__global__ __launch_bounds__(kThreads) void router_dx_kernel(int T, int d, int E,
                                                             const float *__restrict__ dlogit,
                                                             const float *__restrict__ wr,
                                                             float *__restrict__ dx) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (int64_t)T * d) return;
  const int t = (int)(gid / d), c = (int)(gid % d);
  const float *dl = dlogit + (size_t)t * E;
  float s = 0.0f;
  for (int e = 0; e < E; ++e) s = __builtin_fmaf(dl[e], wr[(size_t)e * d + c], s);
  dx[gid] = s;
}

// dW_r[e][c] = sum_t dlogit[t][e] x[t][c]: a block owns 8 experts and 256
// columns and walks all tokens (deterministic, no atomics).
template <int DT>
__global__ __launch_bounds__(kThreads) void router_dw_kernel(int T, int d, int E,
                                                             const float *__restrict__ dlogit,
                                                             const typename Elem<DT>::T *__restrict__ x,
                                                             float *__restrict__ dwr) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const int e0 = blockIdx.y * 8;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < T; ++t) {
    const float xv = c < d ? Elem<DT>::to_f32(x[(size_t)t * d + c]) : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (e0 + j < E) s[j] = __builtin_fmaf(dlogit[(size_t)t * E + e0 + j], xv, s[j]);
  }
  if (c < d)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (e0 + j < E) dwr[(size_t)(e0 + j) * d + c] = s[j];
}

int chunks_per_lane(int row16) { return (row16 + kWave - 1) / kWave; }

}  // namespace

hipError_t launch_grad_combine(const occ_layer_desc &Ld, const void *dy, const occ_brim &b,
                               const void *out_epd, void *d_out_sfd, void *d_out_epd, float *dw,
                               hipStream_t st) {
  if (Ld.T == 0) return hipSuccess;
  const int row16 = Ld.d * 2 / 16;
  const int L = Ld.E / Ld.D;
  const int ld = Ld.T * (Ld.k < Ld.D ? Ld.k : Ld.D);
  const dim3 grid((Ld.T + kTokPerBlock - 1) / kTokPerBlock);
  const int nch = chunks_per_lane(row16);
#define OCC_GC(N)                                                                            \
  grad_combine_kernel<N><<<grid, kThreads, 0, st>>>(                                         \
      Ld.T, Ld.D, L, ld, row16, static_cast<const u32x4 *>(dy), b.brim0, b.brim1, b.epd_w,   \
      static_cast<const u32x4 *>(out_epd), static_cast<u32x4 *>(d_out_sfd),                  \
      static_cast<u32x4 *>(d_out_epd), dw)
  if (nch <= 1) OCC_GC(1);
  else if (nch <= 2) OCC_GC(2);
  else if (nch <= 4) OCC_GC(4);
  else OCC_GC(8);
#undef OCC_GC
  return hipGetLastError();
}

hipError_t launch_router_backward(const occ_layer_desc &Ld, const Placement &pl, const void *x,
                                  const float *w_router, const float *logits,
                                  const int32_t *idx, const float *topk_w, const occ_brim &b,
                                  const float *dw, float *dlogit, float *dx_router,
                                  float *dw_router, hipStream_t st) {
  const int T = Ld.T, E = Ld.E, d = Ld.d, L = Ld.E / Ld.D;
  const int ld = Ld.T * (Ld.k < Ld.D ? Ld.k : Ld.D);
  if (T > 0) {
    router_grad_kernel<<<(T + kTokPerBlock - 1) / kTokPerBlock, kThreads, 0, st>>>(
        T, E, Ld.k, Ld.D, L, ld, Ld.renorm, pl, logits, idx, topk_w, b.brim0, b.brim1, dw,
        dlogit);
    const int64_t n = (int64_t)T * d;
    router_dx_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(
        T, d, E, dlogit, w_router, dx_router);
  }
  const dim3 grid((d + kThreads - 1) / kThreads, (E + 7) / 8);
  if (Ld.dtype == OCC_F32)
    router_dw_kernel<OCC_F32><<<grid, kThreads, 0, st>>>(T, d, E, dlogit,
                                                          static_cast<const float *>(x), dw_router);
  else
    router_dw_kernel<OCC_BF16><<<grid, kThreads, 0, st>>>(
        T, d, E, dlogit, static_cast<const Elem<OCC_BF16>::T *>(x), dw_router);
  return hipGetLastError();
}

}  // namespace occ
