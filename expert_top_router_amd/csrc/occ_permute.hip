// Dispatch (ORI -> SFD -> EPD) and combine (EPD -> SFD -> ORI).
//
// Occult, Figure 4 caption: token tensors ORI, SFD and EPD are stored
// compactly on HBM and the all-to-all and expert computing are guided by the
// BRIMs in both directions.  One wave owns one ORI token:
//   dispatch: read x[t] once into registers, write it to each of its SFD rows
//             (BRIM_0 column t) and each of its EPD rows (BRIM_1 columns of
//             those SFD rows);
//   combine:  for each of its devices (ascending) sum w * out_EPD over the
//             device's experts (local index ascending) in fp32, store that
//             pre-reduced row to out_SFD (the return payload) and add it, as
//             stored, into y[t].
// The conventional strategy of Occult, Figure 2 (one row per (token, expert)
// pair, no deduplication) is the same walk without the SFD stage: dispatch
// writes only the EPD rows, and combine sums w * out_EPD over all of the
// token's rows (device, then local expert ascending) into y in fp32 with a
// single rounding, storing no pre-reduced payload.
// Index lookups are lane-parallel: lane p of a pass holds pair (device
// p / L, local expert p % L); ballots then walk the present rows in
// ascending (device, local) order.  Rows move as 16-byte per-lane chunks,
// 1 KiB per wave instruction, so every row access is fully coalesced.
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = kThreads / kWave;

template <int NCH, bool SFD>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    int T, int D, int L, int ld, int row16, const u32x4 *__restrict__ x,
    const int32_t *__restrict__ brim0, const int32_t *__restrict__ brim1,
    u32x4 *__restrict__ sfd, u32x4 *__restrict__ epd) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;  // whole wave leaves together
  u32x4 v[NCH];
  const u32x4 *src = x + (size_t)t * row16;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = lane + kWave * c;
    if (i < row16) v[c] = src[i];
  }
  const int npairs = D * L;
  for (int p0 = 0; p0 < npairs; p0 += kWave) {
    const int p = p0 + lane;
    int32_t s = -1, r = -1;
    bool first = false;
    if (p < npairs) {
      const int dv = p / L, l = p - dv * L;
      s = brim0[(size_t)dv * T + t];
      first = l == 0;
      if (s >= 0) r = brim1[(size_t)l * ld + s];
    }
    uint64_t ms = SFD ? __ballot(first && s >= 0) : 0;
    uint64_t mr = __ballot(r >= 0);
    while (ms) {
      const int b = __ffsll((long long)ms) - 1;
      ms &= ms - 1;
      const int32_t row = __builtin_amdgcn_readlane(s, b);
      u32x4 *dst = sfd + (size_t)row * row16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane + kWave * c;
        // the send buffer is not read again by this step: non-temporal
        // stores keep it out of the caches the expert GEMM reads through
        if (i < row16) __builtin_nontemporal_store(v[c], dst + i);
      }
    }
    while (mr) {
      const int b = __ffsll((long long)mr) - 1;
      mr &= mr - 1;
      const int32_t row = __builtin_amdgcn_readlane(r, b);
      u32x4 *dst = epd + (size_t)row * row16;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = lane + kWave * c;
        if (i < row16) dst[i] = v[c];
      }
    }
  }
}

// 16-byte chunk <-> fp32 lanes
template <int DT> struct Chunk;
template <> struct Chunk<OCC_BF16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const u32x4 &u, float *f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float *f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
  }
  // value as stored (rounded to bf16), back in fp32
  static __device__ __forceinline__ float stored(float f) { return bf16_to_f32(f32_to_bf16(f)); }
};
template <> struct Chunk<OCC_F32> {
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
  static __device__ __forceinline__ float stored(float f) { return f; }
};

// CSPLIT waves share a token, each owning a contiguous range of its row's
// 16-byte chunks (the per-lane fp32 sums of a wide row would otherwise limit
// the waves, hence the rows, in flight); each walks the token's BRIM entries
// itself.
template <int DT, int NCH, bool PRE, int CSPLIT>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    int T, int D, int L, int ld, int row16, const u32x4 *__restrict__ out_epd,
    const int32_t *__restrict__ brim0, const int32_t *__restrict__ brim1,
    const float *__restrict__ epd_w, const u32x4 *__restrict__ shared, u32x4 *__restrict__ out_sfd,
    u32x4 *__restrict__ y, const float *__restrict__ add32) {
  using CK = Chunk<DT>;
  constexpr int VE = CK::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kTokPerBlock + threadIdx.x / kWave;
  const int t = gw / CSPLIT, part = gw - t * CSPLIT;
  if (t >= T) return;
  // this wave's chunks: [cb, ce) of the row
  const int cb = part * row16 / CSPLIT, ce = (part + 1) * row16 / CSPLIT;
  const int i0 = cb + lane;
  float yacc[NCH][VE], acc[NCH][VE];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = i0 + kWave * c;
    if (shared != nullptr && i < ce) {
      CK::unpack(shared[(size_t)t * row16 + i], yacc[c]);
    } else {
#pragma unroll
      for (int u = 0; u < VE; ++u) yacc[c][u] = 0.0f;
    }
    // an fp32 term (the backward's dx_router), first in the sum; loaded here
    // so that its latency overlaps the EPD row loads
    if (add32 != nullptr && i < ce) {
      const float *ap = add32 + ((size_t)t * row16 + i) * VE;
#pragma unroll
      for (int u = 0; u < VE; ++u) yacc[c][u] += ap[u];
    }
#pragma unroll
    for (int u = 0; u < VE; ++u) acc[c][u] = 0.0f;
  }
  int cur_dev = -1;
  int32_t cur_s = -1;
  auto finish_device = [&]() {
    u32x4 *dst = out_sfd + (size_t)cur_s * row16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int i = i0 + kWave * c;
#pragma unroll
      for (int u = 0; u < VE; ++u) {
        const float v = CK::stored(acc[c][u]);
        acc[c][u] = v;
      }
      // the return payload is not read again by this step (non-temporal)
      if (i < ce) __builtin_nontemporal_store(CK::pack(acc[c]), dst + i);
#pragma unroll
      for (int u = 0; u < VE; ++u) {
        yacc[c][u] += acc[c][u];
        acc[c][u] = 0.0f;
      }
    }
  };
  const int npairs = D * L;
  for (int p0 = 0; p0 < npairs; p0 += kWave) {
    const int p = p0 + lane;
    int32_t s = -1, r = -1;
    float wr = 0.0f;
    if (p < npairs) {
      const int dv = p / L, l = p - dv * L;
      s = brim0[(size_t)dv * T + t];
      if (s >= 0) {
        r = brim1[(size_t)l * ld + s];
        if (r >= 0) wr = epd_w != nullptr ? epd_w[r] : 1.0f;
      }
    }
    uint64_t mr = __ballot(r >= 0);
    while (mr) {
      const int b = __ffsll((long long)mr) - 1;
      mr &= mr - 1;
      const int dv = (p0 + b) / L;
      if (PRE && dv != cur_dev) {
        if (cur_dev >= 0) finish_device();
        cur_dev = dv;
        cur_s = __builtin_amdgcn_readlane(s, b);
      }
      // the row's loads go out before the weight is read from its lane, so
      // they do not wait for the weight's load (one dependent latency fewer)
      const int32_t row = __builtin_amdgcn_readlane(r, b);
      const u32x4 *srcp = out_epd + (size_t)row * row16;
      u32x4 v[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = i0 + kWave * c;
        if (i < ce) v[c] = srcp[i];
      }
      const float wb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(wr), b));
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int i = i0 + kWave * c;
        if (i < ce) {
          float f[VE];
          CK::unpack(v[c], f);
#pragma unroll
          for (int u = 0; u < VE; ++u) {
            if (PRE) acc[c][u] = __builtin_fmaf(wb, f[u], acc[c][u]);
            else yacc[c][u] = __builtin_fmaf(wb, f[u], yacc[c][u]);
          }
        }
      }
    }
  }
  if (PRE && cur_dev >= 0) finish_device();
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = i0 + kWave * c;
    if (i < ce) y[(size_t)t * row16 + i] = CK::pack(yacc[c]);
  }
}

int chunks_per_lane(int row16) { return (row16 + kWave - 1) / kWave; }

}  // namespace

hipError_t launch_dispatch(const occ_layer_desc &Ld, const void *x, const occ_brim &b, void *sfd,
                           void *epd, hipStream_t st) {
  // sfd == nullptr: the conventional dispatch (EPD rows only)
  if (Ld.T == 0) return hipSuccess;
  const int es = Ld.dtype == OCC_F32 ? 4 : 2;
  const int row16 = Ld.d * es / 16;
  const int L = Ld.E / Ld.D;
  const int ld = Ld.T * (Ld.k < Ld.D ? Ld.k : Ld.D);
  const dim3 grid((Ld.T + kTokPerBlock - 1) / kTokPerBlock);
  const u32x4 *xp = static_cast<const u32x4 *>(x);
  u32x4 *sp = static_cast<u32x4 *>(sfd);
  u32x4 *ep = static_cast<u32x4 *>(epd);
  const int nch = chunks_per_lane(row16);
#define OCC_DISPATCH(N)                                                                     \
  do {                                                                                      \
    if (sp != nullptr)                                                                      \
      dispatch_kernel<N, true><<<grid, kThreads, 0, st>>>(Ld.T, Ld.D, L, ld, row16, xp,     \
                                                          b.brim0, b.brim1, sp, ep);        \
    else                                                                                    \
      dispatch_kernel<N, false><<<grid, kThreads, 0, st>>>(Ld.T, Ld.D, L, ld, row16, xp,    \
                                                           b.brim0, b.brim1, sp, ep);       \
  } while (0)
  if (nch <= 1) OCC_DISPATCH(1);
  else if (nch <= 2) OCC_DISPATCH(2);
  else if (nch <= 4) OCC_DISPATCH(4);
  else if (nch <= 8) OCC_DISPATCH(8);
  else OCC_DISPATCH(8);
#undef OCC_DISPATCH
  return hipGetLastError();
}

template <int DT>
static hipError_t combine_dt(const occ_layer_desc &Ld, const void *out_epd, const occ_brim &b,
                             const void *shared_out, void *out_sfd, void *y, hipStream_t st,
                             const float *ew, const float *add32) {
  const int es = DT == OCC_F32 ? 4 : 2;
  const int row16 = Ld.d * es / 16;
  const int L = Ld.E / Ld.D;
  const int ld = Ld.T * (Ld.k < Ld.D ? Ld.k : Ld.D);
  const u32x4 *oe = static_cast<const u32x4 *>(out_epd);
  const u32x4 *sh = static_cast<const u32x4 *>(shared_out);
  u32x4 *os = static_cast<u32x4 *>(out_sfd);
  u32x4 *yp = static_cast<u32x4 *>(y);
  // rows of more than 4 KiB go to two waves (4 chunks per lane each): the
  // fp32 sums of 8 chunks per lane limit the waves in flight (d = 4096
  // bf16: 0.52 of the HBM peak with one wave per token)
  const int nch = chunks_per_lane(row16);
  const int split = nch > 4 ? 2 : 1;
  const dim3 grid(((int64_t)Ld.T * split + kTokPerBlock - 1) / kTokPerBlock);
#define OCC_COMBINE(N, CS)                                                                \
  do {                                                                                    \
    if (os != nullptr)                                                                    \
      combine_kernel<DT, N, true, CS><<<grid, kThreads, 0, st>>>(                         \
          Ld.T, Ld.D, L, ld, row16, oe, b.brim0, b.brim1, ew, sh, os, yp, add32);         \
    else                                                                                  \
      combine_kernel<DT, N, false, CS><<<grid, kThreads, 0, st>>>(                        \
          Ld.T, Ld.D, L, ld, row16, oe, b.brim0, b.brim1, ew, sh, os, yp, add32);         \
  } while (0)
  if (nch <= 1) OCC_COMBINE(1, 1);
  else if (nch <= 2) OCC_COMBINE(2, 1);
  else if (nch <= 4) OCC_COMBINE(4, 1);
  else OCC_COMBINE(4, 2);  // row16 <= 512 (rows of at most 8 KiB)
#undef OCC_COMBINE
  return hipGetLastError();
}

// out_sfd == nullptr: the conventional combine (no pre-reduction)
hipError_t launch_combine(const occ_layer_desc &Ld, const void *out_epd, const occ_brim &b,
                          const void *shared_out, void *out_sfd, void *y, hipStream_t st) {
  if (Ld.T == 0) return hipSuccess;
  return Ld.dtype == OCC_F32
             ? combine_dt<OCC_F32>(Ld, out_epd, b, shared_out, out_sfd, y, st, b.epd_w, nullptr)
             : combine_dt<OCC_BF16>(Ld, out_epd, b, shared_out, out_sfd, y, st, b.epd_w, nullptr);
}

// Gradient of the dispatch (the same walk, unit weights): d_sfd[s] = sum over
// l of d_epd[r], dx[t] = dx_shared[t] (stored rows, may be null) + add32[t]
// (fp32, may be null) + sum over devices of d_sfd[s].
hipError_t launch_grad_dispatch(const occ_layer_desc &Ld, const void *d_epd, const occ_brim &b,
                                const float *add32, const void *dx_shared, void *d_sfd, void *dx,
                                hipStream_t st) {
  if (Ld.T == 0) return hipSuccess;
  return Ld.dtype == OCC_F32
             ? combine_dt<OCC_F32>(Ld, d_epd, b, dx_shared, d_sfd, dx, st, nullptr, add32)
             : combine_dt<OCC_BF16>(Ld, d_epd, b, dx_shared, d_sfd, dx, st, nullptr, add32);
}

}  // namespace occ
