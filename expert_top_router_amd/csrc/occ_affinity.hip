// Home devices for the next layer and the share of assignments served on a
// token's own device.
//
// Expert Coupling in MoE Pretraining, Abstract: token shuffling moves each
// token to the GPU predicted to hold its next-layer experts, which raises the
// share of token-expert assignments served on the token's GPU; ExFlow,
// Abstract: inter-layer expert affinity, the conditional statistics of a
// token's routing across layers.  With affinity counts A[i][j] (tokens that
// chose expert i at this layer and j at the next, from a calibration batch)
// and the next layer's placement:
//   home[t] = argmax over devices d of sum over the token's experts i of
//             sum over the next-layer experts j on d of A[i][j]
//             (int64 sums; lower device index on equal sums)
//   hits   += number of (t, j) with j among the token's next-layer experts
//             and j on device home[t]
// Each block first folds the affinity matrix into per-device sums
// B[i][d] in LDS (at most 32 KiB); then one thread per token needs k1 * D
// LDS reads.
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void home_kernel(int T, int k1, int E1, int E2, int D,
                                                        DeviceOf dv,
                                                        const int32_t *__restrict__ idx1,
                                                        const int32_t *__restrict__ aff,
                                                        int32_t *__restrict__ home) {
  // B[i][d] = sum of affinity[i][j] over the next-layer experts j on device d
  __shared__ long long B[OCC_MAX_E * OCC_MAX_D];
  for (int c = threadIdx.x; c < E1 * D; c += kThreads) {
    const int i = c / D, d = c - i * D;
    long long s = 0;
    for (int j = 0; j < E2; ++j)
      if (dv.dev[j] == d) s += aff[(size_t)i * E2 + j];
    B[c] = s;
  }
  __syncthreads();
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= T) return;
  const int32_t *row = idx1 + (size_t)t * k1;
  int best = 0;
  long long best_score = -1;
  for (int d = 0; d < D; ++d) {
    long long sc = 0;
    for (int q = 0; q < k1; ++q) {
      const int32_t i = row[q];
      if ((unsigned)i < (unsigned)E1) sc += B[i * D + d];  // other ids never used as addresses
    }
    if (sc > best_score) {  // strictly greater: lower device index on ties
      best_score = sc;
      best = d;
    }
  }
  home[t] = best;
}

__global__ __launch_bounds__(kThreads) void zero1_kernel(int32_t *p) {
  if (threadIdx.x == 0) p[0] = 0;
}

__global__ __launch_bounds__(kThreads) void hits_kernel(int T, int k2, int E2, DeviceOf dv,
                                                        const int32_t *__restrict__ idx2,
                                                        const int32_t *__restrict__ home,
                                                        int32_t *__restrict__ hits) {
  __shared__ int32_t part[kThreads / kWave];
  const int t = blockIdx.x * kThreads + threadIdx.x;
  int c = 0;
  if (t < T) {
    const int h = home[t];
    for (int q = 0; q < k2; ++q) {
      const int32_t j = idx2[(size_t)t * k2 + q];
      if ((unsigned)j < (unsigned)E2 && dv.dev[j] == h) ++c;
    }
  }
  for (int off = kWave / 2; off > 0; off >>= 1) c += __shfl_xor(c, off);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) part[wave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kThreads / kWave; ++w) s += part[w];
    if (s != 0) atomicAdd(hits, s);
  }
}

}  // namespace

hipError_t launch_home_device(int T, int k1, int E1, const int32_t *idx1, int E2, int D,
                              const DeviceOf &dv, const int32_t *affinity, int32_t *home,
                              hipStream_t st) {
  if (T > 0)
    home_kernel<<<(T + kThreads - 1) / kThreads, kThreads, 0, st>>>(T, k1, E1, E2, D, dv, idx1,
                                                                     affinity, home);
  return hipGetLastError();
}

hipError_t launch_local_hits(int T, int k2, int E2, const int32_t *idx2, const DeviceOf &dv,
                             const int32_t *home, int32_t *hits, int accumulate, hipStream_t st) {
  if (!accumulate) zero1_kernel<<<1, kThreads, 0, st>>>(hits);
  if (T > 0)
    hits_kernel<<<(T + kThreads - 1) / kThreads, kThreads, 0, st>>>(T, k2, E2, dv, idx2, home,
                                                                    hits);
  return hipGetLastError();
}

}  // namespace occ
