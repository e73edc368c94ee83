// Co-activation (collaboration) counts.
//
// Occult, Abstract: two experts activated by the same token are
// "collaborated"; intra- or inter-collaborated by whether they share a
// device.  counts[i][j] = number of tokens choosing both i and j (the
// diagonal counts tokens per expert).  Each block builds an E x E histogram
// of its tokens in LDS (at most 64 KiB for E = 128) and flushes the non-zero
// entries with integer atomics, whose sum does not depend on their order.
//
// Across two consecutive layers (Expert Coupling in MoE Pretraining,
// Abstract: the experts a token selects at one layer predict those it
// selects at the next; ExFlow, Abstract: inter-layer expert affinity) the
// same kernel counts counts[i][j] = number of tokens choosing expert i at
// the first layer and expert j at the second (E1 x E2).
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void zero_kernel(int32_t *p, int n) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0;
}

__global__ __launch_bounds__(kThreads) void coact_kernel(int T, int k1, int E1, int k2, int E2,
                                                         int tok_per_block,
                                                         const int32_t *__restrict__ idx1,
                                                         const int32_t *__restrict__ idx2,
                                                         int32_t *__restrict__ counts) {
  extern __shared__ int32_t hist[];
  const int n = E1 * E2;
  for (int i = threadIdx.x; i < n; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int t_lo = blockIdx.x * tok_per_block;
  const int t_hi = min(T, t_lo + tok_per_block);
  for (int t = t_lo + threadIdx.x; t < t_hi; t += kThreads) {
    const int32_t *ra = idx1 + (size_t)t * k1;
    const int32_t *rb = idx2 + (size_t)t * k2;
    for (int a = 0; a < k1; ++a) {
      const int32_t ea = ra[a];
      for (int b = 0; b < k2; ++b) {
        const int32_t eb = rb[b];
        // ids outside [0, E) are skipped, never used as addresses
        if ((unsigned)ea < (unsigned)E1 && (unsigned)eb < (unsigned)E2)
          atomicAdd(&hist[ea * E2 + eb], 1);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int32_t c = hist[i];
    if (c != 0) atomicAdd(&counts[i], c);
  }
}

hipError_t coactivation(int T, int k1, int E1, const int32_t *idx1, int k2, int E2,
                        const int32_t *idx2, int32_t *counts, int accumulate, hipStream_t st) {
  const int n = E1 * E2;
  if (!accumulate) zero_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, st>>>(counts, n);
  if (T > 0) {
    // about one block per CU, at least 64 tokens per block
    const int tpb = max(64, (T + 255) / 256 + 63) / 64 * 64;
    const int nblk = (T + tpb - 1) / tpb;
    const size_t lds = sizeof(int32_t) * n;
    if (lds > 48 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&coact_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
      if (e != hipSuccess) return e;
    }
    coact_kernel<<<nblk, kThreads, lds, st>>>(T, k1, E1, k2, E2, tpb, idx1, idx2, counts);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_coactivation(const occ_layer_desc &L, const int32_t *idx, int32_t *counts,
                               int accumulate, hipStream_t st) {
  return coactivation(L.T, L.k, L.E, idx, L.k, L.E, idx, counts, accumulate, st);
}

hipError_t launch_cross_coactivation(int T, int k1, int E1, const int32_t *idx1, int k2, int E2,
                                     const int32_t *idx2, int32_t *counts, int accumulate,
                                     hipStream_t st) {
  return coactivation(T, k1, E1, idx1, k2, E2, idx2, counts, accumulate, st);
}

}  // namespace occ
