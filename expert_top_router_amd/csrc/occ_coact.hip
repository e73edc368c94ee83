// Co-activation (collaboration) counts.
//
// Occult, Abstract: two experts activated by the same token are
// "collaborated"; intra- or inter-collaborated by whether they share a
// device.  counts[i][j] = number of tokens choosing both i and j (the
// diagonal counts tokens per expert).  Each block builds an E x E histogram
// of its tokens in LDS (at most 64 KiB for E = 128) and flushes the non-zero
// entries with integer atomics, whose sum does not depend on their order.
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void zero_kernel(int32_t *p, int n) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0;
}

__global__ __launch_bounds__(kThreads) void coact_kernel(int T, int k, int E, int tok_per_block,
                                                         const int32_t *__restrict__ idx,
                                                         int32_t *__restrict__ counts) {
  extern __shared__ int32_t hist[];
  const int n = E * E;
  for (int i = threadIdx.x; i < n; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int t_lo = blockIdx.x * tok_per_block;
  const int t_hi = min(T, t_lo + tok_per_block);
  for (int t = t_lo + threadIdx.x; t < t_hi; t += kThreads) {
    const int32_t *row = idx + (size_t)t * k;
    for (int a = 0; a < k; ++a) {
      const int32_t ea = row[a];
      for (int b = 0; b < k; ++b) {
        const int32_t eb = row[b];
        // ids outside [0, E) are skipped, never used as addresses
        if ((unsigned)ea < (unsigned)E && (unsigned)eb < (unsigned)E)
          atomicAdd(&hist[ea * E + eb], 1);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int32_t c = hist[i];
    if (c != 0) atomicAdd(&counts[i], c);
  }
}

}  // namespace

hipError_t launch_coactivation(const occ_layer_desc &L, const int32_t *idx, int32_t *counts,
                               int accumulate, hipStream_t st) {
  const int n = L.E * L.E;
  if (!accumulate) zero_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, st>>>(counts, n);
  if (L.T > 0) {
    // about one block per CU, at least 64 tokens per block
    const int tpb = max(64, (L.T + 255) / 256 + 63) / 64 * 64;
    const int nblk = (L.T + tpb - 1) / tpb;
    const size_t lds = sizeof(int32_t) * n;
    if (lds > 48 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&coact_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
      if (e != hipSuccess) return e;
    }
    coact_kernel<<<nblk, kThreads, lds, st>>>(L.T, L.k, L.E, tpb, idx, counts);
  }
  return hipGetLastError();
}

}  // namespace occ
