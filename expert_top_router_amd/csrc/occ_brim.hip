// BRIM construction: the SFD and EPD layouts and the two re-index matrices.
//
// Occult, Figure 5 caption: BRIM_0 is [devices] x [ORI tokens] and BRIM_1 is
// [local experts per device] x [SFD tokens].  Expert Coupling in MoE
// Pretraining, Abstract: a dispatcher sends each token to each GPU once.
//
// SFD = one row per (token, device) pair, device-major, ascending token;
// EPD = one row per (token, expert) pair, slot-major (slot = device*L +
// local), ascending token.  Both orders are stable counting sorts keyed by
// device (resp. slot), done in three passes over blocks of 256 tokens:
//   count: per block and key, ballot popcounts            -> cnt[key][blk]
//   scan:  one workgroup, exclusive scan in key-major order -> offsets
//   fill:  per token, block base + rank among earlier lanes (ballot) ->
//          BRIM_0, sfd_token, BRIM_1, epd_token, epd_sfd, epd_w
// No atomics, so every output is deterministic.
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kTB = 256;  // tokens per block = threads per block
constexpr int kWaves = kTB / kWave;
constexpr int kScanThreads = 1024;

// Per-lane view of one token: device bitmask and slot bitmask (E <= 128).
struct TokenKeys {
  uint32_t dmask;
  uint64_t slo, shi;  // slots 0..63 and 64..127
  int32_t slot[OCC_MAX_K];
  float w[OCC_MAX_K];
};

__device__ __forceinline__ bool slot_bit(const TokenKeys &tk, int g) {
  const uint64_t lo = tk.slo, hi = tk.shi;  // select values, not fields
  const uint64_t word = g < 64 ? lo : hi;
  return (word >> (g & 63)) & 1ull;
}

__device__ __forceinline__ TokenKeys load_keys(int t, int T, int k, int L, const int32_t *idx,
                                               const float *w, const Placement &pl) {
  TokenKeys tk{};
#pragma unroll
  for (int j = 0; j < OCC_MAX_K; ++j) {
    tk.slot[j] = -1;
    tk.w[j] = 0.0f;
    // ids outside [0, OCC_MAX_E) or of no slot are skipped, never used as addresses
    const int e = (t < T && j < k) ? idx[(size_t)t * k + j] : -1;
    const int g = (unsigned)e < (unsigned)OCC_MAX_E ? pl.slot_of[e] : -1;
    if (g >= 0) {
      tk.slot[j] = g;
      tk.w[j] = w != nullptr ? w[(size_t)t * k + j] : 0.0f;
      tk.dmask |= 1u << (g / L);
      const uint64_t bit = 1ull << (g & 63);
      if (g < 64) tk.slo |= bit;
      else tk.shi |= bit;
    }
  }
  return tk;
}

// Per-wave counts of every key (D devices then E slots) into wcnt[wave][key].
__device__ __forceinline__ void wave_counts(const TokenKeys &tk, int D, int E, int32_t *wcnt) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int dv = 0; dv < D; ++dv) {
    const uint64_t b = __ballot((tk.dmask >> dv) & 1u);
    if (lane == 0) wcnt[dv] = __popcll(b);
  }
  for (int g = 0; g < E; ++g) {
    const uint64_t b = __ballot(slot_bit(tk, g));
    if (lane == 0) wcnt[D + g] = __popcll(b);
  }
}

__global__ __launch_bounds__(kTB) void brim_count_kernel(int T, int k, int D, int E, int L,
                                                         int nblk, const int32_t *idx,
                                                         Placement pl, int32_t *cnt) {
  extern __shared__ int32_t wcnt[];  // [kWaves][D + E]
  const int nk = D + E;
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x * kTB + threadIdx.x;
  const TokenKeys tk = load_keys(t, T, k, L, idx, nullptr, pl);
  wave_counts(tk, D, E, wcnt + wave * nk);
  __syncthreads();
  for (int c = threadIdx.x; c < nk; c += kTB) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += wcnt[w * nk + c];
    cnt[(size_t)c * nblk + blockIdx.x] = s;
  }
}

// Exclusive scan of a[0..n) in place by one workgroup; returns the total.
__device__ int32_t block_exclusive_scan(int32_t *a, int n, int32_t *lds) {
  const int tid = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int32_t s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  lds[tid] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t v = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += v;
    __syncthreads();
  }
  int32_t run = tid > 0 ? lds[tid - 1] : 0;
  const int32_t total = lds[kScanThreads - 1];
  for (int i = lo; i < hi; ++i) {
    const int32_t v = a[i];
    a[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kScanThreads) void brim_scan_kernel(int D, int E, int nblk,
                                                                 int32_t *cnt, int32_t *sfd_offset,
                                                                 int32_t *slot_offset,
                                                                 int32_t *S_out) {
  __shared__ int32_t lds[kScanThreads];
  const int32_t S = block_exclusive_scan(cnt, D * nblk, lds);
  const int32_t R = block_exclusive_scan(cnt + (size_t)D * nblk, E * nblk, lds);
  __syncthreads();
  for (int dv = threadIdx.x; dv <= D; dv += kScanThreads)
    sfd_offset[dv] = dv == D ? S : (nblk > 0 ? cnt[(size_t)dv * nblk] : 0);
  for (int g = threadIdx.x; g <= E; g += kScanThreads)
    slot_offset[g] = g == E ? R : (nblk > 0 ? cnt[(size_t)(D + g) * nblk] : 0);
  if (threadIdx.x == 0) S_out[0] = S;
}

__global__ __launch_bounds__(kTB) void brim_fill_kernel(
    int T, int k, int D, int E, int L, int nblk, int ld, const int32_t *idx, const float *w,
    Placement pl, const int32_t *off, int32_t *brim0, int32_t *brim1, int32_t *sfd_token,
    int32_t *epd_token, int32_t *epd_sfd, float *epd_w) {
  extern __shared__ int32_t wcnt[];  // [kWaves][D + E], then turned into bases
  const int nk = D + E;
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x * kTB + threadIdx.x;
  const bool live = t < T;
  const TokenKeys tk = load_keys(t, T, k, L, idx, w, pl);
  wave_counts(tk, D, E, wcnt + wave * nk);
  __syncthreads();
  // bases: block offset of the key plus the counts of earlier waves
  for (int c = threadIdx.x; c < nk; c += kTB) {
    int32_t run = off[(size_t)c * nblk + blockIdx.x];
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const int32_t v = wcnt[w2 * nk + c];
      wcnt[w2 * nk + c] = run;
      run += v;
    }
  }
  __syncthreads();
  const int32_t *base = wcnt + wave * nk;
  const uint64_t lt = lanemask_lt();
  for (int dv = 0; dv < D; ++dv) {
    const bool hasd = live && ((tk.dmask >> dv) & 1u);
    const uint64_t bd = __ballot(hasd);
    const int32_t s = hasd ? base[dv] + __popcll(bd & lt) : -1;
    if (live) brim0[(size_t)dv * T + t] = s;
    if (hasd) sfd_token[s] = t;
    for (int l = 0; l < L; ++l) {
      const int g = dv * L + l;
      const bool hass = live && slot_bit(tk, g);
      const uint64_t bs = __ballot(hass);
      if (hasd) {
        int32_t r = -1;
        if (hass) {
          r = base[D + g] + __popcll(bs & lt);
          float wr = 0.0f;
#pragma unroll
          for (int j = 0; j < OCC_MAX_K; ++j)
            if (tk.slot[j] == g) wr = tk.w[j];
          epd_token[r] = t;
          epd_sfd[r] = s;
          epd_w[r] = wr;
        }
        brim1[(size_t)l * ld + s] = r;
      }
    }
  }
}

}  // namespace

size_t brim_workspace_bytes(int T, int D, int E) {
  const size_t nblk = ((size_t)T + kTB - 1) / kTB;
  const size_t bytes = (size_t)(D + E) * nblk * sizeof(int32_t);
  return (bytes + 255) / 256 * 256 + 256;
}

hipError_t launch_build_brim(const occ_layer_desc &Ld, const int32_t *idx, const float *w,
                             const Placement &pl, const occ_brim &b, void *ws, hipStream_t st) {
  const int T = Ld.T, k = Ld.k, D = Ld.D, E = Ld.E, L = E / D;
  const int nblk = (T + kTB - 1) / kTB;
  const int ld = T * (k < D ? k : D);
  int32_t *cnt = static_cast<int32_t *>(ws);
  const size_t lds = sizeof(int32_t) * kWaves * (D + E);
  if (nblk > 0)
    brim_count_kernel<<<nblk, kTB, lds, st>>>(T, k, D, E, L, nblk, idx, pl, cnt);
  brim_scan_kernel<<<1, kScanThreads, 0, st>>>(D, E, nblk, cnt, b.sfd_offset, b.slot_offset, b.S);
  if (nblk > 0)
    brim_fill_kernel<<<nblk, kTB, lds, st>>>(T, k, D, E, L, nblk, ld, idx, w, pl, cnt, b.brim0,
                                             b.brim1, b.sfd_token, b.epd_token, b.epd_sfd,
                                             b.epd_w);
  return hipGetLastError();
}

}  // namespace occ
