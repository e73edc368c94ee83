// BRIM construction: the SFD and EPD layouts and the two re-index matrices.
//
// Occult, Figure 5 caption: BRIM_0 is [devices] x [ORI tokens] and BRIM_1 is
// [local experts per device] x [SFD tokens].  Expert Coupling in MoE
// Pretraining, Abstract: a dispatcher sends each token to each GPU once.
//
// SFD = one row per (token, device) pair, device-major, ascending token;
// EPD = one row per (token, expert) pair, slot-major (slot = device*L +
// local), ascending token.  Both orders are stable counting sorts keyed by
// device (resp. slot), done in three passes over blocks of 64 tokens:
//   count:   per block and key, ballot popcounts             -> cnt[key][blk]
//   keyscan: one wave per key, exclusive scan over the blocks -> cnt, tot[key]
//   fill:    key prefix (scan of tot) + block prefix + rank among the
//            wave's earlier lanes (ballot) -> BRIM_0, sfd_token, BRIM_1,
//            epd_token, epd_sfd, epd_w; block 0 writes the offsets and S
// No atomics, so every output is deterministic.
//
// Collaboration pruning under an all-to-all budget (Occult, TL;DR:
// routing-score-based pruning to minimise the budget C_T): with budget < D a
// token keeps at most `budget` devices, those with the largest summed routing
// weight of its selected experts (fp32 sums in top-k order; lower device
// index on equal sums); its experts on other devices are dropped, and with
// `rescale` the kept weights are scaled by (sum of all its weights) / (sum of
// the kept ones) so the token's total gate mass is unchanged.  Counting and
// filling apply the same rule, so the layouts stay consistent, and EPD then
// holds fewer than T*k rows (slot_offset[E]).
#include <mutex>

#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kTB = 64;  // tokens per block = one wave's lanes (no intra-block prefix)
// Waves per count / fill block: all of them hold the block's 64 tokens and
// split the keys (devices, slots) among themselves, so a wave's serial loop
// over keys is kWB times shorter.
constexpr int kWB = 4;

// Per-lane view of one token: device bitmask and slot bitmask (E <= 128).
template <int KMAX> struct TokenKeys {
  uint32_t dmask;
  uint64_t slo, shi;  // slots 0..63 and 64..127
  int32_t slot[KMAX];
  float w[KMAX];
};

template <int KMAX>
__device__ __forceinline__ bool slot_bit(const TokenKeys<KMAX> &tk, int g) {
  const uint64_t lo = tk.slo, hi = tk.shi;  // select values, not fields
  const uint64_t word = g < 64 ? lo : hi;
  return (word >> (g & 63)) & 1ull;
}

struct Prune {
  int budget;   // devices kept per token (>= D: no pruning)
  int rescale;  // 1: keep each token's total weight
};

template <int KMAX>
__device__ __forceinline__ TokenKeys<KMAX> load_keys(int t, int T, int k, int L,
                                                     const int32_t *idx, const float *w,
                                                     const Placement &pl, const Prune &pr) {
  TokenKeys<KMAX> tk{};
  int dev[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    tk.slot[j] = -1;
    tk.w[j] = 0.0f;
    dev[j] = -1;
    wt[j] = 0.0f;
    // ids outside [0, OCC_MAX_E) or of no slot are skipped, never used as addresses
    const int e = (t < T && j < k) ? idx[(size_t)t * k + j] : -1;
    const int g = (unsigned)e < (unsigned)OCC_MAX_E ? pl.slot_of[e] : -1;
    if (g >= 0) {
      tk.slot[j] = g;
      dev[j] = g / L;
      wt[j] = w != nullptr ? w[(size_t)t * k + j] : 0.0f;
    }
  }
  float scale = 1.0f;
  if (pr.budget < OCC_MAX_D) {
    // score of each pick's device: fp32 sum of the token's weights on it, in pick order
    float score[KMAX];
    bool first[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      float sc = 0.0f;
      bool f = dev[j] >= 0;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        if (dev[i] == dev[j]) sc += wt[i];
        if (i < j && dev[i] == dev[j]) f = false;
      }
      score[j] = sc;
      first[j] = f;  // the first pick on its device stands for the device
    }
    float total = 0.0f, kept = 0.0f;
    bool keep[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      keep[j] = false;
      if (dev[j] < 0) continue;
      int rank = 0;  // devices ahead of this pick's device
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (first[i] && dev[i] != dev[j] &&
            (score[i] > score[j] || (score[i] == score[j] && dev[i] < dev[j])))
          ++rank;
      keep[j] = rank < pr.budget;
      total += wt[j];
      if (keep[j]) kept += wt[j];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (!keep[j]) dev[j] = -1;  // dropped (or no pick)
    if (pr.rescale && kept > 0.0f) scale = total / kept;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (dev[j] < 0) {
      tk.slot[j] = -1;
      continue;
    }
    const int g = tk.slot[j];
    tk.w[j] = pr.rescale && pr.budget < OCC_MAX_D ? wt[j] * scale : wt[j];
    tk.dmask |= 1u << dev[j];
    const uint64_t bit = 1ull << (g & 63);
    if (g < 64) tk.slo |= bit;
    else tk.shi |= bit;
  }
  return tk;
}

// count: the wave's number of tokens per device and per slot -> cnt[key][blk]
template <int KMAX>
__global__ __launch_bounds__(kTB * kWB) void brim_count_kernel(int T, int k, int D, int E, int L,
                                                               int nblk, const int32_t *idx,
                                                               const float *w, Placement pl,
                                                               Prune pr, int32_t *cnt) {
  const int lane = threadIdx.x % kTB, wv = threadIdx.x / kTB;
  const int t = blockIdx.x * kTB + lane;
  // the weights matter for counting only when pruning decides by them
  const TokenKeys<KMAX> tk =
      load_keys<KMAX>(t, T, k, L, idx, pr.budget < OCC_MAX_D ? w : nullptr, pl, pr);
  for (int dv = wv; dv < D; dv += kWB) {
    const uint64_t b = __ballot((tk.dmask >> dv) & 1u);
    if (lane == 0) cnt[(size_t)dv * nblk + blockIdx.x] = __popcll(b);
  }
  for (int g = wv; g < E; g += kWB) {
    const uint64_t b = __ballot(slot_bit(tk, g));
    if (lane == 0) cnt[(size_t)(D + g) * nblk + blockIdx.x] = __popcll(b);
  }
}

__global__ __launch_bounds__(kTB) void brim_zero_kernel(int32_t *p, int n) {
  for (int i = threadIdx.x; i < n; i += kTB) p[i] = 0;
}

// keyscan: one wave per key c; exclusive scan of cnt[c][0..nblk) in place,
// the key's total into tot[c]
// (the loads of up to 16 chunks of 64 blocks go out before their scans, so
// their latencies overlap instead of following each other)
__global__ __launch_bounds__(kTB) void brim_keyscan_kernel(int nblk, int32_t *cnt,
                                                           int32_t *tot) {
  constexpr int kChunks = 16;
  const int c = blockIdx.x, lane = threadIdx.x;
  int32_t *row = cnt + (size_t)c * nblk;
  int32_t carry = 0;
  for (int g0 = 0; g0 < nblk; g0 += kTB * kChunks) {
    int32_t v[kChunks];
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int b = g0 + kTB * u + lane;
      v[u] = b < nblk ? row[b] : 0;
    }
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      if (g0 + kTB * u >= nblk) break;  // uniform: no scans of empty chunks
      const int b = g0 + kTB * u + lane;
      int32_t x = v[u];
#pragma unroll
      for (int off = 1; off < kTB; off <<= 1) {
        const int32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      if (b < nblk) row[b] = carry + x - v[u];
      carry += __shfl(x, kTB - 1);
    }
  }
  if (lane == 0) tot[c] = carry;
}

// Exclusive prefix of tot[0..n) by one wave into out[0..n); returns the sum.
__device__ __forceinline__ int32_t wave_exclusive(const int32_t *tot, int n, int32_t *out) {
  const int lane = threadIdx.x;
  int32_t carry = 0;
  for (int i0 = 0; i0 < n; i0 += kTB) {
    const int i = i0 + lane;
    const int32_t v = i < n ? tot[i] : 0;
    int32_t x = v;
#pragma unroll
    for (int off = 1; off < kTB; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (i < n) out[i] = carry + x - v;
    carry += __shfl(x, kTB - 1);
  }
  return carry;
}

// fill: rank of each token among the wave's earlier lanes with the same key,
// plus the key's prefix and the block's prefix inside the key
template <int KMAX>
__global__ __launch_bounds__(kTB * kWB) void brim_fill_kernel(
    int T, int k, int D, int E, int L, int nblk, int ld, const int32_t *idx, const float *w,
    Placement pl, Prune pr, const int32_t *within, const int32_t *tot, int32_t *brim0,
    int32_t *brim1,
    int32_t *sfd_token, int32_t *epd_token, int32_t *epd_sfd, float *epd_w, int32_t *sfd_offset,
    int32_t *slot_offset, int32_t *S_out) {
  __shared__ int32_t base[OCC_MAX_D + OCC_MAX_E];
  const int lane = threadIdx.x % kTB, wv = threadIdx.x / kTB;
  // The token's keys and this block's per-key prefixes are loaded first:
  // neither depends on the key totals, so their latency overlaps the scans.
  const int t = blockIdx.x * kTB + lane;
  const bool live = t < T;
  const TokenKeys<KMAX> tk = load_keys<KMAX>(t, T, k, L, idx, w, pl, pr);
  constexpr int KR = (OCC_MAX_D + OCC_MAX_E + kTB - 1) / kTB;  // keys per lane
  int32_t win[KR];
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    const int c = lane + kTB * r;
    win[r] = wv == 0 && nblk > 0 && c < D + E ? within[(size_t)c * nblk + blockIdx.x] : 0;
  }
  // key prefixes (wave 0): devices and slots are two separate exclusive
  // scans; block 0 writes them out, then each key's base moves on by this
  // block's prefix inside the key
  if (wv == 0) {
    const int32_t S = wave_exclusive(tot, D, base);
    const int32_t R = wave_exclusive(tot + D, E, base + D);
    // other lanes wrote those entries: order the reads after their writes
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (blockIdx.x == 0) {
      for (int c = lane; c <= D; c += kTB) sfd_offset[c] = c == D ? S : base[c];
      for (int c = lane; c <= E; c += kTB) slot_offset[c] = c == E ? R : base[D + c];
      if (lane == 0) S_out[0] = S;
    }
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int c = lane + kTB * r;
      if (c < D + E) base[c] += win[r];
    }
  }
  if (nblk == 0) return;  // no tokens: only the offsets above (uniform over the block)
  __syncthreads();
  const uint64_t lt = lanemask_lt();
  for (int dv = wv; dv < D; dv += kWB) {
    const bool hasd = live && ((tk.dmask >> dv) & 1u);
    const uint64_t bd = __ballot(hasd);
    const int32_t s = hasd ? base[dv] + __popcll(bd & lt) : -1;
    if (live) brim0[(size_t)dv * T + t] = s;
    if (hasd) sfd_token[s] = t;
    if (bd == 0) continue;  // no token of this wave on the device (uniform)
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
          for (int j = 0; j < KMAX; ++j)
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

// counts per (key, block), 64-element aligned, then the key totals
size_t brim_count_elems(int T, int D, int E) {
  const size_t nblk = ((size_t)T + kTB - 1) / kTB;
  return ((size_t)(D + E) * nblk + 63) / 64 * 64;
}

template <int KMAX>
void launch_kmax(int T, int k, int D, int E, int L, int nblk, int ld, const int32_t *idx,
                 const float *w, const Placement &pl, const Prune &pr, const occ_brim &b,
                 int32_t *cnt, int32_t *tot, hipStream_t st) {
  if (nblk > 0) {
    brim_count_kernel<KMAX><<<nblk, kTB * kWB, 0, st>>>(T, k, D, E, L, nblk, idx, w, pl, pr, cnt);
    brim_keyscan_kernel<<<D + E, kTB, 0, st>>>(nblk, cnt, tot);
  } else {
    // no tokens: every key total is zero
    brim_zero_kernel<<<1, kTB, 0, st>>>(tot, D + E);
  }
  brim_fill_kernel<KMAX><<<nblk > 0 ? nblk : 1, kTB * kWB, 0, st>>>(
      T, k, D, E, L, nblk, ld, idx, w, pl, pr, cnt, tot, b.brim0, b.brim1, b.sfd_token, b.epd_token,
      b.epd_sfd, b.epd_w, b.sfd_offset, b.slot_offset, b.S);
}

}  // namespace

// Workspace of occ_build_brim_noalloc: one fixed device array per GPU, held
// until the process ends.  In host code `scratch` is only a stand-in for the
// symbol; its device address comes from hipGetSymbolAddress, once per device
// (each GPU has its own copy at its own address).
static __device__ __align__(256) int32_t scratch[kBrimScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];  // device address per device, null until queried
}  // namespace

hipError_t brim_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t brim_workspace_bytes(int T, int D, int E) {
  return (brim_count_elems(T, D, E) + OCC_MAX_D + OCC_MAX_E) * sizeof(int32_t);
}

hipError_t launch_build_brim(const occ_layer_desc &Ld, const int32_t *idx, const float *w,
                             const Placement &pl, const occ_brim &b, void *ws, hipStream_t st,
                             int budget, int rescale) {
  const int T = Ld.T, k = Ld.k, D = Ld.D, E = Ld.E, L = E / D;
  const int nblk = (T + kTB - 1) / kTB;
  const int ld = T * (k < D ? k : D);
  int32_t *cnt = static_cast<int32_t *>(ws);
  int32_t *tot = cnt + brim_count_elems(T, D, E);
  // a budget of D or more keeps every device: the unpruned layouts
  const Prune pr{budget < D ? budget : OCC_MAX_D, rescale};
  if (k <= 2) launch_kmax<2>(T, k, D, E, L, nblk, ld, idx, w, pl, pr, b, cnt, tot, st);
  else if (k <= 4) launch_kmax<4>(T, k, D, E, L, nblk, ld, idx, w, pl, pr, b, cnt, tot, st);
  else if (k <= 8) launch_kmax<8>(T, k, D, E, L, nblk, ld, idx, w, pl, pr, b, cnt, tot, st);
  else launch_kmax<16>(T, k, D, E, L, nblk, ld, idx, w, pl, pr, b, cnt, tot, st);
  return hipGetLastError();
}

}  // namespace occ
