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
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kTB = 64;  // tokens per block = one wave (many blocks, no intra-block prefix)

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

template <int KMAX>
__device__ __forceinline__ TokenKeys<KMAX> load_keys(int t, int T, int k, int L,
                                                     const int32_t *idx, const float *w,
                                                     const Placement &pl) {
  TokenKeys<KMAX> tk{};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
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

// count: the wave's number of tokens per device and per slot -> cnt[key][blk]
template <int KMAX>
__global__ __launch_bounds__(kTB) void brim_count_kernel(int T, int k, int D, int E, int L,
                                                         int nblk, const int32_t *idx,
                                                         Placement pl, int32_t *cnt) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x * kTB + lane;
  const TokenKeys<KMAX> tk = load_keys<KMAX>(t, T, k, L, idx, nullptr, pl);
  for (int dv = 0; dv < D; ++dv) {
    const uint64_t b = __ballot((tk.dmask >> dv) & 1u);
    if (lane == 0) cnt[(size_t)dv * nblk + blockIdx.x] = __popcll(b);
  }
  for (int g = 0; g < E; ++g) {
    const uint64_t b = __ballot(slot_bit(tk, g));
    if (lane == 0) cnt[(size_t)(D + g) * nblk + blockIdx.x] = __popcll(b);
  }
}

__global__ __launch_bounds__(kTB) void brim_zero_kernel(int32_t *p, int n) {
  for (int i = threadIdx.x; i < n; i += kTB) p[i] = 0;
}

// keyscan: one wave per key c; exclusive scan of cnt[c][0..nblk) in place,
// the key's total into tot[c]
__global__ __launch_bounds__(kTB) void brim_keyscan_kernel(int nblk, int32_t *cnt,
                                                           int32_t *tot) {
  const int c = blockIdx.x, lane = threadIdx.x;
  int32_t *row = cnt + (size_t)c * nblk;
  int32_t carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += kTB) {
    const int b = b0 + lane;
    const int32_t v = b < nblk ? row[b] : 0;
    int32_t x = v;
#pragma unroll
    for (int off = 1; off < kTB; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (b < nblk) row[b] = carry + x - v;
    carry += __shfl(x, kTB - 1);
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
__global__ __launch_bounds__(kTB) void brim_fill_kernel(
    int T, int k, int D, int E, int L, int nblk, int ld, const int32_t *idx, const float *w,
    Placement pl, const int32_t *within, const int32_t *tot, int32_t *brim0, int32_t *brim1,
    int32_t *sfd_token, int32_t *epd_token, int32_t *epd_sfd, float *epd_w, int32_t *sfd_offset,
    int32_t *slot_offset, int32_t *S_out) {
  __shared__ int32_t base[OCC_MAX_D + OCC_MAX_E];
  const int lane = threadIdx.x;
  // key prefixes: devices and slots are two separate exclusive scans
  const int32_t S = wave_exclusive(tot, D, base);
  const int32_t R = wave_exclusive(tot + D, E, base + D);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int c = lane; c <= D; c += kTB) sfd_offset[c] = c == D ? S : base[c];
    for (int c = lane; c <= E; c += kTB) slot_offset[c] = c == E ? R : base[D + c];
    if (lane == 0) S_out[0] = S;
  }
  if (nblk == 0) return;  // no tokens: only the offsets above
  for (int c = lane; c < D + E; c += kTB) base[c] += within[(size_t)c * nblk + blockIdx.x];
  __syncthreads();
  const int t = blockIdx.x * kTB + lane;
  const bool live = t < T;
  const TokenKeys<KMAX> tk = load_keys<KMAX>(t, T, k, L, idx, w, pl);
  const uint64_t lt = lanemask_lt();
  for (int dv = 0; dv < D; ++dv) {
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
                 const float *w, const Placement &pl, const occ_brim &b, int32_t *cnt,
                 int32_t *tot, hipStream_t st) {
  if (nblk > 0) {
    brim_count_kernel<KMAX><<<nblk, kTB, 0, st>>>(T, k, D, E, L, nblk, idx, pl, cnt);
    brim_keyscan_kernel<<<D + E, kTB, 0, st>>>(nblk, cnt, tot);
  } else {
    // no tokens: every key total is zero
    brim_zero_kernel<<<1, kTB, 0, st>>>(tot, D + E);
  }
  brim_fill_kernel<KMAX><<<nblk > 0 ? nblk : 1, kTB, 0, st>>>(
      T, k, D, E, L, nblk, ld, idx, w, pl, cnt, tot, b.brim0, b.brim1, b.sfd_token, b.epd_token,
      b.epd_sfd, b.epd_w, b.sfd_offset, b.slot_offset, b.S);
}

}  // namespace

size_t brim_workspace_bytes(int T, int D, int E) {
  return (brim_count_elems(T, D, E) + OCC_MAX_D + OCC_MAX_E) * sizeof(int32_t);
}

hipError_t launch_build_brim(const occ_layer_desc &Ld, const int32_t *idx, const float *w,
                             const Placement &pl, const occ_brim &b, void *ws, hipStream_t st) {
  const int T = Ld.T, k = Ld.k, D = Ld.D, E = Ld.E, L = E / D;
  const int nblk = (T + kTB - 1) / kTB;
  const int ld = T * (k < D ? k : D);
  int32_t *cnt = static_cast<int32_t *>(ws);
  int32_t *tot = cnt + brim_count_elems(T, D, E);
  if (k <= 2) launch_kmax<2>(T, k, D, E, L, nblk, ld, idx, w, pl, b, cnt, tot, st);
  else if (k <= 4) launch_kmax<4>(T, k, D, E, L, nblk, ld, idx, w, pl, b, cnt, tot, st);
  else if (k <= 8) launch_kmax<8>(T, k, D, E, L, nblk, ld, idx, w, pl, b, cnt, tot, st);
  else launch_kmax<16>(T, k, D, E, L, nblk, ld, idx, w, pl, b, cnt, tot, st);
  return hipGetLastError();
}

}  // namespace occ
