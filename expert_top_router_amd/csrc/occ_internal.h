// Internal declarations shared by the HIP sources of liboccult (not part of
// the C ABI).  gfx950 only: wave64, 160 KB LDS per CU, 256 CUs in 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "occ.h"

namespace occ {

constexpr int kWave = 64;

// Native 16-byte vector (HIP's uint4 is a union wrapper that can keep
// register arrays of it in scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kXcds = 8;

// Placement passed by value to kernels, so it needs no device copy:
// slot g = dv * L + l holds expert expert_at[g]; slot_of is its inverse.
struct Placement {
  int32_t expert_at[OCC_MAX_E];
  int32_t slot_of[OCC_MAX_E];
};

// ---- element conversions --------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int DT> struct Elem;
template <> struct Elem<OCC_F32> {
  using T = float;
  static __device__ __forceinline__ float load(const T *p, size_t i) { return p[i]; }
  static __device__ __forceinline__ T from_f32(float v) { return v; }
  static __device__ __forceinline__ float to_f32(T v) { return v; }
};
template <> struct Elem<OCC_BF16> {
  using T = uint16_t;
  static __device__ __forceinline__ float load(const T *p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ T from_f32(float v) { return f32_to_bf16(v); }
  static __device__ __forceinline__ float to_f32(T v) { return bf16_to_f32(v); }
};

// Widen one 16-byte vector of stored elements to fp32 (8 bf16 or 4 fp32).
template <int DT> __device__ __forceinline__ void widen(const u32x4 &u, float *f);
template <> __device__ __forceinline__ void widen<OCC_BF16>(const u32x4 &u, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void widen<OCC_F32>(const u32x4 &u, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
}

// Cross-lane reductions through DPP (no LDS round trips): the quad
// permutations and the half-row and row mirrors combine the 16 lanes of a
// row (every lane ends with its row's value); row_bcast15 / row_bcast31 then
// carry rows 0..2 into row 3, whose last lane holds the wave's value.
template <int CTRL, int RM = 0xf> __device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               RM, 0xf, false));
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dppf<0xb1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dppf<0x4e>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dppf<0x141>(v));  // row_half_mirror
  return fmaxf(v, dppf<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row_sum(float v) {
  v += dppf<0xb1>(v);
  v += dppf<0x4e>(v);
  v += dppf<0x141>(v);
  return v + dppf<0x140>(v);
}
__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max(v);
  v = fmaxf(v, dppf<0x142, 0xa>(v));  // row_bcast15 into rows 1 and 3
  v = fmaxf(v, dppf<0x143, 0xc>(v));  // row_bcast31 into rows 2 and 3
  return lane63(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum(v);
  v += dppf<0x142, 0xa>(v);
  v += dppf<0x143, 0xc>(v);
  return lane63(v);
}

__device__ __forceinline__ int row_min_i(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0xb1, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x4e, 0xf, 0xf, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));
  return min(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));
}
__device__ __forceinline__ int row_sum_i(int v) {
  v += __builtin_amdgcn_update_dpp(v, v, 0xb1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(v, v, 0x4e, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false);
  return v + __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false);
}
// inclusive prefix sum over the 16 lanes of a row (row_shr with zero fill)
__device__ __forceinline__ int row_scan_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  return v + __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (kWave - lane));
}

// Compute units of the current device, queried once per device and cached
// (the persistent GEMMs launch one block per CU).  Returns 0 on a HIP error.
int device_cu_count();

// ---- launchers (each returns hipGetLastError() of its launches) -----------
hipError_t launch_route_topk(const occ_layer_desc &L, const void *x, const float *wr,
                             int32_t *idx, float *w, float *logits, hipStream_t st);
// routing with the logit chains on the matrix cores (K = 1 fp32 MFMAs):
// 32 < E <= 128, k <= 16, d a multiple of 64 (bf16) or 32 (fp32)
bool route_mfma_applies(const occ_layer_desc &L);
hipError_t launch_route_mfma(const occ_layer_desc &L, const void *x, const float *wr,
                             int32_t *idx, float *w, float *logits, hipStream_t st);
// filtered routing (occ_route_topk_ws): applies to bf16 layers with
// 32 <= E <= 128, k <= 16, d % 64 == 0
bool route_filter_applies(const occ_layer_desc &L);
size_t route_filter_workspace_bytes(const occ_layer_desc &L);
hipError_t launch_route_filtered(const occ_layer_desc &L, const void *x, const float *wr,
                                 int32_t *idx, float *w, void *ws, hipStream_t st);

// workspace layout of the BRIM build: counts then scanned offsets
size_t brim_workspace_bytes(int T, int D, int E);
// budget >= D: the plain layouts; budget < D: collaboration pruning (at most
// `budget` devices per token, kept weights rescaled when `rescale` is 1)
// The fixed workspace of occ_build_brim_noalloc (per GPU) and its device
// address on the current device (looked up once per device, then cached).
constexpr size_t kBrimScratchBytes = OCC_NOALLOC_BRIM_SCRATCH_BYTES;
static_assert(kBrimScratchBytes % 256 == 0, "whole 256-byte lines");
hipError_t brim_scratch(void **ptr);
hipError_t launch_build_brim(const occ_layer_desc &L, const int32_t *idx, const float *w,
                             const Placement &pl, const occ_brim &b, void *ws, hipStream_t st,
                             int budget, int rescale);

hipError_t launch_dispatch(const occ_layer_desc &L, const void *x, const occ_brim &b, void *sfd,
                           void *epd, hipStream_t st);

hipError_t launch_combine(const occ_layer_desc &L, const void *out_epd, const occ_brim &b,
                          const void *shared_out, void *out_sfd, void *y, hipStream_t st);

// Backward: grad-combine, grad-dispatch and the router gradient.
hipError_t launch_grad_combine(const occ_layer_desc &L, const void *dy, const occ_brim &b,
                               const void *out_epd, void *d_out_sfd, void *d_out_epd, float *dw,
                               hipStream_t st);
hipError_t launch_grad_dispatch(const occ_layer_desc &L, const void *d_epd, const occ_brim &b,
                                const float *add32, const void *dx_shared, void *d_sfd, void *dx,
                                hipStream_t st);
hipError_t launch_router_backward(const occ_layer_desc &L, const Placement &pl, const void *x,
                                  const float *w_router, const float *logits,
                                  const int32_t *idx, const float *topk_w, const occ_brim &b,
                                  const float *dw, float *dlogit, float *dx_router,
                                  float *dw_router, void *ws, hipStream_t st);
// Workspace bytes of launch_router_backward (partial sums of dW_r).
size_t router_backward_ws_bytes(const occ_layer_desc &L);

hipError_t launch_coactivation(const occ_layer_desc &L, const int32_t *idx, int32_t *counts,
                               int accumulate, hipStream_t st);
hipError_t launch_cross_coactivation(int T, int k1, int E1, const int32_t *idx1, int k2, int E2,
                                     const int32_t *idx2, int32_t *counts, int accumulate,
                                     hipStream_t st);

// Token shuffling toward the next layer's experts.  dev_of: device of each
// next-layer expert id (E2 entries, placement validated on the host).
struct DeviceOf {
  int8_t dev[OCC_MAX_E];
};
hipError_t launch_home_device(int T, int k1, int E1, const int32_t *idx1, int E2, int D,
                              const DeviceOf &dv, const int32_t *affinity, int32_t *home,
                              hipStream_t st);
hipError_t launch_local_hits(int T, int k2, int E2, const int32_t *idx2, const DeviceOf &dv,
                             const int32_t *home, int32_t *hits, int accumulate, hipStream_t st);

// Expert GEMMs.  up: h = swiglu(A W_gu^T); down: out = h W_dn^T.
// Expert backward: recomputes [G | U] into gu ([R][2I]), writes
// [dG | dU] into dgu ([R][2I]) and dEPD ([R][d]), and the fp32 weight
// gradients dW_gate_up [E][2I][d] and dW_down [E][d][I].
hipError_t launch_expert_backward(const occ_layer_desc &L, const int32_t *slot_offset,
                                  const Placement &pl, const void *epd, const void *w_gate_up,
                                  const void *w_down, const void *h, const void *d_out_epd,
                                  void *gu, void *dgu, void *d_epd, float *dw_gate_up,
                                  float *dw_down, hipStream_t st, bool recompute_gu = true);
// fp32 layers: the same products, one thread per output (occ_bwd_f32.hip)
hipError_t launch_expert_backward_f32(const occ_layer_desc &L, const int32_t *slot_offset,
                                      const Placement &pl, const void *epd, const void *w_gate_up,
                                      const void *w_down, const void *h, const void *d_out_epd,
                                      void *gu, void *dgu, void *d_epd, float *dw_gate_up,
                                      float *dw_down, hipStream_t st);
hipError_t launch_shared_backward_f32(const occ_layer_desc &L, const void *x,
                                      const void *w_gate_up_sh, const void *w_down_sh,
                                      const void *h_sh, const void *dy, void *gu, void *dgu,
                                      void *dx_shared, float *dw_gate_up_sh, float *dw_down_sh,
                                      hipStream_t st);
// Shared experts' backward: gu and dgu are [T][n_sh * 2 I_sh] dtype
// workspaces; h_sh the forward's shared activations [T][n_sh * I_sh].
hipError_t launch_shared_backward(const occ_layer_desc &L, const void *x, const void *w_gate_up_sh,
                                  const void *w_down_sh, const void *h_sh, const void *dy,
                                  void *gu, void *dgu, void *dx_shared, float *dw_gate_up_sh,
                                  float *dw_down_sh, hipStream_t st);
// gu: when set (bf16 layers without shared experts), the [G | U] rows are
// also written (bf16 [R][2I])
hipError_t launch_expert_up(const occ_layer_desc &L, const void *epd, const int32_t *slot_offset,
                            const Placement &pl, const void *w_gate_up, void *h,
                            const void *x, const void *w_gate_up_sh, void *h_sh,
                            hipStream_t st, void *gu = nullptr);
hipError_t launch_expert_down(const occ_layer_desc &L, const int32_t *slot_offset,
                              const Placement &pl, const void *w_down, const void *h,
                              void *out_epd, const void *w_down_sh, const void *h_sh,
                              void *shared_out, hipStream_t st);

}  // namespace occ
