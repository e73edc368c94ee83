// Backward of the expert networks for fp32 layers.
//
// The same products as the bf16 backward (Expert Coupling in MoE
// Pretraining, Abstract: the MoE layer runs forward and backward; Occult,
// Figure 4 caption: expert computing on the EPD state), for the small fp32
// layers, where launches, not arithmetic, bound the step: one thread per
// output element, an in-order fp32 FMA chain over K, as the fp32 forward.
//   grouped rows (the slots' EPD rows, or one dense group of ORI rows):
//     C[m][n] = sum_k A(m, k) B_e(k, n), expert e of the row's slot
//     (with the SwiGLU backward: dG = acc U silu'(G), dU = acc G sigmoid(G),
//     from the [G | U] row, written to columns n and N + n)
//   grouped K (weight gradients): C_e[m][n] = sum over the slot's rows r of
//     A(m, r) B(r, n)
// A(m, k) = A[m a_m + k a_k], B_e(k, n) = B[e b_group + k b_k + n b_n].
#include "occ_internal.h"

namespace occ {
namespace {

constexpr int kThreads = 256;

struct F32Prod {
  const float *A;
  int64_t a_m, a_k;
  const float *B;
  int64_t b_k, b_n, b_group;
  float *C;
  int64_t c_m, c_n, c_group;
  const float *aux;  // SwiGLU backward: the [G | U] rows
  int64_t aux_m;
  int M, N, K;
  const int32_t *row_offset;  // [G + 1] on the device; nullptr: one group of `dense` rows
  int G, dense;
  int32_t expert_of_group[OCC_MAX_E];
};

// last group whose first row is <= m
__device__ __forceinline__ int group_of(const int32_t *ro, int G, int m) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ro[mid] <= m) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// MODE 0: grouped rows, plain; 1: grouped rows, SwiGLU backward; 2: grouped K
template <int MODE>
__global__ __launch_bounds__(kThreads) void f32_prod_kernel(F32Prod p, int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= total) return;
  if (MODE == 2) {
    const int64_t mn = (int64_t)p.M * p.N;
    const int g = (int)(gid / mn);
    const int m = (int)((gid - g * mn) / p.N), n = (int)(gid % p.N);
    const int r0 = p.row_offset != nullptr ? p.row_offset[g] : 0;
    const int r1 = p.row_offset != nullptr ? p.row_offset[g + 1] : p.dense;
    float acc = 0.0f;
    for (int r = r0; r < r1; ++r)
      acc = __builtin_fmaf(p.A[m * p.a_m + (int64_t)r * p.a_k], p.B[(int64_t)r * p.b_k + n * p.b_n],
                           acc);
    p.C[(int64_t)p.expert_of_group[g] * p.c_group + m * p.c_m + n * p.c_n] = acc;
    return;
  }
  const int m = (int)(gid / p.N), n = (int)(gid % p.N);
  const int rows = p.row_offset != nullptr ? p.row_offset[p.G] : p.dense;
  if (m >= rows) return;
  const int g = p.row_offset != nullptr ? group_of(p.row_offset, p.G, m) : 0;
  const float *Bp = p.B + (int64_t)p.expert_of_group[g] * p.b_group + n * p.b_n;
  const float *Ap = p.A + m * p.a_m;
  float acc = 0.0f;
  for (int k = 0; k < p.K; ++k) acc = __builtin_fmaf(Ap[k * p.a_k], Bp[k * p.b_k], acc);
  if (MODE == 0) {
    p.C[m * p.c_m + n * p.c_n] = acc;
  } else {
    const float G = p.aux[m * p.aux_m + n], U = p.aux[m * p.aux_m + p.N + n];
    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-G));
    p.C[m * p.c_m + n] = acc * U * (sg * (1.0f + G * (1.0f - sg)));
    p.C[m * p.c_m + p.N + n] = acc * G * sg;
  }
}

template <int MODE>
hipError_t run(const F32Prod &p, int64_t total, hipStream_t st) {
  if (total <= 0) return hipSuccess;
  f32_prod_kernel<MODE><<<(unsigned)((total + kThreads - 1) / kThreads), kThreads, 0, st>>>(
      p, total);
  return hipGetLastError();
}

F32Prod prod(const Placement &pl) {
  F32Prod p{};
  for (int g = 0; g < OCC_MAX_E; ++g) p.expert_of_group[g] = pl.expert_at[g];
  return p;
}

}  // namespace

hipError_t launch_expert_backward_f32(const occ_layer_desc &L, const int32_t *slot_offset,
                                      const Placement &pl, const void *epd, const void *w_gate_up,
                                      const void *w_down, const void *h, const void *d_out_epd,
                                      void *gu, void *dgu, void *d_epd, float *dw_gate_up,
                                      float *dw_down, hipStream_t st) {
  const int64_t d = L.d, I = L.I, R = (int64_t)L.T * L.k, E = L.E;
  hipError_t err;
  // 1. [G | U] = EPD W_gate_up^T (W_gate_up[e] is [2I][d])
  F32Prod p = prod(pl);
  p.row_offset = slot_offset;
  p.G = L.E;
  p.A = static_cast<const float *>(epd);
  p.a_m = d, p.a_k = 1;
  p.B = static_cast<const float *>(w_gate_up);
  p.b_k = 1, p.b_n = d, p.b_group = 2 * I * d;
  p.C = static_cast<float *>(gu);
  p.c_m = 2 * I, p.c_n = 1;
  p.M = (int)R, p.N = (int)(2 * I), p.K = (int)d;
  if ((err = run<0>(p, R * 2 * I, st)) != hipSuccess) return err;
  // 2. dh = d_out_EPD W_down (W_down[e] is [d][I]), SwiGLU backward -> [dG | dU]
  p = prod(pl);
  p.row_offset = slot_offset;
  p.G = L.E;
  p.A = static_cast<const float *>(d_out_epd);
  p.a_m = d, p.a_k = 1;
  p.B = static_cast<const float *>(w_down);
  p.b_k = I, p.b_n = 1, p.b_group = d * I;
  p.aux = static_cast<const float *>(gu);
  p.aux_m = 2 * I;
  p.C = static_cast<float *>(dgu);
  p.c_m = 2 * I;
  p.M = (int)R, p.N = (int)I, p.K = (int)d;
  if ((err = run<1>(p, R * I, st)) != hipSuccess) return err;
  // 3. dW_down[e] = sum over the slot's rows of d_out_EPD^T h   ([d][I])
  p = prod(pl);
  p.row_offset = slot_offset;
  p.G = L.E;
  p.A = static_cast<const float *>(d_out_epd);
  p.a_m = 1, p.a_k = d;
  p.B = static_cast<const float *>(h);
  p.b_k = I, p.b_n = 1;
  p.C = dw_down;
  p.c_m = I, p.c_n = 1, p.c_group = d * I;
  p.M = (int)d, p.N = (int)I;
  if ((err = run<2>(p, E * d * I, st)) != hipSuccess) return err;
  // 4. dW_gate_up[e] = sum over the slot's rows of [dG | dU]^T EPD   ([2I][d])
  p = prod(pl);
  p.row_offset = slot_offset;
  p.G = L.E;
  p.A = static_cast<const float *>(dgu);
  p.a_m = 1, p.a_k = 2 * I;
  p.B = static_cast<const float *>(epd);
  p.b_k = d, p.b_n = 1;
  p.C = dw_gate_up;
  p.c_m = d, p.c_n = 1, p.c_group = 2 * I * d;
  p.M = (int)(2 * I), p.N = (int)d;
  if ((err = run<2>(p, E * 2 * I * d, st)) != hipSuccess) return err;
  // 5. dEPD = [dG | dU] W_gate_up   (K = 2I)
  p = prod(pl);
  p.row_offset = slot_offset;
  p.G = L.E;
  p.A = static_cast<const float *>(dgu);
  p.a_m = 2 * I, p.a_k = 1;
  p.B = static_cast<const float *>(w_gate_up);
  p.b_k = d, p.b_n = 1, p.b_group = 2 * I * d;
  p.C = static_cast<float *>(d_epd);
  p.c_m = d, p.c_n = 1;
  p.M = (int)R, p.N = (int)d, p.K = (int)(2 * I);
  return run<0>(p, R * d, st);
}

hipError_t launch_shared_backward_f32(const occ_layer_desc &L, const void *x,
                                      const void *w_gate_up_sh, const void *w_down_sh,
                                      const void *h_sh, const void *dy, void *gu, void *dgu,
                                      void *dx_shared, float *dw_gate_up_sh, float *dw_down_sh,
                                      hipStream_t st) {
  const int64_t T = L.T, d = L.d, Is = L.I_shared, ns = L.n_shared, W2 = ns * 2 * Is;
  const Placement none{};
  const float *wgu = static_cast<const float *>(w_gate_up_sh);
  const float *wdn = static_cast<const float *>(w_down_sh);
  float *gub = static_cast<float *>(gu);
  float *dgub = static_cast<float *>(dgu);
  hipError_t err;
  // 1. [G | U] of every shared expert: X times the stacked W_gate_up_sh
  F32Prod p = prod(none);
  p.G = 1, p.dense = (int)T;
  p.A = static_cast<const float *>(x);
  p.a_m = d, p.a_k = 1;
  p.B = wgu;
  p.b_k = 1, p.b_n = d;
  p.C = gub;
  p.c_m = W2, p.c_n = 1;
  p.M = (int)T, p.N = (int)W2, p.K = (int)d;
  if ((err = run<0>(p, T * W2, st)) != hipSuccess) return err;
  for (int64_t s = 0; s < ns; ++s) {
    // 2. dh_s = dY W_down_sh[s]; SwiGLU backward into its [dG | dU] columns
    p = prod(none);
    p.G = 1, p.dense = (int)T;
    p.A = static_cast<const float *>(dy);
    p.a_m = d, p.a_k = 1;
    p.B = wdn + s * d * Is;
    p.b_k = Is, p.b_n = 1;
    p.aux = gub + s * 2 * Is;
    p.aux_m = W2;
    p.C = dgub + s * 2 * Is;
    p.c_m = W2;
    p.M = (int)T, p.N = (int)Is, p.K = (int)d;
    if ((err = run<1>(p, T * Is, st)) != hipSuccess) return err;
    // 3. dW_down_sh[s] = dY^T h_s
    p = prod(none);
    p.G = 1, p.dense = (int)T;
    p.A = static_cast<const float *>(dy);
    p.a_m = 1, p.a_k = d;
    p.B = static_cast<const float *>(h_sh) + s * Is;
    p.b_k = ns * Is, p.b_n = 1;
    p.C = dw_down_sh + s * d * Is;
    p.c_m = Is, p.c_n = 1;
    p.M = (int)d, p.N = (int)Is;
    if ((err = run<2>(p, d * Is, st)) != hipSuccess) return err;
  }
  // 4. dW_gate_up_sh = [dG | dU]^T X   (the stacked [n_sh 2 I_sh][d])
  p = prod(none);
  p.G = 1, p.dense = (int)T;
  p.A = dgub;
  p.a_m = 1, p.a_k = W2;
  p.B = static_cast<const float *>(x);
  p.b_k = d, p.b_n = 1;
  p.C = dw_gate_up_sh;
  p.c_m = d, p.c_n = 1;
  p.M = (int)W2, p.N = (int)d;
  if ((err = run<2>(p, W2 * d, st)) != hipSuccess) return err;
  // 5. dx_shared = [dG | dU] W_gate_up_sh (K = n_sh 2 I_sh)
  p = prod(none);
  p.G = 1, p.dense = (int)T;
  p.A = dgub;
  p.a_m = W2, p.a_k = 1;
  p.B = wgu;
  p.b_k = d, p.b_n = 1;
  p.C = static_cast<float *>(dx_shared);
  p.c_m = d, p.c_n = 1;
  p.M = (int)T, p.N = (int)d, p.K = (int)W2;
  return run<0>(p, T * d, st);
}

}  // namespace occ
