/*
 * occ.h -- C ABI of the collaboration-aware MoE layer step (Occult) on one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages describe it:
 *   - each token is routed to k of E experts (Expert Coupling in MoE
 *     Pretraining, Abstract);
 *   - the token tensor passes through three states stored compactly in HBM,
 *     ORI (original order), SFD (one row per token and expert-parallel
 *     device) and EPD (one row per token and expert), guided by two
 *     bidirectional re-index matrices, BRIM_0 [devices x ORI tokens] and
 *     BRIM_1 [local experts per device x SFD tokens] (Occult, Figure 4 and
 *     Figure 5 captions);
 *   - a token is sent to each device once, not once per expert (Expert
 *     Coupling, Abstract), and its co-located expert outputs are reduced
 *     before the way back;
 *   - experts that one token activates together are "collaborated" (Occult,
 *     Abstract); their counts drive correlated placement (Expert Coupling,
 *     Abstract; Occult, TL;DR: expert-placement rescheduling).
 *
 * The expert-parallel devices are logical partitions of one GPU's buffers:
 * device dv owns SFD rows [sfd_offset[dv], sfd_offset[dv+1]) and slots
 * dv*L .. dv*L+L-1, with L = E / D local experts per device.  Every buffer is
 * laid out exactly as it would be sent.
 *
 * Conventions for every entry point:
 *   - Pointers named *_host are host memory; all others are device memory
 *     allocated and owned by the caller.  The library never allocates.
 *   - Row-major, K-contiguous layouts; "dtype" is the layer's storage type
 *     (OCC_F32: float, OCC_BF16: bfloat16 as 16-bit words).
 *   - Calls are asynchronous on the given stream and never synchronise the
 *     host; no call reads device memory on the host.
 *   - Arguments are validated on the host before anything is launched.  On
 *     an error nothing is launched and no output is touched; the return code
 *     says why and occ_last_error() gives the text.
 *   - The library holds no state besides the per-thread error text, the
 *     per-device compute-unit count it caches and the fixed workspace of
 *     occ_build_brim_noalloc; calls on different streams are independent
 *     (except overlapping occ_build_brim_noalloc calls, see there).
 */
#ifndef OCC_H
#define OCC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t occ_status;
#define OCC_OK 0
#define OCC_EINVAL (-1) /* bad shape, null pointer or argument */
#define OCC_EUNSUP (-2) /* valid but outside what the kernels support */
#define OCC_ENOSPC (-3) /* workspace smaller than required */
#define OCC_EHIP (-4)   /* a HIP launch failed; see occ_last_error() */

#define OCC_F32 0
#define OCC_BF16 1

/* Limits checked by every call (OCC_EUNSUP beyond them). */
#define OCC_MAX_E 128 /* routed experts */
#define OCC_MAX_K 16  /* experts per token */
#define OCC_MAX_D 32  /* logical expert-parallel devices */

/* Shape of one MoE layer.  T tokens of hidden size d; E routed experts of
 * intermediate size I, k chosen per token; D logical devices (E % D == 0);
 * n_shared always-active experts of intermediate size I_shared (0 if none);
 * renorm = 1 divides the chosen softmax weights by their sum. */
typedef struct occ_layer_desc {
  int32_t T, d, E, k, D, I;
  int32_t n_shared, I_shared;
  int32_t dtype;
  int32_t renorm;
} occ_layer_desc;

/* The re-index state of one batch (all device memory, caller-allocated).
 * S_max = T * min(k, D); R = T * k.
 *   brim0       int32 [D][T]      SFD row of (device, token), -1 if the token
 *                                 selects no expert on that device
 *   brim1       int32 [L][S_max]  EPD row of (local expert, SFD row), -1 if
 *                                 the token of that SFD row does not select
 *                                 that local expert; columns >= S unspecified
 *   sfd_offset  int32 [D+1]       first SFD row of each device; [D] = S
 *   slot_offset int32 [E+1]       first EPD row of each slot; [E] = R
 *   sfd_token   int32 [S_max]     ORI token of each SFD row (rows < S)
 *   epd_token   int32 [R]         ORI token of each EPD row
 *   epd_sfd     int32 [R]         SFD row of each EPD row
 *   epd_w       float [R]         routing weight of each EPD row
 *   S           int32 [1]         number of SFD rows (dispatched rows)
 * Inside a device (SFD) or a slot (EPD) rows are in ascending token order. */
typedef struct occ_brim {
  int32_t *brim0;
  int32_t *brim1;
  int32_t *sfd_offset;
  int32_t *slot_offset;
  int32_t *sfd_token;
  int32_t *epd_token;
  int32_t *epd_sfd;
  float *epd_w;
  int32_t *S;
} occ_brim;

/* Bytes of device workspace occ_build_brim needs (0 on a bad descriptor). */
size_t occ_workspace_bytes(const occ_layer_desc *desc);

/* Bytes of device workspace occ_expert_ffn / occ_expert_up / occ_expert_down
 * need for the SwiGLU activations h: R*I (+ T*n_shared*I_shared) elements of
 * dtype (0 on a bad descriptor). */
size_t occ_ffn_workspace_bytes(const occ_layer_desc *desc);

/* Routing (Expert Coupling, Abstract: each token goes to k of E experts).
 *   x        dtype [T][d]     ORI tokens
 *   w_router float [E][d]     router weights, fp32 whatever the layer dtype
 *   topk_idx int32 [T][k]     chosen experts, by logit descending, lower
 *                             expert index first on equal logits
 *   topk_w   float [T][k]     softmax over all E logits at the chosen
 *                             experts (divided by their sum if renorm)
 *   logits   float [T][E]     optional (NULL to skip)
 * Each logit is the fp32 chain acc = fma(x[t][j], w_router[e][j], acc) over
 * j = 0..d-1 in order, from +0: bit-reproducible on any IEEE machine. */
occ_status occ_route_topk(const occ_layer_desc *desc, const void *x, const float *w_router,
                          int32_t *topk_idx, float *topk_w, float *logits, hipStream_t stream);

/* Bytes of device workspace occ_route_topk_ws needs; 0 when the descriptor
 * is invalid or outside the filtered path (bf16 layers with 32 <= E <= 128,
 * k <= 16 and d % 64 == 0), where occ_route_topk_ws needs none. */
size_t occ_route_workspace_bytes(const occ_layer_desc *desc);

/* occ_route_topk without the logits output, through a workspace (Expert
 * Coupling, Abstract: k of E experts).  Same topk_idx as occ_route_topk, bit
 * for bit; topk_w within fp32 rounding of it.  On the filtered path the
 * logits are first approximated by bf16 matrix-core products; an error bound
 * per token (from |x_t|, the router rows' norms and their bf16 rounding)
 * leaves the experts that can be among the k largest in-order chains, and
 * only those chains run (a block of 128 tokens with a token of more than 16
 * such experts, or a non-finite value, runs every chain).  The softmax sum
 * takes the other experts' approximate logits.  The filter pays off only
 * when every router row is bf16-representable (a bf16 router widened to
 * fp32); otherwise every chain runs, which is correct but slower than
 * occ_route_topk.  Elsewhere it is occ_route_topk with logits = NULL and ws
 * is not read.
 *   ws, ws_bytes  device workspace of occ_route_workspace_bytes(desc) bytes
 *                 (OCC_ENOSPC when smaller, OCC_EINVAL when NULL and needed) */
occ_status occ_route_topk_ws(const occ_layer_desc *desc, const void *x, const float *w_router,
                             int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* BRIM construction (Occult, Figure 5 caption; Expert Coupling, Abstract:
 * each token to each device once).
 *   topk_idx, topk_w  as written by occ_route_topk
 *   slot_expert_host  int32 [E] host: expert held by slot g = dv*L + l; must
 *                     be a permutation of 0..E-1 (OCC_EINVAL otherwise)
 *   brim              outputs, see occ_brim
 *   ws, ws_bytes      device workspace of occ_workspace_bytes(desc) bytes
 * Deterministic: stable counting sorts, no dependence on atomics order. */
occ_status occ_build_brim(const occ_layer_desc *desc, const int32_t *topk_idx,
                          const float *topk_w, const int32_t *slot_expert_host,
                          const occ_brim *brim, void *ws, size_t ws_bytes, hipStream_t stream);

/* occ_build_brim for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and outputs as occ_build_brim
 * without ws / ws_bytes: the workspace is a fixed device array inside the
 * library, OCC_NOALLOC_BRIM_SCRATCH_BYTES bytes on each GPU the library runs
 * on (held until the process ends; its address is looked up once per
 * device).  Nothing is allocated.  OCC_EUNSUP when occ_workspace_bytes(desc)
 * exceeds that size (about 100 K tokens with D + E = 160 keys).  Every call
 * on one GPU shares that array, so calls that overlap on one GPU (other
 * streams or threads) race and must be serialised by the caller; a call
 * fully overwrites what it reads, so nothing needs clearing between calls. */
#define OCC_NOALLOC_BRIM_SCRATCH_BYTES (1u << 20)
occ_status occ_build_brim_noalloc(const occ_layer_desc *desc, const int32_t *topk_idx,
                                  const float *topk_w, const int32_t *slot_expert_host,
                                  const occ_brim *brim, hipStream_t stream);

/* BRIM build under an all-to-all budget: routing-score-based collaboration
 * pruning (Occult, TL;DR: pruning by routing score to minimise the budget
 * C_T).  The pages give no exact rule; this one is used: each token keeps at
 * most `budget` devices (1 <= budget <= D), those with the largest summed
 * routing weight of the token's selected experts (fp32 sums in top-k order,
 * lower device index on equal sums); its selections on the other devices are
 * dropped.  rescale = 1 multiplies each kept weight by (sum of the token's
 * weights) / (sum of its kept weights), both fp32 sums in top-k order;
 * rescale = 0 keeps the weights.  Outputs as occ_build_brim, except that EPD
 * holds R' = slot_offset[E] <= T*k rows (epd_token, epd_sfd, epd_w valid
 * below R'); budget = D gives exactly occ_build_brim's result.  Every later
 * call works on the pruned layouts unchanged.  EINVAL for a budget outside
 * 1..D or rescale outside {0, 1}. */
occ_status occ_build_brim_pruned(const occ_layer_desc *desc, const int32_t *topk_idx,
                                 const float *topk_w, const int32_t *slot_expert_host,
                                 int32_t budget, int32_t rescale, const occ_brim *brim, void *ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Dispatch ORI -> SFD -> EPD (Occult, Figure 4 caption): bit copies
 *   sfd[s] = x[sfd_token[s]]  (dtype [S_max][d], rows < S written): the
 *            all-to-all send buffer, grouped by device
 *   epd[r] = sfd[epd_sfd[r]]  (dtype [R][d]): the experts' input, by slot
 * Both are written from one read of each ORI row. */
occ_status occ_dispatch(const occ_layer_desc *desc, const void *x, const occ_brim *brim,
                        void *sfd, void *epd, hipStream_t stream);

/* Expert networks on EPD (Expert Coupling, Abstract: "expert networks";
 * SwiGLU without biases).  For EPD row r of slot g, e = slot_expert_host[g]:
 *   h[r]       = silu(W_gate[e] epd[r]) * (W_up[e] epd[r])    (stored in dtype)
 *   out_epd[r] = W_down[e] h[r]                               (dtype [R][d])
 * w_gate_up dtype [E][2I][d] (rows 0..I-1 gate, I..2I-1 up), w_down dtype
 * [E][d][I]; fp32 accumulation.  Shared experts (n_shared > 0) run on the ORI
 * rows with weight 1: shared_out = sum_s FFN_s(x) (dtype [T][d]) from
 * w_gate_up_sh [n_shared][2*I_shared][d] and w_down_sh [n_shared][d][I_shared].
 * h_ws holds h (occ_ffn_workspace_bytes).  x, w_*_sh and shared_out must be
 * NULL when n_shared == 0.  occ_expert_up runs the gate/up GEMM with the SwiGLU
 * epilogue, occ_expert_down the down GEMM; occ_expert_ffn runs both. */
occ_status occ_expert_ffn(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                          const int32_t *slot_expert_host, const void *w_gate_up,
                          const void *w_down, void *h_ws, size_t h_ws_bytes, void *out_epd,
                          const void *x, const void *w_gate_up_sh, const void *w_down_sh,
                          void *shared_out, hipStream_t stream);
occ_status occ_expert_up(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                         const int32_t *slot_expert_host, const void *w_gate_up, void *h_ws,
                         size_t h_ws_bytes, const void *x, const void *w_gate_up_sh,
                         hipStream_t stream);
occ_status occ_expert_down(const occ_layer_desc *desc, const occ_brim *brim,
                           const int32_t *slot_expert_host, const void *w_down,
                           const void *h_ws, size_t h_ws_bytes, void *out_epd,
                           const void *w_down_sh, void *shared_out, hipStream_t stream);

/* Combine (Occult, Figure 4 caption, the way back over the same BRIMs):
 *   out_sfd[s] = sum over l ascending with r = brim1[l][s] >= 0 of
 *                epd_w[r] * out_epd[r]        (dtype [S_max][d]: the
 *                pre-reduced return payload, rows < S written)
 *   y[t]       = shared_out[t] + sum over devices dv ascending with
 *                s = brim0[dv][t] >= 0 of out_sfd[s]        (dtype [T][d])
 * fp32 accumulation, each stored row rounded to dtype (ties to even).
 * shared_out may be NULL. */
occ_status occ_combine(const occ_layer_desc *desc, const void *out_epd, const occ_brim *brim,
                       const void *shared_out, void *out_sfd, void *y, hipStream_t stream);

/* Conventional per-(token, expert) dispatch and combine: the standard
 * strategy that Occult, Figure 2 contrasts with, where every (token, expert)
 * pair is one row of the send buffer and comes back unreduced.  Same
 * occ_build_brim outputs, no SFD stage:
 *   occ_dispatch_direct: epd[r] = x[epd_token[r]]   (dtype [R][d]; the EPD,
 *                        grouped by slot and so by device, is the send buffer)
 *   occ_combine_direct:  y[t] = shared_out[t] + sum over the token's rows r
 *                        (device, then local expert ascending) of
 *                        epd_w[r] * out_epd[r]      (dtype [T][d])
 *                        fp32 accumulation, one rounding to dtype (ties to
 *                        even); shared_out may be NULL.
 * EINVAL on a NULL x / epd / out_epd / y or brim array (T > 0). */
occ_status occ_dispatch_direct(const occ_layer_desc *desc, const void *x, const occ_brim *brim,
                               void *epd, hipStream_t stream);
occ_status occ_combine_direct(const occ_layer_desc *desc, const void *out_epd, const occ_brim *brim,
                              const void *shared_out, void *y, hipStream_t stream);

/* Co-activation (collaboration) counts (Occult, Abstract):
 *   counts int32 [E][E]: counts[i][j] += #tokens choosing both i and j
 *   (diagonal: tokens per expert).  accumulate = 0 zeroes counts first.
 * Integer atomics only, so the result does not depend on scheduling. */
occ_status occ_coactivation(const occ_layer_desc *desc, const int32_t *topk_idx,
                            int32_t *counts, int32_t accumulate, hipStream_t stream);

/* ---- Backward pass through the BRIMs (bf16 and fp32 layers: in an fp32
 * layer every tensor marked bf16 below is fp32 and no step rounds to bf16).
 * Expert Coupling in MoE Pretraining, Abstract: every MoE layer runs its
 * all-to-alls in the forward and the backward pass; Occult, Figure 4
 * caption: the moves between ORI, SFD and EPD are guided by the BRIMs,
 * walked here in the opposite direction.  Call order after a forward
 * (occ_route_topk with logits, occ_build_brim, occ_dispatch, occ_expert_ffn,
 * occ_combine): occ_grad_combine, occ_expert_backward, occ_router_backward,
 * (with shared experts) occ_shared_backward, occ_grad_dispatch.  Top-k
 * selection is a constant. */

/* Bytes of the workspace of occ_expert_backward and occ_router_backward
 * (one buffer may serve both calls in turn; 0 for an invalid or unsupported
 * descriptor). */
size_t occ_backward_workspace_bytes(const occ_layer_desc *desc);

/* Gradient of the combine, given dy (bf16 [T][d]):
 *   d_out_sfd[s] = dy[sfd_token[s]]          (bf16 [S_max][d], rows < S; the
 *                                             backward send buffer; may be NULL)
 *   d_out_epd[r] = epd_w[r] * dy[epd_token[r]]   (bf16 [R][d], rounded)
 *   dw_epd[r]    = sum_c dy[t][c] out_epd[r][c]  (fp32 [R]: gradient of the
 *                                             routing weight of row r) */
occ_status occ_grad_combine(const occ_layer_desc *desc, const void *dy, const occ_brim *brim,
                            const void *out_epd, void *d_out_sfd, void *d_out_epd, float *dw_epd,
                            hipStream_t stream);

/* Gradient of the SwiGLU experts on the EPD rows of each slot:
 *   [G | U] = EPD W_gate_up[e]^T recomputed (bf16, in bwd_ws)
 *   dh      = d_out_epd W_down[e];  dG = dh U silu'(G), dU = dh silu(G)
 *             (bf16, in bwd_ws)
 *   d_epd   = [dG | dU] W_gate_up[e]                      (bf16 [R][d])
 *   dw_gate_up[e] = sum over the slot's rows of [dG | dU]^T EPD
 *                                                  (fp32 [E][2I][d], written)
 *   dw_down[e]    = sum over the slot's rows of d_out_epd^T h
 *                                                  (fp32 [E][d][I], written)
 * h_ws is the forward's workspace (h of every EPD row); bwd_ws holds
 * occ_backward_workspace_bytes(desc) bytes. */
occ_status occ_expert_backward(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                               const int32_t *slot_expert_host, const void *w_gate_up,
                               const void *w_down, const void *h_ws, size_t h_ws_bytes,
                               const void *d_out_epd, void *bwd_ws, size_t bwd_ws_bytes,
                               void *d_epd, float *dw_gate_up, float *dw_down,
                               hipStream_t stream);

/* Training (Expert Coupling in MoE Pretraining, Abstract: the layer runs
 * forward and backward): the pair for steps that keep the experts' pre-activations instead
 * of recomputing them (bf16 layers without shared experts; EUNSUP otherwise):
 * occ_expert_ffn_keep is occ_expert_ffn that also writes
 *   gu[r] = [EPD W_gate^T | EPD W_up^T] of EPD row r   (bf16 [R][2I], rows < R;
 *           the products rounded once, as h's inputs)
 * and occ_expert_backward_kept is occ_expert_backward reading [G | U] from gu
 * (written by occ_expert_ffn_keep for the same layer, weights and BRIM)
 * instead of recomputing it; bwd_ws as for occ_expert_backward.  The results
 * equal occ_expert_ffn's and occ_expert_backward's bit for bit; the pair
 * trades 2 R I bf16 values of device memory for one grouped GEMM. */
occ_status occ_expert_ffn_keep(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                               const int32_t *slot_expert_host, const void *w_gate_up,
                               const void *w_down, void *h_ws, size_t h_ws_bytes, void *gu,
                               void *out_epd, hipStream_t stream);
occ_status occ_expert_backward_kept(const occ_layer_desc *desc, const void *epd,
                                    const occ_brim *brim, const int32_t *slot_expert_host,
                                    const void *w_gate_up, const void *w_down, const void *h_ws,
                                    size_t h_ws_bytes, const void *gu, const void *d_out_epd,
                                    void *bwd_ws, size_t bwd_ws_bytes, void *d_epd,
                                    float *dw_gate_up, float *dw_down, hipStream_t stream);

/* Gradient of the routing: for each token, dp of its picks from dw_epd
 * (through the renormalisation when desc->renorm), then the softmax backward
 * over all E experts, from the forward's fp32 logits:
 *   dlogits[t][e] = p[e] (dp[e] - sum_e' p[e'] dp[e'])      (fp32 [T][E])
 *   dx_router     = dlogits W_r                            (fp32 [T][d])
 *   dw_router     = dlogits^T x                            (fp32 [E][d])
 * Both products accumulate in fp32; dw_router sums its token chunks in a
 * fixed order (deterministic).  The gradient is exact for a BRIM from
 * occ_build_brim.  With one from occ_build_brim_pruned it takes dw_epd (the
 * gradient of each stored weight) as the gradient of that pick's routing
 * weight and gives dropped picks none: with rescale = 0 the exact gradient
 * of the pruned layer (the pruning decision held fixed), with rescale = 1 an
 * approximation that ignores the rescaling factor.  bwd_ws: device workspace of at least
 * occ_backward_workspace_bytes(desc) bytes for the partial sums (ENOSPC when
 * smaller; its contents are not kept). */
occ_status occ_router_backward(const occ_layer_desc *desc, const void *x, const float *w_router,
                               const float *logits, const int32_t *topk_idx,
                               const float *topk_w, const int32_t *slot_expert_host,
                               const occ_brim *brim, const float *dw_epd, float *dlogits,
                               float *dx_router, float *dw_router, void *bwd_ws,
                               size_t bwd_ws_bytes, hipStream_t stream);

/* Gradient of the shared experts (always active, weight 1, on the ORI rows;
 * layers with n_shared > 0, EINVAL otherwise).  For shared expert s, with
 * X the layer's tokens and dY the layer's output gradient:
 *   [G | U]_s = X W_gate_up_sh[s]^T recomputed (bf16, in bwd_ws)
 *   dh_s = dY W_down_sh[s];  dG_s = dh U silu'(G), dU_s = dh silu(G)
 *             (bf16, in bwd_ws)
 *   dw_gate_up_sh[s] = [dG | dU]_s^T X     (fp32 [n_shared][2 I_shared][d], written)
 *   dw_down_sh[s]    = dY^T h_s            (fp32 [n_shared][d][I_shared], written;
 *                                           h_s: the forward's, from h_ws)
 *   dx_shared = sum over s of [dG | dU]_s W_gate_up_sh[s]
 *                                          (bf16 [T][d]; for occ_grad_dispatch)
 * x, w_gate_up_sh, w_down_sh as given to occ_expert_ffn; h_ws its workspace;
 * dy bf16 [T][d]; bwd_ws of occ_backward_workspace_bytes(desc) bytes. */
occ_status occ_shared_backward(const occ_layer_desc *desc, const void *x,
                               const void *w_gate_up_sh, const void *w_down_sh, const void *h_ws,
                               size_t h_ws_bytes, const void *dy, void *bwd_ws,
                               size_t bwd_ws_bytes, void *dx_shared, float *dw_gate_up_sh,
                               float *dw_down_sh, hipStream_t stream);

/* Gradient of the dispatch (the combine's walk with unit weights):
 *   d_sfd[s] = sum over l ascending with r = brim1[l][s] >= 0 of d_epd[r]
 *              (bf16 [S_max][d], rows < S: the backward return payload)
 *   dx[t]    = dx_shared[t] + dx_router[t] + sum over devices of
 *              d_sfd[brim0[dv][t]]
 *              (bf16 [T][d]; fp32 accumulation, one rounding; dx_router may
 *              be NULL; dx_shared, from occ_shared_backward, must be set when
 *              n_shared > 0 and NULL otherwise) */
occ_status occ_grad_dispatch(const occ_layer_desc *desc, const void *d_epd, const occ_brim *brim,
                             const float *dx_router, const void *dx_shared, void *d_sfd, void *dx,
                             hipStream_t stream);

/* Cross-layer co-activation (Expert Coupling in MoE Pretraining, Abstract:
 * the experts a token selects at one layer predict those it selects at the
 * next; ExFlow, Abstract: inter-layer expert affinity):
 *   counts int32 [E1][E2]: counts[i][j] += #tokens t with i among
 *   idx1[t][0..k1) and j among idx2[t][0..k2).  accumulate = 0 zeroes first.
 *   idx1 int32 [T][k1], idx2 int32 [T][k2] (device), ids outside 0..E-1
 *   skipped.  Integer atomics only (order-free). */
occ_status occ_cross_coactivation(int32_t T, int32_t k1, int32_t E1, const int32_t *idx1,
                                  int32_t k2, int32_t E2, const int32_t *idx2, int32_t *counts,
                                  int32_t accumulate, hipStream_t stream);

/* Home device of each token for the next layer (token shuffling, Expert
 * Coupling, Abstract: move each token to the GPU predicted to hold its
 * next-layer experts).  With affinity int32 [E1][E2] (occ_cross_coactivation
 * of a calibration batch) and the next layer's placement (slot_expert2_host,
 * int32 [E2] host, a permutation; D devices of E2/D experts):
 *   home[t] = argmax over d of sum over i in idx1[t] of sum over the experts
 *             j on device d of affinity[i][j]   (int64, lower d on ties)
 *   home int32 [T] (device). */
occ_status occ_home_device(int32_t T, int32_t k1, int32_t E1, const int32_t *idx1, int32_t E2,
                           int32_t D, const int32_t *slot_expert2_host, const int32_t *affinity,
                           int32_t *home, hipStream_t stream);

/* Assignments served on the token's own device (Expert Coupling, Abstract:
 * the share of token-expert assignments served on the token's GPU):
 *   hits[0] += #(t, q) with device(idx2[t][q]) == home[t]
 * for any home assignment home int32 [T] (device): the predicted one of
 * occ_home_device, or a plain sharding such as t * D / T.  hits is a device
 * int32 scalar; accumulate = 0 zeroes it first. */
occ_status occ_local_hits(int32_t T, int32_t k2, int32_t E2, const int32_t *idx2, int32_t D,
                          const int32_t *slot_expert2_host, const int32_t *home, int32_t *hits,
                          int32_t accumulate, hipStream_t stream);

/* Greedy correlated placement on the host (Expert Coupling, Abstract:
 * experts often selected together go on one GPU; Occult, TL;DR: placement
 * rescheduling).  For each device in turn: take the unplaced expert with the
 * most tokens (lower index on ties), then repeatedly the unplaced expert
 * with the largest summed count against the device's experts (ties: more
 * tokens, then lower index) until the device holds E/D experts.
 *   counts_host      int32 [E][E] host (from occ_coactivation)
 *   slot_expert_host int32 [E] host output */
occ_status occ_place_greedy(int32_t E, int32_t D, const int32_t *counts_host,
                            int32_t *slot_expert_host);

/* Text of the last error on the calling thread ("" if none). */
const char *occ_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OCC_H */
