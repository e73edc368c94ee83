// Host side of the C ABI: argument validation, error reporting and launch
// sequencing.  Nothing here reads device memory or synchronises; every
// check happens before the first launch of a call.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>
#include <vector>

#include "occ.h"
#include "occ_internal.h"

namespace {

thread_local std::string g_err;

occ_status fail(occ_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

occ_status ok() {
  g_err.clear();
  return OCC_OK;
}

occ_status hip_status(hipError_t e, const char *where) {
  if (e == hipSuccess) return ok();
  return fail(OCC_EHIP, "%s: %s", where, hipGetErrorString(e));
}

int64_t elem_bytes(const occ_layer_desc &L) { return L.dtype == OCC_F32 ? 4 : 2; }
int64_t s_max(const occ_layer_desc &L) { return (int64_t)L.T * (L.k < L.D ? L.k : L.D); }

// A buffer of n > 0 elements must be set; an empty one may be NULL.
bool missing(const void *p, int64_t n) { return n > 0 && p == nullptr; }

// Shape checks shared by every call.
occ_status check_desc(const occ_layer_desc *p) {
  if (p == nullptr) return fail(OCC_EINVAL, "layer descriptor is NULL");
  const occ_layer_desc &L = *p;
  if (L.T < 0 || L.d <= 0 || L.E <= 0 || L.k <= 0 || L.D <= 0 || L.I <= 0)
    return fail(OCC_EINVAL, "bad shape: T=%d d=%d E=%d k=%d D=%d I=%d", L.T, L.d, L.E, L.k, L.D,
                L.I);
  if (L.dtype != OCC_F32 && L.dtype != OCC_BF16)
    return fail(OCC_EINVAL, "dtype %d is neither OCC_F32 nor OCC_BF16", L.dtype);
  if (L.renorm != 0 && L.renorm != 1) return fail(OCC_EINVAL, "renorm must be 0 or 1");
  if (L.k > L.E) return fail(OCC_EINVAL, "k=%d exceeds E=%d", L.k, L.E);
  if (L.E % L.D != 0) return fail(OCC_EINVAL, "E=%d is not a multiple of D=%d", L.E, L.D);
  if (L.n_shared < 0 || L.I_shared < 0 || (L.n_shared > 0 && L.I_shared <= 0))
    return fail(OCC_EINVAL, "bad shared experts: n_shared=%d I_shared=%d", L.n_shared,
                L.I_shared);
  if (L.E > OCC_MAX_E) return fail(OCC_EUNSUP, "E=%d > %d", L.E, OCC_MAX_E);
  if (L.k > OCC_MAX_K) return fail(OCC_EUNSUP, "k=%d > %d", L.k, OCC_MAX_K);
  if (L.D > OCC_MAX_D) return fail(OCC_EUNSUP, "D=%d > %d", L.D, OCC_MAX_D);
  if ((int64_t)L.T * L.k > INT32_MAX || (int64_t)L.T * L.E > INT32_MAX)
    return fail(OCC_EUNSUP, "T=%d too large for 32-bit row indices", L.T);
  if (L.d % 8 != 0) return fail(OCC_EUNSUP, "d=%d is not a multiple of 8", L.d);
  if (L.d * elem_bytes(L) > 8192)
    return fail(OCC_EUNSUP, "rows of %lld bytes exceed 8192", (long long)(L.d * elem_bytes(L)));
  if (L.dtype == OCC_BF16 && (L.d % 64 != 0 || L.I % 64 != 0 || L.I_shared % 64 != 0))
    return fail(OCC_EUNSUP, "bf16 expert GEMMs need d, I, I_shared multiples of 64");
  if (L.dtype == OCC_BF16) {
    // the bf16 GEMMs address each operand with 32-bit byte offsets
    const int64_t R = (int64_t)L.T * L.k, lim = 0xffffffffll;
    if (R * L.d * 2 > lim || R * L.I * 2 > lim || (int64_t)L.E * 2 * L.I * L.d * 2 > lim ||
        (int64_t)L.T * L.n_shared * L.I_shared * 2 > lim ||
        (int64_t)L.n_shared * 2 * L.I_shared * L.d * 2 > lim)
      return fail(OCC_EUNSUP, "an expert GEMM operand exceeds 4 GiB");
  }
  return OCC_OK;
}

occ_status check_brim(const occ_layer_desc &L, const occ_brim *b, bool need_all) {
  if (b == nullptr) return fail(OCC_EINVAL, "brim is NULL");
  const int64_t R = (int64_t)L.T * L.k, Sm = s_max(L);
  if (missing(b->brim0, (int64_t)L.D * L.T) || missing(b->brim1, (int64_t)(L.E / L.D) * Sm) ||
      !b->slot_offset)
    return fail(OCC_EINVAL, "brim0, brim1 and slot_offset must be set");
  if (need_all && (!b->sfd_offset || missing(b->sfd_token, Sm) || missing(b->epd_token, R) ||
                   missing(b->epd_sfd, R) || missing(b->epd_w, R) || !b->S))
    return fail(OCC_EINVAL, "every occ_brim array must be set");
  return OCC_OK;
}

occ_status make_placement(const occ_layer_desc &L, const int32_t *slot_expert_host,
                          occ::Placement &pl) {
  if (slot_expert_host == nullptr) return fail(OCC_EINVAL, "slot_expert_host is NULL");
  for (int i = 0; i < OCC_MAX_E; ++i) pl.expert_at[i] = pl.slot_of[i] = -1;
  for (int g = 0; g < L.E; ++g) {
    const int e = slot_expert_host[g];
    if (e < 0 || e >= L.E || pl.slot_of[e] != -1)
      return fail(OCC_EINVAL, "slot_expert is not a permutation of 0..%d (slot %d -> %d)",
                  L.E - 1, g, e);
    pl.expert_at[g] = e;
    pl.slot_of[e] = g;
  }
  return OCC_OK;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t h_bytes(const occ_layer_desc &L) {
  return align256((size_t)L.T * L.k * L.I * elem_bytes(L));
}
size_t h_sh_bytes(const occ_layer_desc &L) {
  return (size_t)L.T * L.n_shared * L.I_shared * elem_bytes(L);
}

#define OCC_TRY(expr)                \
  do {                               \
    const occ_status s_ = (expr);    \
    if (s_ != OCC_OK) return s_;     \
  } while (0)

}  // namespace

extern "C" {

const char *occ_last_error(void) { return g_err.c_str(); }

size_t occ_workspace_bytes(const occ_layer_desc *desc) {
  if (check_desc(desc) != OCC_OK) return 0;
  return occ::brim_workspace_bytes(desc->T, desc->D, desc->E);
}

size_t occ_ffn_workspace_bytes(const occ_layer_desc *desc) {
  if (check_desc(desc) != OCC_OK) return 0;
  return h_bytes(*desc) + h_sh_bytes(*desc);
}

occ_status occ_route_topk(const occ_layer_desc *desc, const void *x, const float *w_router,
                          int32_t *topk_idx, float *topk_w, float *logits, hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  const int64_t Td = (int64_t)desc->T * desc->d, Tk = (int64_t)desc->T * desc->k;
  if (missing(x, Td) || !w_router || missing(topk_idx, Tk) || missing(topk_w, Tk))
    return fail(OCC_EINVAL, "x, w_router, topk_idx and topk_w must be set");
  return hip_status(occ::launch_route_topk(*desc, x, w_router, topk_idx, topk_w, logits, stream),
                    "occ_route_topk");
}

size_t occ_route_workspace_bytes(const occ_layer_desc *desc) {
  if (check_desc(desc) != OCC_OK) return 0;
  return occ::route_filter_workspace_bytes(*desc);
}

occ_status occ_route_topk_ws(const occ_layer_desc *desc, const void *x, const float *w_router,
                             int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  const int64_t Td = (int64_t)desc->T * desc->d, Tk = (int64_t)desc->T * desc->k;
  if (missing(x, Td) || !w_router || missing(topk_idx, Tk) || missing(topk_w, Tk))
    return fail(OCC_EINVAL, "x, w_router, topk_idx and topk_w must be set");
  if (!occ::route_filter_applies(*desc))
    return hip_status(
        occ::launch_route_topk(*desc, x, w_router, topk_idx, topk_w, nullptr, stream),
        "occ_route_topk_ws");
  const size_t need = occ::route_filter_workspace_bytes(*desc);
  if (ws == nullptr) return fail(OCC_EINVAL, "workspace is NULL");
  if (ws_bytes < need)
    return fail(OCC_ENOSPC, "workspace of %zu bytes < %zu required", ws_bytes, need);
  return hip_status(
      occ::launch_route_filtered(*desc, x, w_router, topk_idx, topk_w, ws, stream),
      "occ_route_topk_ws");
}

static occ_status build_brim(const char *name, const occ_layer_desc *desc,
                             const int32_t *topk_idx, const float *topk_w,
                             const int32_t *slot_expert_host, const occ_brim *brim, void *ws,
                             size_t ws_bytes, hipStream_t stream, int32_t budget,
                             int32_t rescale) {
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, true));
  const int64_t Tk = (int64_t)desc->T * desc->k;
  if (missing(topk_idx, Tk) || missing(topk_w, Tk))
    return fail(OCC_EINVAL, "topk_idx and topk_w must be set");
  occ::Placement pl;
  OCC_TRY(make_placement(*desc, slot_expert_host, pl));
  const size_t need = occ::brim_workspace_bytes(desc->T, desc->D, desc->E);
  if (ws == nullptr) return fail(OCC_EINVAL, "workspace is NULL");
  if (ws_bytes < need)
    return fail(OCC_ENOSPC, "workspace of %zu bytes < %zu required", ws_bytes, need);
  return hip_status(occ::launch_build_brim(*desc, topk_idx, topk_w, pl, *brim, ws, stream,
                                           budget, rescale),
                    name);
}

occ_status occ_build_brim(const occ_layer_desc *desc, const int32_t *topk_idx,
                          const float *topk_w, const int32_t *slot_expert_host,
                          const occ_brim *brim, void *ws, size_t ws_bytes, hipStream_t stream) {
  return build_brim("occ_build_brim", desc, topk_idx, topk_w, slot_expert_host, brim, ws,
                    ws_bytes, stream, OCC_MAX_D, 0);
}

occ_status occ_build_brim_noalloc(const occ_layer_desc *desc, const int32_t *topk_idx,
                                  const float *topk_w, const int32_t *slot_expert_host,
                                  const occ_brim *brim, hipStream_t stream) {
  // the same checks as occ_build_brim, then the library's fixed array as
  // the workspace; nothing is allocated
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, true));
  const int64_t Tk = (int64_t)desc->T * desc->k;
  if (missing(topk_idx, Tk) || missing(topk_w, Tk))
    return fail(OCC_EINVAL, "topk_idx and topk_w must be set");
  occ::Placement pl;
  OCC_TRY(make_placement(*desc, slot_expert_host, pl));
  const size_t need = occ::brim_workspace_bytes(desc->T, desc->D, desc->E);
  if (need > occ::kBrimScratchBytes)
    return fail(OCC_EUNSUP, "occ_build_brim_noalloc: the layer needs %zu bytes of workspace, "
                "more than the %zu of its fixed array (use occ_build_brim)", need,
                occ::kBrimScratchBytes);
  void *ws = nullptr;
  const hipError_t e = occ::brim_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "occ_build_brim_noalloc (scratch address)");
  return hip_status(occ::launch_build_brim(*desc, topk_idx, topk_w, pl, *brim, ws, stream,
                                           OCC_MAX_D, 0),
                    "occ_build_brim_noalloc");
}

occ_status occ_build_brim_pruned(const occ_layer_desc *desc, const int32_t *topk_idx,
                                 const float *topk_w, const int32_t *slot_expert_host,
                                 int32_t budget, int32_t rescale, const occ_brim *brim, void *ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (desc != nullptr && (budget < 1 || budget > desc->D))
    return fail(OCC_EINVAL, "budget %d outside 1..D", budget);
  if (rescale != 0 && rescale != 1) return fail(OCC_EINVAL, "rescale must be 0 or 1");
  return build_brim("occ_build_brim_pruned", desc, topk_idx, topk_w, slot_expert_host, brim, ws,
                    ws_bytes, stream, budget, rescale);
}

occ_status occ_dispatch(const occ_layer_desc *desc, const void *x, const occ_brim *brim,
                        void *sfd, void *epd, hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const int64_t Td = (int64_t)desc->T * desc->d;
  if (missing(x, Td) || missing(sfd, s_max(*desc)) || missing(epd, Td * desc->k))
    return fail(OCC_EINVAL, "x, sfd and epd must be set");
  return hip_status(occ::launch_dispatch(*desc, x, *brim, sfd, epd, stream), "occ_dispatch");
}

occ_status occ_dispatch_direct(const occ_layer_desc *desc, const void *x, const occ_brim *brim,
                               void *epd, hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const int64_t Td = (int64_t)desc->T * desc->d;
  if (missing(x, Td) || missing(epd, Td * desc->k))
    return fail(OCC_EINVAL, "x and epd must be set");
  return hip_status(occ::launch_dispatch(*desc, x, *brim, nullptr, epd, stream),
                    "occ_dispatch_direct");
}

// Shared-expert pointers: all set when n_shared > 0, all NULL otherwise.
static occ_status check_shared_args(const occ_layer_desc &L, std::initializer_list<const void *> ps,
                                    const char *names) {
  for (const void *p : ps) {
    if (L.n_shared > 0 && p == nullptr) return fail(OCC_EINVAL, "n_shared > 0 needs %s", names);
    if (L.n_shared == 0 && p != nullptr)
      return fail(OCC_EINVAL, "n_shared == 0 but %s given", names);
  }
  return OCC_OK;
}

occ_status occ_expert_up(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                         const int32_t *slot_expert_host, const void *w_gate_up, void *h_ws,
                         size_t h_ws_bytes, const void *x, const void *w_gate_up_sh,
                         hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const occ_layer_desc &L = *desc;
  const int64_t Rd = (int64_t)L.T * L.k * L.d;
  if (missing(epd, Rd) || !w_gate_up || missing(h_ws, (int64_t)(h_bytes(L) + h_sh_bytes(L))))
    return fail(OCC_EINVAL, "epd, w_gate_up and h_ws must be set");
  OCC_TRY(check_shared_args(L, {x, w_gate_up_sh}, "x and w_gate_up_sh"));
  if (h_ws_bytes < h_bytes(L) + h_sh_bytes(L))
    return fail(OCC_ENOSPC, "h workspace of %zu bytes < %zu required", h_ws_bytes,
                h_bytes(L) + h_sh_bytes(L));
  occ::Placement pl;
  OCC_TRY(make_placement(L, slot_expert_host, pl));
  char *h = static_cast<char *>(h_ws);
  return hip_status(occ::launch_expert_up(L, epd, brim->slot_offset, pl, w_gate_up, h, x,
                                          w_gate_up_sh, h + h_bytes(L), stream),
                    "occ_expert_up");
}

occ_status occ_expert_down(const occ_layer_desc *desc, const occ_brim *brim,
                           const int32_t *slot_expert_host, const void *w_down,
                           const void *h_ws, size_t h_ws_bytes, void *out_epd,
                           const void *w_down_sh, void *shared_out, hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const occ_layer_desc &L = *desc;
  const int64_t Rd = (int64_t)L.T * L.k * L.d;
  if (!w_down || missing(h_ws, (int64_t)(h_bytes(L) + h_sh_bytes(L))) || missing(out_epd, Rd))
    return fail(OCC_EINVAL, "w_down, h_ws and out_epd must be set");
  OCC_TRY(check_shared_args(L, {w_down_sh, shared_out}, "w_down_sh and shared_out"));
  if (h_ws_bytes < h_bytes(L) + h_sh_bytes(L))
    return fail(OCC_ENOSPC, "h workspace of %zu bytes < %zu required", h_ws_bytes,
                h_bytes(L) + h_sh_bytes(L));
  occ::Placement pl;
  OCC_TRY(make_placement(L, slot_expert_host, pl));
  const char *h = static_cast<const char *>(h_ws);
  return hip_status(occ::launch_expert_down(L, brim->slot_offset, pl, w_down, h, out_epd,
                                            w_down_sh, h + h_bytes(L), shared_out, stream),
                    "occ_expert_down");
}

occ_status occ_expert_ffn(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                          const int32_t *slot_expert_host, const void *w_gate_up,
                          const void *w_down, void *h_ws, size_t h_ws_bytes, void *out_epd,
                          const void *x, const void *w_gate_up_sh, const void *w_down_sh,
                          void *shared_out, hipStream_t stream) {
  // validate both halves before launching either
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const occ_layer_desc &L = *desc;
  const int64_t Rd = (int64_t)L.T * L.k * L.d;
  if (missing(epd, Rd) || !w_gate_up || !w_down ||
      missing(h_ws, (int64_t)(h_bytes(L) + h_sh_bytes(L))) || missing(out_epd, Rd))
    return fail(OCC_EINVAL, "epd, w_gate_up, w_down, h_ws and out_epd must be set");
  OCC_TRY(check_shared_args(L, {x, w_gate_up_sh, w_down_sh, shared_out},
                            "x, w_gate_up_sh, w_down_sh and shared_out"));
  if (h_ws_bytes < h_bytes(L) + h_sh_bytes(L))
    return fail(OCC_ENOSPC, "h workspace of %zu bytes < %zu required", h_ws_bytes,
                h_bytes(L) + h_sh_bytes(L));
  occ::Placement pl;
  OCC_TRY(make_placement(L, slot_expert_host, pl));
  char *h = static_cast<char *>(h_ws);
  hipError_t e = occ::launch_expert_up(L, epd, brim->slot_offset, pl, w_gate_up, h, x,
                                       w_gate_up_sh, h + h_bytes(L), stream);
  if (e != hipSuccess) return hip_status(e, "occ_expert_ffn (up)");
  return hip_status(occ::launch_expert_down(L, brim->slot_offset, pl, w_down, h, out_epd,
                                            w_down_sh, h + h_bytes(L), shared_out, stream),
                    "occ_expert_ffn (down)");
}

occ_status occ_combine(const occ_layer_desc *desc, const void *out_epd, const occ_brim *brim,
                       const void *shared_out, void *out_sfd, void *y, hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const int64_t Td = (int64_t)desc->T * desc->d;
  if (missing(brim->epd_w, (int64_t)desc->T * desc->k))
    return fail(OCC_EINVAL, "brim->epd_w must be set");
  if (missing(out_epd, Td * desc->k) || missing(out_sfd, s_max(*desc)) || missing(y, Td))
    return fail(OCC_EINVAL, "out_epd, out_sfd and y must be set");
  return hip_status(occ::launch_combine(*desc, out_epd, *brim, shared_out, out_sfd, y, stream),
                    "occ_combine");
}

occ_status occ_combine_direct(const occ_layer_desc *desc, const void *out_epd, const occ_brim *brim,
                              const void *shared_out, void *y, hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const int64_t Td = (int64_t)desc->T * desc->d;
  if (missing(brim->epd_w, (int64_t)desc->T * desc->k))
    return fail(OCC_EINVAL, "brim->epd_w must be set");
  if (missing(out_epd, Td * desc->k) || missing(y, Td))
    return fail(OCC_EINVAL, "out_epd and y must be set");
  return hip_status(occ::launch_combine(*desc, out_epd, *brim, shared_out, nullptr, y, stream),
                    "occ_combine_direct");
}

occ_status occ_coactivation(const occ_layer_desc *desc, const int32_t *topk_idx,
                            int32_t *counts, int32_t accumulate, hipStream_t stream) {
  OCC_TRY(check_desc(desc));
  if (missing(topk_idx, (int64_t)desc->T * desc->k) || !counts)
    return fail(OCC_EINVAL, "topk_idx and counts must be set");
  if (accumulate != 0 && accumulate != 1) return fail(OCC_EINVAL, "accumulate must be 0 or 1");
  return hip_status(occ::launch_coactivation(*desc, topk_idx, counts, accumulate, stream),
                    "occ_coactivation");
}

// ---- backward -------------------------------------------------------------
static occ_status check_backward(const occ_layer_desc *desc) {
  OCC_TRY(check_desc(desc));
  // [G | U] and [dG | dU] (R x 2I bf16, and T x n_shared 2 I_shared for the
  // shared experts) are GEMM operands addressed with 32-bit byte offsets,
  // like every operand check_desc bounds
  if (desc->dtype == OCC_BF16 &&
      ((int64_t)desc->T * desc->k * 2 * desc->I * 2 > 0xffffffffll ||
       (int64_t)desc->T * desc->n_shared * 2 * desc->I_shared * 2 > 0xffffffffll))
    return fail(OCC_EUNSUP, "the backward's [G | U] rows exceed 4 GiB");
  return OCC_OK;
}

// The pair that keeps [G | U] runs the routed bf16 experts only.
static occ_status check_keep(const occ_layer_desc *desc) {
  OCC_TRY(check_backward(desc));
  if (desc->dtype != OCC_BF16)
    return fail(OCC_EUNSUP, "kept pre-activations are for bf16 layers");
  if (desc->n_shared != 0)
    return fail(OCC_EUNSUP, "kept pre-activations are for layers without shared experts");
  return OCC_OK;
}

static size_t gu_bytes(const occ_layer_desc &L) {
  return align256((size_t)L.T * L.k * 2 * L.I * elem_bytes(L));
}
static size_t gu_sh_bytes(const occ_layer_desc &L) {
  return align256((size_t)L.T * L.n_shared * 2 * L.I_shared * elem_bytes(L));
}

size_t occ_backward_workspace_bytes(const occ_layer_desc *desc) {
  if (check_backward(desc) != OCC_OK) return 0;
  return std::max(std::max(2 * gu_bytes(*desc), 2 * gu_sh_bytes(*desc)),
                  occ::router_backward_ws_bytes(*desc));
}

occ_status occ_grad_combine(const occ_layer_desc *desc, const void *dy, const occ_brim *brim,
                            const void *out_epd, void *d_out_sfd, void *d_out_epd, float *dw_epd,
                            hipStream_t stream) {
  OCC_TRY(check_backward(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const int64_t Td = (int64_t)desc->T * desc->d, Rk = (int64_t)desc->T * desc->k;
  if (missing(brim->epd_w, Rk)) return fail(OCC_EINVAL, "brim->epd_w must be set");
  if (missing(dy, Td) || missing(out_epd, Td * desc->k) || missing(d_out_epd, Td * desc->k) ||
      missing(dw_epd, Rk))
    return fail(OCC_EINVAL, "dy, out_epd, d_out_epd and dw_epd must be set");
  return hip_status(occ::launch_grad_combine(*desc, dy, *brim, out_epd, d_out_sfd, d_out_epd,
                                             dw_epd, stream),
                    "occ_grad_combine");
}

occ_status occ_expert_backward(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                               const int32_t *slot_expert_host, const void *w_gate_up,
                               const void *w_down, const void *h_ws, size_t h_ws_bytes,
                               const void *d_out_epd, void *bwd_ws, size_t bwd_ws_bytes,
                               void *d_epd, float *dw_gate_up, float *dw_down,
                               hipStream_t stream) {
  OCC_TRY(check_backward(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const occ_layer_desc &L = *desc;
  const int64_t Rd = (int64_t)L.T * L.k * L.d;
  if (missing(epd, Rd) || !w_gate_up || !w_down || missing(d_out_epd, Rd) || missing(d_epd, Rd) ||
      !dw_gate_up || !dw_down || missing(h_ws, (int64_t)h_bytes(L)) ||
      missing(bwd_ws, (int64_t)(2 * gu_bytes(L))))
    return fail(OCC_EINVAL, "expert backward: an operand is NULL");
  if (h_ws_bytes < h_bytes(L))
    return fail(OCC_ENOSPC, "h workspace of %zu bytes < %zu", h_ws_bytes, h_bytes(L));
  if (bwd_ws_bytes < 2 * gu_bytes(L))
    return fail(OCC_ENOSPC, "backward workspace of %zu bytes < %zu", bwd_ws_bytes,
                2 * gu_bytes(L));
  occ::Placement pl;
  OCC_TRY(make_placement(L, slot_expert_host, pl));
  char *ws = static_cast<char *>(bwd_ws);
  return hip_status(occ::launch_expert_backward(L, brim->slot_offset, pl, epd, w_gate_up, w_down,
                                                h_ws, d_out_epd, ws, ws + gu_bytes(L), d_epd,
                                                dw_gate_up, dw_down, stream),
                    "occ_expert_backward");
}

occ_status occ_expert_ffn_keep(const occ_layer_desc *desc, const void *epd, const occ_brim *brim,
                               const int32_t *slot_expert_host, const void *w_gate_up,
                               const void *w_down, void *h_ws, size_t h_ws_bytes, void *gu,
                               void *out_epd, hipStream_t stream) {
  OCC_TRY(check_keep(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const occ_layer_desc &L = *desc;
  const int64_t Rd = (int64_t)L.T * L.k * L.d;
  if (missing(epd, Rd) || !w_gate_up || !w_down || missing(h_ws, (int64_t)h_bytes(L)) ||
      missing(gu, (int64_t)gu_bytes(L)) || missing(out_epd, Rd))
    return fail(OCC_EINVAL, "epd, w_gate_up, w_down, h_ws, gu and out_epd must be set");
  if (h_ws_bytes < h_bytes(L))
    return fail(OCC_ENOSPC, "h workspace of %zu bytes < %zu required", h_ws_bytes, h_bytes(L));
  occ::Placement pl;
  OCC_TRY(make_placement(L, slot_expert_host, pl));
  char *h = static_cast<char *>(h_ws);
  hipError_t e = occ::launch_expert_up(L, epd, brim->slot_offset, pl, w_gate_up, h, nullptr,
                                       nullptr, nullptr, stream, gu);
  if (e != hipSuccess) return hip_status(e, "occ_expert_ffn_keep (up)");
  return hip_status(occ::launch_expert_down(L, brim->slot_offset, pl, w_down, h, out_epd,
                                            nullptr, nullptr, nullptr, stream),
                    "occ_expert_ffn_keep (down)");
}

occ_status occ_expert_backward_kept(const occ_layer_desc *desc, const void *epd,
                                    const occ_brim *brim, const int32_t *slot_expert_host,
                                    const void *w_gate_up, const void *w_down, const void *h_ws,
                                    size_t h_ws_bytes, const void *gu, const void *d_out_epd,
                                    void *bwd_ws, size_t bwd_ws_bytes, void *d_epd,
                                    float *dw_gate_up, float *dw_down, hipStream_t stream) {
  OCC_TRY(check_keep(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const occ_layer_desc &L = *desc;
  const int64_t Rd = (int64_t)L.T * L.k * L.d;
  if (missing(epd, Rd) || !w_gate_up || !w_down || missing(d_out_epd, Rd) || missing(d_epd, Rd) ||
      !dw_gate_up || !dw_down || missing(h_ws, (int64_t)h_bytes(L)) ||
      missing(gu, (int64_t)gu_bytes(L)) || missing(bwd_ws, (int64_t)(2 * gu_bytes(L))))
    return fail(OCC_EINVAL, "expert backward: an operand is NULL");
  if (h_ws_bytes < h_bytes(L))
    return fail(OCC_ENOSPC, "h workspace of %zu bytes < %zu", h_ws_bytes, h_bytes(L));
  if (bwd_ws_bytes < 2 * gu_bytes(L))
    return fail(OCC_ENOSPC, "backward workspace of %zu bytes < %zu", bwd_ws_bytes,
                2 * gu_bytes(L));
  occ::Placement pl;
  OCC_TRY(make_placement(L, slot_expert_host, pl));
  char *ws = static_cast<char *>(bwd_ws);
  return hip_status(occ::launch_expert_backward(L, brim->slot_offset, pl, epd, w_gate_up, w_down,
                                                h_ws, d_out_epd, const_cast<void *>(gu),
                                                ws + gu_bytes(L), d_epd, dw_gate_up, dw_down,
                                                stream, false),
                    "occ_expert_backward_kept");
}

occ_status occ_router_backward(const occ_layer_desc *desc, const void *x, const float *w_router,
                               const float *logits, const int32_t *topk_idx,
                               const float *topk_w, const int32_t *slot_expert_host,
                               const occ_brim *brim, const float *dw_epd, float *dlogits,
                               float *dx_router, float *dw_router, void *bwd_ws,
                               size_t bwd_ws_bytes, hipStream_t stream) {
  OCC_TRY(check_backward(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const occ_layer_desc &L = *desc;
  const int64_t T = L.T, Tk = T * L.k;
  if (missing(x, T * L.d) || !w_router || missing(logits, T * L.E) || missing(topk_idx, Tk) ||
      missing(topk_w, Tk) || missing(dw_epd, Tk) || missing(dlogits, T * L.E) ||
      missing(dx_router, T * L.d) || !dw_router)
    return fail(OCC_EINVAL, "router backward: an operand is NULL");
  const size_t need = occ::router_backward_ws_bytes(L);
  if (need > 0 && (bwd_ws == nullptr || bwd_ws_bytes < need))
    return fail(OCC_ENOSPC, "router backward: workspace of %zu bytes, need %zu", bwd_ws_bytes,
                need);
  occ::Placement pl;
  OCC_TRY(make_placement(L, slot_expert_host, pl));
  return hip_status(occ::launch_router_backward(L, pl, x, w_router, logits, topk_idx, topk_w, *brim,
                                                dw_epd, dlogits, dx_router, dw_router, bwd_ws,
                                                stream),
                    "occ_router_backward");
}

occ_status occ_shared_backward(const occ_layer_desc *desc, const void *x,
                               const void *w_gate_up_sh, const void *w_down_sh, const void *h_ws,
                               size_t h_ws_bytes, const void *dy, void *bwd_ws,
                               size_t bwd_ws_bytes, void *dx_shared, float *dw_gate_up_sh,
                               float *dw_down_sh, hipStream_t stream) {
  OCC_TRY(check_backward(desc));
  const occ_layer_desc &L = *desc;
  if (L.n_shared == 0) return fail(OCC_EINVAL, "occ_shared_backward: the layer has no shared experts");
  const int64_t Td = (int64_t)L.T * L.d;
  if (missing(x, Td) || !w_gate_up_sh || !w_down_sh || missing(dy, Td) ||
      missing(dx_shared, Td) || !dw_gate_up_sh || !dw_down_sh ||
      missing(h_ws, (int64_t)(h_bytes(L) + h_sh_bytes(L))) ||
      missing(bwd_ws, (int64_t)(2 * gu_sh_bytes(L))))
    return fail(OCC_EINVAL, "shared backward: an operand is NULL");
  if (h_ws_bytes < h_bytes(L) + h_sh_bytes(L))
    return fail(OCC_ENOSPC, "h workspace of %zu bytes < %zu", h_ws_bytes,
                h_bytes(L) + h_sh_bytes(L));
  if (bwd_ws_bytes < 2 * gu_sh_bytes(L))
    return fail(OCC_ENOSPC, "backward workspace of %zu bytes < %zu", bwd_ws_bytes,
                2 * gu_sh_bytes(L));
  char *ws = static_cast<char *>(bwd_ws);
  const char *h = static_cast<const char *>(h_ws);
  return hip_status(occ::launch_shared_backward(L, x, w_gate_up_sh, w_down_sh, h + h_bytes(L), dy,
                                                ws, ws + gu_sh_bytes(L), dx_shared,
                                                dw_gate_up_sh, dw_down_sh, stream),
                    "occ_shared_backward");
}

occ_status occ_grad_dispatch(const occ_layer_desc *desc, const void *d_epd, const occ_brim *brim,
                             const float *dx_router, const void *dx_shared, void *d_sfd, void *dx,
                             hipStream_t stream) {
  OCC_TRY(check_backward(desc));
  OCC_TRY(check_brim(*desc, brim, false));
  const int64_t Td = (int64_t)desc->T * desc->d;
  if (missing(d_epd, Td * desc->k) || missing(d_sfd, s_max(*desc)) || missing(dx, Td))
    return fail(OCC_EINVAL, "d_epd, d_sfd and dx must be set");
  OCC_TRY(check_shared_args(*desc, {dx_shared}, "dx_shared"));
  return hip_status(occ::launch_grad_dispatch(*desc, d_epd, *brim, dx_router, dx_shared, d_sfd, dx,
                                              stream),
                    "occ_grad_dispatch");
}

// ---- cross-layer affinity -------------------------------------------------
static occ_status check_routing(const char *what, int32_t T, int32_t k, int32_t E,
                                const int32_t *idx) {
  if (T < 0 || k < 1 || E < 1 || k > E) return fail(OCC_EINVAL, "%s: bad T=%d k=%d E=%d", what, T, k, E);
  if (E > OCC_MAX_E || k > OCC_MAX_K)
    return fail(OCC_EUNSUP, "%s: E=%d or k=%d beyond the supported maximum", what, E, k);
  if ((int64_t)T * k > INT32_MAX) return fail(OCC_EUNSUP, "%s: T*k beyond int32", what);
  if (T > 0 && idx == nullptr) return fail(OCC_EINVAL, "%s: selections are NULL", what);
  return OCC_OK;
}

static occ_status make_device_of(int32_t E, int32_t D, const int32_t *slot_expert_host,
                                 occ::DeviceOf &dv) {
  if (D < 1 || E % D != 0) return fail(OCC_EINVAL, "bad E=%d D=%d", E, D);
  if (D > OCC_MAX_D) return fail(OCC_EUNSUP, "D=%d beyond %d", D, OCC_MAX_D);
  if (slot_expert_host == nullptr) return fail(OCC_EINVAL, "slot_expert_host is NULL");
  const int L = E / D;
  for (int i = 0; i < OCC_MAX_E; ++i) dv.dev[i] = -1;
  for (int g = 0; g < E; ++g) {
    const int e = slot_expert_host[g];
    if (e < 0 || e >= E || dv.dev[e] != -1)
      return fail(OCC_EINVAL, "slot_expert is not a permutation of 0..%d (slot %d -> %d)",
                  E - 1, g, e);
    dv.dev[e] = (int8_t)(g / L);
  }
  return OCC_OK;
}

occ_status occ_cross_coactivation(int32_t T, int32_t k1, int32_t E1, const int32_t *idx1,
                                  int32_t k2, int32_t E2, const int32_t *idx2, int32_t *counts,
                                  int32_t accumulate, hipStream_t stream) {
  OCC_TRY(check_routing("first layer", T, k1, E1, idx1));
  OCC_TRY(check_routing("second layer", T, k2, E2, idx2));
  if (counts == nullptr) return fail(OCC_EINVAL, "counts is NULL");
  if (accumulate != 0 && accumulate != 1) return fail(OCC_EINVAL, "accumulate must be 0 or 1");
  return hip_status(occ::launch_cross_coactivation(T, k1, E1, idx1, k2, E2, idx2, counts,
                                                   accumulate, stream),
                    "occ_cross_coactivation");
}

occ_status occ_home_device(int32_t T, int32_t k1, int32_t E1, const int32_t *idx1, int32_t E2,
                           int32_t D, const int32_t *slot_expert2_host, const int32_t *affinity,
                           int32_t *home, hipStream_t stream) {
  OCC_TRY(check_routing("first layer", T, k1, E1, idx1));
  if (E2 < 1 || E2 > OCC_MAX_E) return fail(E2 < 1 ? OCC_EINVAL : OCC_EUNSUP, "bad E2=%d", E2);
  occ::DeviceOf dv;
  OCC_TRY(make_device_of(E2, D, slot_expert2_host, dv));
  if (affinity == nullptr || (T > 0 && home == nullptr))
    return fail(OCC_EINVAL, "affinity and home must be set");
  return hip_status(occ::launch_home_device(T, k1, E1, idx1, E2, D, dv, affinity, home, stream),
                    "occ_home_device");
}

occ_status occ_local_hits(int32_t T, int32_t k2, int32_t E2, const int32_t *idx2, int32_t D,
                          const int32_t *slot_expert2_host, const int32_t *home, int32_t *hits,
                          int32_t accumulate, hipStream_t stream) {
  OCC_TRY(check_routing("second layer", T, k2, E2, idx2));
  occ::DeviceOf dv;
  OCC_TRY(make_device_of(E2, D, slot_expert2_host, dv));
  if (hits == nullptr || (T > 0 && home == nullptr))
    return fail(OCC_EINVAL, "home and hits must be set");
  if (accumulate != 0 && accumulate != 1) return fail(OCC_EINVAL, "accumulate must be 0 or 1");
  return hip_status(occ::launch_local_hits(T, k2, E2, idx2, dv, home, hits, accumulate, stream),
                    "occ_local_hits");
}

occ_status occ_place_greedy(int32_t E, int32_t D, const int32_t *counts_host,
                            int32_t *slot_expert_host) {
  if (E <= 0 || D <= 0 || E % D != 0) return fail(OCC_EINVAL, "bad E=%d D=%d", E, D);
  if (!counts_host || !slot_expert_host) return fail(OCC_EINVAL, "NULL counts or output");
  const int L = E / D;
  std::vector<char> placed(E, 0);
  std::vector<int64_t> affinity(E);
  auto n_of = [&](int e) { return counts_host[(size_t)e * E + e]; };
  for (int dv = 0; dv < D; ++dv) {
    // seed: most tokens, lower index on ties
    int seed = -1;
    for (int e = 0; e < E; ++e)
      if (!placed[e] && (seed < 0 || n_of(e) > n_of(seed))) seed = e;
    placed[seed] = 1;
    slot_expert_host[dv * L] = seed;
    for (int e = 0; e < E; ++e) affinity[e] = counts_host[(size_t)e * E + seed];
    for (int l = 1; l < L; ++l) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (placed[e]) continue;
        if (best < 0 || affinity[e] > affinity[best] ||
            (affinity[e] == affinity[best] && n_of(e) > n_of(best)))
          best = e;
      }
      placed[best] = 1;
      slot_expert_host[dv * L + l] = best;
      for (int e = 0; e < E; ++e) affinity[e] += counts_host[(size_t)e * E + best];
    }
  }
  return ok();
}

}  // extern "C"
