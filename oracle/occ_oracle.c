/*
 * occ_oracle.c -- plain, slow, single-threaded CPU oracle of the
 * collaboration-aware MoE layer step (Occult), TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The HIP path never does, and no code is shared with
 * it.  Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (FMAs only where written as fmaf; no flush of denormals).
 *
 * Sources, cited by page and passage:
 *  [OCC-TLDR]   Occult (arXiv 2505.13345), sciencestack.ai page, TL;DR:
 *               BRIM data structures, three token states, expert placement
 *               rescheduling, all-to-all budget C_T.
 *  [OCC-ABS]    same page, Abstract: experts co-activated by one token are
 *               "collaborated"; intra- vs inter-collaboration by device;
 *               Occult delivers exact results with reduced communication.
 *  [OCC-FIG4]   same page, Figure 4 caption: forward workflow over the token
 *               states ORI, SFD, EPD stored on HBM and guided by BRIMs.
 *  [OCC-FIG5]   same page, Figure 5 caption: BRIM_0 is [EP devices] x
 *               [ORI tokens]; BRIM_1 is [local experts per device] x
 *               [SFD tokens].
 *  [OCC-FIG2]   same page, Figure 2 caption: MoE workflows under three
 *               all-to-all strategies across expert-parallel devices (the
 *               plain one sends one row per (token, expert) pair).
 *  [EXF-ABS]    ExFlow (arXiv 2210.17223, bohrium.dp.tech page), Abstract:
 *               inter-layer expert affinity from the conditional statistics
 *               of a token's routing across layers.
 *  [CPL-ABS]    "Expert Coupling in MoE Pretraining" (readsearch.ai page),
 *               Abstract: each token is routed to k of E experts; a
 *               dispatcher that sends each token to each GPU once;
 *               correlated placement puts often co-selected experts on one
 *               GPU; neither changes routing nor expert parameters.
 *
 * Where the pages are silent the plainest reading is taken (all are listed
 * in the design notes): softmax routing over all E experts with selection on
 * the logits (ties: lower expert index first), logits as an in-order fp32 FMA
 * chain, SwiGLU experts without biases, SFD = one row per (token, device)
 * pair grouped by device in ascending token order, EPD = one row per
 * (token, expert) pair grouped by slot (device, local expert) in ascending
 * token order, BRIM entries = global row indices with -1 for "absent".
 *
 * Floating point: expert arithmetic in double; stored results rounded (ties
 * to even) to the layer dtype at the points the layer stores them.
 *
 * parity pins: see tests/test_oracle_*.py (every function here is pinned).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { DT_F32 = 0, DT_BF16 = 1 };

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ECHECK -2 /* an internal consistency check failed */

/* ---- storage helpers ---------------------------------------------------- */

/* Exact widening of a stored element (fp32, or bf16 given as its 16 bits). */
static float load_f32(const void *p, size_t i, int dt) {
  if (dt == DT_F32) return ((const float *)p)[i];
  uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a double to the nearest value of the layer dtype, ties to even.
 * bf16 keeps 8 significant bits and fp32's exponent range. */
static double round_dt(double v, int dt) {
  if (dt == DT_F32) return (double)(float)v;
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  (void)frexp(v, &e);          /* |v| in [2^(e-1), 2^e) */
  if (e < -125) e = -125;      /* below the smallest normal the spacing is 2^-133 */
  double q = ldexp(1.0, e - 8); /* spacing of bf16 values in that binade */
  return nearbyint(v / q) * q;  /* default rounding mode: nearest, ties to even */
}

/* out[i] = round_dt(in[i]) for an array (dt = 0 fp32, 1 bf16, 2 none). */
int orc_round_array(long n, int dt, const double *in, double *out) {
  if (n < 0) return ORC_EINVAL;
  for (long i = 0; i < n; ++i) out[i] = dt == 2 ? in[i] : round_dt(in[i], dt);
  return ORC_OK;
}

/* ---- O1-O3: routing ------------------------------------------------------
 * [CPL-ABS]: each token is routed to k of the E experts.  Softmax gate over
 * all E experts; selection on the logits (softmax is monotone). */

/* logits[t][e] = fp32 chain acc = fmaf(x[t][j], wr[e][j], acc), j = 0..d-1;
 * x stored in dt_x, the router in dt_w (both widened exactly to fp32). */
int orc_logits(int T, int d, int E, int dt_x, const void *x, int dt_w, const void *wr,
               float *logits) {
  if (T < 0 || d <= 0 || E <= 0 || !logits) return ORC_EINVAL;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int j = 0; j < d; ++j)
        acc = fmaf(load_f32(x, (size_t)t * d + j, dt_x), load_f32(wr, (size_t)e * d + j, dt_w),
                   acc);
      logits[(size_t)t * E + e] = acc;
    }
  return ORC_OK;
}

/* Selection key: NaN counts as -infinity. */
static float sel_key(float v) { return isnan(v) ? -INFINITY : v; }

/* Top-k by (logit descending, expert ascending), then softmax weights of the
 * chosen experts, computed in double over all E logits. */
int orc_topk(int T, int E, int k, int renorm, const float *logits, int32_t *idx, float *w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return ORC_EINVAL;
  char *taken = (char *)malloc((size_t)E);
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  if (!taken || !p) { free(taken); free(p); return ORC_EINVAL; }
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        /* strict ">" while scanning upward: the lower index keeps a tie */
        if (best < 0 || sel_key(l[e]) > sel_key(l[best])) best = e;
      }
      taken[best] = 1;
      idx[(size_t)t * k + j] = best;
    }
    double m = -INFINITY;
    for (int e = 0; e < E; ++e) if (sel_key(l[e]) > m) m = sel_key(l[e]);
    double z = 0.0;
    for (int e = 0; e < E; ++e) { p[e] = exp((double)l[e] - m); z += p[e]; }
    for (int e = 0; e < E; ++e) p[e] /= z;
    double sel = 0.0;
    for (int j = 0; j < k; ++j) sel += p[idx[(size_t)t * k + j]];
    for (int j = 0; j < k; ++j) {
      double v = p[idx[(size_t)t * k + j]];
      if (renorm) v /= sel;
      w[(size_t)t * k + j] = (float)v;
    }
  }
  free(taken);
  free(p);
  return ORC_OK;
}

/* ---- O4-O6: SFD / EPD layouts and the two BRIMs --------------------------
 * [OCC-FIG5] BRIM_0 [D][T] over ORI tokens, BRIM_1 [L][SFD tokens];
 * [CPL-ABS] each token is sent to each device once (SFD);
 * [OCC-FIG4] EPD is what the experts consume.
 * slot g = device * L + local; slot_expert[g] is the expert held there. */
int orc_brim(int T, int k, int E, int D, const int32_t *idx, const float *w,
             const int32_t *slot_expert, int32_t *brim0, int32_t *brim1, int ld,
             int32_t *sfd_offset, int32_t *slot_offset, int32_t *sfd_token,
             int32_t *epd_token, int32_t *epd_sfd, float *epd_w, int32_t *S_out) {
  if (T < 0 || k <= 0 || E <= 0 || D <= 0 || E % D != 0) return ORC_EINVAL;
  const int L = E / D;
  int32_t *dev_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!dev_of || !seen) { free(dev_of); free(seen); return ORC_EINVAL; }
  for (int g = 0; g < E; ++g) {
    int e = slot_expert[g];
    if (e < 0 || e >= E || seen[e]) { free(dev_of); free(seen); return ORC_EINVAL; }
    seen[e] = 1;
    dev_of[e] = g / L;
  }
  free(seen);
  if (ld < T * (k < D ? k : D)) { free(dev_of); return ORC_EINVAL; }

  /* SFD: device-major, ascending token inside a device */
  int32_t s = 0;
  for (int dv = 0; dv < D; ++dv) {
    sfd_offset[dv] = s;
    for (int t = 0; t < T; ++t) {
      int hit = 0;
      for (int j = 0; j < k; ++j) {
        int e = idx[(size_t)t * k + j];
        if (e >= 0 && dev_of[e] == dv) hit = 1;  /* e < 0: a pair dropped by pruning */
      }
      if (hit) {
        brim0[(size_t)dv * T + t] = s;
        sfd_token[s] = t;
        ++s;
      } else {
        brim0[(size_t)dv * T + t] = -1;
      }
    }
  }
  sfd_offset[D] = s;
  *S_out = s;
  const int32_t S = s;

  /* EPD: slot-major, ascending token inside a slot */
  for (int l = 0; l < L; ++l)
    for (int32_t c = 0; c < S; ++c) brim1[(size_t)l * ld + c] = -1;
  int32_t r = 0;
  for (int g = 0; g < E; ++g) {
    int e = slot_expert[g], dv = g / L, l = g % L;
    slot_offset[g] = r;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[(size_t)t * k + j] == e) {
          int32_t sc = brim0[(size_t)dv * T + t];
          brim1[(size_t)l * ld + sc] = r;
          epd_token[r] = t;
          epd_sfd[r] = sc;
          epd_w[r] = w[(size_t)t * k + j];
          ++r;
        }
  }
  slot_offset[E] = r;
  free(dev_of);
  /* dropless: one EPD row per selected pair, T*k unless pruning dropped some */
  int32_t pairs = 0;
  for (size_t q = 0; q < (size_t)T * k; ++q) pairs += idx[q] >= 0;
  return r == pairs ? ORC_OK : ORC_ECHECK;
}

/* ---- O5': routing-score-based collaboration pruning ------------------------
 * [OCC-TLDR]: pruning by routing score to minimise the all-to-all budget C_T.
 * The pages give no exact rule; the reading: each token is sent to at most
 * `budget` devices.  A device's score is the fp32 sum, in top-k order, of
 * the token's routing weights on experts it holds; devices are ranked by
 * score (descending, lower device index first) and the first `budget` kept.
 * Selections on other devices become idx = -1, w = 0.  With rescale, each
 * kept weight is multiplied by total / kept (fp32 sums in top-k order of all
 * and of the kept weights), so the token's gate mass is unchanged. */
int orc_prune(int T, int k, int E, int D, const int32_t *slot_expert, int budget, int rescale,
              const int32_t *idx, const float *w, int32_t *idx_out, float *w_out) {
  if (T < 0 || k <= 0 || E <= 0 || D <= 0 || E % D != 0 || budget < 1) return ORC_EINVAL;
  const int L = E / D;
  int32_t *dev_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  float *score = (float *)malloc(sizeof(float) * (size_t)D);
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)D);
  int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (size_t)D);
  if (!dev_of || !score || !order || !keep) {
    free(dev_of); free(score); free(order); free(keep);
    return ORC_EINVAL;
  }
  for (int g = 0; g < E; ++g) dev_of[slot_expert[g]] = g / L;
  for (int t = 0; t < T; ++t) {
    const int32_t *it = idx + (size_t)t * k;
    const float *wt = w + (size_t)t * k;
    int n = 0; /* the token's devices, in first-pick order */
    for (int dv = 0; dv < D; ++dv) { score[dv] = 0.0f; keep[dv] = 0; }
    for (int j = 0; j < k; ++j) {
      int dv = dev_of[it[j]];
      int seen = 0;
      for (int q = 0; q < n; ++q) if (order[q] == dv) seen = 1;
      if (!seen) order[n++] = dv;
      score[dv] = score[dv] + wt[j];
    }
    /* selection of the best `budget` devices: (score desc, device asc) */
    for (int c = 0; c < budget && c < n; ++c) {
      int best = -1;
      for (int q = 0; q < n; ++q) {
        int dv = order[q];
        if (keep[dv]) continue;
        if (best < 0 || score[dv] > score[best] || (score[dv] == score[best] && dv < best))
          best = dv;
      }
      keep[best] = 1;
    }
    float total = 0.0f, kept = 0.0f;
    for (int j = 0; j < k; ++j) {
      total = total + wt[j];
      if (keep[dev_of[it[j]]]) kept = kept + wt[j];
    }
    float scale = (rescale && kept > 0.0f) ? total / kept : 1.0f;
    for (int j = 0; j < k; ++j) {
      if (keep[dev_of[it[j]]]) {
        idx_out[(size_t)t * k + j] = it[j];
        w_out[(size_t)t * k + j] = rescale ? wt[j] * scale : wt[j];
      } else {
        idx_out[(size_t)t * k + j] = -1;
        w_out[(size_t)t * k + j] = 0.0f;
      }
    }
  }
  free(dev_of); free(score); free(order); free(keep);
  return ORC_OK;
}

/* ---- O8-O9: expert networks ---------------------------------------------
 * The pages say only "expert networks"; the layer uses SwiGLU without
 * biases: y = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + e^-z).
 * h is stored in the layer dtype before the down projection. */

/* yacc[c] += sum_i round(silu(a_i) * b_i) * Wd[c][i] for one input row. */
static void swiglu_accum(int d, int I, int dt, const void *xrow_base, size_t xoff,
                         const void *wgu, size_t gu_off, const void *wdn, size_t dn_off,
                         double *h, double *yacc) {
  for (int i = 0; i < I; ++i) {
    double a = 0.0, b = 0.0;
    for (int j = 0; j < d; ++j) {
      double xj = load_f32(xrow_base, xoff + j, dt);
      a += xj * load_f32(wgu, gu_off + (size_t)i * d + j, dt);
      b += xj * load_f32(wgu, gu_off + (size_t)(I + i) * d + j, dt);
    }
    double silu = a / (1.0 + exp(-a));
    h[i] = round_dt(silu * b, dt);
  }
  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += h[i] * load_f32(wdn, dn_off + (size_t)c * I + i, dt);
    yacc[c] += acc;
  }
}

/* out[n][d] = round(FFN_{ex[n]}(x[tok[n]])): routed expert rows.
 * wgu [E][2I][d], wdn [E][d][I]. */
int orc_expert_rows(int n, const int32_t *tok, const int32_t *ex, int d, int I, int dt,
                    const void *x, const void *wgu, const void *wdn, float *out) {
  if (n < 0 || d <= 0 || I <= 0) return ORC_EINVAL;
  double *h = (double *)malloc(sizeof(double) * (size_t)I);
  double *y = (double *)malloc(sizeof(double) * (size_t)d);
  if (!h || !y) { free(h); free(y); return ORC_EINVAL; }
  for (int r = 0; r < n; ++r) {
    for (int c = 0; c < d; ++c) y[c] = 0.0;
    swiglu_accum(d, I, dt, x, (size_t)tok[r] * d, wgu, (size_t)ex[r] * 2 * I * d, wdn,
                 (size_t)ex[r] * d * I, h, y);
    for (int c = 0; c < d; ++c) out[(size_t)r * d + c] = (float)round_dt(y[c], dt);
  }
  free(h);
  free(y);
  return ORC_OK;
}

/* Shared, always-active experts (weight 1): out = round(sum_s FFN_s(x)). */
int orc_shared_rows(int n, const int32_t *tok, int d, int I_sh, int n_sh, int dt,
                    const void *x, const void *wgu_sh, const void *wdn_sh, float *out) {
  if (n < 0 || d <= 0 || I_sh <= 0 || n_sh <= 0) return ORC_EINVAL;
  double *h = (double *)malloc(sizeof(double) * (size_t)I_sh);
  double *y = (double *)malloc(sizeof(double) * (size_t)d);
  if (!h || !y) { free(h); free(y); return ORC_EINVAL; }
  for (int r = 0; r < n; ++r) {
    for (int c = 0; c < d; ++c) y[c] = 0.0;
    for (int sg = 0; sg < n_sh; ++sg)
      swiglu_accum(d, I_sh, dt, x, (size_t)tok[r] * d, wgu_sh, (size_t)sg * 2 * I_sh * d,
                   wdn_sh, (size_t)sg * d * I_sh, h, y);
    for (int c = 0; c < d; ++c) out[(size_t)r * d + c] = (float)round_dt(y[c], dt);
  }
  free(h);
  free(y);
  return ORC_OK;
}

/* ---- O10-O11: pre-reduction and scatter back to ORI -----------------------
 * [OCC-FIG4]: results return over the same BRIMs.  For each requested token
 * t and each device holding it (s = BRIM_0[dv][t] >= 0):
 *   out_SFD[s] = round(sum_{l ascending, BRIM_1[l][s] >= 0} epd_w[r] out_EPD[r])
 * then Y[t] = round(shared[t] + sum_{dv ascending} out_SFD[s]).
 * out_epd rows are looked up through epd_row (r -> row, NULL = identity);
 * out_sfd rows are written through sfd_row (s -> row, NULL = identity; a
 * NULL out_sfd skips storing them).  shared is [ntok][d] or NULL. */
int orc_combine(int ntok, const int32_t *tok, int T, int D, int L, int ld, int d, int dt,
                const int32_t *brim0, const int32_t *brim1, const float *epd_w,
                const float *out_epd, const int32_t *epd_row, const float *shared,
                float *out_sfd, const int32_t *sfd_row, float *y) {
  if (ntok < 0 || d <= 0 || D <= 0 || L <= 0) return ORC_EINVAL;
  double *acc = (double *)malloc(sizeof(double) * (size_t)d);
  double *yt = (double *)malloc(sizeof(double) * (size_t)d);
  if (!acc || !yt) { free(acc); free(yt); return ORC_EINVAL; }
  int rc = ORC_OK;
  for (int q = 0; q < ntok && rc == ORC_OK; ++q) {
    int t = tok[q];
    if (t < 0 || t >= T) { rc = ORC_EINVAL; break; }
    for (int c = 0; c < d; ++c) yt[c] = shared ? (double)shared[(size_t)q * d + c] : 0.0;
    for (int dv = 0; dv < D; ++dv) {
      int32_t s = brim0[(size_t)dv * T + t];
      if (s < 0) continue;
      for (int c = 0; c < d; ++c) acc[c] = 0.0;
      for (int l = 0; l < L; ++l) {
        int32_t r = brim1[(size_t)l * ld + s];
        if (r < 0) continue;
        int32_t row = epd_row ? epd_row[r] : r;
        if (row < 0) { rc = ORC_ECHECK; break; }
        double wr = (double)epd_w[r];
        for (int c = 0; c < d; ++c) acc[c] += wr * (double)out_epd[(size_t)row * d + c];
      }
      for (int c = 0; c < d; ++c) {
        double v = round_dt(acc[c], dt);
        if (out_sfd) {
          int32_t srow = sfd_row ? sfd_row[s] : s;
          if (srow >= 0) out_sfd[(size_t)srow * d + c] = (float)v;
        }
        yt[c] += v;
      }
    }
    for (int c = 0; c < d; ++c) y[(size_t)q * d + c] = (float)round_dt(yt[c], dt);
  }
  free(acc);
  free(yt);
  return rc;
}

/* ---- O13: brute force, no deduplication ----------------------------------
 * The standard MoE layer: Y[t] = round(shared[t] + sum_j w[t][j] FFN_idx(x_t)),
 * with each FFN output rounded as the expert stores it.  [OCC-ABS] says the
 * Occult layouts give exact results, so they must agree with this. */
int orc_bruteforce(int ntok, const int32_t *tok, int d, int I, int k, int dt, const void *x,
                   const int32_t *idx, const float *w, const void *wgu, const void *wdn,
                   const float *shared, float *y) {
  if (ntok < 0 || d <= 0 || I <= 0 || k <= 0) return ORC_EINVAL;
  float *o = (float *)malloc(sizeof(float) * (size_t)d);
  double *yt = (double *)malloc(sizeof(double) * (size_t)d);
  if (!o || !yt) { free(o); free(yt); return ORC_EINVAL; }
  for (int q = 0; q < ntok; ++q) {
    int t = tok[q];
    for (int c = 0; c < d; ++c) yt[c] = shared ? (double)shared[(size_t)q * d + c] : 0.0;
    for (int j = 0; j < k; ++j) {
      int32_t e = idx[(size_t)t * k + j];
      if (e < 0) continue; /* a selection dropped by pruning */
      orc_expert_rows(1, &tok[q], &e, d, I, dt, x, wgu, wdn, o);
      double wj = (double)w[(size_t)t * k + j];
      for (int c = 0; c < d; ++c) yt[c] += wj * (double)o[c];
    }
    for (int c = 0; c < d; ++c) y[(size_t)q * d + c] = (float)round_dt(yt[c], dt);
  }
  free(o);
  free(yt);
  return ORC_OK;
}

/* ---- O10': conventional combine (no deduplication) ------------------------
 * [OCC-FIG2]: the plain strategy returns every (token, expert) row unreduced
 * and the source sums them.  For each requested token, in the same walk as
 * orc_combine (devices ascending, local experts ascending, rows found through
 * BRIM_0 and BRIM_1) but with no per-device rounding:
 *   y[t] = round_dtype(shared[t] + sum_r w[r] * out_epd[r])   (fp64 sum) */
int orc_combine_direct(int ntok, const int32_t *tok, int T, int D, int L, int ld, int d, int dt,
                       const int32_t *brim0, const int32_t *brim1, const float *epd_w,
                       const float *out_epd, const int32_t *epd_row, const float *shared,
                       float *y) {
  if (ntok < 0 || d <= 0 || D <= 0 || L <= 0) return ORC_EINVAL;
  double *yt = (double *)malloc(sizeof(double) * (size_t)d);
  if (!yt) return ORC_EINVAL;
  int rc = ORC_OK;
  for (int q = 0; q < ntok && rc == ORC_OK; ++q) {
    int t = tok[q];
    if (t < 0 || t >= T) { rc = ORC_EINVAL; break; }
    for (int c = 0; c < d; ++c) yt[c] = shared ? (double)shared[(size_t)q * d + c] : 0.0;
    for (int dv = 0; dv < D && rc == ORC_OK; ++dv) {
      int32_t s = brim0[(size_t)dv * T + t];
      if (s < 0) continue;
      for (int l = 0; l < L; ++l) {
        int32_t r = brim1[(size_t)l * ld + s];
        if (r < 0) continue;
        int32_t row = epd_row ? epd_row[r] : r;
        if (row < 0) { rc = ORC_ECHECK; break; }
        double wr = (double)epd_w[r];
        for (int c = 0; c < d; ++c) yt[c] += wr * (double)out_epd[(size_t)row * d + c];
      }
    }
    for (int c = 0; c < d; ++c) y[(size_t)q * d + c] = (float)round_dt(yt[c], dt);
  }
  free(yt);
  return rc;
}

/* ---- O12: co-activation (collaboration) counts ---------------------------
 * [OCC-ABS]: two experts co-activated by one token are "collaborated".
 * C[i][j] = #tokens selecting both i and j; the diagonal counts tokens per
 * expert.  accumulate = 0 starts from zero. */
int orc_coactivation(int T, int k, int E, const int32_t *idx, int32_t *C, int accumulate) {
  if (T < 0 || k <= 0 || E <= 0) return ORC_EINVAL;
  if (!accumulate) memset(C, 0, sizeof(int32_t) * (size_t)E * E);
  for (int t = 0; t < T; ++t)
    for (int a = 0; a < k; ++a)
      for (int b = 0; b < k; ++b)
        C[(size_t)idx[(size_t)t * k + a] * E + idx[(size_t)t * k + b]] += 1;
  return ORC_OK;
}

/* ---- O12': cross-layer co-activation, home devices, local hits ------------
 * [CPL-ABS]: the experts a token selects at one layer predict those at the
 * next; token shuffling moves each token to the GPU predicted to hold its
 * next-layer experts and raises the share of assignments served on the
 * token's GPU.  [EXF-ABS]: inter-layer expert affinity.
 *   A[i][j]  = #tokens choosing i at the first layer and j at the second
 *   home[t]  = argmax_d sum_{i in idx1[t]} sum_{j on device d} A[i][j]
 *              (lower d on equal sums)
 *   hits     = #(t, q) with device(idx2[t][q]) == home[t] */
int orc_cross_coactivation(int T, int k1, int E1, const int32_t *idx1, int k2, int E2,
                           const int32_t *idx2, int32_t *A) {
  if (T < 0 || k1 <= 0 || k2 <= 0 || E1 <= 0 || E2 <= 0) return ORC_EINVAL;
  memset(A, 0, sizeof(int32_t) * (size_t)E1 * E2);
  for (int t = 0; t < T; ++t)
    for (int a = 0; a < k1; ++a)
      for (int b = 0; b < k2; ++b)
        A[(size_t)idx1[(size_t)t * k1 + a] * E2 + idx2[(size_t)t * k2 + b]] += 1;
  return ORC_OK;
}

int orc_home_device(int T, int k1, int E1, const int32_t *idx1, int E2, int D,
                    const int32_t *slot_expert2, const int32_t *A, int32_t *home) {
  if (T < 0 || k1 <= 0 || E1 <= 0 || E2 <= 0 || D <= 0 || E2 % D != 0) return ORC_EINVAL;
  const int L = E2 / D;
  for (int t = 0; t < T; ++t) {
    int best = 0;
    long long best_sum = -1;
    for (int d = 0; d < D; ++d) {
      long long sum = 0;
      for (int l = 0; l < L; ++l) {
        int j = slot_expert2[d * L + l];
        for (int a = 0; a < k1; ++a) sum += A[(size_t)idx1[(size_t)t * k1 + a] * E2 + j];
      }
      if (sum > best_sum) { best_sum = sum; best = d; }
    }
    home[t] = best;
  }
  return ORC_OK;
}

int orc_local_hits(int T, int k2, int E2, const int32_t *idx2, int D, const int32_t *slot_expert2,
                   const int32_t *home, int64_t *hits) {
  if (T < 0 || k2 <= 0 || E2 <= 0 || D <= 0 || E2 % D != 0) return ORC_EINVAL;
  const int L = E2 / D;
  int64_t h = 0;
  for (int t = 0; t < T; ++t)
    for (int q = 0; q < k2; ++q) {
      int j = idx2[(size_t)t * k2 + q];
      int g = 0;
      while (slot_expert2[g] != j) ++g;
      if (g / L == home[t]) ++h;
    }
  *hits = h;
  return ORC_OK;
}

/* ---- O-P: greedy correlated placement ------------------------------------
 * [CPL-ABS] correlated placement puts experts often selected together on the
 * same GPU; [OCC-TLDR] expert placement rescheduling.  The pages give no
 * algorithm; this is the plain greedy: for each device in turn, seed with the
 * unassigned expert of largest n_e (= C[e][e]; ties: lower e), then add the
 * unassigned expert with the largest sum of counts to the device's experts
 * (ties: larger n_e, then lower e) until it holds L experts. */
int orc_greedy_placement(int E, int D, const int32_t *C, int32_t *slot_expert) {
  if (E <= 0 || D <= 0 || E % D != 0) return ORC_EINVAL;
  const int L = E / D;
  char *used = (char *)calloc((size_t)E, 1);
  if (!used) return ORC_EINVAL;
  for (int dv = 0; dv < D; ++dv) {
    int seed = -1;
    for (int e = 0; e < E; ++e) {
      if (used[e]) continue;
      if (seed < 0 || C[(size_t)e * E + e] > C[(size_t)seed * E + seed]) seed = e;
    }
    used[seed] = 1;
    slot_expert[dv * L] = seed;
    for (int l = 1; l < L; ++l) {
      int best = -1;
      long long best_aff = -1;
      for (int e = 0; e < E; ++e) {
        if (used[e]) continue;
        long long aff = 0;
        for (int m = 0; m < l; ++m) aff += C[(size_t)e * E + slot_expert[dv * L + m]];
        int better = best < 0 || aff > best_aff ||
                     (aff == best_aff && C[(size_t)e * E + e] > C[(size_t)best * E + best]);
        if (better) { best = e; best_aff = aff; }
      }
      used[best] = 1;
      slot_expert[dv * L + l] = best;
    }
  }
  free(used);
  return ORC_OK;
}

/* Intra-collaboration share of a placement ([OCC-ABS]): pairs i<j on one
 * device over all pairs i<j, counted with their co-activation counts. */
int orc_intra_share(int E, int D, const int32_t *C, const int32_t *slot_expert,
                    long long *intra, long long *total) {
  if (E <= 0 || D <= 0 || E % D != 0) return ORC_EINVAL;
  const int L = E / D;
  int32_t *dev = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  if (!dev) return ORC_EINVAL;
  for (int g = 0; g < E; ++g) dev[slot_expert[g]] = g / L;
  long long in = 0, all = 0;
  for (int i = 0; i < E; ++i)
    for (int j = i + 1; j < E; ++j) {
      all += C[(size_t)i * E + j];
      if (dev[i] == dev[j]) in += C[(size_t)i * E + j];
    }
  *intra = in;
  *total = all;
  free(dev);
  return ORC_OK;
}

/* Exposed so the tests can pin the dtype rounding by itself. */
double orc_round_dt(double v, int dt) { return round_dt(v, dt); }
