/*
 * ORACLE for the token-choice MoE FFN layer forward (one device's share, no
 * expert parallelism).  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may call it; the GPU library never does.
 * It shares no code, header or constant with the GPU path.
 *
 * Plain, slow, obviously correct: every floating-point quantity is accumulated
 * in binary64 in the order written below; there is no blocking and no fusion.
 *
 * Sources (web pages, cited by title and section):
 *   [EP]     "Expert-parallel MoE training" explainer (blog.vllbc.top,
 *            visual-reading): the router / capacity / drop section, its capacity
 *            calculator, and the walk through one MoE layer (dispatch, experts,
 *            unpermute, gate-weighted sum, residual) plus its memory calculator
 *            (gated FFN with gate / up / down matrices).
 *   [DS7508] DeepSpeed discussion #7508 "The MoE spends too much time on the gate
 *            network", first answer: capacity = ceil((tokens/experts)*cf*k) with
 *            the worked value 10,923.
 *   [SW]     Switch Transformers explainer ("AI 十大论文精讲（七）: Switch Routing"):
 *            §1.1 routing (logits = router weight times x, softmax, argmax,
 *            y = E_i(x) p_i(x)), §1.2 capacity and overflow through the residual,
 *            §2.1 selective precision (router input, logits and softmax in fp32),
 *            §2.3 expert FFN weights W_in / W_out.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - selection is on the fp32 logits, larger first, ties to the lower expert
 *     index; the k choices are ordered that way (choice r = 0 is the best);
 *   - capacity priority is choice-major: every token's first choice before any
 *     second choice, token order inside each ("position" policy of [EP]);
 *   - capacity is ceil(double(T*k) * cf / E), optionally raised to min_capacity;
 *   - a dropped assignment contributes nothing and the remaining gates are not
 *     renormalised; the residual carries a fully dropped token;
 *   - GELU is the exact erf form; SwiGLU is silu(x W_gate) * (x W_up) then W_down;
 *   - weights are stored [out_features, in_features] row-major:
 *     W1, W3: [E][F][H]; W2: [E][H][F]; the router Wg is [H][E] (x . Wg).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_SOFTMAX_TOPK = 0, OR_SOFTMAX_TOPK_RENORM = 1, OR_TOPK_SOFTMAX = 2 };
enum { OR_RELU = 0, OR_GELU = 1, OR_SWIGLU = 2 };
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };
enum { OR_DROP_POSITION = 0, OR_DROP_PROBS = 1 };
enum { OR_SECOND_ALWAYS = 0, OR_SECOND_RANDOM = 1 };

/* A bf16 number is the upper half of an IEEE binary32; its value is exact in binary64. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void *p, int dtype, int64_t i) {
  if (dtype == OR_BF16) return bf16_to_double(((const uint16_t *)p)[i]);
  return (double)((const float *)p)[i];
}

/* Capacity ([EP] router/capacity section: ceil((T*k/E)*cf); [DS7508]: 10,923 at
 * T=32768, E=12, k=4, cf=1).  Returns -1 for dropless (no capacity limit). */
int64_t oracle_capacity(int64_t T, int64_t k, int64_t E, double cf, int64_t min_capacity, int dropless) {
  if (dropless) return -1;
  double c = ceil((double)(T * k) * cf / (double)E);
  int64_t C = (int64_t)c;
  return C < min_capacity ? min_capacity : C;
}

/* Router logits ([EP] router: linear layer Wg in R^{HxE}; [SW] §1.1 h(x) = Wr x,
 * §2.1 fp32 router): l[t,e] = fl32(sum_h x[t,h]*Wg[h,e]  +  bias[e]), the sum in
 * binary64 over h ascending, rounded once to fp32.  bias may be NULL. */
void oracle_logits(int64_t T, int64_t H, int64_t E, int x_dtype, const void *x, const float *Wg,
                   const float *bias, float *logits) {
#pragma omp parallel
  {
    double *acc = (double *)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t e = 0; e < E; ++e) acc[e] = 0.0;
      for (int64_t h = 0; h < H; ++h) {
        double xv = elem(x, x_dtype, t * H + h);
        const float *w = Wg + h * E;
        for (int64_t e = 0; e < E; ++e) acc[e] += xv * (double)w[e];
      }
      for (int64_t e = 0; e < E; ++e)
        logits[t * E + e] = (float)(bias ? acc[e] + (double)bias[e] : acc[e]);
    }
    free(acc);
  }
}

/* Top-k selection for one token ([EP] router: top-k after scoring; [SW] §1.1
 * argmax for k=1): k rounds, each taking the largest remaining logit, the lower
 * index on equal values. */
static void select_topk(const float *l, int64_t E, int k, int32_t *idx) {
  for (int r = 0; r < k; ++r) {
    int32_t best = -1;
    for (int64_t e = 0; e < E; ++e) {
      int taken = 0;
      for (int j = 0; j < r; ++j) taken |= (idx[j] == (int32_t)e);
      if (taken) continue;
      if (best < 0 || l[e] > l[best]) best = (int32_t)e;
    }
    idx[r] = best;
  }
}

/* Gate values of the k choices ([EP] router: softmax then top-k, or top-k then
 * normalise over the selected; [SW] §1.1 p_i = exp(h_i)/sum_j exp(h_j)), binary64
 * from the fp32 logits, rounded once to fp32. */
static void gates(const float *l, int64_t E, int k, int mode, int score, const int32_t *idx, float *g) {
  if (score == OR_SIGMOID && mode != OR_TOPK_SOFTMAX) {
    /* sigmoid scores ([EP] router: softmax or sigmoid before the top-k): the chosen
     * scores themselves, or divided by their sum when renormalised */
    double sc[16], sum = 0.0;
    for (int r = 0; r < k; ++r) {
      sc[r] = 1.0 / (1.0 + exp(-(double)l[idx[r]]));
      sum += sc[r];
    }
    for (int r = 0; r < k; ++r) g[r] = (float)(mode == OR_SOFTMAX_TOPK ? sc[r] : sc[r] / sum);
    return;
  }
  double m = l[idx[0]]; /* the largest logit */
  if (mode == OR_TOPK_SOFTMAX) {
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += exp((double)l[idx[j]] - m);
    for (int r = 0; r < k; ++r) g[r] = (float)(exp((double)l[idx[r]] - m) / den);
    return;
  }
  double den = 0.0;
  for (int64_t e = 0; e < E; ++e) den += exp((double)l[e] - m);
  if (mode == OR_SOFTMAX_TOPK) {
    for (int r = 0; r < k; ++r) g[r] = (float)(exp((double)l[idx[r]] - m) / den);
    return;
  }
  /* OR_SOFTMAX_TOPK_RENORM: p over all E, then p of the chosen divided by their sum */
  double p[16], s = 0.0;
  for (int r = 0; r < k; ++r) {
    p[r] = exp((double)l[idx[r]] - m) / den;
    s += p[r];
  }
  for (int r = 0; r < k; ++r) g[r] = (float)(p[r] / s);
}

/*
 * Routing plan from given fp32 logits: selection, gates, capacity, slot
 * assignment, packing.  C < 0 means dropless.
 *   - selection is on the logits (softmax and sigmoid are both increasing, so
 *     either score picks the same experts in the same order);
 *   - slot assignment, "position" policy ([EP] capacity / drop: drop the
 *     assignments at the end of the batch; over-capacity assignments skip the
 *     expert): walk q = 0 .. T*k-1 with r = q / T, t = q % T; the assignment
 *     (t, r) to e = idx takes slot n_e, then n_e += 1; it is kept iff slot < C.
 *   - GShard second choice ([EP] router: top-2, the second expert taken at random
 *     by its weight; rule read as GShard's: with k = 2 and gates g1, g2, the
 *     second assignment exists iff u_t * (g1 + g2) < 2 * g2 for the caller's
 *     uniform u_t, in binary64 on the fp32 gates); an absent assignment takes no
 *     slot, is not counted in demand and gets dst_row -1;
 *   - "probs" policy ([EP]: drop the lowest-probability ones): per expert, the C
 *     assignments with the largest gate value are kept (equal gates: the earlier
 *     q first); the kept ones take slots in q order.
 *   - packing: offsets = exclusive prefix sum of kept; a kept assignment goes to
 *     packed row offsets[e] + slot (-1 when dropped); row_token inverts it.
 * Returns R = offsets[E], or -1 on bad arguments.
 */
static int cmp_probs(const void *a, const void *b) {
  /* entries are (gate, q) pairs: larger gate first, then smaller q */
  const double *x = (const double *)a, *y = (const double *)b;
  if (x[0] != y[0]) return x[0] > y[0] ? -1 : 1;
  return x[1] < y[1] ? -1 : (x[1] > y[1] ? 1 : 0);
}

int64_t oracle_route_from_logits(int64_t T, int64_t E, int k, int gate_mode, int score_fn, int drop_policy,
                                 int second_policy, const float *second_u, int64_t C, const float *logits,
                                 int32_t *topk_idx, float *topk_gate, int32_t *dst_row, int32_t *demand, int32_t *kept,
                                 int32_t *offsets, int32_t *row_token, int32_t *n_dropped) {
  if (k < 1 || k > 16 || k > E || T < 0) return -1;
  if (second_policy == OR_SECOND_RANDOM && (k != 2 || !second_u)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    select_topk(logits + t * E, E, k, topk_idx + t * k);
    gates(logits + t * E, E, k, gate_mode, score_fn, topk_idx + t * k, topk_gate + t * k);
  }
  int64_t *n = (int64_t *)calloc((size_t)E, sizeof(int64_t));
  int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T * k > 0 ? T * k : 1));
  char *absent = (char *)calloc((size_t)(T * k > 0 ? T * k : 1), 1);
  if (second_policy == OR_SECOND_RANDOM)
    for (int64_t t = 0; t < T; ++t) {
      const double g1 = topk_gate[t * 2], g2 = topk_gate[t * 2 + 1];
      absent[t * 2 + 1] = !((double)second_u[t] * (g1 + g2) < 2.0 * g2);
    }
  for (int64_t q = 0; q < T * k; ++q) {
    int64_t r = q / T, t = q % T;
    int32_t e = topk_idx[t * k + r];
    if (absent[t * k + r]) continue;
    slot[t * k + r] = n[e];
    n[e] += 1;
  }
  if (drop_policy == OR_DROP_PROBS && C >= 0) {
    /* per expert: its assignments in q order, sorted by (gate desc, q asc); the
     * first C are kept and renumbered in q order, the rest get slot C (dropped) */
    double *ent = (double *)malloc(sizeof(double) * 2 * (size_t)(T * k > 0 ? T * k : 1));
    char *keep = (char *)calloc((size_t)(T * k > 0 ? T * k : 1), 1);
    for (int64_t e = 0; e < E; ++e) {
      if (n[e] <= C) continue;
      int64_t m = 0;
      for (int64_t q = 0; q < T * k; ++q) {
        const int64_t ch = q / T, tok = q % T; /* choice-major position q */
        if (topk_idx[tok * k + ch] == (int32_t)e && !absent[tok * k + ch]) {
          ent[2 * m] = (double)topk_gate[tok * k + ch];
          ent[2 * m + 1] = (double)q;
          ++m;
        }
      }
      qsort(ent, (size_t)m, 2 * sizeof(double), cmp_probs);
      for (int64_t j = 0; j < C; ++j) {
        int64_t q = (int64_t)ent[2 * j + 1];
        keep[(q % T) * k + q / T] = 1;
      }
      int64_t next = 0;
      for (int64_t q = 0; q < T * k; ++q) {
        const int64_t ch = q / T, tok = q % T;
        if (topk_idx[tok * k + ch] == (int32_t)e && !absent[tok * k + ch])
          slot[tok * k + ch] = keep[tok * k + ch] ? next++ : C;
      }
    }
    free(ent);
    free(keep);
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) {
    demand[e] = (int32_t)n[e];
    kept[e] = (int32_t)((C < 0 || n[e] < C) ? n[e] : C);
    offsets[e + 1] = offsets[e] + kept[e];
  }
  for (int64_t t = 0; t < T; ++t)
    for (int r = 0; r < k; ++r) {
      int64_t i = t * k + r;
      int32_t e = topk_idx[i];
      if (!absent[i] && (C < 0 || slot[i] < C)) {
        dst_row[i] = (int32_t)(offsets[e] + slot[i]);
        row_token[dst_row[i]] = (int32_t)t;
      } else {
        dst_row[i] = -1;
      }
    }
  *n_dropped = (int32_t)(T * k - offsets[E]);
  free(n);
  free(slot);
  free(absent);
  return offsets[E];
}

/*
 * Router training terms ([EP] router section, the auxiliary-loss and z-loss
 * paragraphs; [SW] "Load balance & capacity"), binary64 from the fp32 logits.
 *   P_e   = (1/T) sum_t softmax(l_t)_e          mean routing probability
 *           (sigmoid scoring: the token's sigmoid scores divided by their sum)
 *   f_e   = demand_e / (T*k)   (aux_mode 0: every choice counts, k in the
 *           denominator -- Switch, Megatron-Core, DeepSpeed top-1 / top-k)
 *         = first_e / T        (aux_mode 1: only each token's first choice,
 *           no division by k -- DeepSpeed's top-2 path)
 *   out[0] = aux_coeff * E * sum_e f_e P_e      (uniform routing gives aux_coeff)
 *   out[1] = z_coeff * (1/T) sum_t logsumexp(l_t)^2
 * demand is the number of choices per expert before any capacity limit.
 * T = 0 gives zeros.
 */
void oracle_router_losses(int64_t T, int64_t E, int k, int score_fn, const float *logits, const int32_t *topk_idx,
                          const int32_t *demand, int aux_mode, double aux_coeff, double z_coeff, double *out) {
  out[0] = out[1] = 0.0;
  if (T <= 0) return;
  double *P = (double *)calloc((size_t)E, sizeof(double));
  double zsum = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const float *l = logits + t * E;
    double m = l[0];
    for (int64_t e = 1; e < E; ++e)
      if (l[e] > m) m = l[e];
    double den = 0.0;
    for (int64_t j = 0; j < E; ++j) den += exp((double)l[j] - m);
    if (score_fn == OR_SIGMOID) { /* P from the token's sigmoid scores divided by their sum */
      double ssum = 0.0;
      for (int64_t j = 0; j < E; ++j) ssum += 1.0 / (1.0 + exp(-(double)l[j]));
      for (int64_t j = 0; j < E; ++j) P[j] += (1.0 / (1.0 + exp(-(double)l[j]))) / ssum;
    } else {
      for (int64_t j = 0; j < E; ++j) P[j] += exp((double)l[j] - m) / den;
    }
    const double lse = m + log(den);
    zsum += lse * lse;
  }
  double dot = 0.0;
  for (int64_t e = 0; e < E; ++e) {
    double f;
    if (aux_mode == 0) {
      f = (double)demand[e] / ((double)T * (double)k);
    } else {
      int64_t first = 0;
      for (int64_t t = 0; t < T; ++t) first += (topk_idx[t * k] == (int32_t)e);
      f = (double)first / (double)T;
    }
    dot += f * (P[e] / (double)T);
  }
  out[0] = aux_coeff * (double)E * dot;
  out[1] = z_coeff * zsum / (double)T;
  free(P);
}

/* Dispatch ([EP] layer walk-through: tokens grouped by target expert):
 * X[row] = x[row_token[row]], a copy of the row's bytes. */
void oracle_dispatch(int64_t R, int64_t H, int dtype, const void *x, const int32_t *row_token, void *X) {
  size_t rb = (size_t)H * (dtype == OR_BF16 ? 2 : 4);
  for (int64_t row = 0; row < R; ++row)
    memcpy((char *)X + (size_t)row * rb, (const char *)x + (size_t)row_token[row] * rb, rb);
}

static double act_relu(double u) { return u > 0.0 ? u : 0.0; }
static double act_gelu(double u) { return 0.5 * u * (1.0 + erf(u / sqrt(2.0))); }
static double act_silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Expert FFN on single rows ([SW] §2.3 W_in / W_out; [EP] memory calculator:
 * gated FFN with gate / up / down): for a row x of expert e, in binary64 with no
 * intermediate rounding,
 *   2-matrix: u = x W_in (u_f = sum_h x_h W1[e][f][h]); h = ReLU(u) or GELU(u);
 *   SwiGLU:   h = silu(x W_gate) * (x W_up)   (W_gate = W1, W_up = W3);
 *   Y_n = sum_f h_f W2[e][n][f].
 * xin: n_rows x H elements of dtype; Y: n_rows x H binary64.
 */
void oracle_expert_rows(int64_t n_rows, const int32_t *expert_of_row, int64_t H, int64_t F, int dtype, int act,
                        const void *xin, const void *W1, const void *W3, const void *W2, double *Y) {
#pragma omp parallel
  {
    double *xr = (double *)malloc(sizeof(double) * (size_t)H);
    double *hr = (double *)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      int64_t e = expert_of_row[i];
      for (int64_t h = 0; h < H; ++h) xr[h] = elem(xin, dtype, i * H + h);
      for (int64_t f = 0; f < F; ++f) {
        int64_t base = (e * F + f) * H;
        double u = 0.0;
        for (int64_t h = 0; h < H; ++h) u += xr[h] * elem(W1, dtype, base + h);
        if (act == OR_SWIGLU) {
          double v = 0.0;
          for (int64_t h = 0; h < H; ++h) v += xr[h] * elem(W3, dtype, base + h);
          hr[f] = act_silu(u) * v;
        } else {
          hr[f] = act == OR_RELU ? act_relu(u) : act_gelu(u);
        }
      }
      for (int64_t n = 0; n < H; ++n) {
        int64_t base = (e * H + n) * F;
        double y = 0.0;
        for (int64_t f = 0; f < F; ++f) y += hr[f] * elem(W2, dtype, base + f);
        Y[i * H + n] = y;
      }
    }
    free(xr);
    free(hr);
  }
}

/* Expert FFN over the packed rows [0, offsets[E]): row of expert e = offsets[e] .. offsets[e+1]-1. */
void oracle_expert_ffn(int64_t E, const int32_t *offsets, int64_t H, int64_t F, int dtype, int act, const void *X,
                       const void *W1, const void *W3, const void *W2, double *Y) {
  int64_t R = offsets[E];
  int32_t *eo = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
  for (int64_t e = 0; e < E; ++e)
    for (int64_t row = offsets[e]; row < offsets[e + 1]; ++row) eo[row] = (int32_t)e;
  oracle_expert_rows(R, eo, H, F, dtype, act, X, W1, W3, W2, Y);
  free(eo);
}

/*
 * Combine ([EP] layer walk-through: unpermute, multiply by the gate, sum, add
 * the residual; [SW] §1.1 y = E_i(x) p_i(x), §1.2 overflow passes through the
 * residual): y[t] = res[t] + sum_{r ascending, dst_row[t,r] >= 0} g[t,r] Y[dst_row[t,r]],
 * in binary64.  Y is binary64 [R][H]; residual (dtype) may be NULL.
 * Only the tokens listed in `tokens` (n_tok of them) are computed when tokens != NULL;
 * y then holds n_tok rows in that order.
 */
void oracle_combine(int64_t T, int64_t H, int k, int dtype, const double *Y, const float *topk_gate,
                    const int32_t *dst_row, const void *residual, int64_t n_tok, const int64_t *tokens, double *y) {
  int64_t n = tokens ? n_tok : T;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t t = tokens ? tokens[i] : i;
    for (int64_t c = 0; c < H; ++c) {
      double acc = residual ? elem(residual, dtype, t * H + c) : 0.0;
      for (int r = 0; r < k; ++r) {
        int32_t d = dst_row[t * k + r];
        if (d >= 0) acc += (double)topk_gate[t * k + r] * Y[(int64_t)d * H + c];
      }
      y[i * H + c] = acc;
    }
  }
}

/*
 * Whole-layer output for selected tokens, from a routing plan this oracle made:
 * y[t] = res[t] + sum over kept choices of g * FFN_e(x[t]).  Dispatch is a copy,
 * so an expert's input row for (t, r) is x[t] itself.
 */
void oracle_token_outputs(int64_t n_tok, const int64_t *tokens, int64_t H, int64_t F, int k, int dtype, int act,
                          const void *x, const int32_t *topk_idx, const float *topk_gate, const int32_t *dst_row,
                          const void *W1, const void *W3, const void *W2, const void *residual, double *y) {
  size_t eb = dtype == OR_BF16 ? 2 : 4;
  int64_t nr = 0;
  for (int64_t i = 0; i < n_tok; ++i)
    for (int r = 0; r < k; ++r) nr += dst_row[tokens[i] * k + r] >= 0;
  char *xs = (char *)calloc((size_t)(nr > 0 ? nr : 1) * (size_t)H, eb);
  int32_t *es = (int32_t *)calloc((size_t)(nr > 0 ? nr : 1), sizeof(int32_t));
  double *Ys = (double *)malloc(sizeof(double) * (size_t)(nr > 0 ? nr : 1) * (size_t)H);
  int64_t j = 0;
  for (int64_t i = 0; i < n_tok; ++i)
    for (int r = 0; r < k; ++r)
      if (dst_row[tokens[i] * k + r] >= 0) {
        memcpy(xs + (size_t)j * H * eb, (const char *)x + (size_t)tokens[i] * H * eb, (size_t)H * eb);
        es[j++] = topk_idx[tokens[i] * k + r];
      }
  oracle_expert_rows(nr, es, H, F, dtype, act, xs, W1, W3, W2, Ys);
  j = 0;
  for (int64_t i = 0; i < n_tok; ++i) {
    int64_t t = tokens[i];
    for (int64_t c = 0; c < H; ++c) y[i * H + c] = residual ? elem(residual, dtype, t * H + c) : 0.0;
    for (int r = 0; r < k; ++r)
      if (dst_row[t * k + r] >= 0) {
        double g = (double)topk_gate[t * k + r];
        for (int64_t c = 0; c < H; ++c) y[i * H + c] += g * Ys[j * H + c];
        ++j;
      }
  }
  free(xs);
  free(es);
  free(Ys);
}
