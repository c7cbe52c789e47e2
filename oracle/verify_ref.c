/* verify_ref.c - plain fp64 C oracle of one round of draft-token verification.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or run it.  The product path (the HIP
 * library and its Python binding) never calls it and shares no code with it.
 * It computes what oracle/verify.py computes, written a second time in C: the
 * two oracles check each other, and this one runs on every host core.
 *
 * Pages, cited by title and section:
 *   [CZ]   chzhyang, "Speculative Decoding: Medusa, MTP, EAGLE, DFlash, DDTree,
 *          and DSpark"
 *   [VLLM] vLLM blog post "speculative-decoding-amd-gpus"
 *
 * What is computed:
 *   - drafts are verified left to right; the first rejection ends the round
 *     and the drafts after it are discarded ([VLLM] "Core idea of speculative
 *     decoding"; [CZ] section 1, the A B C D -> A B R example);
 *   - a stochastic draft y_i is kept with probability min(1, p_i(y_i)/q_i(y_i)),
 *     p_i the target's tempered distribution and q_i the draft's ([CZ]
 *     section 1, the acceptance probability alpha_i);
 *   - after the first rejection one token is drawn from [p_i - q_i]_+
 *     normalised; with no rejection one more token is drawn from the target's
 *     last row ([CZ] section 1, the paragraph after alpha_i);
 *   - greedy requests keep a draft while it is the target's argmax and commit
 *     the argmax at the first mismatch ([CZ] section 1 "Greedy equivalence";
 *     [VLLM] "A simple accept/reject example");
 *   - the accepted length does not count the final token ([CZ] section 2).
 *
 * Readings where the pages leave a step open (the same as the NumPy oracle):
 *   R1 p = softmax(z/T), q = softmax(d/T), one fp32 temperature widened
 *      exactly to fp64;
 *   R2 greedy ignores T and takes the lowest id among tied maxima;
 *   R3 with u in [0, 1): keep y iff u q(y) < p(y);
 *   R4 one uniform per draft position, one per request for the final draw;
 *   R5 inverse CDF in ascending id: the first t whose running sum exceeds
 *      w times the total; if rounding leaves none, the last id with weight;
 *   R6 a residual whose total is exactly 0 falls back to drawing from p;
 *   R7 request b has k_b drafts, k_b + 1 target rows (the last one is the
 *      bonus row) and k_b draft rows, packed request after request.
 *
 * Plain on purpose: each row is copied to fp64 and walked in ascending id,
 * every sum is sequential in fp64, exp() is the C library's.  Requests are
 * independent, so the only parallelism (OpenMP over requests) changes no
 * arithmetic: any thread count gives the same bits.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* ------------------------------------------------------------ single steps */

/* R1: the temperature the kernels are given is fp32; widen it exactly. */
double oracle_widen_temperature(double T) { return (double)(float)T; }

/* p_v = exp((z_v - max z) / T) / sum over the row ([CZ] section 1: p_i and q_i
 * are the tempered softmax of the target's and the draft's logits). */
void oracle_tempered_softmax(const double *z, int64_t V, double T, double *p) {
  double m = z[0];
  for (int64_t v = 1; v < V; ++v)
    if (z[v] > m) m = z[v];
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) {
    p[v] = exp((z[v] - m) / T);
    s += p[v];
  }
  for (int64_t v = 0; v < V; ++v) p[v] = p[v] / s;
}

/* Greedy target choice: the lowest id attaining the row maximum (R2). */
int64_t oracle_lowest_argmax(const double *z, int64_t V) {
  int64_t best = 0;
  for (int64_t v = 1; v < V; ++v)
    if (z[v] > z[best]) best = v;
  return best;
}

/* The ratio test of [CZ] section 1 in the form of R3. */
int oracle_keeps_draft(double u, double p_y, double q_y) { return u * q_y < p_y; }

/* Relative distance of the ratio test from its boundary:
 * |u q(y) - p(y)| / max(u q(y), p(y)), and 1 when both sides are 0. */
double oracle_accept_margin(double u, double p_y, double q_y) {
  const double a = u * q_y, b = p_y;
  const double top = a > b ? a : b;
  return top == 0.0 ? 1.0 : fabs(a - b) / top;
}

/* r_v = max(p_v - q_v, 0) ([CZ] section 1, the correction distribution). */
void oracle_positive_residual(const double *p, const double *q, int64_t V, double *r) {
  for (int64_t v = 0; v < V; ++v) {
    const double d = p[v] - q[v];
    r[v] = d > 0.0 ? d : 0.0;
  }
}

/* Draw with one uniform u from the unnormalised weights wt[0..n) (R5).
 * *tok: the drawn id; *total: the sequential sum of the weights; *margin: the
 * distance of u * total from the nearer edge of the drawn id's cumulative
 * interval, relative to the total (0 when the total is 0).  Returns 0, or -1
 * when no weight is positive. */
int oracle_inverse_cdf(const double *wt, int64_t n, double u, int64_t *tok, double *total,
                       double *margin) {
  double c = 0.0;
  for (int64_t v = 0; v < n; ++v) c += wt[v];
  const double tot = c;
  const double thr = u * tot;
  int64_t t = -1;
  double lo = 0.0, hi = 0.0;
  c = 0.0;
  for (int64_t v = 0; v < n; ++v) {
    const double before = c;
    c += wt[v];
    if (c > thr) {
      t = v;
      lo = before;
      hi = c;
      break;
    }
  }
  if (t < 0) {                        /* no crossing: the last id with weight */
    for (int64_t v = n - 1; v >= 0; --v)
      if (wt[v] > 0.0) {
        t = v;
        break;
      }
    if (t < 0) return -1;
    c = 0.0;
    for (int64_t v = 0; v <= t; ++v) {
      lo = c;
      c += wt[v];
    }
    hi = c;
  }
  *tok = t;
  *total = tot;
  *margin = tot > 0.0 ? fmin(fabs(lo - thr), fabs(hi - thr)) / tot : 0.0;
  return 0;
}

/* ------------------------------------------------------------ one request */

typedef struct {
  const void *target, *draft;
  int elem_bytes;                  /* 4: fp32 logits, 8: fp64 logits */
  int64_t target_ld, draft_ld, V;
  const int64_t *tokens;
  const double *u_accept;
  double T;
} Inputs;

/* Row `row` of a logit matrix, widened exactly to fp64, into z[0..V). */
static void load_row(const void *base, int elem_bytes, int64_t row, int64_t ld, int64_t V,
                     double *z) {
  for (int64_t v = 0; v < V; ++v) {
    if (elem_bytes == 4)
      z[v] = (double)((const float *)base)[row * ld + v];
    else
      z[v] = ((const double *)base)[row * ld + v];
  }
}

typedef struct {
  int64_t a, final_tok;
  double resid, margin;
} Result;

/* Greedy request: target rows t0 .. t0 + k, drafts tokens[d0 .. d0 + k). */
static Result greedy_request(const Inputs *in, int64_t t0, int64_t d0, int64_t k, double *z) {
  Result r = {k, -1, -1.0, INFINITY};
  for (int64_t i = 0; i < k; ++i) {
    load_row(in->target, in->elem_bytes, t0 + i, in->target_ld, in->V, z);
    const int64_t g = oracle_lowest_argmax(z, in->V);
    if (in->tokens[d0 + i] != g) {
      r.a = i;
      r.final_tok = g;
      return r;
    }
  }
  load_row(in->target, in->elem_bytes, t0 + k, in->target_ld, in->V, z);
  r.final_tok = oracle_lowest_argmax(z, in->V);
  return r;
}

/* Stochastic request.  early_exit = 0: every position's p, q (and p(y),
 * q(y)) is formed, tests stop at the first rejection; early_exit = 1: a
 * position's distributions are formed only when its test is reached.
 * Returns -1 in r->a when a draw finds no positive weight. */
static Result stochastic_request(const Inputs *in, int64_t t0, int64_t d0, int64_t k, double w,
                                 int early_exit, double *z, double *p, double *q, double *res,
                                 double *p_draft, double *q_draft) {
  Result r = {k, -1, -1.0, INFINITY};
  int cut = 0;
  const int64_t V = in->V;
  for (int64_t i = 0; i < k; ++i) {
    if (cut && early_exit) break;
    load_row(in->target, in->elem_bytes, t0 + i, in->target_ld, V, z);
    oracle_tempered_softmax(z, V, in->T, p);
    load_row(in->draft, in->elem_bytes, d0 + i, in->draft_ld, V, z);
    oracle_tempered_softmax(z, V, in->T, q);
    const int64_t y = in->tokens[d0 + i];
    p_draft[d0 + i] = p[y];
    q_draft[d0 + i] = q[y];
    if (cut) continue;                /* later rows decide nothing */
    const double u = in->u_accept[d0 + i];
    r.margin = fmin(r.margin, oracle_accept_margin(u, p[y], q[y]));
    if (oracle_keeps_draft(u, p[y], q[y])) continue;
    cut = 1;
    r.a = i;
    oracle_positive_residual(p, q, V, res);
    double Z = 0.0;
    for (int64_t v = 0; v < V; ++v) Z += res[v];
    int64_t t;
    double tot, m;
    int rc;
    if (Z > 0.0) {
      rc = oracle_inverse_cdf(res, V, w, &t, &tot, &m);
      r.resid = tot;
    } else {                          /* R6 */
      rc = oracle_inverse_cdf(p, V, w, &t, &tot, &m);
      r.resid = 0.0;
    }
    if (rc != 0) {
      r.a = -1;
      return r;
    }
    r.final_tok = t;
    r.margin = fmin(r.margin, m);
  }
  if (!cut) {                         /* every draft kept: the bonus from row k */
    load_row(in->target, in->elem_bytes, t0 + k, in->target_ld, V, z);
    oracle_tempered_softmax(z, V, in->T, p);
    int64_t t;
    double tot, m;
    if (oracle_inverse_cdf(p, V, w, &t, &tot, &m) != 0) {
      r.a = -1;
      return r;
    }
    r.final_tok = t;
    r.margin = fmin(r.margin, m);
  }
  return r;
}

/* ------------------------------------------------------------ packed batch */

/* A packed batch in the layout of the C ABI: target row of (b, i) is
 * off[b] + b + i (i = 0 .. k_b), draft row of (b, i) is off[b] + i, with
 * off[b] the sum of k over the requests before b.  greedy may be NULL (every
 * request greedy); draft may be NULL when every request is greedy.
 * Outputs (caller-owned): accepted_len[B], out_tokens[K+B] (-1 in unused
 * slots), p_draft[K], q_draft[K] (-1 for greedy requests and, with
 * early_exit, after the cut), resid_mass[B] (-1 unless a residual was drawn
 * from), margin[B] (the smallest deciding margin; +inf for greedy requests).
 * threads: OpenMP threads over requests (<= 0: the runtime's default).
 * Returns 0; -1 when a stochastic request's draft token lies outside [0, V);
 * -2 for inconsistent arguments; -3 when memory runs out; -4 when a draw
 * finds no positive weight. */
int oracle_verify_batch(const void *target, const void *draft, int elem_bytes,
                        int64_t target_ld, int64_t draft_ld, const int64_t *tokens,
                        const int64_t *num_draft, const uint8_t *greedy, int64_t B, int64_t V,
                        double temperature, const double *u_accept, const double *u_final,
                        int early_exit, int threads, int64_t *accepted_len, int64_t *out_tokens,
                        double *p_draft, double *q_draft, double *resid_mass, double *margin) {
  if (B < 0 || V <= 0 || (elem_bytes != 4 && elem_bytes != 8) || !target) return -2;
  int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B + 1));
  if (!off) return -3;
  off[0] = 0;
  for (int64_t b = 0; b < B; ++b) {
    if (num_draft[b] < 0) {
      free(off);
      return -2;
    }
    off[b + 1] = off[b] + num_draft[b];
  }
  const int64_t K = off[B];
  for (int64_t b = 0; b < B; ++b) {
    const int g = greedy ? greedy[b] != 0 : 1;
    if (!g && !draft) {
      free(off);
      return -2;
    }
    for (int64_t i = 0; !g && i < num_draft[b]; ++i) {
      const int64_t y = tokens[off[b] + i];
      if (y < 0 || y >= V) {
        free(off);
        return -1;
      }
    }
  }
  for (int64_t j = 0; j < K + B; ++j) out_tokens[j] = -1;
  for (int64_t j = 0; j < K; ++j) p_draft[j] = q_draft[j] = -1.0;

  Inputs in;
  in.target = target;
  in.draft = draft;
  in.elem_bytes = elem_bytes;
  in.target_ld = target_ld;
  in.draft_ld = draft_ld;
  in.V = V;
  in.tokens = tokens;
  in.u_accept = u_accept;
  in.T = oracle_widen_temperature(temperature);

  int status = 0;
  if (threads <= 0) threads = 1;
#pragma omp parallel num_threads(threads)
  {
    double *buf = (double *)malloc(sizeof(double) * (size_t)V * 4);
    if (!buf) {
#pragma omp atomic write
      status = -3;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
      if (!buf) continue;
      const int64_t k = num_draft[b], t0 = off[b] + b, d0 = off[b];
      const int g = greedy ? greedy[b] != 0 : 1;
      Result r;
      if (g)
        r = greedy_request(&in, t0, d0, k, buf);
      else
        r = stochastic_request(&in, t0, d0, k, (double)u_final[b], early_exit, buf, buf + V,
                               buf + 2 * V, buf + 3 * V, p_draft, q_draft);
      if (r.a < 0) {
#pragma omp atomic write
        status = -4;
        continue;
      }
      accepted_len[b] = r.a;
      for (int64_t i = 0; i < r.a; ++i) out_tokens[t0 + i] = tokens[d0 + i];
      out_tokens[t0 + r.a] = r.final_tok;
      resid_mass[b] = r.resid;
      margin[b] = r.margin;
    }
    free(buf);
  }
  free(off);
  return status;
}
