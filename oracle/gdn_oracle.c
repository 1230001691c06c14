/*
 * Gated DeltaNet layer oracle: plain, slow, double-precision CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library shares no
 * code, header, table or helper with it, and never calls it.
 *
 * What it computes, step by step, for one sequence of the Gated DeltaNet
 * ("GDR", the gated delta rule) linear-attention layer of Qwen3.5 /
 * Qwen3-Next:
 *
 *   1. conv      fused [q|k|v] depthwise causal conv1d over the last K raw
 *                inputs, then SiLU
 *                (pegainfer PR #1003 "shard linear-attention/GDR state per TP
 *                rank", PR body, weight_loader bullet: the fused qkv weight
 *                has q, k and v segments and conv1d has one weight per
 *                channel; cortex commit 95dc874 "TP-aware Qwen3-Next", Architecture
 *                pieces, TpQwen3_5GatedDeltaNet: in_proj_qkv and conv1d.weight
 *                are fused tensors with three regions [key|key|value]).
 *   2. split     channel order [q (Hk*dk) | k (Hk*dk) | v (Hv*dv)], head-major
 *                inside each region (same two passages).
 *   3. l2norm    q and k per K-head, q additionally scaled by 1/sqrt(dk)
 *                (cortex commit 95dc874, "Reuses unchanged" paragraph: l2norm).
 *   4. gates     g = -exp(A_log[h]) * softplus(a + dt_bias[h]), beta = sigmoid(b)
 *                (cortex commit 95dc874, TpQwen3_5GatedDeltaNet: in_proj_a,
 *                in_proj_b, A_log, dt_bias; Helpers: softplus).  V-head h reads
 *                K-head floor(h / (Hv/Hk)) (Helpers: repeat_interleave).
 *   5. recurrence, per V-head, with the post-update state used for the output:
 *                S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - e^{g_t} S_{t-1}^T k_t)^T
 *                o_t = S_t^T q_t
 *                (the per-V-head delta-rule state of cortex commit 95dc874,
 *                TpQwen3_5GatedDeltaNet bullet; the GDR recurrence as defined
 *                in Yang, Kautz & Hatamizadeh, "Gated Delta Networks: Improving
 *                Mamba2 with Delta Rule", ICLR 2025, eq. for S_t).
 *   6. gated RMSNorm   y = w * o / sqrt(mean(o^2) + eps) * SiLU(z), w shared by
 *                all V-heads (pegainfer PR #1003, PR body, batch_decode and
 *                weights bullets: the gated norm runs per local V-head with
 *                one replicated weight; cortex commit 95dc874, "Reuses
 *                unchanged": the gated Qwen3_5RmsNormGated tail).
 *
 * Readings taken where the pages are silent: no conv bias; the conv weight tap
 * K-1 multiplies the current token; the conv window holds the last K raw
 * inputs, oldest first; l2norm is x / sqrt(sum x^2 + eps); the norm weight
 * multiplies as given.
 *
 * No intermediate rounding: every input is taken as given (already rounded to
 * its storage type by the caller) and all arithmetic is double.
 *
 * The chunkwise routine at the end is NOT a second oracle of the layer: it is
 * the blocked (WY / UT) rewriting of step 5, kept here so that tests can show,
 * in double precision, that the blocked form equals the token loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int num_k_heads;  /* Hk */
  int num_v_heads;  /* Hv, a multiple of Hk */
  int head_k_dim;   /* dk */
  int head_v_dim;   /* dv */
  int conv_kernel;  /* K */
  double l2norm_eps;
  double rmsnorm_eps;
  double scale;     /* <= 0 means 1/sqrt(dk) */
} ogdn_geom;

typedef struct {
  const double* conv_w;  /* [C][K] */
  const double* A_log;   /* [Hv] */
  const double* dt_bias; /* [Hv] */
  const double* norm_w;  /* [dv] */
} ogdn_weights;

static int channels(const ogdn_geom* g) {
  return 2 * g->num_k_heads * g->head_k_dim + g->num_v_heads * g->head_v_dim;
}

static double q_scale(const ogdn_geom* g) {
  return g->scale > 0.0 ? g->scale : 1.0 / sqrt((double)g->head_k_dim);
}

static int geom_ok(const ogdn_geom* g) {
  if (!g) return 0;
  if (g->num_k_heads <= 0 || g->num_v_heads <= 0 || g->head_k_dim <= 0 ||
      g->head_v_dim <= 0 || g->conv_kernel <= 0)
    return 0;
  return g->num_v_heads % g->num_k_heads == 0;
}

/* ---------------------------------------------------------------- step 1 */

double ogdn_silu(double x) { return x / (1.0 + exp(-x)); }

/* Causal depthwise conv of one channel.  stream[0..K-1] is the window before
 * the first token (oldest first), stream[K+t] is token t.  Token t sees the K
 * most recent inputs ending at itself: stream[t+1 .. t+K]; weight tap j
 * multiplies stream[t+1+j], so tap K-1 meets the current token.  Returns the
 * pre-activation; the caller applies SiLU. */
static double conv_at(const double* w, int K, const double* stream, int t) {
  double acc = 0.0;
  for (int j = 0; j < K; ++j) acc += w[j] * stream[t + 1 + j];
  return acc;
}

/* Conv + SiLU of channel ch over T tokens.  window: [K][C] (oldest first),
 * x: [T][C].  out[t] for t < T.  Scratch stream of K+T doubles. */
void ogdn_conv_channel(int C, int K, const double* w_ch, const double* window,
                       const double* x, int T, int ch, double* stream,
                       double* out, int out_stride) {
  for (int j = 0; j < K; ++j) stream[j] = window[(size_t)j * C + ch];
  for (int t = 0; t < T; ++t) stream[K + t] = x[(size_t)t * C + ch];
  for (int t = 0; t < T; ++t)
    out[(size_t)t * out_stride] = ogdn_silu(conv_at(w_ch, K, stream, t));
}

/* Window after T tokens: the last K entries of [window ; x]. */
void ogdn_conv_window_advance(int C, int K, double* window, const double* x,
                              int T) {
  double* old = (double*)malloc(sizeof(double) * (size_t)K * C);
  memcpy(old, window, sizeof(double) * (size_t)K * C);
  for (int j = 0; j < K; ++j) {
    int s = T + j; /* index into [old ; x], length K + T */
    const double* src = s < K ? old + (size_t)s * C : x + (size_t)(s - K) * C;
    memcpy(window + (size_t)j * C, src, sizeof(double) * C);
  }
  free(old);
}

/* ---------------------------------------------------------------- step 3 */

void ogdn_l2norm(const double* x, int n, double eps, double mult,
                 double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = mult / sqrt(ss + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * inv;
}

/* ---------------------------------------------------------------- step 4 */

double ogdn_softplus(double x) {
  /* log(1 + e^x), written so that large x does not overflow */
  return x > 30.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

void ogdn_gates(double A_log, double dt_bias, double a, double b, double* g,
                double* beta) {
  *g = -exp(A_log) * ogdn_softplus(a + dt_bias);
  *beta = 1.0 / (1.0 + exp(-b));
}

/* ---------------------------------------------------------------- step 5 */

/* One token of the gated delta rule on S [dk][dv] (row i = key index,
 * column j = value index), in place; o = S_t^T q with the updated state. */
void ogdn_gdr_step(int dk, int dv, double g, double beta, const double* k,
                   const double* v, const double* q, double* S, double* o) {
  double decay = exp(g);
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= decay;
  for (int j = 0; j < dv; ++j) {
    double pred = 0.0; /* (e^g S_{t-1})^T k, column j */
    for (int i = 0; i < dk; ++i) pred += S[(size_t)i * dv + j] * k[i];
    double u = beta * (v[j] - pred);
    for (int i = 0; i < dk; ++i) S[(size_t)i * dv + j] += k[i] * u;
  }
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
    o[j] = acc;
  }
}

/* ---------------------------------------------------------------- step 6 */

void ogdn_gated_rmsnorm(int dv, const double* o, const double* z,
                        const double* w, double eps, double* y) {
  double ms = 0.0;
  for (int j = 0; j < dv; ++j) ms += o[j] * o[j];
  ms /= dv;
  double inv = 1.0 / sqrt(ms + eps);
  for (int j = 0; j < dv; ++j) y[j] = w[j] * o[j] * inv * ogdn_silu(z[j]);
}

/* ------------------------------------------------ one V-head of a sequence */

typedef struct {
  const ogdn_geom* g;
  const ogdn_weights* w;
  int T;
  const double* x;      /* [T][C] */
  const double* z;      /* [T][Hv][dv] */
  const double* a;      /* [T][Hv] */
  const double* b;      /* [T][Hv] */
  const double* window; /* [K][C], the window BEFORE the first token */
  double* S;            /* [Hv][dk][dv] */
  double* y;            /* [T][Hv][dv] or NULL */
  double* o;            /* [T][Hv][dv] or NULL */
  int chunk;            /* 0: token loop; > 0: blocked form with this length */
} head_job;

/* Conv + SiLU + split + l2norm of the channels that V-head h reads:
 * qh, kh: [T][dk] (normalised, q scaled), vh: [T][dv]. */
static void head_inputs(const head_job* J, int h, double* qh, double* kh,
                        double* vh) {
  const ogdn_geom* g = J->g;
  int C = channels(g), K = g->conv_kernel, T = J->T;
  int dk = g->head_k_dim, dv = g->head_v_dim;
  int r = g->num_v_heads / g->num_k_heads;
  int m = h / r; /* repeat_interleave of K-heads onto V-heads */
  int q0 = m * dk, k0 = g->num_k_heads * dk + m * dk;
  int v0 = 2 * g->num_k_heads * dk + h * dv;
  double* stream = (double*)malloc(sizeof(double) * (size_t)(K + T));
  for (int i = 0; i < dk; ++i) {
    ogdn_conv_channel(C, K, J->w->conv_w + (size_t)(q0 + i) * K, J->window,
                      J->x, T, q0 + i, stream, qh + i, dk);
    ogdn_conv_channel(C, K, J->w->conv_w + (size_t)(k0 + i) * K, J->window,
                      J->x, T, k0 + i, stream, kh + i, dk);
  }
  for (int j = 0; j < dv; ++j)
    ogdn_conv_channel(C, K, J->w->conv_w + (size_t)(v0 + j) * K, J->window,
                      J->x, T, v0 + j, stream, vh + j, dv);
  free(stream);
  double sc = q_scale(g);
  for (int t = 0; t < T; ++t) {
    ogdn_l2norm(qh + (size_t)t * dk, dk, g->l2norm_eps, sc, qh + (size_t)t * dk);
    ogdn_l2norm(kh + (size_t)t * dk, dk, g->l2norm_eps, 1.0, kh + (size_t)t * dk);
  }
}

static void head_token_loop(const head_job* J, int h, const double* qh,
                            const double* kh, const double* vh, double* ot) {
  const ogdn_geom* g = J->g;
  int Hv = g->num_v_heads, dk = g->head_k_dim, dv = g->head_v_dim;
  double* S = J->S + (size_t)h * dk * dv;
  for (int t = 0; t < J->T; ++t) {
    double gt, bt;
    ogdn_gates(J->w->A_log[h], J->w->dt_bias[h], J->a[(size_t)t * Hv + h],
               J->b[(size_t)t * Hv + h], &gt, &bt);
    ogdn_gdr_step(dk, dv, gt, bt, kh + (size_t)t * dk, vh + (size_t)t * dv,
                  qh + (size_t)t * dk, S, ot + (size_t)t * dv);
  }
}

/* Blocked rewriting of the token loop over chunks of length L (the last one
 * may be shorter).  Within a chunk with gamma_i = sum_{j<=i} g_j:
 *   A_ij = beta_i e^{gamma_i-gamma_j} k_i.k_j (j < i),   Tm = (I + A)^{-1}
 *   W = Tm diag(beta e^gamma) K,   U = Tm diag(beta) V,   V' = U - W S
 *   O = diag(e^gamma) Q S + (mask_{j<=i} e^{gamma_i-gamma_j} Q K^T) V'
 *   S <- e^{gamma_last} S + sum_i e^{gamma_last-gamma_i} k_i V'_i^T
 * Derivation: unrolling the recurrence inside the chunk gives
 * u_t = beta_t (v_t - e^{gamma_t} S_0^T k_t - sum_{j<t} e^{gamma_t-gamma_j}
 * (k_t.k_j) u_j), a unit lower-triangular system in the rows u_t. */
static void head_chunkwise(const head_job* J, int h, const double* qh,
                           const double* kh, const double* vh, double* ot) {
  const ogdn_geom* g = J->g;
  int Hv = g->num_v_heads, dk = g->head_k_dim, dv = g->head_v_dim;
  int L = J->chunk;
  double* S = J->S + (size_t)h * dk * dv;
  double* gam = (double*)malloc(sizeof(double) * L);
  double* bet = (double*)malloc(sizeof(double) * L);
  double* A = (double*)malloc(sizeof(double) * L * L);
  double* Tm = (double*)malloc(sizeof(double) * L * L);
  double* W = (double*)malloc(sizeof(double) * (size_t)L * dk);
  double* U = (double*)malloc(sizeof(double) * (size_t)L * dv);
  double* Vp = (double*)malloc(sizeof(double) * (size_t)L * dv);
  for (int c0 = 0; c0 < J->T; c0 += L) {
    int n = J->T - c0 < L ? J->T - c0 : L;
    const double* Q = qh + (size_t)c0 * dk;
    const double* Kc = kh + (size_t)c0 * dk;
    const double* V = vh + (size_t)c0 * dv;
    double run = 0.0;
    for (int i = 0; i < n; ++i) {
      double gi, bi;
      ogdn_gates(J->w->A_log[h], J->w->dt_bias[h],
                 J->a[(size_t)(c0 + i) * Hv + h], J->b[(size_t)(c0 + i) * Hv + h],
                 &gi, &bi);
      run += gi;
      gam[i] = run;
      bet[i] = bi;
    }
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) {
        double v = 0.0;
        if (j < i) {
          for (int d = 0; d < dk; ++d) v += Kc[(size_t)i * dk + d] * Kc[(size_t)j * dk + d];
          v *= bet[i] * exp(gam[i] - gam[j]);
        }
        A[i * L + j] = v;
      }
    /* Tm = (I + A)^{-1} by forward substitution, column by column */
    for (int col = 0; col < n; ++col)
      for (int i = 0; i < n; ++i) {
        double v = (i == col) ? 1.0 : 0.0;
        for (int j = col; j < i; ++j) v -= A[i * L + j] * Tm[j * L + col];
        Tm[i * L + col] = (i < col) ? 0.0 : v;
      }
    for (int i = 0; i < n; ++i) {
      for (int d = 0; d < dk; ++d) {
        double acc = 0.0;
        for (int j = 0; j <= i; ++j)
          acc += Tm[i * L + j] * bet[j] * exp(gam[j]) * Kc[(size_t)j * dk + d];
        W[(size_t)i * dk + d] = acc;
      }
      for (int e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int j = 0; j <= i; ++j) acc += Tm[i * L + j] * bet[j] * V[(size_t)j * dv + e];
        U[(size_t)i * dv + e] = acc;
      }
    }
    for (int i = 0; i < n; ++i)
      for (int e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d) acc += W[(size_t)i * dk + d] * S[(size_t)d * dv + e];
        Vp[(size_t)i * dv + e] = U[(size_t)i * dv + e] - acc;
      }
    for (int i = 0; i < n; ++i)
      for (int e = 0; e < dv; ++e) {
        double inter = 0.0;
        for (int d = 0; d < dk; ++d) inter += Q[(size_t)i * dk + d] * S[(size_t)d * dv + e];
        double intra = 0.0;
        for (int j = 0; j <= i; ++j) {
          double qk = 0.0;
          for (int d = 0; d < dk; ++d) qk += Q[(size_t)i * dk + d] * Kc[(size_t)j * dk + d];
          intra += exp(gam[i] - gam[j]) * qk * Vp[(size_t)j * dv + e];
        }
        ot[(size_t)(c0 + i) * dv + e] = exp(gam[i]) * inter + intra;
      }
    double last = gam[n - 1];
    for (int d = 0; d < dk; ++d)
      for (int e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int i = 0; i < n; ++i)
          acc += exp(last - gam[i]) * Kc[(size_t)i * dk + d] * Vp[(size_t)i * dv + e];
        S[(size_t)d * dv + e] = exp(last) * S[(size_t)d * dv + e] + acc;
      }
  }
  free(gam); free(bet); free(A); free(Tm); free(W); free(U); free(Vp);
}

static void run_head(const head_job* J, int h) {
  const ogdn_geom* g = J->g;
  int T = J->T, Hv = g->num_v_heads, dk = g->head_k_dim, dv = g->head_v_dim;
  double* qh = (double*)malloc(sizeof(double) * (size_t)T * dk + 8);
  double* kh = (double*)malloc(sizeof(double) * (size_t)T * dk + 8);
  double* vh = (double*)malloc(sizeof(double) * (size_t)T * dv + 8);
  double* ot = (double*)malloc(sizeof(double) * (size_t)T * dv + 8);
  head_inputs(J, h, qh, kh, vh);
  if (J->chunk > 0)
    head_chunkwise(J, h, qh, kh, vh, ot);
  else
    head_token_loop(J, h, qh, kh, vh, ot);
  for (int t = 0; t < T; ++t) {
    const double* o_t = ot + (size_t)t * dv;
    size_t off = ((size_t)t * Hv + h) * dv;
    if (J->o) memcpy(J->o + off, o_t, sizeof(double) * dv);
    if (J->y)
      ogdn_gated_rmsnorm(dv, o_t, J->z + off, J->w->norm_w, g->rmsnorm_eps,
                         J->y + off);
  }
  free(qh); free(kh); free(vh); free(ot);
}

/* ------------------------------------------- work sharing over V-heads */

typedef struct {
  const head_job* jobs; /* one per sequence */
  const int* items;     /* pairs (job index, head) */
  int n_items;
  int next;
  pthread_mutex_t lock;
} pool_t;

static void* worker(void* arg) {
  pool_t* P = (pool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&P->lock);
    int i = P->next++;
    pthread_mutex_unlock(&P->lock);
    if (i >= P->n_items) break;
    run_head(&P->jobs[P->items[2 * i]], P->items[2 * i + 1]);
  }
  return NULL;
}

static void run_items(const head_job* jobs, const int* items, int n_items,
                      int nthreads) {
  if (n_items <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_items) nthreads = n_items;
  pool_t P;
  P.jobs = jobs; P.items = items; P.n_items = n_items; P.next = 0;
  pthread_mutex_init(&P.lock, NULL);
  if (nthreads == 1) {
    worker(&P);
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &P);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&P.lock);
}

/* ---------------------------------------------------------- public entry */

/*
 * Several independent sequences of the layer.
 *   cu_seqlens [N+1]: sequence n owns tokens [cu[n], cu[n+1]) of x, z, a, b, y, o.
 *   S     [N][Hv][dk][dv]  in: state before the first token; out: after the last.
 *   window[N][K][C]        in: conv window before the first token; out: after.
 *   head_mask [Hv] or NULL: only heads with a nonzero entry are computed (their
 *          y/o rows and S blocks are written; other heads are left untouched).
 *   chunk  0 for the token loop, > 0 for the blocked rewriting.
 * Returns 0, or -1 on a malformed argument.
 */
int ogdn_sequences(const ogdn_geom* g, const ogdn_weights* w, int N,
                   const int* cu_seqlens, const double* x, const double* z,
                   const double* a, const double* b, double* S, double* window,
                   double* y, double* o, const unsigned char* head_mask,
                   int chunk, int nthreads) {
  if (!geom_ok(g) || !w || N < 0 || !cu_seqlens || chunk < 0) return -1;
  int C = channels(g), K = g->conv_kernel, Hv = g->num_v_heads;
  int dk = g->head_k_dim, dv = g->head_v_dim;
  if (cu_seqlens[0] != 0) return -1;
  for (int n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  head_job* jobs = (head_job*)malloc(sizeof(head_job) * (N > 0 ? N : 1));
  double* win0 = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * K * C);
  int* items = (int*)malloc(sizeof(int) * 2 * (size_t)(N > 0 ? N : 1) * Hv);
  int n_items = 0;
  for (int n = 0; n < N; ++n) {
    int t0 = cu_seqlens[n], T = cu_seqlens[n + 1] - t0;
    memcpy(win0 + (size_t)n * K * C, window + (size_t)n * K * C,
           sizeof(double) * (size_t)K * C);
    head_job* J = &jobs[n];
    J->g = g; J->w = w; J->T = T;
    J->x = x + (size_t)t0 * C;
    J->z = z ? z + (size_t)t0 * Hv * dv : NULL;
    J->a = a + (size_t)t0 * Hv;
    J->b = b + (size_t)t0 * Hv;
    J->window = win0 + (size_t)n * K * C;
    J->S = S + (size_t)n * Hv * dk * dv;
    J->y = (y && z) ? y + (size_t)t0 * Hv * dv : NULL;
    J->o = o ? o + (size_t)t0 * Hv * dv : NULL;
    J->chunk = chunk;
    if (T == 0) continue;
    for (int h = 0; h < Hv; ++h)
      if (!head_mask || head_mask[h]) {
        items[2 * n_items] = n;
        items[2 * n_items + 1] = h;
        ++n_items;
      }
  }
  run_items(jobs, items, n_items, nthreads);
  for (int n = 0; n < N; ++n) {
    int t0 = cu_seqlens[n], T = cu_seqlens[n + 1] - t0;
    ogdn_conv_window_advance(C, K, window + (size_t)n * K * C,
                             x + (size_t)t0 * C, T);
  }
  free(jobs); free(win0); free(items);
  return 0;
}

/*
 * Slot-pool form used by both batched decode (every sequence has one token)
 * and packed prefill.  pool_S [P][Hv][dk][dv], pool_conv [P][K][C].
 * Sequence n runs on slot slot_idx[n]; a negative slot marks a padding entry,
 * whose y/o rows are set to zero and which touches no slot.  When has_init is
 * given and has_init[n] == 0 the sequence starts from zero state and a zero
 * window instead of the slot's contents.  The final state and window are
 * written back to the slot; slots not named are untouched.
 */
int ogdn_pool_run(const ogdn_geom* g, const ogdn_weights* w, double* pool_S,
                  double* pool_conv, int P, int N, const int* cu_seqlens,
                  const int* slot_idx, const unsigned char* has_init,
                  const double* x, const double* z, const double* a,
                  const double* b, double* y, double* o, int nthreads) {
  if (!geom_ok(g) || N < 0 || P < 0) return -1;
  int C = channels(g), K = g->conv_kernel, Hv = g->num_v_heads;
  int dk = g->head_k_dim, dv = g->head_v_dim;
  size_t sS = (size_t)Hv * dk * dv, sW = (size_t)K * C;
  for (int n = 0; n < N; ++n) {
    if (slot_idx[n] >= P) return -1;
    for (int m = 0; m < n; ++m)
      if (slot_idx[n] >= 0 && slot_idx[m] == slot_idx[n]) return -1;
  }
  double* S = (double*)calloc((size_t)(N > 0 ? N : 1) * sS, sizeof(double));
  double* W = (double*)calloc((size_t)(N > 0 ? N : 1) * sW, sizeof(double));
  for (int n = 0; n < N; ++n) {
    int s = slot_idx[n];
    if (s < 0 || (has_init && !has_init[n])) continue;
    memcpy(S + n * sS, pool_S + (size_t)s * sS, sizeof(double) * sS);
    memcpy(W + n * sW, pool_conv + (size_t)s * sW, sizeof(double) * sW);
  }
  int rc = ogdn_sequences(g, w, N, cu_seqlens, x, z, a, b, S, W, y, o, NULL,
                          0, nthreads);
  if (rc == 0) {
    for (int n = 0; n < N; ++n) {
      int s = slot_idx[n];
      size_t t0 = (size_t)cu_seqlens[n], t1 = (size_t)cu_seqlens[n + 1];
      if (s < 0) {
        if (y) memset(y + t0 * Hv * dv, 0, sizeof(double) * (t1 - t0) * Hv * dv);
        if (o) memset(o + t0 * Hv * dv, 0, sizeof(double) * (t1 - t0) * Hv * dv);
        continue;
      }
      memcpy(pool_S + (size_t)s * sS, S + n * sS, sizeof(double) * sS);
      memcpy(pool_conv + (size_t)s * sW, W + n * sW, sizeof(double) * sW);
    }
  }
  free(S); free(W);
  return rc;
}

/* State compaction on retire: slot dst[i] receives a copy of slot src[i]
 * (recurrent state and conv window); everything else is untouched.  The
 * copies are taken from a snapshot, so the result does not depend on order
 * (pegainfer issue #1001, Splits, "TP CUDA Graph": slot-indexed per-rank
 * recurrent/conv state, D2D compaction on retire). */
int ogdn_compact(const ogdn_geom* g, double* pool_S, double* pool_conv, int P,
                 const int* src, const int* dst, int n) {
  if (!geom_ok(g) || n < 0) return -1;
  int C = channels(g), K = g->conv_kernel;
  size_t sS = (size_t)g->num_v_heads * g->head_k_dim * g->head_v_dim;
  size_t sW = (size_t)K * C;
  for (int i = 0; i < n; ++i)
    if (src[i] < 0 || src[i] >= P || dst[i] < 0 || dst[i] >= P) return -1;
  double* snapS = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * sS);
  double* snapW = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * sW);
  for (int i = 0; i < n; ++i) {
    memcpy(snapS + i * sS, pool_S + (size_t)src[i] * sS, sizeof(double) * sS);
    memcpy(snapW + i * sW, pool_conv + (size_t)src[i] * sW, sizeof(double) * sW);
  }
  for (int i = 0; i < n; ++i) {
    memcpy(pool_S + (size_t)dst[i] * sS, snapS + i * sS, sizeof(double) * sS);
    memcpy(pool_conv + (size_t)dst[i] * sW, snapW + i * sW, sizeof(double) * sW);
  }
  free(snapS); free(snapW);
  return 0;
}
