/*
 * Oracle for the Domino draft-head path.  TEST INFRASTRUCTURE ONLY: the
 * product path never links, loads or calls this file; only the tests, the
 * smoke check and the bench's CPU-baseline leg do.
 *
 * Plain, slow, obviously correct CPU code.  Every sum is taken in double;
 * bf16 inputs are widened exactly (bits << 16); results that the GPU stores
 * as fp32 are rounded once, at the end.  No blocking, no fusion, no
 * reordering beyond the definitions cited on each function.  OpenMP only
 * splits independent outer loops (vocabulary rows, GRU units).
 *
 * Sources (the pages are web summaries of the Domino paper, arXiv
 * 2605.29707, and of DominoTree, arXiv 2607.08642):
 *   [Domino/nl]  gist.science Dutch summary, "Methodologie: Domino",
 *                parts 1 (parallel draft backbone) and 2 (Domino-head).
 *   [Domino/zh]  163.com explainer, sections 3 and 4 (Domino head).
 *   [Domino/ko]  dimensionstp.github.io review, section 3-2 (module
 *                breakdown, final-logits equation).
 *   [Tree/zh]    gist.science Chinese DominoTree summary, technical
 *                abstract, "方法论 / 核心组件" (conditional best-first heap,
 *                top-M candidate restriction).
 *
 * Readings taken where the pages are silent: GRU in the torch.nn.GRUCell form with gate blocks
 * (r, z, n); initial state zero; the first GRU input is the anchor token;
 * concat order [H_i ; S]; argmax ties go to the lowest index; tree
 * children scored by a log-softmax over the M corrected candidate logits,
 * heap key (score desc, parent index asc, candidate rank asc).
 *
 * Sampling at temperature T > 0 (the pages report decoding at T = 1 next
 * to greedy decoding: 163.com explainer, section 6; DominoTree summary,
 * experiments at T in {0, 0.5, 1}) is written as the Gumbel-max trick:
 * argmax_v (L_v + T g_v) with g_v standard Gumbel noise, which draws v with
 * probability softmax(L / T)_v.  The noise comes from the counter-based
 * generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), written here from that
 * definition; its counter layout is fixed below so the GPU path can draw
 * the same numbers from its own implementation.
 *
 * Verification inputs of a drafted tree follow the standard tree-attention
 * verification that DominoTree reuses unchanged (DominoTree summary,
 * "方法论 / 核心组件", verification: an ancestor-only causal mask).
 *
 * Parity pins: tests/test_oracle_*.py (hand values, torch float64
 * library routines, brute-force tree enumeration, closed forms, the
 * generator's published known-answer vectors, distribution tests).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t hidden;     /* d  */
  int32_t vocab;      /* V  */
  int32_t gru_hidden; /* Hs */
  int32_t rank;       /* r  */
  int32_t block;      /* P  */
  int32_t dtype;      /* 0 = fp32 storage, 1 = bf16 storage (H and all weight matrices) */
} od_dims;

typedef struct {
  const void *lm_head;  /* [V][d]            */
  const void *embed;    /* [V][d]            */
  const void *w_ih;     /* [3Hs][d]  r, z, n */
  const void *w_hh;     /* [3Hs][Hs] r, z, n */
  const float *b_ih;    /* [3Hs] or NULL     */
  const float *b_hh;    /* [3Hs] or NULL     */
  const void *w1;       /* [r][d+Hs]         */
  const float *b1;      /* [r] or NULL       */
  const void *w2;       /* [V][r]            */
  const float *b2;      /* [V] or NULL       */
} od_weights;

/* exact value of element i of a stored fp32 or bf16 array */
static double elem(const void *base, int dtype, size_t i) {
  if (dtype == 0) return (double)((const float *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double bias(const float *b, size_t i) { return b ? (double)b[i] : 0.0; }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* SiLU(z) = z * sigmoid(z)  [Domino/zh s4; Domino/nl low-rank head] */
double oracle_silu(double z) { return z * oracle_sigmoid(z); }

/*
 * Base logits through the frozen LM head, all block positions at once:
 *   Lb[m][v] = sum_k H[m][k] * W_lm[v][k]          [Domino/nl part 1; Domino/zh s3]
 * H holds `rows` rows of length d.  Result rounded once to fp32.
 */
void oracle_base_logits(const od_dims *D, const void *lm_head, const void *H, int32_t rows, float *out) {
  const int d = D->hidden, V = D->vocab, dt = D->dtype;
#pragma omp parallel for schedule(static)
  for (int v = 0; v < V; ++v) {
    for (int m = 0; m < rows; ++m) {
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += elem(H, dt, (size_t)m * d + k) * elem(lm_head, dt, (size_t)v * d + k);
      out[(size_t)m * V + v] = (float)s;
    }
  }
}

/*
 * One GRU step, torch.nn.GRUCell form (gate blocks r, z, n):
 *   r  = sigmoid(W_ir x + b_ir + W_hr h + b_hr)
 *   z  = sigmoid(W_iz x + b_iz + W_hz h + b_hz)
 *   n  = tanh(W_in x + b_in + r * (W_hn h + b_hn))
 *   h' = (1 - z) * n + z * h
 * The causal encoder is a GRU of width Hs that reads the embeddings of the
 * drafted tokens one at a time [Domino/zh s4; Domino/nl part 2].
 * x has d entries, h and out have Hs entries (out may not alias h).
 */
void oracle_gru_cell(const od_dims *D, const od_weights *W, const double *x, const double *h, double *out) {
  const int d = D->hidden, Hs = D->gru_hidden, dt = D->dtype;
#pragma omp parallel for schedule(static)
  for (int j = 0; j < Hs; ++j) {
    double gi[3], gh[3];
    for (int g = 0; g < 3; ++g) {
      const size_t row = (size_t)g * Hs + j;
      double si = bias(W->b_ih, row), sh = bias(W->b_hh, row);
      for (int k = 0; k < d; ++k) si += elem(W->w_ih, dt, row * d + k) * x[k];
      for (int k = 0; k < Hs; ++k) sh += elem(W->w_hh, dt, row * Hs + k) * h[k];
      gi[g] = si;
      gh[g] = sh;
    }
    const double r = oracle_sigmoid(gi[0] + gh[0]);
    const double z = oracle_sigmoid(gi[1] + gh[1]);
    const double n = tanh(gi[2] + r * gh[2]);
    out[j] = (1.0 - z) * n + z * h[j];
  }
}

/*
 * Low-rank bottleneck of the correction head on the concatenation [H_i ; S]:
 *   a = SiLU(W1 [H_i ; S] + b1)                     [Domino/nl part 2; Domino/zh s4]
 * Hrow is one stored row of H (d entries), S the GRU state (Hs), a has r entries.
 */
void oracle_head_bottleneck(const od_dims *D, const od_weights *W, const void *Hrow, const double *S, double *a) {
  const int d = D->hidden, Hs = D->gru_hidden, r = D->rank, dt = D->dtype;
  const int in = d + Hs;
#pragma omp parallel for schedule(static)
  for (int k = 0; k < r; ++k) {
    double s = bias(W->b1, k);
    for (int i = 0; i < d; ++i) s += elem(W->w1, dt, (size_t)k * in + i) * elem(Hrow, dt, i);
    for (int j = 0; j < Hs; ++j) s += elem(W->w1, dt, (size_t)k * in + d + j) * S[j];
    a[k] = oracle_silu(s);
  }
}

/*
 * Final logits of one position: L = Lb + dL with dL = W2 a + b2
 *                                             [Domino/nl part 2; Domino/ko 3-2 eq.]
 * Lbrow is the fp32 base-logit row (V entries), out has V entries.
 */
void oracle_final_logits(const od_dims *D, const od_weights *W, const float *Lbrow, const double *a, double *out) {
  const int V = D->vocab, r = D->rank, dt = D->dtype;
#pragma omp parallel for schedule(static)
  for (int v = 0; v < V; ++v) {
    double s = bias(W->b2, v);
    for (int k = 0; k < r; ++k) s += elem(W->w2, dt, (size_t)v * r + k) * a[k];
    out[v] = (double)Lbrow[v] + s;
  }
}

/* greedy token: first index of the maximum; margin = best minus runner-up */
int32_t oracle_argmax(const double *L, int32_t n, double *margin) {
  int32_t best = 0;
  for (int32_t v = 1; v < n; ++v)
    if (L[v] > L[best]) best = v;
  if (margin) {
    double second = -INFINITY;
    for (int32_t v = 0; v < n; ++v)
      if (v != best && L[v] > second) second = L[v];
    *margin = n > 1 ? L[best] - second : INFINITY;
  }
  return best;
}

/*
 * The sequential correction chain over one draft block, for B sequences.
 * Position p uses the GRU state after reading t0, tok[0], ..., tok[p-1]
 * (the encoder starts at the block's first position and, at position i,
 * holds the tokens before i [Domino/zh s4]); the token fed back is the one
 * just drafted, or forced[b][p] when a forced prefix is given (the
 * teacher-forced reading of [Domino/nl, Trainingsstrategie 1]).
 *   H      [B][P][d]   stored dtype
 *   Lb     [B][P][V]   fp32
 *   t0     [B]
 *   forced [B][P] or NULL
 * Outputs: tokens [B][P]; logits [B][P][V] (double) or NULL;
 *          margins [B][P] (double) or NULL.
 */
void oracle_chain(const od_dims *D, const od_weights *W, int32_t B, const void *H, const float *Lb,
                  const int32_t *t0, const int32_t *forced, int32_t *tokens, double *logits, double *margins) {
  const int d = D->hidden, V = D->vocab, Hs = D->gru_hidden, r = D->rank, P = D->block, dt = D->dtype;
  double *x = malloc(sizeof(double) * d);
  double *h = malloc(sizeof(double) * Hs);
  double *hn = malloc(sizeof(double) * Hs);
  double *a = malloc(sizeof(double) * r);
  double *L = malloc(sizeof(double) * V);
  const size_t hrow_bytes = dt == 0 ? 4 : 2;
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < Hs; ++j) h[j] = 0.0;
    int32_t prev = t0[b];
    for (int p = 0; p < P; ++p) {
      for (int k = 0; k < d; ++k) x[k] = elem(W->embed, dt, (size_t)prev * d + k);
      oracle_gru_cell(D, W, x, h, hn);
      memcpy(h, hn, sizeof(double) * Hs);
      const size_t row = (size_t)b * P + p;
      oracle_head_bottleneck(D, W, (const char *)H + row * d * hrow_bytes, h, a);
      oracle_final_logits(D, W, Lb + row * V, a, L);
      double m;
      const int32_t t = oracle_argmax(L, V, &m);
      tokens[row] = t;
      if (margins) margins[row] = m;
      if (logits) memcpy(logits + row * V, L, sizeof(double) * V);
      prev = forced ? forced[row] : t;
    }
  }
  free(x);
  free(h);
  free(hn);
  free(a);
  free(L);
}

/*
 * Top-M candidates of one base-logit row, ordered by (value desc, index asc).
 * The tree restricts every expansion to the M best marginal candidates of
 * its depth [Tree/zh, Top-M].  Plain insertion into a sorted list.
 */
void oracle_topm(const float *row, int32_t V, int32_t M, int32_t *idx, float *val) {
  int32_t filled = 0;
  for (int32_t v = 0; v < V; ++v) {
    const float x = row[v];
    if (filled == M && !(x > val[M - 1])) continue; /* equal value, larger index: loses */
    int32_t pos = filled < M ? filled : M - 1;
    while (pos > 0 && x > val[pos - 1]) {
      val[pos] = val[pos - 1];
      idx[pos] = idx[pos - 1];
      --pos;
    }
    val[pos] = x;
    idx[pos] = v;
    if (filled < M) ++filled;
  }
}

typedef struct {
  double score;
  int32_t parent; /* index of the popped parent, -1 for the anchor */
  int32_t rank;   /* position of the token in its depth's candidate list */
  int32_t token;
  int32_t depth;  /* 1-based; the node was scored with base-logit row depth-1 */
} od_entry;

/* heap order: higher score first, then lower parent index, then lower rank */
static int od_before(const od_entry *a, const od_entry *b) {
  if (a->score != b->score) return a->score > b->score;
  if (a->parent != b->parent) return a->parent < b->parent;
  return a->rank < b->rank;
}

/*
 * Push the M children of one node.  The node sits at depth delta with GRU
 * state S; its children are scored on block position delta:
 *   l_j = Lb[delta][C_j] + (W2 a)[C_j] + b2[C_j],  a = SiLU(W1 [H_delta ; S] + b1)
 *   child score = parent score + l_j - logsumexp_j(l)
 * Only the M candidate columns of W2 are touched [Tree/zh, Top-M].
 */
static void expand(const od_dims *D, const od_weights *W, const void *Hrow, const float *Lbrow, const int32_t *cand,
                   int32_t M, const double *S, double parent_score, int32_t node, int32_t delta, double *a, double *l,
                   od_entry *heap, int32_t *nheap) {
  const int r = D->rank, dt = D->dtype;
  oracle_head_bottleneck(D, W, Hrow, S, a);
  double mx = -INFINITY;
  for (int j = 0; j < M; ++j) {
    const int32_t c = cand[j];
    double s = (double)Lbrow[c] + bias(W->b2, c);
    for (int k = 0; k < r; ++k) s += elem(W->w2, dt, (size_t)c * r + k) * a[k];
    l[j] = s;
    if (s > mx) mx = s;
  }
  double se = 0.0;
  for (int j = 0; j < M; ++j) se += exp(l[j] - mx);
  const double lse = mx + log(se);
  for (int j = 0; j < M; ++j) {
    od_entry e = {parent_score + (l[j] - lse), node, j, cand[j], delta + 1};
    heap[(*nheap)++] = e;
  }
}

/*
 * Best-first draft tree with per-path (conditional) scoring
 * [Tree/zh, conditional best-first heap; Top-M].
 * For each sequence the anchor t0 is the root (not counted); its state is
 * GRU(E[t0], 0) and it is expanded at depth 0.  The entry popped k-th
 * becomes node k; unless it sits at depth P or is the last of the budget,
 * its state GRU(E[token], S_parent) is formed and it is expanded.
 * Slots left when the tree runs out of nodes hold parent -1, token -1,
 * depth 0, score -inf.
 * Outputs [B][N]: parents, tokens, depth (may be NULL), scores (may be NULL).
 */
void oracle_tree(const od_dims *D, const od_weights *W, int32_t B, const void *H, const float *Lb,
                 const int32_t *t0, int32_t N, int32_t M, int32_t *parents, int32_t *tokens, int32_t *depth,
                 double *scores) {
  const int d = D->hidden, V = D->vocab, Hs = D->gru_hidden, r = D->rank, P = D->block, dt = D->dtype;
  const size_t hrow_bytes = dt == 0 ? 4 : 2;
  int32_t *cand = malloc(sizeof(int32_t) * (size_t)P * M);
  float *cval = malloc(sizeof(float) * (size_t)P * M);
  double *state = malloc(sizeof(double) * (size_t)(N + 1) * Hs); /* slot 0: anchor, slot k+1: node k */
  double *x = malloc(sizeof(double) * d);
  double *zero = calloc((size_t)Hs, sizeof(double));
  double *a = malloc(sizeof(double) * r);
  double *l = malloc(sizeof(double) * M);
  od_entry *heap = malloc(sizeof(od_entry) * (size_t)(N + 1) * M);

  for (int b = 0; b < B; ++b) {
    const float *Lb_b = Lb + (size_t)b * P * V;
    const char *H_b = (const char *)H + (size_t)b * P * d * hrow_bytes;
    for (int p = 0; p < P; ++p) oracle_topm(Lb_b + (size_t)p * V, V, M, cand + (size_t)p * M, cval + (size_t)p * M);

    int32_t nheap = 0;
    for (int i = 0; i < d; ++i) x[i] = elem(W->embed, dt, (size_t)t0[b] * d + i);
    oracle_gru_cell(D, W, x, zero, state);
    if (P > 0) expand(D, W, H_b, Lb_b, cand, M, state, 0.0, -1, 0, a, l, heap, &nheap);

    for (int k = 0; k < N; ++k) {
      const size_t o = (size_t)b * N + k;
      if (nheap == 0) {
        parents[o] = -1;
        tokens[o] = -1;
        if (depth) depth[o] = 0;
        if (scores) scores[o] = -INFINITY;
        continue;
      }
      int best = 0;
      for (int i = 1; i < nheap; ++i)
        if (od_before(&heap[i], &heap[best])) best = i;
      const od_entry e = heap[best];
      heap[best] = heap[--nheap];
      parents[o] = e.parent;
      tokens[o] = e.token;
      if (depth) depth[o] = e.depth;
      if (scores) scores[o] = e.score;
      if (e.depth < P && k + 1 < N) {
        double *S = state + (size_t)(k + 1) * Hs;
        for (int i = 0; i < d; ++i) x[i] = elem(W->embed, dt, (size_t)e.token * d + i);
        oracle_gru_cell(D, W, x, state + (size_t)(e.parent + 1) * Hs, S);
        const int32_t delta = e.depth;
        expand(D, W, H_b + (size_t)delta * d * hrow_bytes, Lb_b + (size_t)delta * V, cand + (size_t)delta * M, M, S,
               e.score, k, delta, a, l, heap, &nheap);
      }
    }
  }
  free(cand);
  free(cval);
  free(state);
  free(x);
  free(zero);
  free(a);
  free(l);
  free(heap);
}

/* ---- sampling at temperature T ------------------------------------------------ */

/*
 * Philox4x32-10: 10 rounds on a 128-bit counter (c0..c3) under a 64-bit key
 * (k0, k1).  A round multiplies c0 and c2 by the constants 0xD2511F53 and
 * 0xCD9E8D57 into 64-bit products (hi, lo) and returns
 *   (hi(c2 M1) ^ c1 ^ k0, lo(c2 M1), hi(c0 M0) ^ c3 ^ k1, lo(c0 M0));
 * before every round after the first the key is advanced by the Weyl
 * constants (0x9E3779B9, 0xBB67AE85).
 */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/*
 * The standard Gumbel noise of sequence b (its index in the whole batch),
 * block position p and vocabulary entry v under `seed`:
 *   x = word (b & 1) of Philox4x32-10(counter (v, p, b >> 1, 0), key (seed lo, seed hi)),
 *   u = (2 (x >> 9) + 1) / 2^24          (in (0, 1), exact in fp32),
 *   g = -log(-log(u)).
 */
double oracle_gumbel(uint64_t seed, int32_t b, int32_t p, int32_t v) {
  const uint32_t ctr[4] = {(uint32_t)v, (uint32_t)p, (uint32_t)b >> 1, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t x[4];
  oracle_philox4x32_10(ctr, key, x);
  const double u = (2.0 * (double)(x[b & 1] >> 9) + 1.0) / 16777216.0;
  return -log(-log(u));
}

/*
 * The correction chain with the token of every position drawn at
 * temperature T >= 0 (Gumbel-max): the chain of oracle_chain, except that
 *   tokens[b][p] = argmax_v (L[b][p][v] + T g(seed, b, p, v))
 * (first index on exact ties) and the token fed back is that draw (or
 * forced[b][p]).  T = 0 is the greedy chain.  logits are the unperturbed L;
 * margins are the top-2 margins of the perturbed values.  b counts from
 * `seq0` in the whole batch (the noise depends on it).
 */
void oracle_chain_sampled(const od_dims *D, const od_weights *W, int32_t B, int32_t seq0, const void *H,
                          const float *Lb, const int32_t *t0, const int32_t *forced, double temperature,
                          uint64_t seed, int32_t *tokens, double *logits, double *margins) {
  const int d = D->hidden, V = D->vocab, Hs = D->gru_hidden, r = D->rank, P = D->block, dt = D->dtype;
  double *x = malloc(sizeof(double) * d);
  double *h = malloc(sizeof(double) * Hs);
  double *hn = malloc(sizeof(double) * Hs);
  double *a = malloc(sizeof(double) * r);
  double *L = malloc(sizeof(double) * V);
  double *Lp = malloc(sizeof(double) * V);
  const size_t hrow_bytes = dt == 0 ? 4 : 2;
  for (int b = 0; b < B; ++b) {
    for (int j = 0; j < Hs; ++j) h[j] = 0.0;
    int32_t prev = t0[b];
    for (int p = 0; p < P; ++p) {
      for (int k = 0; k < d; ++k) x[k] = elem(W->embed, dt, (size_t)prev * d + k);
      oracle_gru_cell(D, W, x, h, hn);
      memcpy(h, hn, sizeof(double) * Hs);
      const size_t row = (size_t)b * P + p;
      oracle_head_bottleneck(D, W, (const char *)H + row * d * hrow_bytes, h, a);
      oracle_final_logits(D, W, Lb + row * V, a, L);
#pragma omp parallel for schedule(static)
      for (int v = 0; v < V; ++v) Lp[v] = temperature > 0.0 ? L[v] + temperature * oracle_gumbel(seed, seq0 + b, p, v) : L[v];
      double m;
      const int32_t t = oracle_argmax(Lp, V, &m);
      tokens[row] = t;
      if (margins) margins[row] = m;
      if (logits) memcpy(logits + row * V, L, sizeof(double) * V);
      prev = forced ? forced[row] : t;
    }
  }
  free(x);
  free(h);
  free(hn);
  free(a);
  free(L);
  free(Lp);
}

/* ---- verification inputs of a drafted tree ------------------------------------------ */

/*
 * The flattened tree of one sequence as the target model verifies it:
 * entry 0 is the anchor, entry k + 1 is node k.  Node k is part of the tree
 * when its token is >= 0 and its parent is the anchor (-1) or an earlier
 * node (0 <= parent < k) that is itself part of the tree; other slots are
 * padding.  For a tree node, its depth is 1 + its parent's (anchor 0).
 *   out_tokens[i]    anchor token, node tokens; -1 for padding
 *   out_positions[i] start + depth; -1 for padding
 *   out_mask[i][j]   1 when entry j is entry i itself or one of its
 *                    ancestors (the anchor is an ancestor of every tree
 *                    node); a padding row holds only its own diagonal
 * Arrays per sequence: parents, tokens [N]; out_mask [N+1][N+1] bytes,
 * out_positions and out_tokens [N+1].
 */
void oracle_tree_verify_inputs(int32_t B, int32_t N, const int32_t *parents, const int32_t *tokens,
                               const int32_t *first_tokens, const int32_t *start_positions, uint8_t *out_mask,
                               int32_t *out_positions, int32_t *out_tokens) {
  const int E = N + 1;
  int32_t *depth = malloc(sizeof(int32_t) * (size_t)E);
  int32_t *in_tree = malloc(sizeof(int32_t) * (size_t)E);
  for (int b = 0; b < B; ++b) {
    const int32_t *par = parents + (size_t)b * N, *tok = tokens + (size_t)b * N;
    uint8_t *mask = out_mask + (size_t)b * E * E;
    const int32_t start = start_positions ? start_positions[b] : 0;
    in_tree[0] = 1;
    depth[0] = 0;
    for (int k = 0; k < N; ++k) {
      const int32_t q = par[k];
      const int ok = tok[k] >= 0 && q >= -1 && q < k && in_tree[q + 1];
      in_tree[k + 1] = ok;
      depth[k + 1] = ok ? depth[q + 1] + 1 : 0;
    }
    for (int i = 0; i < E; ++i) {
      for (int j = 0; j < E; ++j) mask[(size_t)i * E + j] = 0;
      mask[(size_t)i * E + i] = 1;
      if (in_tree[i] && i > 0) {
        /* walk up the parent links to the anchor */
        int e = i;
        while (e != 0) {
          e = par[e - 1] + 1;
          mask[(size_t)i * E + e] = 1;
        }
      }
      out_positions[(size_t)b * E + i] = in_tree[i] ? start + depth[i] : -1;
      out_tokens[(size_t)b * E + i] = i == 0 ? first_tokens[b] : (in_tree[i] ? tok[i - 1] : -1);
    }
  }
  free(depth);
  free(in_tree);
}
