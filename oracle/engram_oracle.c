/*
 * Engram conditional-memory forward pass (and its gradients): the ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, single-threaded
 * definition of what the forward pass computes, written from the two Engram
 * pages (the architecture walk-through at yaoyuxiang.cn/news/830577 and the
 * formula sheet at kwkr.cn/news/37585).  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark load it; the product library never
 * does, and the two share no code.
 *
 * Arithmetic: integers exactly (64-bit two's complement, as the pages' numpy
 * int64 code); every real-valued step in double precision, reading inputs in
 * their stored type (float32 or bfloat16) and keeping intermediates in double.
 * No blocking, fusion or reordering beyond the definitions below.
 *
 * Readings where the pages are silent or garbled (each fixed once here):
 *  - the token k positions back is multiplied by multiplier m_k (so m_0 goes
 *    with the current token), one multiplier array shared by every order and
 *    head; heads of one order differ only in their prime modulus;
 *  - the mix is wrapping int64 and "mod" is the floored modulo of numpy, so
 *    hash indices lie in [0, p);
 *  - positions before the start of a sequence hash pad_id (never masked);
 *  - e_t concatenates the rows order by order, head by head within an order;
 *  - the key and value projections have no bias;
 *  - RMSNorm is x * (mean(x^2) + eps)^-1/2 * gamma with a learnable gamma per
 *    branch; the d in 1/sqrt(d) is the hidden size;
 *  - the short conv is linear, depthwise over hc*d channels, causal with zero
 *    history, taps w[..][j] applied to position t - (K-1-j)*dilation, no bias;
 *  - the module returns V_gated + Conv(V_gated) (no add into the hidden state).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MAX_ORDERS 8
#define ORC_MAX_HEADS 64

typedef struct {
  int32_t batch, seqlen;
  int32_t n_orders;
  int32_t orders[ORC_MAX_ORDERS];  /* ascending n-gram orders, each >= 1 */
  int32_t heads_per_order;         /* K hash heads per order */
  int32_t head_dim;                /* Dh, embedding width of one head */
  int32_t hidden, hc_mult;         /* d, number of branches */
  int32_t conv_kernel, conv_dilation;
  int32_t pad_id;
  int32_t dtype;                   /* storage of real inputs: 0 float32, 1 bfloat16 bits */
  double norm_eps, gate_clamp;
  int64_t multipliers[ORC_MAX_ORDERS];
  int64_t primes[ORC_MAX_HEADS];   /* p_{n,j}, order-major */
} orc_config;

/* A row source: dense (keys == NULL, row r at data + r*row_elems) or sparse
 * (keys[i] ascending; the row with key keys[i] is at data + i*row_elems). */
typedef struct {
  const void *data;
  const int64_t *keys;
  int64_t n;
} orc_rows;

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_EMISSING = -2, ORC_ENOMEM = -3 };

static int max_order(const orc_config *c) { return c->orders[c->n_orders - 1]; }
static int n_heads(const orc_config *c) { return c->n_orders * c->heads_per_order; }

static int check(const orc_config *c) {
  if (c->batch < 0 || c->seqlen < 0 || c->n_orders < 1 || c->n_orders > ORC_MAX_ORDERS) return ORC_EINVAL;
  if (c->heads_per_order < 1 || n_heads(c) > ORC_MAX_HEADS) return ORC_EINVAL;
  for (int i = 0; i < c->n_orders; i++)
    if (c->orders[i] < 1 || (i && c->orders[i] <= c->orders[i - 1])) return ORC_EINVAL;
  for (int h = 0; h < n_heads(c); h++)
    if (c->primes[h] < 1) return ORC_EINVAL;
  if (c->head_dim < 1 || c->hidden < 1 || c->hc_mult < 1 || c->conv_kernel < 1 || c->conv_dilation < 1)
    return ORC_EINVAL;
  return ORC_OK;
}

/* stored element i of a real array, as a double */
static double ld(const void *p, int64_t i, int dtype) {
  if (dtype == 0) return (double)((const float *)p)[i];
  uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static const void *row_ptr(const orc_rows *r, int64_t key, int64_t row_bytes) {
  if (r->keys == NULL) {
    if (key < 0 || key >= r->n) return NULL;
    return (const char *)r->data + key * row_bytes;
  }
  int64_t lo = 0, hi = r->n - 1;
  while (lo <= hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (r->keys[mid] == key) return (const char *)r->data + mid * row_bytes;
    if (r->keys[mid] < key) lo = mid + 1; else hi = mid - 1;
  }
  return NULL;
}

/* Time shift (formula sheet, section 4.2): shift_k(x)[b][t] = x[b][t-k] for
 * t >= k; before the start it is hist[b][(max_order-1) + t - k] when a token
 * history (oldest first) is given, else pad_id. */
int orc_shift(const orc_config *c, const int32_t *x, const int32_t *hist, int k, int32_t *out) {
  if (check(c) || k < 0 || k >= max_order(c)) return ORC_EINVAL;
  const int H = max_order(c) - 1;
  for (int64_t b = 0; b < c->batch; b++)
    for (int64_t t = 0; t < c->seqlen; t++) {
      int32_t v;
      if (t - k >= 0) v = x[b * c->seqlen + t - k];
      else if (hist) v = hist[b * H + H + (t - k)];
      else v = c->pad_id;
      out[b * c->seqlen + t] = v;
    }
  return ORC_OK;
}

/* Floored modulo of a signed 64-bit value by p > 0 (numpy's `%`). */
static int64_t floor_mod(int64_t a, int64_t p) {
  int64_t r = a % p;           /* C truncates toward zero */
  if (r < 0) r += p;
  return r;
}

/* Compressed-token remap + shifts + multi-head n-gram hash (formula sheet,
 * section 1.2 steps 1-2 and the full formula in 1.3; walk-through section
 * 4.2).  For order n and head j of that order:
 *   mix  = (s_0 * m_0) xor (s_1 * m_1) xor ... xor (s_{n-1} * m_{n-1})
 *   idx  = mix mod p_{n,j}
 * with s_k = shift_k(x)[b][t] and wrapping int64 products.
 * remap == NULL means ids are already compressed.  idx: [B][T][H] int64. */
int orc_hash(const orc_config *c, const int32_t *remap, int32_t vocab, const int32_t *ids,
             const int32_t *hist, int64_t *idx) {
  if (check(c)) return ORC_EINVAL;
  const int64_t n = (int64_t)c->batch * c->seqlen;
  const int mo = max_order(c), H = n_heads(c);
  if (n == 0) return ORC_OK;
  int32_t *x = malloc(sizeof(int32_t) * n);
  int32_t *sh = malloc(sizeof(int32_t) * n * mo);
  if (!x || !sh) { free(x); free(sh); return ORC_ENOMEM; }
  for (int64_t i = 0; i < n; i++) {
    if (remap) {
      if (ids[i] < 0 || ids[i] >= vocab) { free(x); free(sh); return ORC_EINVAL; }
      x[i] = remap[ids[i]];
    } else {
      x[i] = ids[i];
    }
  }
  for (int k = 0; k < mo; k++) orc_shift(c, x, hist, k, sh + k * n);
  for (int64_t i = 0; i < n; i++) {
    int h = 0;
    for (int oi = 0; oi < c->n_orders; oi++) {
      const int order = c->orders[oi];
      uint64_t mix = 0;
      for (int k = 0; k < order; k++) {
        uint64_t tok = (uint64_t)(int64_t)sh[k * n + i];
        mix ^= tok * (uint64_t)c->multipliers[k];
      }
      for (int j = 0; j < c->heads_per_order; j++, h++)
        idx[i * H + h] = floor_mod((int64_t)mix, c->primes[h]);
    }
  }
  free(x);
  free(sh);
  return ORC_OK;
}

/* First table row of each head: heads are stacked order-major in one table. */
static void head_offsets(const orc_config *c, int64_t *off) {
  int64_t acc = 0;
  for (int h = 0; h < n_heads(c); h++) { off[h] = acc; acc += c->primes[h]; }
}

/* Multi-head embedding lookup and concatenation into e_t (walk-through
 * sections 2.2-1 and 4.3): e[t][h*Dh + i] = table[off_h + idx[t][h]][i],
 * copied bit for bit in the stored type. */
int orc_gather(const orc_config *c, const orc_rows *table, const int64_t *idx, int64_t n_tok, void *e_out) {
  if (check(c)) return ORC_EINVAL;
  const int H = n_heads(c), Dh = c->head_dim;
  const int64_t esz = c->dtype == 0 ? 4 : 2, row_bytes = esz * Dh;
  int64_t off[ORC_MAX_HEADS];
  head_offsets(c, off);
  for (int64_t t = 0; t < n_tok; t++)
    for (int h = 0; h < H; h++) {
      const int64_t r = idx[t * H + h];
      if (r < 0 || r >= c->primes[h]) return ORC_EINVAL;
      const void *src = row_ptr(table, off[h] + r, row_bytes);
      if (!src) return ORC_EMISSING;
      memcpy((char *)e_out + (t * H + h) * row_bytes, src, row_bytes);
    }
  return ORC_OK;
}

/* Key projections of every branch and the shared value projection (formula
 * sheet 2.2 steps 1 and 3): kv[t][o] = sum_i W[o][i] * e[t][i], rows o of W
 * being hc blocks of d key rows followed by d value rows. */
int orc_project(const orc_config *c, const void *w_kv, const void *e, int64_t n_tok, double *kv) {
  if (check(c)) return ORC_EINVAL;
  const int64_t E = (int64_t)n_heads(c) * c->head_dim, O = (int64_t)(c->hc_mult + 1) * c->hidden;
  for (int64_t t = 0; t < n_tok; t++)
    for (int64_t o = 0; o < O; o++) {
      double acc = 0.0;
      for (int64_t i = 0; i < E; i++) acc += ld(w_kv, o * E + i, c->dtype) * ld(e, t * E + i, c->dtype);
      kv[t * O + o] = acc;
    }
  return ORC_OK;
}

/* Context-aware gate (formula sheet 2.2 steps 1-2 and 2.3), per token t and
 * branch h with K = key of branch h and Q = hidden[t][h]:
 *   s = sum_c RMSNorm_k(K)_c * RMSNorm_q(Q)_c / sqrt(d)
 *   g = sigmoid(sign(s) * sqrt(max(|s|, clamp)))
 * score (nullable) receives s. */
int orc_gate(const orc_config *c, const void *gamma_k, const void *gamma_q, const double *kv, const void *hidden,
             int64_t n_tok, double *score, double *g) {
  if (check(c)) return ORC_EINVAL;
  const int hc = c->hc_mult;
  const int64_t d = c->hidden, O = (int64_t)(hc + 1) * d;
  for (int64_t t = 0; t < n_tok; t++)
    for (int h = 0; h < hc; h++) {
      const double *K = kv + t * O + (int64_t)h * d;
      const int64_t q0 = (t * hc + h) * d;
      double kk = 0.0, qq = 0.0;
      for (int64_t i = 0; i < d; i++) {
        const double q = ld(hidden, q0 + i, c->dtype);
        kk += K[i] * K[i];
        qq += q * q;
      }
      const double rk = 1.0 / sqrt(kk / (double)d + c->norm_eps);
      const double rq = 1.0 / sqrt(qq / (double)d + c->norm_eps);
      double dot = 0.0;
      for (int64_t i = 0; i < d; i++) {
        const double kn = K[i] * rk * ld(gamma_k, (int64_t)h * d + i, c->dtype);
        const double qn = ld(hidden, q0 + i, c->dtype) * rq * ld(gamma_q, (int64_t)h * d + i, c->dtype);
        dot += kn * qn;
      }
      const double s = dot / sqrt((double)d);
      const double sgn = s > 0.0 ? 1.0 : (s < 0.0 ? -1.0 : 0.0);
      const double a = sgn * sqrt(fmax(fabs(s), c->gate_clamp));
      if (score) score[t * hc + h] = s;
      g[t * hc + h] = 1.0 / (1.0 + exp(-a));
    }
  return ORC_OK;
}

/* Value fusion, short conv and residual (formula sheet 2.2 step 3 and 3.2;
 * walk-through 2.2-3): Vg[t][h][c] = g[t][h] * V[t][c] and
 *   y[t][h][c] = Vg[t][h][c] + sum_j w[h][c][j] * Vg[t - (K-1-j)*D][h][c]
 * with Vg = 0 before the start of the sequence. kv/g/y are [B][T][..]. */
int orc_conv(const orc_config *c, const void *conv_w, const double *kv, const double *g, double *y) {
  if (check(c)) return ORC_EINVAL;
  const int hc = c->hc_mult, K = c->conv_kernel, D = c->conv_dilation;
  const int64_t d = c->hidden, O = (int64_t)(hc + 1) * d, T = c->seqlen;
  for (int64_t b = 0; b < c->batch; b++)
    for (int64_t t = 0; t < T; t++)
      for (int h = 0; h < hc; h++)
        for (int64_t ch = 0; ch < d; ch++) {
          const int64_t n = b * T + t;
          double acc = g[n * hc + h] * kv[n * O + (int64_t)hc * d + ch];
          for (int j = 0; j < K; j++) {
            const int64_t tau = t - (int64_t)(K - 1 - j) * D;
            if (tau < 0) continue;
            const int64_t m = b * T + tau;
            const double vg = g[m * hc + h] * kv[m * O + (int64_t)hc * d + ch];
            acc += ld(conv_w, ((int64_t)h * d + ch) * K + j, c->dtype) * vg;
          }
          y[(n * hc + h) * d + ch] = acc;
        }
  return ORC_OK;
}

/* The whole module over dense arrays (walk-through 4.3, Engram.forward). */
int orc_forward(const orc_config *c, const int32_t *remap, int32_t vocab, const int32_t *ids, const orc_rows *table,
                const void *w_kv, const void *gamma_k, const void *gamma_q, const void *conv_w, const void *hidden,
                double *y) {
  if (check(c)) return ORC_EINVAL;
  const int64_t n = (int64_t)c->batch * c->seqlen;
  if (n == 0) return ORC_OK;
  const int H = n_heads(c), hc = c->hc_mult;
  const int64_t E = (int64_t)H * c->head_dim, O = (int64_t)(hc + 1) * c->hidden;
  const int64_t esz = c->dtype == 0 ? 4 : 2;
  int64_t *idx = malloc(sizeof(int64_t) * n * H);
  void *e = malloc(esz * n * E);
  double *kv = malloc(sizeof(double) * n * O), *g = malloc(sizeof(double) * n * hc);
  int rc = ORC_ENOMEM;
  if (idx && e && kv && g) {
    rc = orc_hash(c, remap, vocab, ids, NULL, idx);
    if (!rc) rc = orc_gather(c, table, idx, n, e);
    if (!rc) rc = orc_project(c, w_kv, e, n, kv);
    if (!rc) rc = orc_gate(c, gamma_k, gamma_q, kv, hidden, n, NULL, g);
    if (!rc) rc = orc_conv(c, conv_w, kv, g, y);
  }
  free(idx); free(e); free(kv); free(g);
  return rc;
}

static int cmp_i64(const void *a, const void *b) {
  const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
  return (x > y) - (x < y);
}

static int64_t find_key(const int64_t *keys, int64_t n, int64_t key) {
  int64_t lo = 0, hi = n - 1;
  while (lo <= hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (keys[mid] == key) return mid;
    if (keys[mid] < key) lo = mid + 1; else hi = mid - 1;
  }
  return -1;
}

/* The module's output at chosen positions only (flat keys b*T + t), with the
 * table and the hidden states given as row sources (hidden keyed by b*T + t).
 * It evaluates e, K, V and g at every position the causal conv of a chosen
 * position reads, then the same value fusion, conv and residual as
 * orc_conv.  y: [n_pos][hc][d]. */
int orc_forward_at(const orc_config *c, const int32_t *remap, int32_t vocab, const int32_t *ids,
                   const orc_rows *table, const void *w_kv, const void *gamma_k, const void *gamma_q,
                   const void *conv_w, const orc_rows *hidden, int64_t n_pos, const int64_t *pos, double *y) {
  if (check(c)) return ORC_EINVAL;
  const int64_t T = c->seqlen, n = (int64_t)c->batch * T;
  const int H = n_heads(c), hc = c->hc_mult, K = c->conv_kernel, D = c->conv_dilation;
  const int64_t d = c->hidden, E = (int64_t)H * c->head_dim, O = (int64_t)(hc + 1) * d;
  const int64_t esz = c->dtype == 0 ? 4 : 2;
  for (int64_t i = 0; i < n_pos; i++)
    if (pos[i] < 0 || pos[i] >= n) return ORC_EINVAL;
  if (n_pos == 0) return ORC_OK;

  int64_t *idx = malloc(sizeof(int64_t) * n * H);
  int64_t *need = malloc(sizeof(int64_t) * n_pos * K);
  int rc = ORC_ENOMEM;
  if (!idx || !need) goto out0;
  rc = orc_hash(c, remap, vocab, ids, NULL, idx);
  if (rc) goto out0;

  /* every position a chosen output reads */
  int64_t m = 0;
  for (int64_t i = 0; i < n_pos; i++) {
    const int64_t b = pos[i] / T, t = pos[i] % T;
    for (int j = 0; j < K; j++) {
      const int64_t tau = t - (int64_t)(K - 1 - j) * D;
      if (tau >= 0) need[m++] = b * T + tau;
    }
  }
  qsort(need, m, sizeof(int64_t), cmp_i64);
  int64_t u = 0;
  for (int64_t i = 0; i < m; i++)
    if (u == 0 || need[i] != need[u - 1]) need[u++] = need[i];

  void *e = malloc(esz * E);
  void *q = malloc(esz * hc * d);
  double *kv = malloc(sizeof(double) * O);
  double *V = malloc(sizeof(double) * u * d), *g = malloc(sizeof(double) * u * hc);
  if (!e || !q || !kv || !V || !g) { rc = ORC_ENOMEM; goto out1; }
  orc_config one = *c;
  one.batch = 1;
  one.seqlen = 1;
  for (int64_t i = 0; i < u; i++) {
    const int64_t key = need[i];
    rc = orc_gather(&one, table, idx + key * H, 1, e);
    if (rc) goto out1;
    rc = orc_project(&one, w_kv, e, 1, kv);
    if (rc) goto out1;
    const void *hrow = row_ptr(hidden, key, esz * hc * d);
    if (!hrow) { rc = ORC_EMISSING; goto out1; }
    memcpy(q, hrow, esz * hc * d);
    rc = orc_gate(&one, gamma_k, gamma_q, kv, q, 1, NULL, g + i * hc);
    if (rc) goto out1;
    memcpy(V + i * d, kv + (int64_t)hc * d, sizeof(double) * d);
  }
  for (int64_t i = 0; i < n_pos; i++) {
    const int64_t b = pos[i] / T, t = pos[i] % T;
    const int64_t self = find_key(need, u, pos[i]);
    for (int h = 0; h < hc; h++)
      for (int64_t ch = 0; ch < d; ch++) {
        double acc = g[self * hc + h] * V[self * d + ch];
        for (int j = 0; j < K; j++) {
          const int64_t tau = t - (int64_t)(K - 1 - j) * D;
          if (tau < 0) continue;
          const int64_t r = find_key(need, u, b * T + tau);
          acc += ld(conv_w, ((int64_t)h * d + ch) * K + j, c->dtype) * (g[r * hc + h] * V[r * d + ch]);
        }
        y[(i * hc + h) * d + ch] = acc;
      }
  }
  rc = ORC_OK;
out1:
  free(e); free(q); free(kv); free(V); free(g);
out0:
  free(idx); free(need);
  return rc;
}

/* Value fusion and gate backward of one token (the steps "value fusion",
 * "gate" and "RMSNorm" of the gradients below): from dVg [hc][d] and the
 * token's K/V (double [hc+1][d]), query row q [hc][d] (stored type), gates g
 * and scores s [hc], writes dKV [hc+1][d] (dK of each branch, then dV) and
 * d hidden [hc][d], and adds the token's terms to d_gk, d_gq [hc][d] when
 * they are not NULL. */
static void gate_backward_token(const orc_config *c, const double *kv, const void *q, const void *gamma_k,
                                const void *gamma_q, const double *dvg, const double *g, const double *s,
                                double *dkv, double *d_hidden, double *d_gk, double *d_gq) {
  const int hc = c->hc_mult;
  const int64_t d = c->hidden;
  const double *V = kv + (int64_t)hc * d;
  for (int64_t ch = 0; ch < d; ch++) {
    double acc = 0.0;
    for (int h = 0; h < hc; h++) acc += g[h] * dvg[(int64_t)h * d + ch];
    dkv[(int64_t)hc * d + ch] = acc;
  }
  for (int h = 0; h < hc; h++) {
    const double *Kv = kv + (int64_t)h * d;
    const int64_t q0 = (int64_t)h * d;
    double dg = 0.0, kk = 0.0, qq = 0.0;
    for (int64_t ch = 0; ch < d; ch++) {
      const double qv = ld(q, q0 + ch, c->dtype);
      dg += dvg[q0 + ch] * V[ch];
      kk += Kv[ch] * Kv[ch];
      qq += qv * qv;
    }
    const double gv = g[h], sv = s[h];
    const double da = dg * gv * (1.0 - gv);
    const double ds = (sv != 0.0 && fabs(sv) >= c->gate_clamp) ? da / (2.0 * sqrt(fabs(sv))) : 0.0;
    const double rk = 1.0 / sqrt(kk / (double)d + c->norm_eps);
    const double rq = 1.0 / sqrt(qq / (double)d + c->norm_eps);
    const double sd = sqrt((double)d);
    double A = 0.0, B = 0.0;
    for (int64_t ch = 0; ch < d; ch++) {
      const double gk = ld(gamma_k, (int64_t)h * d + ch, c->dtype), gq = ld(gamma_q, (int64_t)h * d + ch, c->dtype);
      const double qv = ld(q, q0 + ch, c->dtype);
      const double u = Kv[ch] * rk * gk, v = qv * rq * gq;
      const double du = ds * v / sd, dv = ds * u / sd;
      A += du * gk * Kv[ch];
      B += dv * gq * qv;
      if (d_gk) d_gk[(int64_t)h * d + ch] += du * Kv[ch] * rk;
      if (d_gq) d_gq[(int64_t)h * d + ch] += dv * qv * rq;
    }
    for (int64_t ch = 0; ch < d; ch++) {
      const double gk = ld(gamma_k, (int64_t)h * d + ch, c->dtype), gq = ld(gamma_q, (int64_t)h * d + ch, c->dtype);
      const double qv = ld(q, q0 + ch, c->dtype);
      const double du = ds * qv * rq * gq / sd, dv = ds * Kv[ch] * rk * gk / sd;
      dkv[(int64_t)h * d + ch] = rk * gk * du - rk * rk * rk * Kv[ch] * A / (double)d;
      d_hidden[q0 + ch] = rq * gq * dv - rq * rq * rq * qv * B / (double)d;
    }
  }
}

/* Gradients of the module's output (the backward pass of a training step;
 * the pages train the module, walk-through 4.4).  Nothing here is on the
 * pages: these are the exact derivatives of the forward definitions above,
 * taken step by step backwards (chain rule), in double precision.  Given
 * dy = dL/dy [B][T][hc][d] (double), with L a scalar loss of y:
 *   conv + residual:  dVg[t] = dy[t] + sum_j w[j] dy[t + (K-1-j)D]  (inside the sequence)
 *                     dw[h][c][j] = sum_t dy[t][h][c] Vg[t - (K-1-j)D][h][c]
 *   value fusion:     dV[t][c] = sum_h g[t][h] dVg[t][h][c],  dg[t][h] = sum_c dVg[t][h][c] V[t][c]
 *   gate:             da = dg g (1-g);  ds = da / (2 sqrt|s|) where |s| >= clamp and s != 0, else 0
 *                     (a = sign(s) sqrt(max(|s|, clamp)) is flat in s inside the clamp)
 *   s = sum_c u_c v_c / sqrt(d), u = K rk gk, v = Q rq gq:
 *                     du = ds v / sqrt(d),  dv = ds u / sqrt(d)
 *   RMSNorm:          dK_c = rk gk_c du_c - rk^3 K_c (sum_i du_i gk_i K_i) / d   (rk = (mean K^2 + eps)^-1/2)
 *                     dgk_c += du_c K_c rk;  likewise dQ (= d hidden) and dgq
 *   projections:      dW[o][i] = sum_t dKV[t][o] e[t][i],  de[t][i] = sum_o dKV[t][o] W[o][i]
 *   gather:           dtable[row of (t, head)] += de[t][that head's slice]
 * Outputs (all overwritten): d_table [sum p][Dh], d_w [(hc+1)d][E], d_gk and
 * d_gq [hc][d], d_cw [hc][d][K], d_hidden [B][T][hc][d]. */
int orc_backward(const orc_config *c, const int32_t *remap, int32_t vocab, const int32_t *ids, const orc_rows *table,
                 const void *w_kv, const void *gamma_k, const void *gamma_q, const void *conv_w, const void *hidden,
                 const double *dy, double *d_table, double *d_w, double *d_gk, double *d_gq, double *d_cw,
                 double *d_hidden) {
  if (check(c)) return ORC_EINVAL;
  const int64_t T = c->seqlen, n = (int64_t)c->batch * T;
  const int H = n_heads(c), hc = c->hc_mult, K = c->conv_kernel, D = c->conv_dilation;
  const int64_t d = c->hidden, Dh = c->head_dim, E = (int64_t)H * Dh, O = (int64_t)(hc + 1) * d;
  const int64_t esz = c->dtype == 0 ? 4 : 2;
  int64_t rows = 0;
  for (int h = 0; h < H; h++) rows += c->primes[h];
  memset(d_table, 0, sizeof(double) * rows * Dh);
  memset(d_w, 0, sizeof(double) * O * E);
  memset(d_gk, 0, sizeof(double) * hc * d);
  memset(d_gq, 0, sizeof(double) * hc * d);
  memset(d_cw, 0, sizeof(double) * hc * d * K);
  if (n == 0) return ORC_OK;

  int64_t *idx = malloc(sizeof(int64_t) * n * H), off[ORC_MAX_HEADS];
  void *e = malloc(esz * n * E);
  double *kv = malloc(sizeof(double) * n * O), *s = malloc(sizeof(double) * n * hc);
  double *g = malloc(sizeof(double) * n * hc), *dvg = malloc(sizeof(double) * n * hc * d);
  double *dkv = malloc(sizeof(double) * n * O), *de = malloc(sizeof(double) * n * E);
  int rc = ORC_ENOMEM;
  if (!idx || !e || !kv || !s || !g || !dvg || !dkv || !de) goto out;
  /* the forward quantities the derivatives use */
  rc = orc_hash(c, remap, vocab, ids, NULL, idx);
  if (!rc) rc = orc_gather(c, table, idx, n, e);
  if (!rc) rc = orc_project(c, w_kv, e, n, kv);
  if (!rc) rc = orc_gate(c, gamma_k, gamma_q, kv, hidden, n, s, g);
  if (rc) goto out;
  head_offsets(c, off);

  /* conv + residual */
  for (int64_t b = 0; b < c->batch; b++)
    for (int64_t t = 0; t < T; t++)
      for (int h = 0; h < hc; h++)
        for (int64_t ch = 0; ch < d; ch++) {
          const int64_t nn = b * T + t;
          const double dyv = dy[(nn * hc + h) * d + ch];
          double acc = dyv;
          for (int j = 0; j < K; j++) {
            const double w = ld(conv_w, ((int64_t)h * d + ch) * K + j, c->dtype);
            const int64_t ahead = t + (int64_t)(K - 1 - j) * D, back = t - (int64_t)(K - 1 - j) * D;
            if (ahead < T) acc += w * dy[((b * T + ahead) * hc + h) * d + ch];
            if (back >= 0) {
              const int64_t m = b * T + back;
              d_cw[((int64_t)h * d + ch) * K + j] += dyv * g[m * hc + h] * kv[m * O + (int64_t)hc * d + ch];
            }
          }
          dvg[(nn * hc + h) * d + ch] = acc;
        }
  /* value fusion and gate */
  for (int64_t nn = 0; nn < n; nn++)
    gate_backward_token(c, kv + nn * O, (const uint8_t *)hidden + nn * hc * d * esz, gamma_k, gamma_q,
                        dvg + nn * hc * d, g + nn * hc, s + nn * hc, dkv + nn * O, d_hidden + nn * hc * d, d_gk, d_gq);
  /* projections */
  for (int64_t o = 0; o < O; o++)
    for (int64_t i = 0; i < E; i++) {
      double acc = 0.0;
      for (int64_t nn = 0; nn < n; nn++) acc += dkv[nn * O + o] * ld(e, nn * E + i, c->dtype);
      d_w[o * E + i] = acc;
    }
  for (int64_t nn = 0; nn < n; nn++)
    for (int64_t i = 0; i < E; i++) {
      double acc = 0.0;
      for (int64_t o = 0; o < O; o++) acc += dkv[nn * O + o] * ld(w_kv, o * E + i, c->dtype);
      de[nn * E + i] = acc;
    }
  /* gather */
  for (int64_t nn = 0; nn < n; nn++)
    for (int h = 0; h < H; h++) {
      const int64_t r = off[h] + idx[nn * H + h];
      for (int64_t j = 0; j < Dh; j++) d_table[r * Dh + j] += de[nn * E + (int64_t)h * Dh + j];
    }
  rc = ORC_OK;
out:
  free(idx); free(e); free(kv); free(s); free(g); free(dvg); free(dkv); free(de);
  return rc;
}

/* The gradients that belong to single positions, at chosen flat positions
 * pos[i] = b*T + t, by the same steps as orc_backward: d_hidden [n_pos][hc][d]
 * and, when de is not NULL, de [n_pos][E], the gradient of the gathered
 * vector e at that position (table row r of head h receives the sum of head
 * h's slice of de over the positions whose index is r).  A position reads e,
 * K, V, g and hidden at itself only, and dy at itself and D, 2D, ...,
 * (K-1)D positions later in its sequence: hidden and dy are row sources keyed
 * by flat position, one [hc][d] row each in the stored type.
 * Optional outputs (each NULL to skip): dkv [n_pos][(hc+1)*d], the gradient of
 * the position's keys and value (the weight gradient is the sum over
 * positions of dkv[p] (x) e[p]); d_gk and d_gq [hc][d], to which the
 * positions' terms of the RMSNorm scales' gradients are added. */
int orc_backward_at(const orc_config *c, const int32_t *remap, int32_t vocab, const int32_t *ids,
                    const orc_rows *table, const void *w_kv, const void *gamma_k, const void *gamma_q,
                    const void *conv_w, const orc_rows *hidden, const orc_rows *dy, int64_t n_pos,
                    const int64_t *pos, double *d_hidden, double *de, double *dkv_out, double *d_gk,
                    double *d_gq) {
  if (check(c)) return ORC_EINVAL;
  const int64_t T = c->seqlen, n = (int64_t)c->batch * T;
  const int H = n_heads(c), hc = c->hc_mult, K = c->conv_kernel, D = c->conv_dilation;
  const int64_t d = c->hidden, E = (int64_t)H * c->head_dim, O = (int64_t)(hc + 1) * d;
  const int64_t esz = c->dtype == 0 ? 4 : 2;
  for (int64_t i = 0; i < n_pos; i++)
    if (pos[i] < 0 || pos[i] >= n) return ORC_EINVAL;
  if (n_pos == 0) return ORC_OK;

  int64_t *idx = malloc(sizeof(int64_t) * n * H);
  void *e = malloc(esz * E);
  double *kv = malloc(sizeof(double) * O), *dkv = malloc(sizeof(double) * O);
  double *dvg = malloc(sizeof(double) * hc * d), *g = malloc(sizeof(double) * hc), *s = malloc(sizeof(double) * hc);
  int rc = ORC_ENOMEM;
  if (!idx || !e || !kv || !dkv || !dvg || !g || !s) goto out;
  rc = orc_hash(c, remap, vocab, ids, NULL, idx);
  if (rc) goto out;
  orc_config one = *c;
  one.batch = 1;
  one.seqlen = 1;
  for (int64_t i = 0; i < n_pos; i++) {
    const int64_t p = pos[i], t = p % T;
    /* forward quantities at the position */
    rc = orc_gather(&one, table, idx + p * H, 1, e);
    if (!rc) rc = orc_project(&one, w_kv, e, 1, kv);
    if (rc) goto out;
    const void *q = row_ptr(hidden, p, esz * hc * d);
    if (!q) { rc = ORC_EMISSING; goto out; }
    rc = orc_gate(&one, gamma_k, gamma_q, kv, q, 1, s, g);
    if (rc) goto out;
    /* conv + residual: dy at the position and at the K-1 positions its Vg feeds */
    const void *dy0 = row_ptr(dy, p, esz * hc * d);
    if (!dy0) { rc = ORC_EMISSING; goto out; }
    for (int64_t k = 0; k < hc * d; k++) dvg[k] = ld(dy0, k, c->dtype);
    for (int j = 0; j < K; j++) {
      const int64_t ahead = t + (int64_t)(K - 1 - j) * D;
      if (ahead >= T) continue;
      const void *dyr = row_ptr(dy, p + (ahead - t), esz * hc * d);
      if (!dyr) { rc = ORC_EMISSING; goto out; }
      for (int h = 0; h < hc; h++)
        for (int64_t ch = 0; ch < d; ch++)
          dvg[(int64_t)h * d + ch] +=
              ld(conv_w, ((int64_t)h * d + ch) * K + j, c->dtype) * ld(dyr, (int64_t)h * d + ch, c->dtype);
    }
    gate_backward_token(c, kv, q, gamma_k, gamma_q, dvg, g, s, dkv, d_hidden + i * hc * d, d_gk, d_gq);
    if (dkv_out) memcpy(dkv_out + i * O, dkv, sizeof(double) * O);
    if (de)
      for (int64_t k = 0; k < E; k++) {
        double acc = 0.0;
        for (int64_t o = 0; o < O; o++) acc += dkv[o] * ld(w_kv, o * E + k, c->dtype);
        de[i * E + k] = acc;
      }
  }
  rc = ORC_OK;
out:
  free(idx); free(e); free(kv); free(dkv); free(dvg); free(g); free(s);
  return rc;
}
