/*
 * Paged-attention decode oracle: a plain, slow CPU implementation of what the
 * decode computes.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may call it; the product path never
 * does.  It shares no code, header, table or constant with the GPU library.
 *
 * What it computes (FlyDSL paged-attention decode pages: aiter PR #4332 "Add
 * paged-attention Tile kernel" host-wrapper fragments for the tensor shapes;
 * aiter PR #6617, Validation, for the FP32-reference check; aiter PR #7079,
 * "Partition merges" and the test catalogue, for sinks at the merge, empty
 * rows and the float64 reference):
 *
 * For sequence s, query row i in [0, QL), q-head h and KV head g = h / G
 * (G = Hq / Hkv, contiguous groups):
 *   L   = context_lens[s] clamped to [0, table capacity]
 *   pos = L - QL + i when causal, else L - 1
 *   visible set V = { t : 0 <= t < L, t <= pos, and (W == 0 or t > pos - W) }
 *   k_t[d], v_t[d]  dequantised from the paged caches (FP8 code * scale;
 *                   BF16 exact)
 *   x_t = softmax_scale * sum_d q[d] * k_t[d]           (double accumulation)
 *   m   = max({x_t : t in V} U {sink_h if sinks})
 *   out[d] = sum_{t in V} e^(x_t - m) v_t[d] / (sum_{t in V} e^(x_t - m)
 *                                               + [sinks] e^(sink_h - m))
 *   V empty -> out = 0.
 *
 * Token address: dense tables give page = block_tables[s][t / page_size],
 * slot = t mod page_size; token tables give a physical slot S =
 * block_tables[s][t], page = S / page_size, slot = S mod page_size; top-k
 * index tables (two-level, token_table = 2) give a logical position
 * P = topk[s][t] of the sequence's paged context, clamped to the table's
 * extent [0, table_stride * page_size), then page = block_tables[s][P /
 * page_size], slot = P mod page_size (the sparse front end: top-k logical
 * positions through the block table, aiter PR #7079, summary and Performance
 * setup).  For token tables context_lens[s] counts the row's tokens.
 *
 * Layouts (x = 16 bytes / element size):
 *   K packed      [pages, Hkv, D/x, page, x]
 *   V plain       [pages, Hkv, D, page]
 *   V transposed  [pages, Hkv, page/x, D, x]
 *   per-token scales [pages, Hkv, page]; per-tensor scales one float.
 *
 * The FP8 e4m3fn decoder is written from the OCP 8-bit floating point
 * definition: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals at exponent 0, S.1111.111 is NaN, no infinities.
 *
 * MXFP4 caches (the MXFP4 K/V of aiter PR #7079's merge of #7056, which
 * states only that such caches take 256-token partitions; the format is the
 * OCP Microscaling (MX) one): each token's K or V row is cut into blocks of
 * 32 consecutive head dims; a block holds 32 FP4 E2M1 codes and one E8M0
 * scale, and element = fp4(code) * 2^(scale - 127).  FP4 E2M1: 1 sign bit,
 * 2 exponent bits with bias 1, 1 mantissa bit, subnormal at exponent 0
 * (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), no NaN or
 * infinity.  E8M0: an unsigned exponent, 0xFF is NaN.  Two codes share a
 * byte, the lower index in the low nibble.  Layouts:
 *   K  [pages, Hkv, D/32, page, 16 bytes]   (the 32 codes of block d/32)
 *   V  [pages, Hkv, D, page/2 bytes]        (row d: token 2j low nibble)
 *   k and v scales: one byte per block, [pages, Hkv, page, D/32].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BF16 0
#define ORC_FP16 1
#define ORC_FP8 2
#define ORC_MXFP4 3

#define ORC_SCALE_NONE 0
#define ORC_SCALE_TENSOR 1
#define ORC_SCALE_TOKEN 2
#define ORC_SCALE_MX 3

typedef struct {
  int num_seqs, query_len, num_q_heads, num_kv_heads, head_dim, page_size;
  int num_pages, table_stride;
  int q_kind;      /* ORC_BF16 or ORC_FP16 */
  int kv_kind;     /* ORC_BF16, ORC_FP8 or ORC_MXFP4 */
  int v_transposed;
  int scale_mode;
  int causal, window, has_sinks, token_table;
  double softmax_scale;
  int index_stride;    /* top-k index tables: row stride of topk */
  const int32_t* topk; /* top-k index tables: logical positions [num_seqs][index_stride] */
} orc_problem;

/* ---- scalar format decoders (from the format definitions) ---- */

double orc_fp8_e4m3fn(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6); /* subnormal: 0.mmm * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

double orc_bf16(uint16_t b) {
  /* bfloat16 is the upper half of an IEEE binary32 */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double orc_fp16(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0x1F) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m / 1024.0, -14);
  else v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return sign ? -v : v;
}

double orc_fp4_e2m1(uint8_t c) {
  int sign = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1); /* subnormal: 0.m * 2^(1-1) */
  return sign ? -v : v;
}

double orc_e8m0(uint8_t e) { return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127); }

static double orc_nibble(const uint8_t* bytes, long byte_index, int high) {
  uint8_t b = bytes[byte_index];
  return orc_fp4_e2m1(high ? (uint8_t)(b >> 4) : (uint8_t)(b & 0xF));
}

/* ---- addressing ---- */

static int orc_clamped_len(const orc_problem* p, const int32_t* context_lens, int s) {
  long cap = p->token_table == 2 ? (long)p->index_stride
             : p->token_table    ? (long)p->table_stride
                                 : (long)p->table_stride * p->page_size;
  long L = context_lens[s];
  if (L < 0) L = 0;
  if (L > cap) L = cap;
  return (int)L;
}

/* physical (page, slot) of logical token t of sequence s */
static void orc_locate(const orc_problem* p, const int32_t* block_tables, int s, int t, long* page, int* slot) {
  if (p->token_table == 2) {
    long P = p->topk[(long)s * p->index_stride + t];
    long extent = (long)p->table_stride * p->page_size;
    if (P < 0) P = 0;
    if (P > extent - 1) P = extent - 1;
    *page = block_tables[(long)s * p->table_stride + P / p->page_size];
    *slot = (int)(P % p->page_size);
  } else if (p->token_table) {
    long S = block_tables[(long)s * p->table_stride + t];
    *page = S / p->page_size;
    *slot = (int)(S % p->page_size);
  } else {
    *page = block_tables[(long)s * p->table_stride + t / p->page_size];
    *slot = t % p->page_size;
  }
}

static double orc_kv_elem(const orc_problem* p, const void* cache, long byte_index_elems) {
  if (p->kv_kind == ORC_FP8) return orc_fp8_e4m3fn(((const uint8_t*)cache)[byte_index_elems]);
  return orc_bf16(((const uint16_t*)cache)[byte_index_elems]);
}

static double orc_scale(const orc_problem* p, const float* sc, long page, int g, int slot) {
  if (p->kv_kind != ORC_FP8 || p->scale_mode == ORC_SCALE_NONE || sc == NULL) return 1.0;
  if (p->scale_mode == ORC_SCALE_TENSOR) return (double)sc[0];
  return (double)sc[(page * p->num_kv_heads + g) * p->page_size + slot];
}

/* block scale of (page, slot, KV head g, block b) of an MXFP4 cache */
static double orc_mx_scale(const orc_problem* p, const void* sc, long page, int g, int slot, int b) {
  const uint8_t* e = (const uint8_t*)sc;
  return orc_e8m0(e[((page * p->num_kv_heads + g) * p->page_size + slot) * (p->head_dim / 32) + b]);
}

/* dequantised K row of token (page, slot) for KV head g */
static void orc_k_row(const orc_problem* p, const void* k_cache, const float* k_scale, long page, int slot, int g,
                      double* out) {
  int D = p->head_dim, ps = p->page_size;
  if (p->kv_kind == ORC_MXFP4) {
    long base = (page * p->num_kv_heads + g) * (long)(D / 2) * ps;
    for (int d = 0; d < D; ++d) {
      int b = d / 32, j = d % 32;
      out[d] = orc_nibble((const uint8_t*)k_cache, base + ((long)b * ps + slot) * 16 + j / 2, j & 1) *
               orc_mx_scale(p, k_scale, page, g, slot, b);
    }
    return;
  }
  int x = p->kv_kind == ORC_FP8 ? 16 : 8;
  double sc = orc_scale(p, k_scale, page, g, slot);
  long base = (page * p->num_kv_heads + g) * (long)D * ps;
  for (int d = 0; d < D; ++d) {
    long idx = base + ((long)(d / x) * ps + slot) * x + d % x;
    out[d] = orc_kv_elem(p, k_cache, idx) * sc;
  }
}

static void orc_v_row(const orc_problem* p, const void* v_cache, const float* v_scale, long page, int slot, int g,
                      double* out) {
  int D = p->head_dim, ps = p->page_size;
  if (p->kv_kind == ORC_MXFP4) {
    long base = (page * p->num_kv_heads + g) * (long)D * (ps / 2);
    for (int d = 0; d < D; ++d)
      out[d] = orc_nibble((const uint8_t*)v_cache, base + (long)d * (ps / 2) + slot / 2, slot & 1) *
               orc_mx_scale(p, v_scale, page, g, slot, d / 32);
    return;
  }
  int x = p->kv_kind == ORC_FP8 ? 16 : 8;
  double sc = orc_scale(p, v_scale, page, g, slot);
  long base = (page * p->num_kv_heads + g) * (long)D * ps;
  for (int d = 0; d < D; ++d) {
    long idx;
    if (p->v_transposed)
      idx = base + ((long)(slot / x) * D + d) * x + slot % x;
    else
      idx = base + (long)d * ps + slot;
    out[d] = orc_kv_elem(p, v_cache, idx) * sc;
  }
}

static double orc_q_elem(const orc_problem* p, const uint16_t* q, long idx) {
  return p->q_kind == ORC_FP16 ? orc_fp16(q[idx]) : orc_bf16(q[idx]);
}

/* visible token range [lo, hi] (inclusive) of query row i; returns 0 if empty */
static int orc_row_range(const orc_problem* p, int L, int i, int* lo, int* hi) {
  long pos = p->causal ? (long)L - p->query_len + i : (long)L - 1;
  long a = 0, b = pos;
  if (b > L - 1) b = L - 1;
  if (p->window > 0 && pos - p->window + 1 > a) a = pos - p->window + 1;
  if (b < a) return 0;
  *lo = (int)a;
  *hi = (int)b;
  return 1;
}

/*
 * Unnormalised attention state of one (sequence, row, head) over the visible
 * tokens that also lie in [t_begin, t_end):  m = max x_t (-inf if none),
 * l = sum e^(x_t - m), o[d] = sum e^(x_t - m) v_t[d].  Two passes: the
 * maximum first, then the weighted sums.
 */
void orc_partial(const orc_problem* p, const uint16_t* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, const float* k_scale,
                 const float* v_scale, int s, int i, int h, int t_begin, int t_end, double* m_out, double* l_out,
                 double* o_out) {
  int D = p->head_dim, G = p->num_q_heads / p->num_kv_heads, g = h / G;
  int L = orc_clamped_len(p, context_lens, s);
  int lo, hi;
  double* kr = (double*)malloc(sizeof(double) * D * 2);
  double* vr = kr + D;
  double* qv = (double*)malloc(sizeof(double) * D);
  for (int d = 0; d < D; ++d) o_out[d] = 0.0;
  *m_out = -INFINITY;
  *l_out = 0.0;
  if (!orc_row_range(p, L, i, &lo, &hi)) goto done;
  if (lo < t_begin) lo = t_begin;
  if (hi > t_end - 1) hi = t_end - 1;
  if (hi < lo) goto done;
  {
    long qbase = ((long)(s * p->query_len + i) * p->num_q_heads + h) * D;
    for (int d = 0; d < D; ++d) qv[d] = orc_q_elem(p, q, qbase + d);
    int n = hi - lo + 1;
    double* x = (double*)malloc(sizeof(double) * n);
    double m = -INFINITY;
    for (int t = lo; t <= hi; ++t) {
      long page;
      int slot;
      orc_locate(p, block_tables, s, t, &page, &slot);
      orc_k_row(p, k_cache, k_scale, page, slot, g, kr);
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += qv[d] * kr[d];
      x[t - lo] = p->softmax_scale * acc;
      if (x[t - lo] > m) m = x[t - lo];
    }
    double l = 0.0;
    for (int t = lo; t <= hi; ++t) {
      long page;
      int slot;
      double w = exp(x[t - lo] - m);
      orc_locate(p, block_tables, s, t, &page, &slot);
      orc_v_row(p, v_cache, v_scale, page, slot, g, vr);
      l += w;
      for (int d = 0; d < D; ++d) o_out[d] += w * vr[d];
    }
    *m_out = m;
    *l_out = l;
    free(x);
  }
done:
  free(kr);
  free(qv);
}

/*
 * Merge unnormalised partial states by the log-sum-exp rule, in the order
 * given, optionally with a sink logit that joins the denominator only:
 *   M = max(max_p m_p, sink); w_p = e^(m_p - M);
 *   out = sum_p w_p o_p / (sum_p w_p l_p + [sink] e^(sink - M));
 * no visible token in any part -> out = 0.
 */
void orc_merge(int n, const double* m, const double* l, const double* o, int D, int has_sink, double sink,
               double* out) {
  double M = -INFINITY, den = 0.0;
  int any = 0;
  for (int p = 0; p < n; ++p)
    if (l[p] > 0.0) {
      any = 1;
      if (m[p] > M) M = m[p];
    }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (!any) return;
  if (has_sink && sink > M) M = sink;
  for (int p = 0; p < n; ++p) {
    if (!(l[p] > 0.0)) continue;
    double w = exp(m[p] - M);
    den += w * l[p];
    for (int d = 0; d < D; ++d) out[d] += w * o[(long)p * D + d];
  }
  if (has_sink) den += exp(sink - M);
  for (int d = 0; d < D; ++d) out[d] /= den;
}

/* one output row (sequence s, query row i, head h) */
static void orc_one(const orc_problem* p, const uint16_t* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, const float* k_scale,
                    const float* v_scale, const float* sinks, int s, int i, int h, float* out) {
  int D = p->head_dim;
  double m, l;
  double* o = (double*)malloc(sizeof(double) * D * 2);
  double* r = o + D;
  orc_partial(p, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, s, i, h, 0, 0x7fffffff, &m,
              &l, o);
  orc_merge(1, &m, &l, o, D, p->has_sinks && sinks != NULL, sinks ? (double)sinks[h] : 0.0, r);
  for (int d = 0; d < D; ++d) out[d] = (float)r[d];
  free(o);
}

typedef struct {
  const orc_problem* p;
  const uint16_t* q;
  const void *k, *v;
  const int32_t *bt, *cl;
  const float *ks, *vs, *sinks;
  const int32_t* sel; /* pairs (token_row, head) or NULL */
  long n_items;
  float* out;
  long next;
  pthread_mutex_t mu;
} orc_job;

static void* orc_worker(void* arg) {
  orc_job* J = (orc_job*)arg;
  const orc_problem* p = J->p;
  int D = p->head_dim;
  for (;;) {
    long it;
    pthread_mutex_lock(&J->mu);
    it = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (it >= J->n_items) break;
    int row, h;
    float* dst;
    if (J->sel) {
      row = J->sel[2 * it];
      h = J->sel[2 * it + 1];
      dst = J->out + it * D;
    } else {
      row = (int)(it / p->num_q_heads);
      h = (int)(it % p->num_q_heads);
      dst = J->out + it * D;
    }
    int s = row / p->query_len, i = row % p->query_len;
    orc_one(p, J->q, J->k, J->v, J->bt, J->cl, J->ks, J->vs, J->sinks, s, i, h, dst);
  }
  return NULL;
}

/*
 * Attention output for every (row, head) (sel == NULL; out is [rows, Hq, D])
 * or for the n_sel (row, head) pairs in sel (out is [n_sel, D]), threaded
 * over output rows.  Returns the number of threads used.
 */
int orc_attend(const orc_problem* p, const uint16_t* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, const float* k_scale, const float* v_scale,
               const float* sinks, const int32_t* sel, long n_sel, float* out, int nthreads) {
  orc_job J;
  J.p = p;
  J.q = q;
  J.k = k_cache;
  J.v = v_cache;
  J.bt = block_tables;
  J.cl = context_lens;
  J.ks = k_scale;
  J.vs = v_scale;
  J.sinks = sinks;
  J.sel = sel;
  J.n_items = sel ? n_sel : (long)p->num_seqs * p->query_len * p->num_q_heads;
  J.out = out;
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0;
  for (int k = 1; k < nthreads; ++k)
    if (pthread_create(&th[started], NULL, orc_worker, &J) == 0) ++started;
  orc_worker(&J);
  for (int k = 0; k < started; ++k) pthread_join(th[k], NULL);
  pthread_mutex_destroy(&J.mu);
  return started + 1;
}
