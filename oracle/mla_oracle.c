/*
 * CPU oracle for weight-absorbed MLA decode over a paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link or call
 * this file; it exists so that tests, the smoke check and the benchmark's
 * CPU baseline can compare the HIP kernels against a plain, slow, obviously
 * correct computation.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (all arithmetic in IEEE double):
 *
 *   Absorbed score, from "MLA 在极长上下文下的显存带宽突围" section
 *   "运行期矩阵吸收避免潜在张量展开": the query already carries W_UK, so the
 *   score of query row (b,s,h) against cached token j is
 *       z_j = scale * ( q_nope . c_j  +  q_rope . k_rope_j )
 *   where the cached latent row of token j is [c_j (512) | k_rope_j (64)]
 *   ("MLA & DSA 推理性能优化指南" §1.1 figure: only c_t^KV (d_c = 512) and
 *   the 64-dim RoPE key are cached).
 *
 *   Value: the same latent c_j (512 dims) is the value, so the output is
 *       out = sum_j softmax(z)_j * c_j          (512 dims per head)
 *       lse = log( sum_j exp(z_j) )              (natural log)
 *   computed as m = max z, l = sum exp(z - m), lse = m + log l,
 *   p_j = exp(z_j - lse).  An empty visible set gives out = 0, lse = -inf.
 *
 *   Visible set of row (b, s, h) with L = cache_seqlens[b]:
 *     dense:  j in [0, L), and with causal also j <= L - Sq + s
 *             (the Sq new tokens are already appended to the cache, as in
 *             the decode flow of "MLA & DSA 推理性能优化指南" §4 figure,
 *             "Output Token append to cache");
 *     sparse: the listed positions indices[b][s][t] with 0 <= idx < L
 *             (DSA reads only the k selected tokens, same page, §1.2 and §4.2).
 *   Paging: token j of sequence b lives in page block_table[b][j / 64] at row
 *   j % 64.  A token whose logical page j / 64 is at or past the table's row
 *   length (bt_stride), or whose page entry lies outside [0, num_pages), is
 *   not visible: the table gives it no resident page.
 *
 *   fp8 cache: each element is an OCP e4m3fn code (1 sign, 4 exponent bits
 *   with bias 7, 3 mantissa bits, subnormals, S.1111.111 = NaN, no infinity)
 *   and the token's value is code * kv_scales[page][row]
 *   ("MLA & DSA 推理性能优化指南" §5.3 table: FP8 cache ~576 B per token).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_DC 512
#define OR_DR 64
#define OR_D (OR_DC + OR_DR)
#define OR_PAGE 64

/* Bytes one cached token occupies per layer: (d_c + d_rope) * bytes/element
 * ("MLA & DSA 推理性能优化指南" §4.1; the fp8 figure there leaves out the
 * per-token scale, which this layout stores separately). */
long oracle_kv_bytes_per_token(int bytes_per_element) {
  return (long)OR_D * bytes_per_element;
}

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP e4m3fn decoding from the format definition. */
double oracle_e4m3fn_to_double(uint8_t v) {
  int sign = v >> 7;
  int e = (v >> 3) & 15;
  int m = v & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);          /* m/8 * 2^(1-7) */
  else
    mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

typedef struct {
  const uint16_t *q_nope, *q_rope; /* bf16 bits */
  const void *kv;                  /* bf16 bits or e4m3 codes */
  const float *kv_scales;
  int fp8, num_pages;
  const int32_t *block_table;
  int bt_stride;
  const int32_t *seqlens;
  int B, Sq, H;
  double scale;
  int causal;
  const int32_t *indices; /* NULL: dense */
  int topk;
  const int64_t *rows; /* NULL: every row; else flat row ids b*Sq*H + s*H + h */
  long nrows;
  double *out, *lse;
  long next; /* work counter */
  pthread_mutex_t mu;
} job_t;

/* Latent element d of token (page p, row r). */
static double kv_elem(const job_t *J, long p, int r, int d) {
  long off = ((long)p * OR_PAGE + r) * OR_D + d;
  if (J->fp8)
    return oracle_e4m3fn_to_double(((const uint8_t *)J->kv)[off]) *
           (double)J->kv_scales[(long)p * OR_PAGE + r];
  return bf16_bits_to_double(((const uint16_t *)J->kv)[off]);
}

/* Physical (page, row) of logical token j of sequence b; 0 if not resident.
 * The block table row of sequence b holds bt_stride entries: a token whose
 * logical page j / 64 is at or past that has no entry and is not visible. */
static int locate(const job_t *J, int b, long j, long *p, int *r) {
  if (j < 0 || j / OR_PAGE >= J->bt_stride) return 0;
  long pg = J->block_table[(long)b * J->bt_stride + j / OR_PAGE];
  if (pg < 0 || pg >= J->num_pages) return 0;
  *p = pg;
  *r = (int)(j % OR_PAGE);
  return 1;
}

static void one_row(const job_t *J, long row, double *o, double *lse_out,
                    double *zbuf, long *pbuf, int *rbuf) {
  int h = (int)(row % J->H);
  int s = (int)((row / J->H) % J->Sq);
  int b = (int)(row / ((long)J->H * J->Sq));
  long L = J->seqlens[b];
  double q[OR_D];
  for (int d = 0; d < OR_DC; d++) q[d] = bf16_bits_to_double(J->q_nope[row * OR_DC + d]);
  for (int d = 0; d < OR_DR; d++) q[OR_DC + d] = bf16_bits_to_double(J->q_rope[row * OR_DR + d]);

  /* 1. the visible set */
  long n = 0;
  if (J->indices) {
    const int32_t *ix = J->indices + ((long)b * J->Sq + s) * J->topk;
    for (int t = 0; t < J->topk; t++) {
      long j = ix[t];
      if (j < 0 || j >= L) continue;
      if (locate(J, b, j, &pbuf[n], &rbuf[n])) n++;
    }
  } else {
    long last = J->causal ? L - J->Sq + s : L - 1; /* inclusive */
    if (last > L - 1) last = L - 1;
    for (long j = 0; j <= last; j++)
      if (locate(J, b, j, &pbuf[n], &rbuf[n])) n++;
  }

  for (int d = 0; d < OR_DC; d++) o[d] = 0.0;
  if (n == 0) {
    *lse_out = -INFINITY;
    return;
  }

  /* 2. scores z_j = scale * (q_nope . c_j + q_rope . k_rope_j) */
  double m = -INFINITY;
  for (long t = 0; t < n; t++) {
    double acc = 0.0;
    for (int d = 0; d < OR_D; d++) acc += q[d] * kv_elem(J, pbuf[t], rbuf[t], d);
    zbuf[t] = J->scale * acc;
    if (zbuf[t] > m) m = zbuf[t];
  }

  /* 3. log-sum-exp */
  double l = 0.0;
  for (long t = 0; t < n; t++) l += exp(zbuf[t] - m);
  double lse = m + log(l);
  *lse_out = lse;

  /* 4. out = sum_j p_j c_j with p_j = exp(z_j - lse) */
  for (long t = 0; t < n; t++) {
    double p = exp(zbuf[t] - lse);
    for (int d = 0; d < OR_DC; d++) o[d] += p * kv_elem(J, pbuf[t], rbuf[t], d);
  }
}

static long max_visible(const job_t *J) {
  if (J->indices) return J->topk;
  long mx = 0;
  for (int b = 0; b < J->B; b++)
    if (J->seqlens[b] > mx) mx = J->seqlens[b];
  return mx;
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  long cap = max_visible(J) + 1;
  double *z = (double *)malloc(sizeof(double) * cap);
  long *pb = (long *)malloc(sizeof(long) * cap);
  int *rb = (int *)malloc(sizeof(int) * cap);
  for (;;) {
    pthread_mutex_lock(&J->mu);
    long k = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (k >= J->nrows) break;
    long row = J->rows ? J->rows[k] : k;
    one_row(J, row, J->out + k * OR_DC, J->lse + k, z, pb, rb);
  }
  free(z);
  free(pb);
  free(rb);
  return NULL;
}

/*
 * Computes `out` [nrows, 512] and `lse` [nrows] (double) for the rows listed
 * in `rows` (flat ids b*Sq*H + s*H + h), or for every row in (b, s, h) order
 * when `rows` is NULL.  `indices` NULL selects the dense path.
 * Returns 0 on success, -1 on bad arguments.
 */
int oracle_mla_decode(const uint16_t *q_nope, const uint16_t *q_rope, const void *kv_pages,
                      const float *kv_scales, int kv_is_fp8, int num_pages,
                      const int32_t *block_table, int bt_stride, const int32_t *cache_seqlens,
                      int B, int Sq, int H, double softmax_scale, int causal,
                      const int32_t *indices, int topk, const int64_t *rows, long nrows,
                      double *out, double *lse, int nthreads) {
  if (!q_nope || !q_rope || !kv_pages || !block_table || !cache_seqlens || !out || !lse)
    return -1;
  if (B <= 0 || Sq <= 0 || H <= 0 || (kv_is_fp8 && !kv_scales) || (indices && topk <= 0))
    return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q_nope = q_nope;
  J.q_rope = q_rope;
  J.kv = kv_pages;
  J.kv_scales = kv_scales;
  J.fp8 = kv_is_fp8;
  J.num_pages = num_pages;
  J.block_table = block_table;
  J.bt_stride = bt_stride;
  J.seqlens = cache_seqlens;
  J.B = B;
  J.Sq = Sq;
  J.H = H;
  J.scale = softmax_scale;
  J.causal = causal;
  J.indices = indices;
  J.topk = topk;
  J.rows = rows;
  J.nrows = rows ? nrows : (long)B * Sq * H;
  J.out = out;
  J.lse = lse;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, worker, &J);
  for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J.mu);
  return 0;
}
