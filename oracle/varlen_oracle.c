/*
 * Packed variable-length scaled-dot-product attention -- fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This library exists to check the GPU library
 * against a plain, slow, obviously correct definition. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg load it; the product
 * path (the HIP library and its Python binding) never calls, links or imports
 * anything here, and nothing here calls the product path.
 *
 * Sources (the crate onnx-runtime-ep-cuda, docs.rs source pages):
 *   [PVA] src/kernels/packed_varlen_attention.rs (0.1.0-dev.6)
 *   [ATT] src/kernels/attention.rs                (0.1.0-dev.6)
 *   [STD] src/kernels/standard_attention.rs       (latest page, 0.1.0-dev.5)
 *   [GQA] src/kernels/group_query_attention.rs    (latest page)
 *
 * What is computed, for every sequence b of the packed batch, every query
 * head h and every query row i of that sequence (plain definition, written
 * out in fp64; no blocking, no online softmax, no reordering):
 *
 *   q0 = cu_q[b],  L_q  = cu_q[b+1]  - q0        [PVA] module doc,
 *   k0 = cu_kv[b], L_kv = cu_kv[b+1] - k0              "Packed layout &
 *                                                       cumulative offsets"
 *   g  = h / (Hq / Hkv)                           [PVA] "Schema (v1)",
 *                                                       kv_num_heads; row
 *                                                       kernel head mapping
 *   s_j = sum_p (Q[q0+i,h,p] * sqrt(scale)) * (K[k0+j,g,p] * sqrt(scale))
 *                                                 [PVA] row kernel stage 1;
 *                                                 [STD] "Semantics"
 *   s_j = softcap * tanh(s_j / softcap)   iff softcap != 0
 *                                                 [PVA] row kernel stage 2
 *                                                 (applied before the mask)
 *   s_j = -inf  iff causal and j > i + (L_kv - L_q)
 *                                                 [PVA] "Causal alignment",
 *                                                 row kernel stage 3
 *   s_j = -inf  iff W > 0 and j < i + (L_kv - L_q) + 1 - W
 *                                                 (local window of W keys
 *                                                 ending at the row's
 *                                                 tail-aligned diagonal, with
 *                                                 or without the causal mask:
 *                                                 [ATT] softmax kernel source,
 *                                                 local_min; [GQA] the
 *                                                 local_window_size attribute
 *                                                 and the kernel's local_start)
 *   m = max_j s_j; a row with no keys or m = -inf is all zeros;
 *   otherwise e_j = exp(s_j - m), l = sum_j e_j,
 *   O[q0+i,h,c] = sum_j e_j * V[k0+j,g,c] / l     [PVA] row kernel stages 4-5;
 *                                                 [STD] "Semantics"
 *                                                 (fully-masked -> 0)
 *
 * scale: the caller's value, or 1/sqrt(head_size) when the caller passes 0
 * ([PVA] "Schema (v1)", scale attribute default). All arithmetic is fp64;
 * the inputs are read as the exact values their storage type holds.
 *
 * Optional outputs for tests: lse = m + ln(l) per row (-inf for an empty or
 * fully masked row), and a restriction of every sequence's keys to the local
 * index window [key_begin, key_end) so that the softmax over any partition of
 * the keys can be formed and recombined.
 *
 * Rows are independent, so the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* Exact value of one stored element as a double. */
static double load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == ORACLE_F32) {
    return (double)((const float*)base)[idx];
  }
  uint16_t bits = ((const uint16_t*)base)[idx];
  if (dtype == ORACLE_BF16) {
    /* bfloat16 is the upper half of an IEEE binary32. */
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
  }
  /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 10) & 0x1f;
  int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 / 2^10 */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp(1.0 + (double)frac / 1024.0, expo - 15);
  }
  return sign ? -mag : mag;
}

typedef struct {
  const void *q, *k, *v;
  int dtype;
  const int32_t *cu_q, *cu_kv;
  int32_t batch, hq, hkv, d, dv;
  double scale, softcap;
  int causal;
  int32_t local_window; /* <= 0: no window */
  int32_t key_begin, key_end;
  const int64_t* rows; /* row id = token * hq + head; NULL -> all rows */
  int64_t n_rows;
  double* out; /* [n_rows, dv] */
  double* lse; /* [n_rows] or NULL */
  int64_t max_kv;
  int n_threads;
} oracle_job;

typedef struct {
  const oracle_job* job;
  int tid;
  int status;
} oracle_worker;

/* Sequence that owns packed query token t: the b with cu_q[b] <= t < cu_q[b+1]
 * ([PVA] "Packed layout & cumulative offsets"). Empty sequences own nothing. */
static int32_t owner_of(const oracle_job* job, int64_t t) {
  int32_t lo = 0, hi = job->batch; /* answer in [lo, hi) */
  while (hi - lo > 1) {
    int32_t mid = lo + (hi - lo) / 2;
    if (job->cu_q[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

/* One output row: query token t, query head h. */
static void attend_row(const oracle_job* job, int64_t t, int32_t h, double* s,
                       double* out_row, double* lse_out) {
  const int32_t b = owner_of(job, t);
  const int64_t q0 = job->cu_q[b];
  const int64_t lq = (int64_t)job->cu_q[b + 1] - q0;
  const int64_t k0 = job->cu_kv[b];
  const int64_t lkv = (int64_t)job->cu_kv[b + 1] - k0;
  const int64_t i = t - q0;
  const int64_t offset = lkv - lq;
  const int32_t group = job->hq / job->hkv;
  const int32_t g = h / group;
  const double root = sqrt(job->scale);
  int64_t j0 = job->key_begin < 0 ? 0 : job->key_begin;
  int64_t j1 = (job->key_end < 0 || job->key_end > lkv) ? lkv : job->key_end;
  if (j1 < j0) j1 = j0;

  /* Stage 1-3: scores, softcap, causal mask. */
  double m = -INFINITY;
  for (int64_t j = j0; j < j1; ++j) {
    double acc = 0.0;
    const int64_t qbase = (t * job->hq + h) * (int64_t)job->d;
    const int64_t kbase = ((k0 + j) * job->hkv + g) * (int64_t)job->d;
    for (int32_t p = 0; p < job->d; ++p) {
      acc += (load_elem(job->q, qbase + p, job->dtype) * root) *
             (load_elem(job->k, kbase + p, job->dtype) * root);
    }
    if (job->softcap != 0.0) {
      acc = job->softcap * tanh(acc / job->softcap);
    }
    if (job->causal && j > i + offset) {
      acc = -INFINITY;
    }
    if (job->local_window > 0 && j < i + offset + 1 - job->local_window) {
      acc = -INFINITY;
    }
    s[j - j0] = acc;
    if (acc > m) m = acc;
  }

  /* Stage 4-5: stable softmax and the weighted sum of value rows. */
  for (int32_t c = 0; c < job->dv; ++c) out_row[c] = 0.0;
  if (j1 == j0 || m == -INFINITY) {
    if (lse_out) *lse_out = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = j0; j < j1; ++j) {
    s[j - j0] = exp(s[j - j0] - m);
    l += s[j - j0];
  }
  for (int64_t j = j0; j < j1; ++j) {
    const int64_t vbase = ((k0 + j) * job->hkv + g) * (int64_t)job->dv;
    for (int32_t c = 0; c < job->dv; ++c) {
      out_row[c] += s[j - j0] * load_elem(job->v, vbase + c, job->dtype);
    }
  }
  for (int32_t c = 0; c < job->dv; ++c) out_row[c] /= l;
  if (lse_out) *lse_out = m + log(l);
}

static void* worker_main(void* arg) {
  oracle_worker* w = (oracle_worker*)arg;
  const oracle_job* job = w->job;
  double* s = (double*)malloc(sizeof(double) * (size_t)(job->max_kv > 0 ? job->max_kv : 1));
  if (!s) {
    w->status = -2;
    return NULL;
  }
  for (int64_t r = w->tid; r < job->n_rows; r += job->n_threads) {
    const int64_t row = job->rows ? job->rows[r] : r;
    const int64_t t = row / job->hq;
    const int32_t h = (int32_t)(row % job->hq);
    attend_row(job, t, h, s, job->out + r * (int64_t)job->dv, job->lse ? job->lse + r : NULL);
  }
  free(s);
  w->status = 0;
  return NULL;
}

/*
 * Public entry point.
 *   q  [total_q, hq, d], k [total_kv, hkv, d], v [total_kv, hkv, dv], all of
 *      storage type dtype (0 f32, 1 f16, 2 bf16), contiguous, host memory.
 *   cu_q, cu_kv: int32 [batch + 1] exclusive prefix sums.
 *   scale: the caller's scale; 0 selects 1/sqrt(d).
 *   local_window: W > 0 restricts row i to keys j >= i + L_kv - L_q + 1 - W;
 *         <= 0 means no window.
 *   rows: NULL for all total_q*hq rows in (token, head) order, else n_rows
 *         row ids (token * hq + head).
 *   key_begin/key_end: local key window per sequence (-1, -1 for all keys).
 *   out: [n_rows, dv] fp64; lse: [n_rows] fp64 or NULL.
 *   n_threads: 0 selects all online cores.
 * Returns 0, -1 on inconsistent arguments, -2 when memory runs out.
 */
int pva_oracle_attention(const void* q, const void* k, const void* v, int dtype,
                         const int32_t* cu_q, const int32_t* cu_kv, int32_t batch,
                         int64_t total_q, int64_t total_kv, int32_t hq, int32_t hkv,
                         int32_t d, int32_t dv, double scale, int causal, double softcap,
                         int32_t local_window, const int64_t* rows, int64_t n_rows, int32_t key_begin,
                         int32_t key_end, double* out, double* lse, int n_threads) {
  if (batch < 1 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || dv <= 0) return -1;
  if (dtype < ORACLE_F32 || dtype > ORACLE_BF16) return -1;
  if (cu_q[0] != 0 || cu_kv[0] != 0) return -1;
  if (cu_q[batch] != total_q || cu_kv[batch] != total_kv) return -1;
  int64_t max_kv = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (cu_q[b + 1] < cu_q[b] || cu_kv[b + 1] < cu_kv[b]) return -1;
    if (cu_kv[b + 1] - cu_kv[b] > max_kv) max_kv = cu_kv[b + 1] - cu_kv[b];
  }
  if (!rows) n_rows = total_q * hq;
  for (int64_t r = 0; rows && r < n_rows; ++r) {
    if (rows[r] < 0 || rows[r] >= total_q * hq) return -1;
  }
  if (n_rows == 0) return 0;
  oracle_job job;
  job.q = q; job.k = k; job.v = v; job.dtype = dtype;
  job.cu_q = cu_q; job.cu_kv = cu_kv; job.batch = batch;
  job.hq = hq; job.hkv = hkv; job.d = d; job.dv = dv;
  job.scale = scale != 0.0 ? scale : 1.0 / sqrt((double)d);
  job.softcap = softcap; job.causal = causal != 0;
  job.local_window = local_window;
  job.key_begin = key_begin; job.key_end = key_end;
  job.rows = rows; job.n_rows = n_rows; job.out = out; job.lse = lse;
  job.max_kv = max_kv;
  int nt = n_threads > 0 ? n_threads : (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nt < 1) nt = 1;
  if ((int64_t)nt > n_rows) nt = (int)n_rows;
  job.n_threads = nt;

  oracle_worker* workers = (oracle_worker*)calloc((size_t)nt, sizeof(oracle_worker));
  pthread_t* threads = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
  if (!workers || !threads) {
    free(workers);
    free(threads);
    return -2;
  }
  int status = 0;
  for (int i = 0; i < nt; ++i) {
    workers[i].job = &job;
    workers[i].tid = i;
    workers[i].status = -2;
    if (i > 0 && pthread_create(&threads[i], NULL, worker_main, &workers[i]) != 0) {
      worker_main(&workers[i]); /* could not start a thread: run it here */
      threads[i] = 0;
    }
  }
  worker_main(&workers[0]);
  for (int i = 1; i < nt; ++i) {
    if (threads[i]) pthread_join(threads[i], NULL);
  }
  for (int i = 0; i < nt; ++i) {
    if (workers[i].status != 0) status = workers[i].status;
  }
  free(workers);
  free(threads);
  return status;
}

/* Number of worker threads a call with n_threads = 0 would use. */
int pva_oracle_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}
