/*
 * Plain CPU fp64 oracle for paged decode attention and the paged K/V append.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the HIP path: its layout offsets,
 * format decoders and arithmetic are written here from the definitions.
 *
 * What it computes
 * ----------------
 * The first page (TensorRT-LLM concept page, "key mechanisms" and "compile-time
 * graph optimization" sections) keeps each sequence's K/V in fixed-size pages
 * and looks up a page table to turn a logical token position into a physical
 * page, for both reads and writes; its "runtime execution model" section has
 * each decode iteration's attention read and update those pages.  The
 * attention itself is the usual single-query softmax attention:
 *
 *   for sequence b, query head h, kv head g = h / (Hq / Hkv), L = seq_lens[b]:
 *     page(t) = block_tables[b][t / P], slot(t) = t % P           (t < L)
 *     k_t = dec(K[page(t)][g][slot(t)][:]) * sK(page(t), g)
 *     v_t = dec(V[page(t)][g][slot(t)][:]) * sV(page(t), g)
 *     s_t = scale * sum_d q[b][h][d] * k_t[d]
 *     out[b][h][:] = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)
 *   with out = 0 when L = 0.  dec() widens fp32, bf16, fp8-e4m3, int8 or int4
 *   exactly; sK, sV are the per-(page, kv head) fp32 scales for fp8, int8 and
 *   int4, 1 otherwise.  int4 elements are two's complement nibbles, two per
 *   byte, element 2i in the low nibble of byte i (of the chunk, or of a row of
 *   k_new / v_new / the gather output).
 *   Everything after decoding is fp64, with libm exp.
 *
 * Element layout of one (page, kv head) chunk of P tokens x D elements
 * (E = elements per 16-byte group: 128 / element bits, TB = 4E):
 *   K (j, d): ((d / E) * P + j) * E + d % E
 *   V (j, d): blk = j / TB, r = j % TB, c = (r % 16) / 4,
 *             e = 4 * (r / 16) + r % 4  ->  blk*TB*D + (c*D + d)*E + e
 *   chunk (pg, g) starts at element (pg * Hkv + g) * P * D.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_I8 = 3, ORC_I4 = 4 };

static int elem_bits(int dt) {
  return dt == ORC_F32 ? 32 : dt == ORC_BF16 ? 16 : (dt == ORC_FP8 || dt == ORC_I8) ? 8 : dt == ORC_I4 ? 4 : 0;
}

/* int4: nibble idx of a packed array (two's complement code 0..15). */
static int get_nib(const void* base, int64_t idx) {
  uint8_t byte = ((const uint8_t*)base)[idx >> 1];
  return (idx & 1) ? byte >> 4 : byte & 15;
}
static void set_nib(void* base, int64_t idx, int code) {
  uint8_t* p = (uint8_t*)base + (idx >> 1);
  if (idx & 1)
    *p = (uint8_t)((*p & 0x0F) | ((code & 15) << 4));
  else
    *p = (uint8_t)((*p & 0xF0) | (code & 15));
}

/* Copy one stored element (any format) from src[si] to dst[di]. */
static void copy_elem(void* dst, int64_t di, const void* src, int64_t si, int bits) {
  if (bits == 4) {
    set_nib(dst, di, get_nib(src, si));
  } else {
    int eb = bits / 8;
    memcpy((char*)dst + di * eb, (const char*)src + si * eb, (size_t)eb);
  }
}

/* bf16: the top half of a binary32. */
double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP fp8 e4m3 ("fn"): sign, 4-bit exponent (bias 7), 3-bit mantissa;
 * exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity. */
double orc_e4m3_to_f64(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

static double load_elem(const void* base, int dt, int64_t idx) {
  switch (dt) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t*)base)[idx]);
    case ORC_I8: return (double)((const int8_t*)base)[idx];   /* two's complement byte */
    case ORC_I4: return (double)((get_nib(base, idx) ^ 8) - 8);  /* two's complement nibble */
    default: return orc_e4m3_to_f64(((const uint8_t*)base)[idx]);
  }
}

static int64_t k_off(int j, int d, int P, int E) {
  return ((int64_t)(d / E) * P + j) * E + d % E;
}

static int64_t v_off(int j, int d, int P, int D, int E) {
  int TB = 4 * E;
  int blk = j / TB, r = j % TB;
  int c = (r % 16) / 4, e = 4 * (r / 16) + r % 4;
  (void)P;
  return (int64_t)blk * TB * D + ((int64_t)c * D + d) * E + e;
}

typedef struct {
  const void* q;
  int q_dtype;
  const void* k_pool;
  const void* v_pool;
  int kv_dtype;
  const float* k_scales;
  const float* v_scales;
  const int32_t* bt;
  int max_pages;
  const int32_t* seq_lens;
  int B, NP, Hq, Hkv, D, P;
  double scale;
  const int32_t* pairs;
  int n_pairs;
  double* out;
  int nthreads;
  int tid;
  int err;
} job_t;

/* One (b, h) output row.  Returns 0, or -1 if a page id used is out of range. */
static int one_row(const job_t* J, int b, int h, double* s_buf, double* acc) {
  const int D = J->D, P = J->P, E = 128 / elem_bits(J->kv_dtype);
  const int G = J->Hq / J->Hkv, g = h / G;
  const int L = J->seq_lens[b] > 0 ? J->seq_lens[b] : 0;
  double* o = J->out + ((int64_t)b * J->Hq + h) * D;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (L == 0) return 0;
  const int64_t qbase = ((int64_t)b * J->Hq + h) * D;
  /* logits */
  double m = -INFINITY;
  for (int t = 0; t < L; ++t) {
    int pg = J->bt[(int64_t)b * J->max_pages + t / P];
    if (pg < 0 || pg >= J->NP) return -1;
    int j = t % P;
    int64_t cbase = ((int64_t)pg * J->Hkv + g) * P * D;
    double sk = J->k_scales ? (double)J->k_scales[(int64_t)pg * J->Hkv + g] : 1.0;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) {
      double qd = load_elem(J->q, J->q_dtype, qbase + d);
      double kd = load_elem(J->k_pool, J->kv_dtype, cbase + k_off(j, d, P, E)) * sk;
      dot += qd * kd;
    }
    s_buf[t] = J->scale * dot;
    if (s_buf[t] > m) m = s_buf[t];
  }
  /* weights and weighted sum of values */
  double l = 0.0;
  for (int d = 0; d < D; ++d) acc[d] = 0.0;
  for (int t = 0; t < L; ++t) {
    int pg = J->bt[(int64_t)b * J->max_pages + t / P];
    int j = t % P;
    int64_t cbase = ((int64_t)pg * J->Hkv + g) * P * D;
    double sv = J->v_scales ? (double)J->v_scales[(int64_t)pg * J->Hkv + g] : 1.0;
    double w = exp(s_buf[t] - m);
    l += w;
    for (int d = 0; d < D; ++d)
      acc[d] += w * (load_elem(J->v_pool, J->kv_dtype, cbase + v_off(j, d, P, D, E)) * sv);
  }
  for (int d = 0; d < D; ++d) o[d] = acc[d] / l;
  return 0;
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  int maxL = J->max_pages * J->P;
  double* s_buf = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)J->D);
  int64_t n = J->pairs ? J->n_pairs : (int64_t)J->B * J->Hq;
  for (int64_t i = J->tid; i < n; i += J->nthreads) {
    int b, h;
    if (J->pairs) {
      b = J->pairs[2 * i];
      h = J->pairs[2 * i + 1];
    } else {
      b = (int)(i / J->Hq);
      h = (int)(i % J->Hq);
    }
    if (one_row(J, b, h, s_buf, acc)) J->err = -1;
  }
  free(s_buf);
  free(acc);
  return NULL;
}

/* Decode attention into out[B][Hq][D] (fp64).  If pairs != NULL only the listed
 * (b, h) rows are computed.  Returns 0, -1 on a bad page id, -2 on bad arguments. */
int orc_decode(const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
               const float* k_scales, const float* v_scales, const int32_t* block_tables,
               int max_pages, const int32_t* seq_lens, int batch, int num_pages,
               int num_q_heads, int num_kv_heads, int head_dim, int page_size, float scale,
               const int32_t* pairs, int n_pairs, double* out, int nthreads) {
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out) return -2;
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 || page_size <= 0) return -2;
  if (!elem_bits(kv_dtype)) return -2;
  for (int b = 0; b < batch; ++b)
    if (seq_lens[b] > max_pages * page_size) return -2;
  if (nthreads < 1) nthreads = 1;
  job_t base = {q, q_dtype, k_pool, v_pool, kv_dtype, k_scales, v_scales, block_tables,
                max_pages, seq_lens, batch, num_pages, num_q_heads, num_kv_heads, head_dim,
                page_size, (double)scale, pairs, n_pairs, out, nthreads, 0, 0};
  job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nthreads);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].tid = i;
    pthread_create(&th[i], NULL, worker, &jobs[i]);
  }
  int err = 0;
  for (int i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    if (jobs[i].err) err = jobs[i].err;
  }
  free(jobs);
  free(th);
  return err;
}

/* Append: for each b with L = seq_lens[b] >= 1, copy token row L-1 of k_new/v_new
 * ([B][Hkv][D]) into slot (L-1) % P of page block_tables[b][(L-1) / P]. */
int orc_append(const void* k_new, const void* v_new, int kv_dtype, const int32_t* block_tables,
               int max_pages, const int32_t* seq_lens, int batch, void* k_pool, void* v_pool,
               int num_pages, int num_kv_heads, int head_dim, int page_size) {
  int bits = elem_bits(kv_dtype);
  if (!bits) return -2;
  int E = 128 / bits, D = head_dim, P = page_size;
  for (int b = 0; b < batch; ++b) {
    int L = seq_lens[b];
    if (L <= 0) continue;
    int t = L - 1;
    if (t / P >= max_pages) return -2;
    int pg = block_tables[(int64_t)b * max_pages + t / P];
    if (pg < 0 || pg >= num_pages) return -1;
    int j = t % P;
    for (int g = 0; g < num_kv_heads; ++g) {
      int64_t cbase = ((int64_t)pg * num_kv_heads + g) * P * D;
      int64_t src = ((int64_t)b * num_kv_heads + g) * D;
      for (int d = 0; d < D; ++d) {
        copy_elem(k_pool, cbase + k_off(j, d, P, E), k_new, src + d, bits);
        copy_elem(v_pool, cbase + v_off(j, d, P, D, E), v_new, src + d, bits);
      }
    }
  }
  return 0;
}

/* Gather: k_out/v_out are [B][Hkv][max_pages*P][D] elements; token t < L of
 * sequence b is copied to row t.  Rows at or past L are left untouched. */
int orc_gather(const void* k_pool, const void* v_pool, int kv_dtype, const int32_t* block_tables,
               int max_pages, const int32_t* seq_lens, int batch, int num_pages,
               int num_kv_heads, int head_dim, int page_size, void* k_out, void* v_out) {
  int bits = elem_bits(kv_dtype);
  if (!bits) return -2;
  int E = 128 / bits, D = head_dim, P = page_size;
  int64_t rows = (int64_t)max_pages * P;
  for (int b = 0; b < batch; ++b) {
    int L = seq_lens[b];
    if (L > rows) return -2;
    for (int t = 0; t < L; ++t) {
      int pg = block_tables[(int64_t)b * max_pages + t / P];
      if (pg < 0 || pg >= num_pages) return -1;
      int j = t % P;
      for (int g = 0; g < num_kv_heads; ++g) {
        int64_t cbase = ((int64_t)pg * num_kv_heads + g) * P * D;
        int64_t dst = (((int64_t)b * num_kv_heads + g) * rows + t) * D;
        for (int d = 0; d < D; ++d) {
          copy_elem(k_out, dst + d, k_pool, cbase + k_off(j, d, P, E), bits);
          copy_elem(v_out, dst + d, v_pool, cbase + v_off(j, d, P, D, E), bits);
        }
      }
    }
  }
  return 0;
}
