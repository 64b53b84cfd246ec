/*
 * oracle.c -- plain fp64 CPU reference for single-query (decode) paged attention
 * with grouped-query heads.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code with the GPU library.
 *
 * What it computes (page "Paged Attention Kernel Architecture for BI-V100",
 * section 1 "Problem Definition"): for every sequence b and query head h,
 *
 *     out[b,h,:] = softmax_t( scale * Q[b,h] . K[t] ) . V[t],   t in [0, L_b)
 *
 * where token t of sequence b lives in physical block block_table[b][t / bs] at
 * offset t % bs (same page, section 3 "Paged K/V Gather"; the decode-path example
 * of the paged-attention docs page, where cache_seqlens gives L_b and -1 marks an
 * unassigned table entry). Query head h reads KV head h / G with G = H_q / H_kv:
 * consecutive query heads form one group (same page, section 4 "GQA Handling":
 * G query heads share one KV head).
 *
 * Deliberately the plain definition: two passes (all scores, then weights), a
 * full softmax with the maximum subtracted, no online update, no split. fp64
 * throughout; fp16 and bf16 values are widened by decoders written here from the
 * IEEE binary16 / bfloat16 bit layouts so that NaN poison survives.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

enum {
  OR_OK = 0,
  OR_EARG = -1,      /* bad shape argument */
  OR_ETABLE = -2,    /* a table entry read for an attended token is outside [0, NB) */
  OR_ESEQLEN = -3,   /* cache length negative or beyond max_blocks_per_seq * block_size */
  OR_ENOMEM = -4,
};

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-10 * 2^-14 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f | 0x400), e - 25); /* (1024 + f) * 2^(e - 15 - 10) */
  }
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_decode_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float x;
  memcpy(&x, &u, sizeof x);
  return (double)x;
}

typedef struct {
  int B, Hq, Hkv, D, bs, NB, MBS, dtype;
  const float* q;
  const void* k;
  const void* v;
  int64_t ks[3]; /* block, head, token strides of K in elements */
  int64_t vs[3];
  const int32_t* table;
  const int32_t* seqlens;
  double scale;
} problem;

static double load_elem(const problem* p, const void* base, const int64_t* st, int64_t blk, int hk,
                        int off, int i) {
  int64_t idx = blk * st[0] + (int64_t)hk * st[1] + (int64_t)off * st[2] + i;
  switch (p->dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_F16: return oracle_decode_f16(((const uint16_t*)base)[idx]);
    default: return oracle_decode_bf16(((const uint16_t*)base)[idx]);
  }
}

/* Physical block and offset holding token t of sequence b, or -1 if the table
 * entry is outside [0, NB). */
static int64_t slot_of(const problem* p, int b, int t, int* off) {
  int32_t phys = p->table[(int64_t)b * p->MBS + t / p->bs];
  *off = t % p->bs;
  if (phys < 0 || phys >= p->NB) return -1;
  return phys;
}

/* Softmax of scale * q . K[t] over tokens t in [0, L) of sequence b, KV head
 * hk, applied to V: out[0..D) in fp64 (zeros when L = 0). s is caller scratch
 * of at least L doubles. Two passes: all scores first, then the weights. */
static int attend(const problem* p, const float* qv, int b, int hk, int L, double* s, double* out) {
  for (int i = 0; i < p->D; i++) out[i] = 0.0;
  if (L == 0) return OR_OK;
  /* pass 1: scores */
  double M = -INFINITY;
  for (int t = 0; t < L; t++) {
    int off;
    int64_t phys = slot_of(p, b, t, &off);
    if (phys < 0) return OR_ETABLE;
    double dot = 0.0;
    for (int i = 0; i < p->D; i++) dot += (double)qv[i] * load_elem(p, p->k, p->ks, phys, hk, off, i);
    s[t] = p->scale * dot;
    if (s[t] > M || t == 0) M = s[t];
  }
  /* pass 2: weights and the weighted sum of V */
  double Z = 0.0;
  for (int t = 0; t < L; t++) {
    int off;
    int64_t phys = slot_of(p, b, t, &off);
    double w = exp(s[t] - M);
    Z += w;
    for (int i = 0; i < p->D; i++) out[i] += w * load_elem(p, p->v, p->vs, phys, hk, off, i);
  }
  for (int i = 0; i < p->D; i++) out[i] /= Z;
  return OR_OK;
}

/* One (b, h) pair of the decode: the query is row b of q, the keys are the
 * L_b cached tokens. */
static int one_head(const problem* p, int b, int h, double* s, double* out) {
  int L = p->seqlens[b];
  int G = p->Hq / p->Hkv;
  const float* qv = p->q + ((int64_t)b * p->Hq + h) * p->D;
  if (L < 0 || (int64_t)L > (int64_t)p->MBS * p->bs) {
    for (int i = 0; i < p->D; i++) out[i] = 0.0;
    return OR_ESEQLEN;
  }
  return attend(p, qv, b, h / G, L, s, out);
}

typedef struct {
  const problem* p;
  const int32_t* pairs; /* npairs x (b, h) */
  int npairs;
  double* out;          /* npairs x D */
  int next;             /* shared work counter */
  int status;
  pthread_mutex_t lock;
} job;

static void* worker(void* arg) {
  job* j = (job*)arg;
  const problem* p = j->p;
  double* s = (double*)malloc(sizeof(double) * ((size_t)p->MBS * p->bs + 1));
  if (!s) {
    pthread_mutex_lock(&j->lock);
    j->status = OR_ENOMEM;
    pthread_mutex_unlock(&j->lock);
    return NULL;
  }
  for (;;) {
    pthread_mutex_lock(&j->lock);
    int k = j->next++;
    pthread_mutex_unlock(&j->lock);
    if (k >= j->npairs) break;
    int b = j->pairs[2 * k], h = j->pairs[2 * k + 1];
    int rc = one_head(p, b, h, s, j->out + (int64_t)k * p->D);
    if (rc != OR_OK) {
      pthread_mutex_lock(&j->lock);
      if (j->status == OR_OK) j->status = rc;
      pthread_mutex_unlock(&j->lock);
    }
  }
  free(s);
  return NULL;
}

static int check_shape(int B, int Hq, int Hkv, int D, int bs, int NB, int MBS, int dtype) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || NB < 0 || MBS <= 0) return OR_EARG;
  if (Hq % Hkv) return OR_EARG;
  if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return OR_EARG;
  return OR_OK;
}

/*
 * Attention output for the listed (b, h) pairs.
 *   q          fp32 [B, Hq, D] contiguous
 *   k, v       pools, element (blk, head, off, i) at blk*s[0] + head*s[1] + off*s[2] + i
 *   table      int32 [B, MBS];  seqlens int32 [B]
 *   pairs      int32 [npairs, 2] of (b, h);  out fp64 [npairs, D]
 *   nthreads   worker threads (>= 1)
 * Returns OR_OK or a negative OR_E* code; invalid table entries are never
 * dereferenced.
 */
int oracle_paged_attn_pairs(int B, int Hq, int Hkv, int D, int bs, int NB, int MBS, int dtype,
                            const float* q, const void* k, const void* v, const int64_t* kstrides,
                            const int64_t* vstrides, const int32_t* table, const int32_t* seqlens,
                            double scale, const int32_t* pairs, int npairs, double* out,
                            int nthreads) {
  int rc = check_shape(B, Hq, Hkv, D, bs, NB, MBS, dtype);
  if (rc != OR_OK) return rc;
  for (int k2 = 0; k2 < npairs; k2++) {
    if (pairs[2 * k2] < 0 || pairs[2 * k2] >= B || pairs[2 * k2 + 1] < 0 || pairs[2 * k2 + 1] >= Hq)
      return OR_EARG;
  }
  problem p = {B, Hq, Hkv, D, bs, NB, MBS, dtype, q, k, v,
               {kstrides[0], kstrides[1], kstrides[2]}, {vstrides[0], vstrides[1], vstrides[2]},
               table, seqlens, scale};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > npairs) nthreads = npairs > 0 ? npairs : 1;
  job j = {&p, pairs, npairs, out, 0, OR_OK, PTHREAD_MUTEX_INITIALIZER};
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  if (!th) return OR_ENOMEM;
  int started = 0;
  for (int t = 1; t < nthreads; t++) {
    if (pthread_create(&th[t], NULL, worker, &j) == 0) started++;
    else break;
  }
  worker(&j);
  for (int t = 1; t <= started; t++) pthread_join(th[t], NULL);
  free(th);
  return j.status;
}

/* Paged prefill (varlen queries), one (row, h) pair at a time. Query rows
 * cu_q[b] .. cu_q[b+1]-1 belong to sequence b (q_len_b of them) and the keys are
 * its L_b = seqlens_k[b] cached tokens, the new ones included. Row i of the
 * sequence sits at position L_b - q_len_b + i: causal, it attends tokens
 * [0, L_b - q_len_b + i] (none when that is negative), else all L_b. */
int oracle_paged_prefill_pairs(int B, int Hq, int Hkv, int D, int bs, int NB, int MBS, int dtype,
                               const float* q, const void* k, const void* v,
                               const int64_t* kstrides, const int64_t* vstrides,
                               const int32_t* table, const int32_t* cu_q, const int32_t* seqlens_k,
                               int causal, double scale, const int32_t* pairs, int npairs,
                               double* out) {
  int rc = check_shape(B, Hq, Hkv, D, bs, NB, MBS, dtype);
  if (rc != OR_OK) return rc;
  if (cu_q[0] != 0) return OR_EARG;
  for (int b = 0; b < B; b++) {
    if (cu_q[b + 1] < cu_q[b]) return OR_EARG;
    if (seqlens_k[b] < 0 || (int64_t)seqlens_k[b] > (int64_t)MBS * bs) return OR_ESEQLEN;
  }
  const int total_q = cu_q[B];
  problem p = {B, Hq, Hkv, D, bs, NB, MBS, dtype, q, k, v,
               {kstrides[0], kstrides[1], kstrides[2]}, {vstrides[0], vstrides[1], vstrides[2]},
               table, seqlens_k, scale};
  double* s = (double*)malloc(sizeof(double) * ((size_t)MBS * bs + 1));
  if (!s) return OR_ENOMEM;
  const int G = Hq / Hkv;
  for (int k2 = 0; k2 < npairs; k2++) {
    const int row = pairs[2 * k2], h = pairs[2 * k2 + 1];
    if (row < 0 || row >= total_q || h < 0 || h >= Hq) {
      free(s);
      return OR_EARG;
    }
    int b = 0;
    while (cu_q[b + 1] <= row) b++; /* the sequence holding the row */
    const int qlen = cu_q[b + 1] - cu_q[b], L = seqlens_k[b];
    int kend = L;
    if (causal) {
      kend = L - qlen + (row - cu_q[b]) + 1;
      if (kend < 0) kend = 0;
      if (kend > L) kend = L;
    }
    rc = attend(&p, q + ((int64_t)row * Hq + h) * D, b, h / G, kend, s, out + (int64_t)k2 * D);
    if (rc != OR_OK) {
      free(s);
      return rc;
    }
  }
  free(s);
  return OR_OK;
}

/* Where token t of sequence b lives: writes the table entry and the offset.
 * Returns OR_OK, or OR_ETABLE when the entry is outside [0, NB). Used to pin the
 * token -> slot rule against the docs page's worked example. */
int oracle_token_slot(const int32_t* table, int MBS, int bs, int NB, int b, int t, int32_t* phys,
                      int32_t* off) {
  problem p;
  memset(&p, 0, sizeof p);
  p.table = table;
  p.MBS = MBS;
  p.bs = bs;
  p.NB = NB;
  int o;
  int64_t ph = slot_of(&p, b, t, &o);
  *phys = table[(int64_t)b * MBS + t / bs];
  *off = o;
  return ph < 0 ? OR_ETABLE : OR_OK;
}
