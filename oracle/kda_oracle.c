/*
 * kda_oracle.c — plain fp64 CPU oracle of the gated delta rule.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline load this library. It shares no code, header, table or helper with
 * the GPU library; inputs reach it as plain host arrays.
 *
 * The recurrence is written exactly as printed on the page "Modele hybrydowe:
 * co Gated DeltaNet zastępuje w cache KV" (trefon.com):
 *   - section "Gated DeltaNet: dodaj zanik":
 *       S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   - section "Atencja liniowa: stan o stałym rozmiarze": state is d_v x d_k
 *     per head, read-out o_t = S_t q_t (the state after the token's update).
 *   - section "Reguła delta: zapisz poprawkę, nie sumę": read what the state
 *     predicts for k_t, write only the error, scaled by beta_t.
 * Expanding the product gives, with S' = S_{t-1} Diag(a_t):
 *       S_t = S' - beta_t (S' k_t) k_t^T + beta_t v_t k_t^T = S' + u_t k_t^T,
 *       u_t = beta_t (v_t - S' k_t).
 * The per-key-channel (KDA) gate replaces alpha_t by Diag(a_t) on the key
 * axis, applied first; with all a_t[j] equal it is the printed scalar form.
 *
 * Row i of S only ever touches row i (each term above acts on rows
 * independently), so the work is split over (sequence, head, block of rows);
 * each row is updated token by token in fp64 with plain sequential sums.
 * There is no chunking, blocking or reordering of the token loop.
 *
 * Snapshots follow section "Co stan rekurencyjny zmienia przy serwowaniu",
 * item 1: the state at position N is kept, here at N = m * interval.
 *
 * Pins (tests/test_oracle_pins.py, tests/test_chunk_rederivation.py) fix the
 * scalar form, the channel-uniform per-key form and, for non-uniform per-key
 * decay, the decayed linear-attention reduction (orthogonal keys, where the
 * read S' k_t vanishes). Parity unpinned: for non-uniform a_t with keys that
 * overlap, no page prints where Diag(a_t) sits relative to the read S' k_t;
 * the printed scalar order (decay first, then read and write) is carried over.
 */
#define _GNU_SOURCE
#include "../include/kda_oracle.h"

#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

/* bf16 -> fp64 exactly: a bf16 value is the upper half of an fp32 value. */
static double bf16_to_double(uint16_t x) {
  uint32_t bits = ((uint32_t)x) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double load_elem(const void* base, int is_bf16, int64_t idx) {
  if (is_bf16) return bf16_to_double(((const uint16_t*)base)[idx]);
  return (double)((const float*)base)[idx];
}

int kda_oracle_snapshot_count(int32_t num_seqs, const int64_t* cu, int64_t interval,
                              int64_t* n_snap) {
  if (num_seqs < 0 || !cu || !n_snap || interval < 0) return KDA_ORACLE_ERR_ARG;
  if (cu[0] != 0) return KDA_ORACLE_ERR_ARG;
  int64_t total = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    int64_t len = cu[n + 1] - cu[n];
    if (len < 0) return KDA_ORACLE_ERR_ARG;
    if (interval > 0) total += len / interval;
  }
  *n_snap = total;
  return KDA_ORACLE_OK;
}

typedef struct {
  /* problem */
  int32_t num_seqs, H, dk, dv, is_bf16, per_key;
  int64_t interval;
  const int64_t* cu;
  const int64_t* snap_base; /* [num_seqs] first slot of each sequence */
  const void *q, *k, *v;
  const float *alpha, *beta, *init;
  double *o, *fin, *snap;
  /* work split */
  int32_t rows_per_block, blocks_per_head;
  int64_t n_units;
  int64_t next_unit; /* shared counter, guarded by lock */
  pthread_mutex_t lock;
} oracle_job;

/* One unit: sequence n, head h, rows [i0, i1) of the state. */
static void run_unit(const oracle_job* J, int64_t unit, double* S, double* kt,
                     double* qt, double* at) {
  const int32_t H = J->H, dk = J->dk, dv = J->dv;
  const int64_t per_seq = (int64_t)H * J->blocks_per_head;
  const int32_t n = (int32_t)(unit / per_seq);
  const int32_t h = (int32_t)((unit % per_seq) / J->blocks_per_head);
  const int32_t blk = (int32_t)(unit % J->blocks_per_head);
  const int32_t i0 = blk * J->rows_per_block;
  int32_t i1 = i0 + J->rows_per_block;
  if (i1 > dv) i1 = dv;
  if (i0 >= i1) return;
  const int32_t rows = i1 - i0;

  /* 1. initial state rows (fp32 -> fp64 exactly), or zeros */
  for (int32_t i = 0; i < rows; ++i)
    for (int32_t j = 0; j < dk; ++j)
      S[(int64_t)i * dk + j] =
          J->init ? (double)J->init[(((int64_t)n * H + h) * dv + (i0 + i)) * dk + j] : 0.0;

  const int64_t t_begin = J->cu[n], len = J->cu[n + 1] - J->cu[n];
  for (int64_t t = 0; t < len; ++t) {
    const int64_t tok = t_begin + t;
    const int64_t qk_off = (tok * H + h) * (int64_t)dk;
    for (int32_t j = 0; j < dk; ++j) {
      kt[j] = load_elem(J->k, J->is_bf16, qk_off + j);
      qt[j] = load_elem(J->q, J->is_bf16, qk_off + j);
      at[j] = J->per_key ? (double)J->alpha[qk_off + j] : (double)J->alpha[tok * H + h];
    }
    const double beta = (double)J->beta[tok * H + h];
    for (int32_t i = 0; i < rows; ++i) {
      double* s = S + (int64_t)i * dk;
      const double vi = load_elem(J->v, J->is_bf16, (tok * H + h) * (int64_t)dv + i0 + i);
      /* 2. decay: S' = S Diag(a_t) (scalar gate: every a_t[j] = alpha_t) */
      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] * at[j];
      /* 3. prediction p = S' k_t */
      double p = 0.0;
      for (int32_t j = 0; j < dk; ++j) p += s[j] * kt[j];
      /* 4. written error u = beta_t (v_t - p) */
      const double u = beta * (vi - p);
      /* 5. S_t = S' + u k_t^T */
      for (int32_t j = 0; j < dk; ++j) s[j] = s[j] + u * kt[j];
      /* 6. read-out o_t = S_t q_t */
      if (J->o) {
        double r = 0.0;
        for (int32_t j = 0; j < dk; ++j) r += s[j] * qt[j];
        J->o[(tok * H + h) * (int64_t)dv + i0 + i] = r;
      }
    }
    /* 7. snapshot of the state after the first (t+1) tokens */
    if (J->interval > 0 && J->snap && (t + 1) % J->interval == 0) {
      const int64_t slot = J->snap_base[n] + (t + 1) / J->interval - 1;
      for (int32_t i = 0; i < rows; ++i)
        memcpy(J->snap + ((slot * H + h) * dv + (i0 + i)) * (int64_t)dk,
               S + (int64_t)i * dk, sizeof(double) * (size_t)dk);
    }
  }
  if (J->fin)
    for (int32_t i = 0; i < rows; ++i)
      memcpy(J->fin + (((int64_t)n * H + h) * dv + (i0 + i)) * (int64_t)dk,
             S + (int64_t)i * dk, sizeof(double) * (size_t)dk);
}

static void* worker(void* arg) {
  oracle_job* J = (oracle_job*)arg;
  double* S = (double*)malloc(sizeof(double) * (size_t)J->rows_per_block * (size_t)J->dk);
  double* kt = (double*)malloc(sizeof(double) * (size_t)J->dk * 3);
  if (!S || !kt) { free(S); free(kt); return NULL; }
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int64_t unit = J->next_unit++;
    pthread_mutex_unlock(&J->lock);
    if (unit >= J->n_units) break;
    run_unit(J, unit, S, kt, kt + J->dk, kt + 2 * J->dk);
  }
  free(S);
  free(kt);
  return NULL;
}

static int affinity_cpus(void) {
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  return 1;
}

static double now_seconds(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

static int validate(int32_t num_seqs, const int64_t* cu, int32_t H, int32_t dk, int32_t dv,
                    int64_t interval, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, int32_t per_key) {
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || interval < 0 || !cu) return KDA_ORACLE_ERR_ARG;
  if (cu[0] != 0) return KDA_ORACLE_ERR_ARG;
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu[n + 1] < cu[n]) return KDA_ORACLE_ERR_ARG;
  const int64_t T = cu[num_seqs];
  if (T > 0 && (!q || !k || !v || !alpha || !beta)) return KDA_ORACLE_ERR_ARG;
  const int64_t na = per_key ? T * H * (int64_t)dk : T * H;
  for (int64_t i = 0; i < na; ++i)
    if (!(alpha[i] > 0.0f && alpha[i] <= 1.0f)) return KDA_ORACLE_ERR_DOMAIN;
  for (int64_t i = 0; i < T * H; ++i)
    if (!(beta[i] >= 0.0f && beta[i] <= 1.0f)) return KDA_ORACLE_ERR_DOMAIN;
  return KDA_ORACLE_OK;
}

static int run_internal(int32_t num_seqs, const int64_t* cu, int32_t H, int32_t dk, int32_t dv,
                        int32_t is_bf16, int32_t per_key, int64_t interval, const void* q,
                        const void* k, const void* v, const float* alpha, const float* beta,
                        const float* init, int32_t num_threads, double* o, double* fin,
                        double* snap, int32_t* threads_used) {
  int rc = validate(num_seqs, cu, H, dk, dv, interval, q, k, v, alpha, beta, per_key);
  if (rc != KDA_ORACLE_OK) return rc;
  int64_t* base = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_seqs > 0 ? num_seqs : 1));
  if (!base) return KDA_ORACLE_ERR_ARG;
  int64_t acc = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    base[n] = acc;
    if (interval > 0) acc += (cu[n + 1] - cu[n]) / interval;
  }

  int nthreads = num_threads > 0 ? num_threads : affinity_cpus();
  oracle_job J;
  memset(&J, 0, sizeof J);
  J.num_seqs = num_seqs; J.H = H; J.dk = dk; J.dv = dv; J.is_bf16 = is_bf16; J.per_key = per_key;
  J.interval = interval; J.cu = cu; J.snap_base = base;
  J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.init = init;
  J.o = o; J.fin = fin; J.snap = snap;
  /* Row blocks: enough units to keep every thread busy, at least 8 rows each. */
  const int64_t seq_heads = (int64_t)num_seqs * H;
  int32_t blocks = 1;
  while (blocks < dv && seq_heads * blocks < 4 * (int64_t)nthreads && dv / (blocks * 2) >= 8) blocks *= 2;
  J.blocks_per_head = blocks;
  J.rows_per_block = (dv + blocks - 1) / blocks;
  J.n_units = seq_heads * blocks;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads > J.n_units) nthreads = (int)(J.n_units > 0 ? J.n_units : 1);

  /* The calling thread is worker 0; helpers 1..nthreads-1 that fail to start
   * are simply not counted (the shared queue still covers every unit). */
  pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  char* ok = (char*)calloc((size_t)nthreads, 1);
  for (int i = 1; tids && ok && i < nthreads; ++i)
    ok[i] = pthread_create(&tids[i], NULL, worker, &J) == 0;
  worker(&J);
  int joined = 1;
  for (int i = 1; tids && ok && i < nthreads; ++i)
    if (ok[i] && pthread_join(tids[i], NULL) == 0) ++joined;
  free(ok);
  free(tids);
  pthread_mutex_destroy(&J.lock);
  free(base);
  if (threads_used) *threads_used = joined;
  return KDA_ORACLE_OK;
}

int kda_oracle_run(int32_t num_seqs, const int64_t* cu, int32_t H, int32_t dk, int32_t dv,
                   int32_t is_bf16, int32_t per_key, int64_t interval, const void* q,
                   const void* k, const void* v, const float* alpha, const float* beta,
                   const float* init, int32_t num_threads, double* o, double* fin,
                   double* snap) {
  return run_internal(num_seqs, cu, H, dk, dv, is_bf16, per_key, interval, q, k, v, alpha, beta,
                      init, num_threads, o, fin, snap, NULL);
}

/* max|x - r| / max|r| over one contiguous slice of `count` elements. */
static double slice_rel(const float* x, const double* r, int64_t count, int* nonfinite) {
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < count; ++i) {
    double xv = (double)x[i];
    if (!isfinite(xv) || !isfinite(r[i])) { *nonfinite = 1; continue; }
    double d = fabs(xv - r[i]);
    if (d > num) num = d;
    if (fabs(r[i]) > den) den = fabs(r[i]);
  }
  if (den < 1e-30) den = 1e-30;
  return num / den;
}

int kda_recurrent_ref_check(int32_t num_seqs, const int64_t* cu, int32_t H, int32_t dk,
                            int32_t dv, int32_t is_bf16, int32_t per_key, int64_t interval,
                            const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* init, const float* o_cand,
                            const float* final_cand, const float* snap_cand, double o_tol,
                            double state_tol, int32_t num_threads, double* o_ref,
                            double* final_ref, double* snap_ref, kda_check_report* report) {
  if (!report) return KDA_ORACLE_ERR_ARG;
  memset(report, 0, sizeof *report);
  int rc = validate(num_seqs, cu, H, dk, dv, interval, q, k, v, alpha, beta, per_key);
  if (rc != KDA_ORACLE_OK) return rc;
  int64_t n_snap = 0;
  kda_oracle_snapshot_count(num_seqs, cu, interval, &n_snap);
  const int64_t T = cu[num_seqs];
  const int64_t state_elems = (int64_t)dv * dk;

  double* o_buf = o_ref ? o_ref : (double*)malloc(sizeof(double) * (size_t)(T * H * dv + 1));
  double* f_buf = final_ref ? final_ref
                            : (double*)malloc(sizeof(double) * (size_t)((int64_t)num_seqs * H * state_elems + 1));
  double* s_buf = snap_ref ? snap_ref : (double*)malloc(sizeof(double) * (size_t)(n_snap * H * state_elems + 1));
  if (!o_buf || !f_buf || !s_buf) {
    if (!o_ref) free(o_buf);
    if (!final_ref) free(f_buf);
    if (!snap_ref) free(s_buf);
    return KDA_ORACLE_ERR_ARG;
  }
  double t0 = now_seconds();
  int32_t used = 0;
  rc = run_internal(num_seqs, cu, H, dk, dv, is_bf16, per_key, interval, q, k, v, alpha, beta,
                    init, num_threads, o_buf, f_buf, n_snap > 0 ? s_buf : NULL, &used);
  report->seconds = now_seconds() - t0;
  report->threads = used;
  report->n_snap = n_snap;
  if (rc == KDA_ORACLE_OK) {
    int nonfinite = 0;
    /* o: slice (seq n, head h) = tokens of n, all d_v channels of head h */
    if (o_cand) {
      for (int32_t n = 0; n < num_seqs; ++n)
        for (int32_t h = 0; h < H; ++h) {
          double num = 0.0, den = 0.0;
          for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t off = (t * H + h) * (int64_t)dv;
            for (int32_t i = 0; i < dv; ++i) {
              double xv = (double)o_cand[off + i], rv = o_buf[off + i];
              if (!isfinite(xv) || !isfinite(rv)) { nonfinite = 1; continue; }
              double d = fabs(xv - rv);
              if (d > num) num = d;
              if (fabs(rv) > den) den = fabs(rv);
            }
          }
          if (cu[n + 1] > cu[n]) {
            double rel = num / (den < 1e-30 ? 1e-30 : den);
            if (rel > report->o_rel) report->o_rel = rel;
          }
        }
    }
    if (final_cand)
      for (int64_t s = 0; s < (int64_t)num_seqs * H; ++s) {
        double rel = slice_rel(final_cand + s * state_elems, f_buf + s * state_elems, state_elems, &nonfinite);
        if (rel > report->final_rel) report->final_rel = rel;
      }
    if (snap_cand)
      for (int64_t s = 0; s < n_snap * H; ++s) {
        double rel = slice_rel(snap_cand + s * state_elems, s_buf + s * state_elems, state_elems, &nonfinite);
        if (rel > report->snap_rel) report->snap_rel = rel;
      }
    report->nonfinite = nonfinite;
    int pass = !nonfinite && (!o_cand || report->o_rel <= o_tol) &&
               (!final_cand || report->final_rel <= state_tol) &&
               (!snap_cand || report->snap_rel <= state_tol);
    rc = pass ? KDA_ORACLE_OK : KDA_ORACLE_MISMATCH;
  }
  if (!o_ref) free(o_buf);
  if (!final_ref) free(f_buf);
  if (!snap_ref) free(s_buf);
  return rc;
}

/* ------------------------------------------------------------------------- *
 * Backward pass (gradients of the recurrence above).
 *
 * For a loss that depends on the outputs o_t and on the final states, the
 * gradients with respect to q, k, v, the gate a, beta and the initial state
 * follow from the chain rule applied to the token update in reverse token
 * order. With S' = S_{t-1} Diag(a_t), p = S' k_t, u = v_t - p (so that
 * S_t = S' + beta_t u k_t^T) and dS the gradient arriving at S_t from later
 * tokens and the final state:
 *   6'  read-out o_t = S_t q_t:     dS <- dS + do_t q_t^T,  dq_t = S_t^T do_t
 *   5'  S_t = S' + beta u k^T:      w = dS k,  dbeta_t = u . w,
 *                                   du = beta w,  dk_t = beta dS^T u,
 *                                   dS' = dS - du k^T
 *   4'  u = v - p:                  dv_t = du,  dp = -du
 *   3'  p = S' k:                   dS' <- dS' + dp k^T (folded into 5'),
 *                                   dk_t <- dk_t + S'^T dp
 *   2'  S' = S_{t-1} Diag(a):       da_t[j] = sum_i dS'[i][j] S_{t-1}[i][j]
 *                                   (scalar gate: the sum over j as well),
 *                                   dS_{t-1} = dS' Diag(a_t)
 * and the gradient of the initial state is dS after the first token. The
 * states S_{t-1} are recomputed forward from checkpoints kept every CK tokens
 * (CK about sqrt(len)), with the same token update as the forward loop, so
 * each backward step sees exactly the forward's values. One (sequence, head)
 * is one unit of work: the rows of dS are coupled through dk.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t num_seqs, H, dk, dv, is_bf16, per_key;
  const int64_t* cu;
  const void *q, *k, *v;
  const float *alpha, *beta, *init, *d_o, *d_final;
  double *dq, *dk_out, *dv_out, *dalpha, *dbeta, *d_init;
  int64_t n_units, next_unit;
  pthread_mutex_t lock;
  int failed;
} bwd_job;

/* one forward token update of the whole d_v x d_k state, in place */
static void fwd_token(const bwd_job* J, int32_t h, int64_t tok, double* S, double* kt, double* at) {
  const int32_t H = J->H, dk = J->dk, dv = J->dv;
  const int64_t qk_off = (tok * H + h) * (int64_t)dk;
  for (int32_t j = 0; j < dk; ++j) {
    kt[j] = load_elem(J->k, J->is_bf16, qk_off + j);
    at[j] = J->per_key ? (double)J->alpha[qk_off + j] : (double)J->alpha[tok * H + h];
  }
  const double beta = (double)J->beta[tok * H + h];
  for (int32_t i = 0; i < dv; ++i) {
    double* s = S + (int64_t)i * dk;
    const double vi = load_elem(J->v, J->is_bf16, (tok * H + h) * (int64_t)dv + i);
    for (int32_t j = 0; j < dk; ++j) s[j] = s[j] * at[j];
    double p = 0.0;
    for (int32_t j = 0; j < dk; ++j) p += s[j] * kt[j];
    const double u = beta * (vi - p);
    for (int32_t j = 0; j < dk; ++j) s[j] = s[j] + u * kt[j];
  }
}

static int bwd_unit(bwd_job* J, int64_t unit) {
  const int32_t H = J->H, dk = J->dk, dv = J->dv;
  const int32_t n = (int32_t)(unit / H), h = (int32_t)(unit % H);
  const int64_t t_begin = J->cu[n], len = J->cu[n + 1] - J->cu[n];
  const int64_t se = (int64_t)dv * dk;
  int64_t CK = 1;
  while (CK * CK < len) ++CK;
  const int64_t nck = len > 0 ? (len + CK - 1) / CK : 0;
  double* ckpt = (double*)malloc(sizeof(double) * (size_t)((nck > 0 ? nck : 1) * se));
  double* buf = (double*)malloc(sizeof(double) * (size_t)((CK + 1) * se));
  double* dS = (double*)malloc(sizeof(double) * (size_t)se);
  double* vec = (double*)malloc(sizeof(double) * (size_t)(5 * dk + 4 * dv));
  if (!ckpt || !buf || !dS || !vec) { free(ckpt); free(buf); free(dS); free(vec); return -1; }
  double *kt = vec, *qt = vec + dk, *at = vec + 2 * dk, *dkt = vec + 3 * dk, *dat = vec + 4 * dk;
  double *dot = vec + 5 * dk, *u = dot + dv, *w = u + dv, *vt = w + dv;

  /* forward: the state before token m*CK of the sequence, m = 0 .. nck-1 */
  double* S = buf;
  for (int64_t e = 0; e < se; ++e)
    S[e] = J->init ? (double)J->init[((int64_t)n * H + h) * se + e] : 0.0;
  for (int64_t t = 0; t < len; ++t) {
    if (t % CK == 0) memcpy(ckpt + (t / CK) * se, S, sizeof(double) * (size_t)se);
    fwd_token(J, h, t_begin + t, S, kt, at);
  }

  for (int64_t e = 0; e < se; ++e)
    dS[e] = J->d_final ? (double)J->d_final[((int64_t)n * H + h) * se + e] : 0.0;

  for (int64_t m = nck - 1; m >= 0; --m) {
    const int64_t t0 = m * CK, t1 = (t0 + CK < len) ? t0 + CK : len;
    /* buf[r] = state before token t0 + r, r = 0 .. t1 - t0 (the last: after t1 - 1) */
    memcpy(buf, ckpt + m * se, sizeof(double) * (size_t)se);
    for (int64_t t = t0; t < t1; ++t) {
      memcpy(buf + (t - t0 + 1) * se, buf + (t - t0) * se, sizeof(double) * (size_t)se);
      fwd_token(J, h, t_begin + t, buf + (t - t0 + 1) * se, kt, at);
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const int64_t tok = t_begin + t;
      const double* Sp = buf + (t - t0) * se;      /* S_{t-1} */
      const double* St = buf + (t - t0 + 1) * se;  /* S_t */
      const int64_t qk_off = (tok * H + h) * (int64_t)dk, v_off = (tok * H + h) * (int64_t)dv;
      for (int32_t j = 0; j < dk; ++j) {
        kt[j] = load_elem(J->k, J->is_bf16, qk_off + j);
        qt[j] = load_elem(J->q, J->is_bf16, qk_off + j);
        at[j] = J->per_key ? (double)J->alpha[qk_off + j] : (double)J->alpha[tok * H + h];
      }
      const double beta = (double)J->beta[tok * H + h];
      for (int32_t i = 0; i < dv; ++i) {
        dot[i] = (double)J->d_o[v_off + i];
        vt[i] = load_elem(J->v, J->is_bf16, v_off + i);
      }
      /* forward quantities of this token: u = v - S' k */
      for (int32_t i = 0; i < dv; ++i) {
        double p = 0.0;
        for (int32_t j = 0; j < dk; ++j) p += Sp[(int64_t)i * dk + j] * at[j] * kt[j];
        u[i] = vt[i] - p;
      }
      /* 6' read-out */
      for (int32_t i = 0; i < dv; ++i)
        for (int32_t j = 0; j < dk; ++j) dS[(int64_t)i * dk + j] += dot[i] * qt[j];
      for (int32_t j = 0; j < dk; ++j) {
        double r = 0.0;
        for (int32_t i = 0; i < dv; ++i) r += St[(int64_t)i * dk + j] * dot[i];
        J->dq[qk_off + j] = r;
      }
      /* 5' the written correction */
      double db = 0.0;
      for (int32_t i = 0; i < dv; ++i) {
        double r = 0.0;
        for (int32_t j = 0; j < dk; ++j) r += dS[(int64_t)i * dk + j] * kt[j];
        w[i] = r;
        db += u[i] * r;
      }
      J->dbeta[tok * H + h] = db;
      for (int32_t j = 0; j < dk; ++j) {
        double r = 0.0;
        for (int32_t i = 0; i < dv; ++i) r += dS[(int64_t)i * dk + j] * u[i];
        dkt[j] = beta * r;
      }
      /* 4' / 3': du = beta w = dv_t, dp = -du */
      for (int32_t i = 0; i < dv; ++i) J->dv_out[v_off + i] = beta * w[i];
      for (int32_t j = 0; j < dk; ++j) {
        double r = 0.0;
        for (int32_t i = 0; i < dv; ++i) r += Sp[(int64_t)i * dk + j] * at[j] * (beta * w[i]);
        dkt[j] -= r;
        J->dk_out[qk_off + j] = dkt[j];
      }
      /* dS' = dS - du k^T, then 2' the decay */
      for (int32_t j = 0; j < dk; ++j) dat[j] = 0.0;
      for (int32_t i = 0; i < dv; ++i)
        for (int32_t j = 0; j < dk; ++j) {
          const double g = dS[(int64_t)i * dk + j] - beta * w[i] * kt[j];
          dat[j] += g * Sp[(int64_t)i * dk + j];
          dS[(int64_t)i * dk + j] = g * at[j];
        }
      if (J->per_key) {
        for (int32_t j = 0; j < dk; ++j) J->dalpha[qk_off + j] = dat[j];
      } else {
        double r = 0.0;
        for (int32_t j = 0; j < dk; ++j) r += dat[j];
        J->dalpha[tok * H + h] = r;
      }
    }
  }
  if (J->d_init) memcpy(J->d_init + ((int64_t)n * H + h) * se, dS, sizeof(double) * (size_t)se);
  free(ckpt); free(buf); free(dS); free(vec);
  return 0;
}

static void* bwd_worker(void* arg) {
  bwd_job* J = (bwd_job*)arg;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int64_t unit = J->next_unit++;
    pthread_mutex_unlock(&J->lock);
    if (unit >= J->n_units) break;
    if (bwd_unit(J, unit) != 0) {
      pthread_mutex_lock(&J->lock);
      J->failed = 1;
      pthread_mutex_unlock(&J->lock);
    }
  }
  return NULL;
}

int kda_oracle_backward(int32_t num_seqs, const int64_t* cu, int32_t H, int32_t dk, int32_t dv,
                        int32_t is_bf16, int32_t per_key, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const float* init, const float* d_o,
                        const float* d_final, int32_t num_threads, double* dq, double* dk_out,
                        double* dv_out, double* dalpha, double* dbeta, double* d_init) {
  int rc = validate(num_seqs, cu, H, dk, dv, 0, q, k, v, alpha, beta, per_key);
  if (rc != KDA_ORACLE_OK) return rc;
  const int64_t T = cu[num_seqs];
  if (T > 0 && (!d_o || !dq || !dk_out || !dv_out || !dalpha || !dbeta)) return KDA_ORACLE_ERR_ARG;
  int nthreads = num_threads > 0 ? num_threads : affinity_cpus();
  bwd_job J;
  memset(&J, 0, sizeof J);
  J.num_seqs = num_seqs; J.H = H; J.dk = dk; J.dv = dv; J.is_bf16 = is_bf16; J.per_key = per_key;
  J.cu = cu; J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.init = init;
  J.d_o = d_o; J.d_final = d_final;
  J.dq = dq; J.dk_out = dk_out; J.dv_out = dv_out; J.dalpha = dalpha; J.dbeta = dbeta; J.d_init = d_init;
  J.n_units = (int64_t)num_seqs * H;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads > J.n_units) nthreads = (int)(J.n_units > 0 ? J.n_units : 1);
  pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  char* ok = (char*)calloc((size_t)nthreads, 1);
  for (int i = 1; tids && ok && i < nthreads; ++i)
    ok[i] = pthread_create(&tids[i], NULL, bwd_worker, &J) == 0;
  bwd_worker(&J);
  for (int i = 1; tids && ok && i < nthreads; ++i)
    if (ok[i]) pthread_join(tids[i], NULL);
  free(ok);
  free(tids);
  pthread_mutex_destroy(&J.lock);
  return J.failed ? KDA_ORACLE_ERR_ARG : KDA_ORACLE_OK;
}
