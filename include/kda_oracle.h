/*
 * kda_oracle.h — C ABI of the CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY. This library (liboracle_kda.so, built from oracle/)
 * is the slow, obviously correct fp64 reference that the GPU library is checked
 * against. It shares no code and no header with the GPU library (kda.h); the
 * product path never links or loads it.
 *
 * What it computes (page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache
 * KV", trefon.com, sections "Atencja liniowa: stan o stałym rozmiarze",
 * "Reguła delta: zapisz poprawkę, nie sumę" and "Gated DeltaNet: dodaj zanik"):
 * per sequence and head, a d_v x d_k state S is updated token by token,
 *
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t                      (read-out uses the updated state),
 *
 * where a_t = alpha_t * 1 for the scalar gate (the printed Gated DeltaNet form)
 * and a_t in (0,1]^{d_k} for the per-key-channel (KDA) gate. The per-key form
 * is not printed on the pages; the decay is read as acting on the key axis
 * before the delta correction, which keeps the printed order (decay multiplies
 * S_{t-1} first) and reduces to the scalar form when all channels are equal.
 * Parity unpinned for that one point: with non-uniform a_t and overlapping
 * keys, nothing on the pages fixes the placement; the pins cover the scalar
 * and channel-uniform forms and the orthogonal-key (linear attention) case.
 *
 * Snapshots (same page, section "Co stan rekurencyjny zmienia przy
 * serwowaniu", item 1: prefix reuse needs the state taken at position N):
 * with interval I > 0, the state after the first m*I tokens of each sequence
 * (m = 1 .. floor(len/I)) is written to slot base_n + m - 1, where base_n is
 * the number of snapshots of all earlier sequences (sequence-major order).
 *
 * Layouts (all HOST pointers, row-major, contiguous):
 *   cu_seqlens    int64 [num_seqs+1], cu[0] = 0, nondecreasing; T = cu[num_seqs]
 *   q, k          [T, H, d_k]  bf16 (uint16 bit patterns) or fp32
 *   v             [T, H, d_v]  same dtype as q, k
 *   alpha         fp32 [T, H] (scalar gate) or [T, H, d_k] (per-key gate), in (0, 1]
 *   beta          fp32 [T, H], in [0, 1]
 *   initial_state fp32 [num_seqs, H, d_v, d_k] or NULL (zeros)
 *   o             fp64 [T, H, d_v]
 *   final_state   fp64 [num_seqs, H, d_v, d_k]
 *   snapshots     fp64 [n_snap, H, d_v, d_k] (may be NULL when interval == 0)
 *
 * Errors: negative return codes, nothing written except possibly partial
 * outputs when a non-finite value is found (see report->nonfinite).
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KDA_ORACLE_OK = 0,
  KDA_ORACLE_MISMATCH = 1,   /* check only: a candidate exceeds its tolerance */
  KDA_ORACLE_ERR_ARG = -1,   /* NULL pointer, bad dimension, bad cu_seqlens   */
  KDA_ORACLE_ERR_DOMAIN = -2 /* alpha outside (0,1] or beta outside [0,1]     */
};

/* Number of snapshot slots for the given packing (sum over sequences of
 * floor(len/interval); 0 when interval == 0). Returns KDA_ORACLE_ERR_ARG on a
 * malformed cu_seqlens or a negative interval. */
int kda_oracle_snapshot_count(int32_t num_seqs, const int64_t* cu_seqlens,
                              int64_t interval, int64_t* n_snap);

/* Runs the fp64 token-by-token recurrence. num_threads <= 0 uses every CPU in
 * the process affinity mask. Outputs may be NULL when not wanted. */
int kda_oracle_run(int32_t num_seqs, const int64_t* cu_seqlens,
                   int32_t num_heads, int32_t d_k, int32_t d_v,
                   int32_t qkv_is_bf16, int32_t per_key_gate, int64_t interval,
                   const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta,
                   const float* initial_state, int32_t num_threads,
                   double* o, double* final_state, double* snapshots);

/* Backward pass of the same recurrence in fp64: for the loss
 *   sum_t <d_o_t, o_t> + sum_n <d_final_n, S_final_n>
 * writes its gradients with respect to q, k, v ([T, H, d]), alpha (like
 * alpha), beta ([T, H]) and the initial state ([num_seqs, H, d_v, d_k]; may be
 * NULL). d_o: fp32 [T, H, d_v]; d_final: fp32 [num_seqs, H, d_v, d_k] or NULL
 * (zero). The token update is differentiated in reverse token order with the
 * states recomputed from checkpoints; nothing is chunked. Returns
 * KDA_ORACLE_ERR_ARG on bad arguments or when memory runs out,
 * KDA_ORACLE_ERR_DOMAIN as kda_oracle_run. */
int kda_oracle_backward(int32_t num_seqs, const int64_t* cu_seqlens,
                        int32_t num_heads, int32_t d_k, int32_t d_v,
                        int32_t qkv_is_bf16, int32_t per_key_gate,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta,
                        const float* initial_state, const float* d_o,
                        const float* d_final, int32_t num_threads,
                        double* dq, double* dk, double* dv, double* dalpha,
                        double* dbeta, double* d_initial_state);

typedef struct {
  double o_rel;      /* max over (seq, head) of max|o - o_ref| / max|o_ref|     */
  double final_rel;  /* same over (seq, head) final-state slices                 */
  double snap_rel;   /* same over (snapshot, head) slices                        */
  int64_t n_snap;    /* snapshot slots compared                                  */
  int32_t threads;   /* threads the oracle ran on                                */
  int32_t nonfinite; /* 1 if a candidate or reference value is NaN/Inf           */
  double seconds;    /* wall time of the reference computation                   */
} kda_check_report;

/* Computes the reference (as kda_oracle_run) and compares the fp32 candidates
 * (each may be NULL to skip it) with the slice-max-normalised error above.
 * Returns KDA_ORACLE_OK if every supplied candidate is within its tolerance,
 * KDA_ORACLE_MISMATCH otherwise (or on any non-finite value), negative on an
 * argument error. o_ref / final_ref / snap_ref receive the fp64 reference when
 * non-NULL. */
int kda_recurrent_ref_check(int32_t num_seqs, const int64_t* cu_seqlens,
                            int32_t num_heads, int32_t d_k, int32_t d_v,
                            int32_t qkv_is_bf16, int32_t per_key_gate,
                            int64_t interval,
                            const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta,
                            const float* initial_state,
                            const float* o_cand, const float* final_cand,
                            const float* snap_cand,
                            double o_tol, double state_tol, int32_t num_threads,
                            double* o_ref, double* final_ref, double* snap_ref,
                            kda_check_report* report);

#ifdef __cplusplus
}
#endif
#endif /* KDA_ORACLE_H */
