/*
 * kda.h — C ABI of libkda.so: the gated delta rule (Gated DeltaNet / KDA) on
 * MI355X (gfx950), as hand-written HIP kernels.
 *
 * The operation (page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache
 * KV", trefon.com, section "Gated DeltaNet: dodaj zanik", with the read-out of
 * section "Atencja liniowa: stan o stałym rozmiarze"): per sequence and head a
 * d_v x d_k fp32 state S evolves token by token as
 *
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 *
 * with a_t = alpha_t * 1 for the scalar gate and a_t in (0,1]^{d_k} for the
 * per-key-channel (KDA) gate, applied on the key axis before the delta
 * correction. No 1/sqrt(d_k) scale is applied to q: callers pre-scale it.
 *
 * Common conventions
 *   - Every tensor is caller-owned device memory, row-major and contiguous.
 *     The library never allocates: temporary storage comes from the caller's
 *     workspace. Pointers must stay valid until the stream's work completes.
 *   - q, k: [T, H, d_k]; v: [T, H, d_v] in bf16 (KDA_BF16) or fp32 (KDA_F32).
 *     alpha: fp32 [T, H] (KDA_GATE_SCALAR) or [T, H, d_k] (KDA_GATE_PER_KEY),
 *     values in (0, 1]. beta: fp32 [T, H] in [0, 1]. States are fp32
 *     [.., H, d_v, d_k] (d_k contiguous). o is fp32 [T, H, d_v].
 *   - Supported: d_k and d_v each 64 or 128 (the state is d_v x d_k, page
 *     "Modele hybrydowe…", section "Atencja liniowa: stan o stałym rozmiarze");
 *     kda_prefill_backward and kda_layer_front need d_k = d_v (KDA_ERR_SHAPE
 *     otherwise: their kernels run square heads only); chunk = 64.
 *   - Outputs must not overlap inputs or each other (KDA_ERR_ARG), except
 *     where an entry point states an exact alias it allows.
 *   - Alignment: q, k, v, per-key alpha, every state and the prefill's o
 *     16 bytes (8 bytes for bf16 q, k in kda_decode_step); scalar alpha,
 *     beta and the decode steps' o 4 bytes; cu_seqlens_dev 8 bytes;
 *     workspace 16 bytes. Otherwise KDA_ERR_ALIGN.
 *   - All compute entry points are asynchronous on the caller's hipStream_t
 *     (passed as void*, NULL = default stream).
 *   - Errors: negative status codes are detected on the host before anything
 *     is enqueued; outputs are then untouched. KDA_ERR_DEVICE reports a HIP
 *     launch failure (work may be partly enqueued). kda_last_error() gives the
 *     text of the calling thread's last failure.
 *   - Determinism: no atomics; results are bitwise reproducible run to run.
 *     With a fixed segment plan (see kda_prefill_chunked) a sequence's
 *     results do not depend on the other sequences of the pack.
 *
 * Numerical preconditions of the chunked prefill (its matrix products run on
 * fp16 MFMA with fp32 accumulation; see kda_prefill_chunked):
 *     |q|, |k| entries <= 16, |v| entries <= 4096, state entries <= 4096, and,
 *     for the per-key gate, within each aligned block of 16 tokens of a chunk
 *     every key channel's decay product stays above 2^-100 (any alpha above
 *     0.0131 per token satisfies it). The page's gate is any alpha in (0, 1);
 *     below this limit a decay factor formed relative to the block's first
 *     token leaves the fp32 range and the outputs become inf or NaN. The
 *     library does not read alpha on the host, so it cannot reject such input.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum {
  KDA_OK = 0,
  KDA_ERR_ARG = -1,       /* NULL pointer, unsupported enum, negative size      */
  KDA_ERR_SHAPE = -2,     /* unsupported d_k/d_v/chunk, bad cu_seqlens, interval */
  KDA_ERR_ALIGN = -3,     /* a pointer is misaligned for the accesses made on it */
  KDA_ERR_WORKSPACE = -4, /* workspace missing or too small                      */
  KDA_ERR_DEVICE = -5     /* HIP error while enqueueing                          */
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;
typedef enum { KDA_GATE_SCALAR = 0, KDA_GATE_PER_KEY = 1 } kda_gate;

typedef struct {
  int32_t num_heads; /* H, 1 .. 65535                       */
  int32_t d_k;       /* key / query channels per head       */
  int32_t d_v;       /* value channels per head             */
  int32_t qkv_dtype; /* kda_dtype of q, k, v                */
  int32_t gate;      /* kda_gate: layout of alpha           */
} kda_shape;

/* ABI version of the loaded library (KDA_ABI_VERSION at build time). */
int kda_abi_version(void);

/* Text of the calling thread's last non-OK status ("" if none). */
const char* kda_last_error(void);

/* Number of snapshot slots: sum over sequences of floor(len / interval), 0
 * when interval == 0. Host-only. Page "Modele hybrydowe…", section "Co stan
 * rekurencyjny zmienia przy serwowaniu", item 1 (state kept at position N).
 * Errors: KDA_ERR_ARG (NULL), KDA_ERR_SHAPE (cu_seqlens not starting at 0 or
 * decreasing, negative interval). */
int kda_snapshot_count(int32_t num_seqs, const int64_t* cu_seqlens_host, int64_t interval,
                       int64_t* n_snap);

/* Bytes of device workspace kda_prefill_chunked needs for this packing
 * (host-only). Same error codes as kda_prefill_chunked's validation. */
int kda_prefill_workspace_size(const kda_shape* shape, int32_t num_seqs,
                               const int64_t* cu_seqlens_host, int32_t chunk,
                               int64_t snapshot_interval, int64_t segment_tokens,
                               size_t* bytes);

/* Chunkwise-parallel prefill over a varlen pack.
 *
 * Same page, closing paragraph of "Co stan rekurencyjny zmienia przy
 * serwowaniu": inside a chunk of tokens the updates are dense matrix
 * products and only the passage from chunk to chunk is sequential. Chunks of
 * `chunk` tokens restart at every sequence start (the last one may be
 * partial). Per chunk the kernels form the decayed key Gram matrix, solve the
 * unit-lower-triangular system of the UT/WY form in LDS, and pass the fp32
 * state to the next chunk with MFMA products.
 *
 * Segments: a run of chunks maps the state affinely, S_end = S_start M + N.
 * When the (sequence, head) chains are too few to fill the GPU, long
 * sequences are cut into segments of `segment_tokens` tokens: one pass
 * computes every middle segment's (M, N) and runs the first segment, a fp32
 * scan composes the segment start states, and a last pass reruns the
 * segments from their true start states.
 *
 * cu_seqlens_host / cu_seqlens_dev: the same int64 [num_seqs+1] offsets on
 *   host (validation, grid sizing) and device (indexing); cu[0] = 0,
 *   nondecreasing, T = cu[num_seqs]. Empty sequences are allowed.
 * chunk: must be 64.
 * segment_tokens: -1 = automatic (segments only when num_seqs * H is below
 *   the device's compute-unit count; the plan then depends on the whole
 *   pack, so a sequence's rounding can differ from a solo run, within the
 *   tolerances), 0 = never segment, > 0 = segment length, a multiple of 64.
 *   With a fixed value (0 or > 0) each sequence's results are bitwise
 *   independent of the rest of the pack.
 * snapshot_interval: 0, or a positive multiple of `chunk`. The state after
 *   the first m*interval tokens of each sequence (m = 1..floor(len/interval))
 *   is written to snapshots[base_n + m - 1], base_n = slots of the earlier
 *   sequences ([n_snap, H, d_v, d_k], see kda_snapshot_count).
 * initial_state: [num_seqs, H, d_v, d_k] or NULL (zeros). May alias
 *   final_state.
 * o: [T, H, d_v]; final_state: [num_seqs, H, d_v, d_k]; neither may overlap
 *   an input (KDA_ERR_ARG), except final_state = initial_state exactly;
 * snapshots: NULL iff the slot count is 0. Device memory, or pinned host
 *   memory (hipHostMalloc; torch pin_memory=True): the kernels then write the
 *   snapshot states over the bus while the prefill runs, which offloads them
 *   to host RAM for prefix reuse without a separate copy (same page, section
 *   "Co stan rekurencyjny zmienia przy serwowaniu", item 1 and the rule on
 *   planning host memory for checkpoints). Pageable host memory is rejected
 *   with KDA_ERR_ARG.
 * workspace: device memory of at least kda_prefill_workspace_size bytes.
 * Rectangular heads: rows of the state evolve independently (row i sees only
 *   value channel i), so d_v = 2 d_k runs each head as two value heads of d_k
 *   rows sharing q, k and the gates, and d_k = 2 d_v pads v and the states
 *   with zero rows to d_k inside the workspace (zero rows stay zero) and
 *   copies o, the final states and the snapshots back.
 */
int kda_prefill_chunked(const kda_shape* shape, int32_t num_seqs,
                        const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                        int32_t chunk, int64_t snapshot_interval, int64_t segment_tokens,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta,
                        const float* initial_state,
                        float* o, float* final_state, float* snapshots,
                        void* workspace, size_t workspace_bytes, void* hip_stream);

/* kda_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture,
 * serving loops that forbid allocation, harnesses that allow none. It calls no
 * allocating routine; the work table lives in a static device array of the
 * library (1 MiB per GPU, held until the process ends).
 * Arguments and results as kda_prefill_chunked with segment_tokens = 0 (each
 * (sequence, head) chain runs in one workgroup, never segmented).
 * Limit: the call's work table must fit the 1 MiB array, which holds about
 * 23000 sequences when d_v >= d_k; with d_k = 2 d_v the zero-padded values
 * and states come from it too, so only calls of a few hundred tokens fit.
 * Beyond it: KDA_ERR_WORKSPACE, nothing enqueued.
 * Calls on one GPU share that array: two calls that overlap in time on one
 * GPU (different streams, or different host threads) race and must not be
 * issued; calls ordered on one stream are safe. KDA_ERR_DEVICE if the
 * array's device address cannot be looked up on the current device. */
int kda_prefill_chunked_noalloc(const kda_shape* shape, int32_t num_seqs,
                                const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                                int32_t chunk, int64_t snapshot_interval,
                                const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* initial_state,
                                float* o, float* final_state, float* snapshots, void* hip_stream);

/* One decode step for `batch` independent sequences (one new token each),
 * updating the fp32 state in place: O(1) work per token, one read and one
 * write of S (page "kda-graft", ailist.pro, section "2. Decode: O(1) против
 * O(L)": the step only touches the fixed-size state).
 * q, k: [batch, H, d_k]; v: [batch, H, d_v]; alpha: [batch, H] or
 * [batch, H, d_k]; beta: [batch, H]; state: [batch, H, d_v, d_k] (read and
 * overwritten); o: [batch, H, d_v]. batch == 0 is a no-op. */
int kda_decode_step(const kda_shape* shape, int32_t batch,
                    const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta,
                    float* state, float* o, void* hip_stream);

/* Several new tokens per sequence in one call -- a speculative draft, or a
 * short extension of a prompt -- with the state after every token kept for
 * rollback (page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache KV",
 * trefon.com, section "Co stan rekurencyjny zmienia przy serwowaniu", item 2:
 * once the state has absorbed draft tokens that are then rejected, the
 * engine needs the state from before them back). Each token is exactly one
 * kda_decode_step; the state stays on chip between the tokens of a call.
 * q, k: [batch, n_tok, H, d_k]; v: [batch, n_tok, H, d_v]; alpha:
 * [batch, n_tok, H] or [batch, n_tok, H, d_k]; beta: [batch, n_tok, H]
 * (token-major within each sequence, i.e. a varlen pack of equal lengths).
 * state: [batch, H, d_v, d_k], read; overwritten with the state after the
 *   first commit[b] tokens of sequence b (left untouched where that is 0).
 * o: [batch, n_tok, H, d_v], written for every token.
 * token_states: NULL, or [batch, n_tok, H, d_v, d_k]: the state after each
 *   token (16-byte aligned).
 * commit: NULL (commit all n_tok tokens), or device int32 [batch]; values
 *   are clamped to [0, n_tok]. Two ways to roll back: run the draft with
 *   commit = 0 (scores only, state unchanged) and then rerun the accepted
 *   prefix with commit = its length; or run once with token_states and keep
 *   the state of the last accepted token.
 * batch == 0 or n_tok == 0 is a no-op. Alignment as kda_decode_step;
 * commit 4 bytes. */
int kda_decode_tokens(const kda_shape* shape, int32_t batch, int32_t n_tok,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta,
                      float* state, float* o, float* token_states, const int32_t* commit,
                      void* hip_stream);

/* Front end of a KDA layer, the step between the q/k/v and gate projections
 * and the recurrence (page "kda-graft: Qwen2.5-0.5B с трансплантированным
 * KDA", ailist.pro, section "Идея и архитектура": a 4-tap convolution
 * initialised as an identity tap, the alpha gate with bias +5, beta). The page
 * gives no formulas; computed here, per sequence of the pack:
 *   q, k, v = SiLU(conv4(x)), conv4 causal and depthwise over the sequence's
 *             tokens, taps oldest first (identity = {0, 0, 0, 1}), the 3
 *             positions before its first token read conv_state_in (or 0);
 *   q, k   /= sqrt(sum over d of squares + 1e-6)   per (token, head);
 *   alpha   = sigmoid(alpha_logit + alpha_bias);  beta = sigmoid(beta_logit).
 * The outputs are laid out as kda_prefill_chunked takes them.
 * xq, xk, xv: [T, H, d] (qkv dtype; d = d_k = d_v); conv_w: fp32 [3, H, d, 4]
 * (q, k, v). conv_state_in: NULL or [num_seqs, 3, 3, H, d] (q, k, v; 3 carried
 * inputs oldest first; qkv dtype). alpha_logit: fp32 [T, H] or [T, H, d_k]
 * (gate of the shape); beta_logit: fp32 [T, H]. q, k, v: [T, H, d] (qkv
 * dtype); alpha, beta: fp32 like their logits. conv_state_out: NULL or
 * [num_seqs, 3, 3, H, d]: each sequence's last 3 conv inputs, shifted in from
 * conv_state_in when the sequence is shorter (must not alias conv_state_in).
 * Alignment: 16 bytes for every tensor except scalar-gate logits/alpha and
 * beta (4) and cu_seqlens_dev (8). q, k, v may not be any of xq, xk, xv
 * (KDA_ERR_ARG: a workgroup reads the 3 rows before its first token, which
 * another one writes). Errors as kda_prefill_chunked. */
int kda_layer_front(const kda_shape* shape, int32_t num_seqs,
                    const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                    const void* xq, const void* xk, const void* xv, const float* conv_w,
                    const void* conv_state_in, const float* alpha_logit, float alpha_bias,
                    const float* beta_logit, void* q, void* k, void* v, float* alpha, float* beta,
                    void* conv_state_out, void* hip_stream);

/* Back end of a KDA layer (same page and section: RMSNorm and the output
 * gate): out = o * rsqrt(mean over d_v of o^2 + eps) * norm_w * sigmoid(g_logit)
 * per (token, head). o, g_logit: fp32 [num_tokens, H, d_v]; norm_w: fp32 [d_v];
 * out: [num_tokens, H, d_v] in out_dtype (KDA_BF16 or KDA_F32), may alias
 * neither input. All pointers 16-byte aligned. */
int kda_layer_back(const kda_shape* shape, int64_t num_tokens, const float* o,
                   const float* g_logit, const float* norm_w, float eps, int32_t out_dtype,
                   void* out, void* hip_stream);

/* Bytes of device workspace kda_layer_prefill needs (host-only; errors as
 * kda_layer_prefill's validation). */
int kda_layer_prefill_workspace_size(const kda_shape* shape, int32_t num_seqs,
                                     const int64_t* cu_seqlens_host, int32_t chunk,
                                     int64_t snapshot_interval, int64_t segment_tokens,
                                     size_t* bytes);

/* The recurrence and the back end of a KDA layer in one call (page "kda-graft:
 * Qwen2.5-0.5B с трансплантированным KDA", ailist.pro, section "Идея и
 * архитектура": the recurrence sits between the layer's projections and its
 * norm and output gate):
 *   out = o * rsqrt(mean over d of o^2 + eps) * norm_w * sigmoid(g_logit)
 * per (token, head), o being what kda_prefill_chunked computes for the same
 * arguments. For the scalar gate with bf16 q, k, v at d = 128, when the plan
 * splits every non-empty sequence into segments (segment_tokens shorter than
 * each of them, or -1 with fewer (sequence, head) chains than compute units), the
 * last pass of the prefill applies the back end to each chunk's output tile
 * on chip and o never reaches memory. Otherwise the prefill writes an fp32 o
 * into the workspace and the back-end kernel of kda_layer_back reads it. Either
 * way out has the bits of kda_prefill_chunked followed by kda_layer_back with
 * g_logit widened to fp32.
 * Arguments as kda_prefill_chunked (final_state, snapshots and their rules
 * included), with d_k = d_v (KDA_ERR_SHAPE otherwise) and
 *   g_logit: [T, H, d] in the qkv dtype; norm_w: fp32 [d]; eps >= 0;
 *   out: [T, H, d] in out_dtype (KDA_BF16 or KDA_F32), overlapping no input;
 *   workspace: at least kda_layer_prefill_workspace_size bytes.
 * Alignment: g_logit, norm_w and out 16 bytes. */
int kda_layer_prefill(const kda_shape* shape, int32_t num_seqs,
                      const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                      int32_t chunk, int64_t snapshot_interval, int64_t segment_tokens,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const float* initial_state,
                      const void* g_logit, const float* norm_w, float eps, int32_t out_dtype,
                      void* out, float* final_state, float* snapshots,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes of kda_prefill_backward for this packing (device memory,
 * caller-owned, 16-byte aligned). It holds the recomputed forward (its states
 * after every 64 tokens) and about 1 MB per (chunk, head) at d = 128
 * (0.3 MB at d = 64) of intermediate fp32 arrays. Heads are independent, so
 * when that would exceed 96 GiB the backward runs the heads in the fewest
 * equal groups that fit (each group's inputs gathered into the workspace and
 * its gradients scattered back); the environment variable
 * KDA_BACKWARD_BUDGET_BYTES, read at every call, replaces the 96 GiB. */
int kda_prefill_backward_workspace_size(const kda_shape* shape, int32_t num_seqs,
                                        const int64_t* cu_seqlens_host, size_t* bytes);

/* Backward pass of kda_prefill_chunked: the gradients of the loss
 *   sum_t <d_o_t, o_t> + sum_n <d_final_state_n, S_final_n>
 * with respect to q, k, v, alpha, beta and the initial state, for the update
 * of page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache KV"
 * (trefon.com), section "Gated DeltaNet: dodaj zanik", differentiated through
 * the chunked form (closing paragraph of "Co stan rekurencyjny zmienia przy
 * serwowaniu"). The forward is recomputed inside (states every 64 tokens);
 * the gradients of each chunk are dense fp32 products, and the gradient of
 * the state runs over the chunks of each sequence in reverse.
 * Inputs as kda_prefill_chunked (q, k, v, alpha, beta, initial_state or NULL,
 * cu_seqlens on host and device). d_o: fp32 [T, H, d_v]. d_final_state: fp32
 * [num_seqs, H, d_v, d_k] or NULL (zero). Outputs, all fp32: dq, dk [T, H, d_k],
 * dv [T, H, d_v], dalpha shaped like alpha, dbeta [T, H], d_initial_state
 * [num_seqs, H, d_v, d_k] or NULL (not wanted). Outputs must not overlap the
 * inputs, except that d_initial_state may be d_final_state.
 * Alignment: q, k, v, per-key alpha and dalpha, initial_state,
 * d_final_state, dq, dk, dv, d_initial_state and workspace 16 bytes; the
 * rest 4 (cu_seqlens_dev 8).
 * Precondition (beyond kda_prefill_chunked's): within each 64-token chunk the
 * decay over any 32 consecutive tokens is at least 2^-120 per channel, so the
 * decay factors relative to the chunk's middle row stay inside fp32.
 * Errors as kda_prefill_chunked; KDA_ERR_WORKSPACE if workspace_bytes is below
 * kda_prefill_backward_workspace_size. num_seqs == 0 is a no-op.
 * d_initial_state may be the d_final_state buffer (it is written after every
 * read of d_final_state); no other output may overlap an input. */
int kda_prefill_backward(const kda_shape* shape, int32_t num_seqs,
                         const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const float* initial_state,
                         const float* d_o, const float* d_final_state,
                         float* dq, float* dk, float* dv, float* dalpha, float* dbeta,
                         float* d_initial_state, void* workspace, size_t workspace_bytes,
                         void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
